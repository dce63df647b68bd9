// QSA top-k block selection for gfx950.
//
// "[Kernel][SM70] Accelerate exact Qwen3.8 decode", Implementation: the
// selection finds the k highest block scores with radix passes over the score
// keys (four 8-bit digit passes) and resolves ties at the pivot score by
// keeping the lowest block indices.  The result is exact: for each row, the
// kept set is the first k blocks in (score descending, index ascending) order,
// reported in increasing index order.
//
// Keys.  A score's fp32 bit pattern u becomes the unsigned key
// u ^ (sign ? 0xFFFFFFFF : 0x80000000), which orders scores like IEEE 754
// totalOrder (-NaN < -inf < ... < -0 < +0 < ... < +inf < +NaN).
//
// One workgroup of 1024 threads (16 waves) works on one row at a time; with
// one workgroup per compute unit, workgroup w takes rows w, w + G, ... (G
// workgroups).  Thread t holds elements j = 4096 i + 4 t + c (register slot
// i, component c) as raw fp32 bits in VGPRs, so a row of up to 65,536 blocks
// is read from HBM once, with 16-byte coalesced non-temporal loads.
// Elements past the row's length hold -inf.  The first half of the next row is loaded into
// the registers the candidate pass frees, slot by slot as it goes, and is in
// flight while the current row is in phases 3-5, which need only LDS.
//   1. Threshold T (rows longer than 4096 blocks, k <= 1024): each lane's
//      maximum in key order (from max/min of the signed raw bits), then each
//      wave's ceil(k/16)-th largest lane maximum with its low 16 bits
//      cleared, by a 16-step ballot bisection over the high bits, and T =
//      the minimum over the 16 waves.  Every lane holds a full first slot,
//      so every lane maximum is an eligible block and at least k keys are
//      >= T (the cleared bits only lower it, by under 1% of its value for
//      normal floats).  Shorter rows take every eligible block.
//   2. Candidates: blocks that are not below T as floats (a superset of the
//      keys >= T) are appended, in one pass, to their wave's LDS region as
//      (raw bits, block index) by ballot and mbcnt.  About 1.5% of a row of
//      independent scores when k is 1/128 of the row.  Each region has one
//      step of slack past the 256 candidates a wave may hold, and stores
//      start at the wave's scalar count clamped to 256, so no lane's store
//      needs a bounds check of its own; a count above 256 is an overflow
//      (phase 3 then takes the exact passes).
//   3. Pivot P, the k-th largest key: MSB-first 8-bit histogram passes over
//      the candidates with key >= T, skipping the leading bytes that T and the
//      row's largest key share (all such candidates share them).  Every wave
//      adds its own region to the shared bins and scans the 256 bins itself,
//      so a pass costs one barrier; three histogram buffers rotate.  `need`
//      is how many keys equal to P are kept, `eq` how many there are.  The
//      first pass checks that at least k candidates reach T and that no
//      region overflowed; otherwise (adversarial inputs) four exact passes
//      run over the whole row, re-read from memory.
//   4. Kept blocks (key > P, or key >= P when every tie is kept) are marked in
//      an LDS bitmap from the candidates; when eq > need the tied blocks go to
//      a second bitmap of which a block-wide popcount scan keeps the first
//      `need` in index order.  After the exact fallback the bitmaps come from
//      a re-read of the row.
//   5. Ordered output: thread t owns bitmap words 2t and 2t+1 (blocks 64t ..
//      64t+63); a block-wide exclusive scan of their popcounts gives each
//      thread its first output position, and it writes its blocks in order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "launch_util.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kThreads = kTopkThreads;
constexpr int kWaves = kThreads / 64;
constexpr int kSlotElems = 4 * kThreads;    // elements one register slot covers
constexpr int kRegion = 256;                  // candidates a wave may hold
constexpr int kRegionStride = kRegion + 64;   // its LDS region: one step of slack
constexpr int kCandCap = kWaves * kRegionStride;  // LDS candidates (raw bits, block index)
constexpr int kThreshMin = kSlotElems;      // rows longer than this use a threshold
constexpr int kBmWords = kTopkMaxBlocks / 32;
constexpr uint32_t kNegInfBits = 0xFF800000u;
static_assert(kBmWords == 2 * kThreads, "each thread owns two bitmap words");

struct TopkShared {
  uint2 cand[kCandCap];       // (raw score bits, block index)
  uint32_t keep[kBmWords];    // bit j: block j is kept
  uint32_t tied[kBmWords];    // bit j: block j's key equals the pivot (eq > need only)
  uint32_t hist[3][256];
  uint32_t twave[kWaves];
  uint32_t tmax[kWaves];
  uint32_t wsum[2][kWaves];
  uint32_t wcnt[kWaves];      // candidates per wave region
};

__device__ __forceinline__ uint32_t key_of_bits(uint32_t u) {
  return u ^ (static_cast<uint32_t>(static_cast<int32_t>(u) >> 31) | 0x80000000u);
}
__device__ __forceinline__ uint32_t bits_of_key(uint32_t k) {
  return (k & 0x80000000u) ? (k ^ 0x80000000u) : ~k;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// 16 bytes of scores, loaded with the non-temporal hint: each score is read
// once (the exact fallback's re-read aside), so the row streams past the
// caches instead of displacing what the other rows' waves still use.
typedef uint32_t u4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_scores16(const float* a) {
  const u4v v = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(a));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Inclusive prefix sum across the 64 lanes of a wave with DPP: a
// Hillis-Steele scan inside each 16-lane row (row_shr 1, 2, 4, 8), then the
// row totals carried across rows (row_bcast 15 into rows 1 and 3, row_bcast 31
// into rows 2 and 3).  Lanes without a source lane add 0.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

// Maximum across the 64 lanes of a wave (same DPP pattern as the scan; lanes
// without a source lane see 0, the identity for unsigned max).
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, false)));
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, false)));
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, false)));
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, false)));
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0u, x, 0x142, 0xA, 0xF, false)));
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0u, x, 0x143, 0xC, 0xF, false)));
  return __builtin_amdgcn_readlane(x, 63);
}

// Exclusive prefix sum over the workgroup in thread order.  Contains a
// barrier; `wsum` must not be in use by another scan in flight.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t c, uint32_t* wsum) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t incl = wave_incl_scan(c);
  if (lane_id() == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t base = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) base += w < wave ? wsum[w] : 0u;
  return base + incl - c;
}

// The m-th largest (1 <= m <= 64) of the wave's 64 lane values, by bisection
// on the bits from the top: at bit b, c lanes agree with the answer so far
// and have bit b set; the answer has bit b set iff c >= m.  With LOW > 0
// the bisection stops there: the m-th largest with its bits below LOW
// cleared, a lower bound that at least m lanes reach.
template <int LOW = 0>
__device__ __forceinline__ uint32_t wave_mth_largest(uint32_t x, uint32_t m) {
  uint32_t res = 0;
#pragma unroll
  for (int b = 31; b >= LOW; --b) {
    const uint32_t trial = res | (1u << b);
    const uint32_t c = static_cast<uint32_t>(__popcll(__ballot((x >> b) == (trial >> b))));
    if (c >= m)
      res = trial;
    else
      m -= c;
  }
  return res;
}

// Number of set bits of `mask` in lanes below this one.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

struct Digit {
  uint32_t digit;    // bin holding the rem-th largest key
  uint32_t above;    // keys in higher bins
  uint32_t in_bin;   // keys in that bin
  uint32_t total;    // keys in all bins
};

// Every wave reads the 256 bins (lane l: bins 255-4l .. 252-4l) and finds the
// bin holding the rem-th largest key, scanning from the top.  If the bins
// hold fewer than rem keys, digit and above are 0.
__device__ __forceinline__ Digit find_digit(const uint32_t* hist, uint32_t rem) {
  const int lane = lane_id();
  const uint4 v = *reinterpret_cast<const uint4*>(&hist[252 - 4 * lane]);
  const uint32_t h[4] = {v.w, v.z, v.y, v.x};
  const uint32_t s = h[0] + h[1] + h[2] + h[3];
  const uint32_t incl = wave_incl_scan(s);
  uint32_t c = incl - s;
  bool found = false;
  uint32_t fd = 0, fc = 0, fh = 0;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    if (!found && c < rem && rem <= c + h[m]) {
      found = true;
      fd = 255 - 4 * lane - m;
      fc = c;
      fh = h[m];
    }
    c += h[m];
  }
  const uint64_t fm = __ballot(found);
  Digit r;
  r.total = __builtin_amdgcn_readlane(incl, 63);
  if (fm == 0) {
    r.digit = r.above = r.in_bin = 0;
  } else {
    const int src = __ffsll(static_cast<unsigned long long>(fm)) - 1;
    r.digit = __builtin_amdgcn_readlane(fd, src);
    r.above = __builtin_amdgcn_readlane(fc, src);
    r.in_bin = __builtin_amdgcn_readlane(fh, src);
  }
  return r;
}

struct Pivot {
  uint32_t key;   // the k-th largest key
  uint32_t need;  // keys equal to `key` among the first k
  uint32_t eq;    // keys equal to `key` in the whole multiset
  bool ok;        // the first pass saw at least k keys (and `accept` held)
};

// Block-wide pivot search: the k-th largest key of the multiset the visitor
// enumerates (visit(f) calls f(act, key) with whole waves), four 8-bit
// passes, one barrier each.  Requires hist[0] and hist[1] zeroed before a
// barrier.  Used by the exact fallback over a whole row.
template <class Visit>
__device__ __forceinline__ Pivot pivot_block(TopkShared& sh, uint32_t k, Visit visit) {
  uint32_t prefix = 0, rem = k;
  Pivot pv{0, 0, 0, true};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int shift = 24 - 8 * q;
    const uint32_t hi_mask = q == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
    uint32_t* hist = sh.hist[q % 3];
    visit([&](bool act, uint32_t key) {
      if (act && ((key ^ prefix) & hi_mask) == 0) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    });
    __syncthreads();
    // Zero the buffer of pass q + 2: every wave finished reading it (pass
    // q - 1) before this barrier, and pass q + 2 adds to it only after the
    // next one.
    if (threadIdx.x < 256) sh.hist[(q + 2) % 3][threadIdx.x] = 0;
    const Digit d = find_digit(hist, rem);
    prefix |= d.digit << shift;
    rem -= d.above;
    pv.eq = d.in_bin;
  }
  pv.key = prefix;
  pv.need = rem;
  return pv;
}

// Block-wide pivot search over the per-wave candidate regions (keys >= T
// count; all of them share the top `first` bytes of T): every wave
// histograms its own region into the shared bins, one barrier per 8-bit
// pass, and every wave finds the digit itself.  Three histogram buffers
// rotate (all three zeroed before the first barrier of the call).  ok is
// false, for every wave alike, if a region overflowed or fewer than k keys
// reach T.
__device__ __forceinline__ Pivot pivot_regions(TopkShared& sh, uint32_t k, uint32_t T, int first,
                                               const uint2* region, uint32_t used) {
  const int lane = lane_id();
  bool overflow = false;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) overflow |= sh.wcnt[w] > static_cast<uint32_t>(kRegion);
  Pivot pv{0, 0, 0, true};
  uint32_t prefix = first == 0 ? 0u : (T & (0xFFFFFFFFu << (32 - 8 * first)));
  uint32_t rem = k;
  for (int q = first; q < 4; ++q) {
    const int shift = 24 - 8 * q;
    const uint32_t hi_mask = q == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
    uint32_t* hist = sh.hist[q % 3];
    for (uint32_t b = 0; b < used; b += 64) {
      const uint32_t e = b + lane;
      const uint32_t key = key_of_bits(e < used ? region[e].x : 0u);
      if (e < used && key >= T && ((key ^ prefix) & hi_mask) == 0)
        atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    // Zero the buffer of pass q + 2: every wave finished reading it (pass
    // q - 1) before this barrier, and pass q + 2 adds to it only after the
    // next one.
    if (threadIdx.x < 256) sh.hist[(q + 2) % 3][threadIdx.x] = 0;
    const Digit d = find_digit(hist, rem);
    if (q == first && (d.total < k || overflow)) {
      pv.ok = false;
      return pv;
    }
    prefix |= d.digit << shift;
    rem -= d.above;
    pv.eq = d.in_bin;
  }
  pv.key = prefix;
  pv.need = rem;
  return pv;
}

// Phases 3-5 of one row, once the candidates are in the wave regions:
// pivot, bitmaps, ordered output (and the exact fallback over the row in
// memory when the candidate pass cannot decide).
__device__ __forceinline__ void finish_row(TopkShared& sh, const TopkParams& p, int row,
                                           int32_t k, int32_t nv, int tid, int lane, uint32_t T,
                                           uint32_t top, bool float_cand, const uint2* region,
                                           uint32_t used, const float* src, int32_t* out) {
  // ---- 3. the pivot over the candidates with key >= T (all waves, each
  // over its own region).  Candidates with key in [T, top] share the leading
  // bytes of T and top.
  const uint32_t kk = static_cast<uint32_t>(k);
  int first = 0;
  if (float_cand) {
    const uint32_t diff = T ^ top;
    first = diff == 0 ? 3 : (__clz(diff) >> 3);
  }
  Pivot pv = pivot_regions(sh, kk, T, first, region, used);
  const bool fast_pivot = pv.ok;
  if (!fast_pivot) {
    // Exact passes over the whole row, re-read from memory, once every wave
    // has left the candidate passes.
    __syncthreads();
    if (tid < 256) {
      sh.hist[0][tid] = 0;
      sh.hist[1][tid] = 0;
    }
    __syncthreads();
    pv = pivot_block(sh, kk, [&](auto f) {
      for (int32_t b = 0; b < nv; b += kThreads) {
        const int32_t j = b + tid;
        f(j < nv, j < nv ? key_of_bits(__float_as_uint(src[j])) : 0u);
      }
    });
  }
  const uint32_t P = pv.key;
  const bool split_ties = pv.eq != pv.need;  // only some of the pivot's ties are kept

  // ---- 4. bitmaps of kept and (when only some are kept) tied blocks.
  auto mark = [&](uint32_t key, uint32_t j) {
    const uint32_t bit = 1u << (j & 31);
    if (split_ties ? key > P : key >= P) atomicOr(&sh.keep[j >> 5], bit);
    if (split_ties && key == P) atomicOr(&sh.tied[j >> 5], bit);
  };
  if (fast_pivot) {
    // Every block with key >= P >= T is a candidate.
    for (uint32_t b = 0; b < used; b += 64) {
      const uint32_t e = b + lane;
      if (e < used) {
        const uint2 cj = region[e];
        mark(key_of_bits(cj.x), cj.y);
      }
    }
  } else {
    for (int32_t b = 0; b < nv; b += kThreads) {
      const int32_t j = b + tid;
      if (j < nv) mark(key_of_bits(__float_as_uint(src[j])), static_cast<uint32_t>(j));
    }
  }
  __syncthreads();
  uint32_t w0 = sh.keep[2 * tid];
  uint32_t w1 = sh.keep[2 * tid + 1];
  if (split_ties) {
    // Keep the first `need` tied blocks in index order.
    uint32_t q0 = sh.tied[2 * tid];
    uint32_t q1 = sh.tied[2 * tid + 1];
    const uint32_t qc = __popc(q0) + __popc(q1);
    const uint32_t before = block_excl_scan(qc, sh.wsum[0]);
    uint32_t take = before < pv.need ? pv.need - before : 0u;
    while (take > 0 && q0) {
      w0 |= q0 & (0u - q0);
      q0 &= q0 - 1u;
      --take;
    }
    while (take > 0 && q1) {
      w1 |= q1 & (0u - q1);
      q1 &= q1 - 1u;
      --take;
    }
  }

  // ---- 5. ordered output of blocks 64 tid .. 64 tid + 63.
  uint32_t pos = block_excl_scan(__popc(w0) + __popc(w1), sh.wsum[1]);
  while (w0) {
    const int b = __ffs(w0) - 1;
    if (pos < kk) out[pos] = 64 * tid + b;
    ++pos;
    w0 &= w0 - 1u;
  }
  while (w1) {
    const int b = __ffs(w1) - 1;
    if (pos < kk) out[pos] = 64 * tid + 32 + b;
    ++pos;
    w1 &= w1 - 1u;
  }
  if (tid == 0 && p.out_count) p.out_count[row] = k;
}

// Row r's eligible length n_valid[r] clamped to [0, n_blocks].
__device__ __forceinline__ int32_t row_valid(const TopkParams& p, int row) {
  const int32_t nv = p.n_valid ? p.n_valid[row] : p.n_blocks;
  return nv < 0 ? 0 : (nv > p.n_blocks ? p.n_blocks : nv);
}

// Loads register slots I0 .. I1 - 1 of row `row` into x: element (i, c) of
// this thread is j = 4096 i + 4 tid + c, valid when j < nv.  Invalid elements
// hold -inf.
template <int ITEMS, bool VEC, int I0, int I1>
__device__ __forceinline__ void load_row(uint32_t (&x)[ITEMS][4], const TopkParams& p, int row,
                                         int32_t nv, uint32_t skip = 0) {
  const int tid = threadIdx.x;
  const float* src = p.scores + static_cast<int64_t>(row) * p.row_stride;
  const int32_t lim = nv - 4 * tid;
#pragma unroll
  for (int i = I0; i < I1; ++i) {
    if ((skip >> i) & 1u) continue;  // already loaded
#pragma unroll
    for (int c = 0; c < 4; ++c) x[i][c] = kNegInfBits;
    if (i * kSlotElems < nv) {
      if (VEC) {
        if (i * kSlotElems < lim) {
          const uint4 v = load_scores16(src + i * kSlotElems + 4 * tid);
          x[i][0] = v.x;
          if ((i + 1) * kSlotElems <= nv) {  // the whole slot is eligible
            x[i][1] = v.y;
            x[i][2] = v.z;
            x[i][3] = v.w;
          } else {
            x[i][1] = i * kSlotElems + 1 < lim ? v.y : kNegInfBits;
            x[i][2] = i * kSlotElems + 2 < lim ? v.z : kNegInfBits;
            x[i][3] = i * kSlotElems + 3 < lim ? v.w : kNegInfBits;
          }
        }
      } else {
        // Uniform per-slot base, one lane offset for every slot; loads are
        // unconditional (clamped into the row in the partial slot).
        const uint32_t* sb = reinterpret_cast<const uint32_t*>(src) + i * kSlotElems;
        if ((i + 1) * kSlotElems <= nv) {
#pragma unroll
          for (int c = 0; c < 4; ++c) x[i][c] = sb[4 * tid + c];
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const bool ok = i * kSlotElems + c < lim;
            const uint32_t v = sb[ok ? 4 * tid + c : 0];
            x[i][c] = ok ? v : kNegInfBits;
          }
        }
      }
    }
  }
}

// Issues the loads of register slot i of a row whose slot is wholly
// eligible ((i + 1) * 4096 <= nv): plain loads, no selects after them, so
// no wait follows.
template <bool VEC>
__device__ __forceinline__ void issue_full_slot(uint32_t (&xi)[4], const float* src, int i,
                                                int tid) {
  if (VEC) {
    const uint4 v = load_scores16(src + i * kSlotElems + 4 * tid);
    xi[0] = v.x;
    xi[1] = v.y;
    xi[2] = v.z;
    xi[3] = v.w;
  } else {
    const uint32_t* sb = reinterpret_cast<const uint32_t*>(src) + i * kSlotElems;
#pragma unroll
    for (int c = 0; c < 4; ++c) xi[c] = sb[4 * tid + c];
  }
}

// Workgroup w takes rows w, w + G, w + 2G, ... (G = gridDim.x).  A row's
// scores are needed in registers only up to the candidate pass: as that pass
// finishes with slot i (i < kPre), slot i of the next row is loaded into its
// registers, so those loads are issued spread through the pass (not in one
// burst after it, which stalls the issuing waves at the address unit) and
// are in flight while this row's pivot, bitmaps and output run on LDS (all
// slots in flight there would exceed the 128 registers a 16-wave workgroup
// has); the next row's other slots are loaded when that row starts.
template <int ITEMS, bool VEC>
__global__ __launch_bounds__(kThreads) void topk_kernel(TopkParams p) {
  constexpr int kPre = ITEMS > 1 ? ITEMS / 2 : ITEMS;
  __shared__ TopkShared sh;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t k = p.k;
  int row = blockIdx.x;
  int32_t nv = row_valid(p, row);
  uint32_t x[ITEMS][4];
  if (nv > k && k > 0) load_row<ITEMS, VEC, 0, kPre>(x, p, row, nv);
  for (; row < p.rows; row += gridDim.x) {
  // An opaque copy of the thread index per row: index arithmetic derived
  // from it is recomputed in each row instead of being hoisted out of the
  // loop and held in registers (spilled) across rows.
  int tid_row = static_cast<int>(threadIdx.x);
  asm volatile("" : "+v"(tid_row));
  const int tid = tid_row;
  const int next = row + static_cast<int>(gridDim.x);
  const int32_t nv_next = next < p.rows ? row_valid(p, next) : 0;
  const bool load_next = next < p.rows && nv_next > k && k > 0;
  int32_t* out = p.out_idx + static_cast<int64_t>(row) * k;
  const float* src = p.scores + static_cast<int64_t>(row) * p.row_stride;
  const int32_t lim = nv - 4 * tid;

  if (nv <= k || k == 0) {  // every eligible block is kept (none when k = 0)
    for (int j = tid; j < k; j += kThreads) out[j] = j < nv ? j : -1;
    if (tid == 0 && p.out_count) p.out_count[row] = nv <= k ? nv : 0;
    if (load_next) load_row<ITEMS, VEC, 0, kPre>(x, p, next, nv_next);
    nv = nv_next;
    continue;
  }
  load_row<ITEMS, VEC, kPre, ITEMS>(x, p, row, nv);
  // Slots of the next row loaded during this row's candidate pass: the
  // wholly eligible ones among the first kPre.
  const float* src_next = p.scores + static_cast<int64_t>(next) * p.row_stride;
  uint32_t pre_next = 0;
  if (load_next) {
    const int full = nv_next / kSlotElems;
    pre_next = (1u << (full < kPre ? full : kPre)) - 1u;
  }

  // Shared state for the phases below.
  if (tid < 256) {
    sh.hist[0][tid] = 0;
    sh.hist[1][tid] = 0;
    sh.hist[2][tid] = 0;
  }
  sh.keep[2 * tid] = 0;
  sh.keep[2 * tid + 1] = 0;
  sh.tied[2 * tid] = 0;
  sh.tied[2 * tid + 1] = 0;


  // ---- 1. threshold.  Rows longer than one slot give every thread a full
  // first slot, so every lane maximum is an eligible block.  The lane maximum
  // in key order: the largest signed raw value if any is non-negative, else
  // the smallest (the negative score closest to zero).
  const bool thresh = nv > kThreshMin && k <= kThreads;
  if (thresh) {
    int32_t mx = INT32_MIN, mn = INT32_MAX;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int32_t v = static_cast<int32_t>(x[i][c]);
        mx = v > mx ? v : mx;
        mn = v < mn ? v : mn;
      }
    const uint32_t lane_max = key_of_bits(static_cast<uint32_t>(mx >= 0 ? mx : mn));
    const uint32_t t_w =
        wave_mth_largest<16>(lane_max, (static_cast<uint32_t>(k) + kWaves - 1) / kWaves);
    const uint32_t m_w = wave_max(lane_max);
    if (lane == 0) {
      sh.twave[wave] = t_w;
      sh.tmax[wave] = m_w;
    }
  }
  __syncthreads();
  uint32_t T = 0, top = 0xFFFFFFFFu;
  if (thresh) {
    T = 0xFFFFFFFFu;
    top = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      T = sh.twave[w] < T ? sh.twave[w] : T;
      top = sh.tmax[w] > top ? sh.tmax[w] : top;
    }
    T = __builtin_amdgcn_readfirstlane(T);
    top = __builtin_amdgcn_readfirstlane(top);
  }
  // A float test against T is a superset of the keys >= T (it also lets
  // negative NaNs through) as long as T is a number above -inf, which keeps
  // the -inf fillers out.
  const bool float_cand = thresh && T >= 0x00800000u && T <= 0xFF800000u;

  // ---- 2. candidates into this wave's region: (raw bits, block index).
  uint32_t cnt = 0;  // this wave's candidates (wave-uniform)
  auto append = [&](auto by_float) {
    constexpr bool kFloat = decltype(by_float)::value;
    uint2* region = sh.cand + kRegionStride * wave;
    const float tf = __uint_as_float(bits_of_key(T));
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      if (i * kSlotElems < nv) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const bool cand = kFloat ? !(__uint_as_float(x[i][c]) < tf) : (i * kSlotElems + c < lim);
          const uint64_t m = __ballot(cand);
          if (m) {
            // The base is clamped at kRegion, so a step's 64 entries always
            // land inside the region's slack; a step can start past kRegion
            // only once the count already exceeds it, which marks the wave
            // overflowed.
            const uint32_t base = min(cnt, static_cast<uint32_t>(kRegion));
            if (cand)
              (region + base)[lanes_below(m)] =
                  make_uint2(x[i][c], static_cast<uint32_t>(i * kSlotElems + 4 * tid + c));
            cnt += static_cast<uint32_t>(__popcll(m));
          }
        }
      }
      // Slot i is consumed.  If slot i of the next row is wholly eligible
      // and among the first kPre, it is loaded into these registers now, so
      // the next row's loads are spread through this pass.
      if ((pre_next >> i) & 1u) issue_full_slot<VEC>(x[i], src_next, i, tid);
    }
  };
  if (float_cand)
    append(std::true_type{});
  else
    append(std::false_type{});
  cnt = __builtin_amdgcn_readfirstlane(cnt);
  if (lane == 0) sh.wcnt[wave] = cnt;
  const uint32_t used = cnt < static_cast<uint32_t>(kRegion) ? cnt : kRegion;
  const uint2* region = sh.cand + kRegionStride * wave;
  __syncthreads();
  // The next row's first kPre slots that are not wholly eligible (loaded
  // with their masks) once this row's scores are no longer needed.
  if (load_next) load_row<ITEMS, VEC, 0, kPre>(x, p, next, nv_next, pre_next);

  finish_row(sh, p, row, k, nv, tid, lane, T, top, float_cand, region, used, src, out);
  nv = nv_next;
  // Every thread has read this row's bitmaps before the next row clears them.
  __syncthreads();
  }
}

template <int ITEMS>
hipError_t launch_items(const TopkParams& p, bool vec, hipStream_t stream) {
  // One workgroup per compute unit (16 waves of up to 128 VGPRs: one fits),
  // each walking its rows.
  const dim3 grid(static_cast<unsigned>(p.rows < p.grid ? p.rows : p.grid));
  if (vec) return pgqa_launch::launch(topk_kernel<ITEMS, true>, grid, dim3(kThreads), 0, stream, p);
  return pgqa_launch::launch(topk_kernel<ITEMS, false>, grid, dim3(kThreads), 0, stream, p);
}

}  // namespace

hipError_t launch_topk(const TopkParams& p, bool vec, hipStream_t stream) {
  if (p.rows <= 0) return hipSuccess;
  const int64_t slots = (static_cast<int64_t>(p.n_blocks) + kSlotElems - 1) / kSlotElems;
  if (slots <= 1) return launch_items<1>(p, vec, stream);
  if (slots <= 2) return launch_items<2>(p, vec, stream);
  if (slots <= 4) return launch_items<4>(p, vec, stream);
  if (slots <= 8) return launch_items<8>(p, vec, stream);
  return launch_items<16>(p, vec, stream);
}

}  // namespace qsa
