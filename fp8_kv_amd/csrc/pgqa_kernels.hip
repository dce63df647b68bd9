// gfx950 kernels for paged grouped-query attention over an FP16 or FP8-E4M3
// KV pool (decode batches and sparse prefill rows share the same kernel).
//
// Sources, by page title and section:
//   "[Kernel][SM70] Scale NVFP4 E4M3 decode batches", Purpose: GQA-6, D256
//     paged decode with FP8-E4M3 KV, paired (wide) KV loads, long-context
//     routes.  Here: 16-byte loads that read whole K/V rows per instruction,
//     and key-range splits merged by log-sum-exp for long contexts.
//   "[Kernel][SM70] Accelerate Qwen3.8 QSA paged prefill", Changes: virtual
//     page-4 tables, contiguous or interleaved strides without copies, rows
//     clamped to their live length, invalid rows inert, page ids of a tile
//     staged ahead of its loads.
//
// Work decomposition.  One workgroup of NW (kWavesPerWg) waves owns one (sequence or row
// b, kv head g, split s): the tokens [s*chunk, min((s+1)*chunk, L_b)).  Wave
// w takes the 16-token tiles w, w+4, w+8, ... of that range and keeps its own
// online-softmax state; the four states are merged through LDS at the end.
// In a whole call with unequal lengths the n*S workgroups of a kv head are
// re-dealt by length (the balanced plan below), so short sequences leave no
// workgroup idle.  With one split and many rows the decomposition is one
// (row, kv head) per wave instead (RW): each wave walks all of its row's
// tiles and stores its output itself, with no merge through LDS.
// With one split the workgroup writes the fp16 output; with several it writes
// a normalised fp32 partial and its base-2 log-sum-exp, merged by merge_kernel
// in a second launch (a kernel boundary makes the partials visible; fencing
// them from inside the first kernel writes back the whole L2 of an XCD per
// workgroup and costs far more).
//
// Per tile (lane = 16*qd + r, r = lane % 16, qd = lane / 16):
//   QK^T on MFMA 16x16x32 f16: M = the 16 tokens (A = K rows, lane r holds
//     token r), N = the query heads of the group padded to 16 (B = q^T, zero
//     for heads >= group), K = head dim in 8 steps of 32.  The head dim is
//     contracted in a permuted order that lets lane (r, qd) read four
//     16-byte pieces of token r's row, so one load instruction covers whole
//     64-byte runs of 16 rows.  Output: lane (r, qd) holds the logits of head
//     r for tokens 4qd .. 4qd+3.
//   Online softmax in the log2 domain on those 4 logits per lane; the row max
//     needs only two cross-lane steps (lanes r, r+16, r+32, r+48).
//   PV on MFMA 16x16x16 f16: M = 16 head-dim slots, N = heads, K = the 16
//     tokens.  The probabilities are already in B-operand layout (lane (r,qd)
//     = head r, tokens 4qd..4qd+3).  The A operand (V^T) wants 4 tokens of
//     one dim per lane; lane (r, qd) loads 16 contiguous bytes of each of the
//     tokens 4qd..4qd+3 (so one instruction reads 4 whole rows) and the 16
//     MFMAs take the dims of those bytes in turn; a byte permute per pair of
//     tokens builds each operand.  Output dim d of MFMA j, slot m is
//     16*m + j (FP8) or 128*(j/8) + 8*m + j%8 (FP16).
#include <type_traits>

#include "launch_util.h"
#include "pgqa_internal.h"

namespace pgqa {
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

constexpr int kLdsRow = kHeadDim + 4;  // padded fp32 row of the merge buffer

// Tile buffers per wave (tiles in flight while one is computed: depth - 1).
// Depth 3 was measured slower at every length (more VGPRs, fewer waves in
// flight per CU), as were 8-wave workgroups.
constexpr int kPipelineDepth = 2;
// Tiles by which page-table entries are loaded ahead of their K/V loads.
constexpr int kPageLookahead = 1;

// ------------------------------------------------------------ ragged balance
// A whole decode call over sequences of unequal length spreads the live tokens
// of each kv head evenly over its n*S workgroup slots.  All sequences share one
// chunk length c = m*A (A = the split granularity, a power of two): the
// smallest with sum_b ceil(L_b / c) <= n*S.  Sequence b then owns the
// ceil(L_b / c) consecutive chunk indices after those of sequences 0..b-1,
// and chunk index J is stored in partial slot (J / S, J % S), i.e. where the
// static plan keeps split J % S of sequence J / S.  When every L_b equals
// max_len the plan is the static one (sequence b owns J = b*S .. b*S + S-1),
// which both kernels detect before any division.
//
// Lengths live in registers of one wave: lane l holds sequences t*64 + l for
// t < ceil(n / 64); every wave that needs the plan computes it itself.
constexpr int kBalancePer = kBalanceMaxSeqs / 64;

// Inclusive prefix sum over the 64 lanes (DPP row shifts, then the two row
// broadcasts that carry rows 0 and 0..1 into the rows above them).
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

__device__ __forceinline__ int wave_sum(int x) {
  return __builtin_amdgcn_readlane(wave_incl_scan(x), 63);
}

struct Balance {
  int L[kBalancePer];  // clamped lengths (0 past n)
  int u[kBalancePer];  // the same in units of A, rounded up
  int rows;            // ceil(n / 64)
  bool full;           // every L_b == max_len: the static plan
};

// Issue the loads of the raw lengths (kept apart from balance_finish so they
// overlap other loads).
// n >= 1.  Lanes past n re-read the last length (balance_finish ignores
// them), so the first row is one unconditional load.
__device__ __forceinline__ void balance_load(int (&raw)[kBalancePer], const int32_t* lens, int n,
                                             int lane) {
  raw[0] = lens[min(lane, n - 1)];
#pragma unroll
  for (int t = 1; t < kBalancePer; ++t) {
    raw[t] = 0;
    if (t * 64 < n) raw[t] = lens[min(t * 64 + lane, n - 1)];
  }
}

__device__ __forceinline__ Balance balance_finish(const int (&raw)[kBalancePer], int n,
                                                  int max_len, int a_shift, int lane) {
  Balance B;
  B.rows = (n + 63) >> 6;
  bool short_seq = false;
#pragma unroll
  for (int t = 0; t < kBalancePer; ++t) {
    B.L[t] = 0;
    B.u[t] = 0;
    if (t < B.rows) {  // rows past the first only wait for their own loads when they exist
      const bool in = t * 64 + lane < n;
      const int L = in ? max(0, min(raw[t], max_len)) : 0;
      B.L[t] = L;
      B.u[t] = (L + (1 << a_shift) - 1) >> a_shift;
      short_seq |= in & (L != max_len);
    }
  }
  B.full = __ballot(short_seq) == 0;
  return B;
}

// The chunk length in units of A (0 when no sequence has a live token).
// ceil(U / slots) <= m <= ceil(U / (slots - nonempty)) bounds the search:
// sum_b ceil(u_b / m) < U/m + nonempty, so the upper end always fits.
// Requires slots > n (S >= 2).
__device__ __forceinline__ int balance_units(const Balance& B, int slots) {
  int su = 0, sne = 0;
#pragma unroll
  for (int t = 0; t < kBalancePer; ++t)
    if (t < B.rows) {
      su += B.u[t];
      sne += B.u[t] > 0 ? 1 : 0;
    }
  const int U = wave_sum(su);
  const int nne = wave_sum(sne);
  if (U == 0) return 0;
  int lo = max(1, (U + slots - 1) / slots);
  int hi = (U + (slots - nne) - 1) / (slots - nne);
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    int c = 0;
#pragma unroll
    for (int t = 0; t < kBalancePer; ++t)
      if (t < B.rows) c += (B.u[t] + mid - 1) / mid;
    if (wave_sum(c) <= slots) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}

// Chunk index J -> (sequence, chunk within it, its clamped length).  False
// when J is past the last chunk (the slot has no work).
__device__ __forceinline__ bool balance_locate(const Balance& B, int m, int J, int& seq,
                                               int& k, int& L) {
  int base = 0;
#pragma unroll
  for (int t = 0; t < kBalancePer; ++t)
    if (t < B.rows) {
      const int nb = (B.u[t] + m - 1) / m;
      const int incl = wave_incl_scan(nb);
      const int tot = __builtin_amdgcn_readlane(incl, 63);
      if (J < base + tot) {
        const uint64_t own = __ballot((J < base + incl) & (J >= base + incl - nb));
        const int lo = __builtin_ctzll(own);
        seq = t * 64 + lo;
        k = J - base - __builtin_amdgcn_readlane(incl - nb, lo);
        L = __builtin_amdgcn_readlane(B.L[t], lo);
        return true;
      }
      base += tot;
    }
  return false;
}

// Sequence -> its first chunk index and chunk count.
__device__ __forceinline__ void balance_range(const Balance& B, int m, int seq, int& start,
                                              int& cnt) {
  int base = 0;
  start = 0;
  cnt = 0;
#pragma unroll
  for (int t = 0; t < kBalancePer; ++t)
    if (t < B.rows) {
      const int nb = (B.u[t] + m - 1) / m;
      const int incl = wave_incl_scan(nb);
      if ((seq >> 6) == t) {
        const int lo = seq & 63;
        start = base + __builtin_amdgcn_readlane(incl - nb, lo);
        cnt = __builtin_amdgcn_readlane(nb, lo);
      }
      base += __builtin_amdgcn_readlane(incl, 63);
    }
}

// ------------------------------------------------------------ E4M3 decode
// Two E4M3 codes (bytes 2*HI, 2*HI+1 of w) to two fp16 values.  Every E4M3
// value is exactly a binary16 value, so with a unit scale this is exact.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_f16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
}

// Eight codes (bytes 8*HALF .. 8*HALF+7 of a 16-byte chunk) to an MFMA operand.
template <int HALF>
__device__ __forceinline__ h8_t e4m3x8_to_h8(u4_t c) {
  u4_t r;
  r[0] = e4m3x2_to_f16x2<false>(c[2 * HALF]);
  r[1] = e4m3x2_to_f16x2<true>(c[2 * HALF]);
  r[2] = e4m3x2_to_f16x2<false>(c[2 * HALF + 1]);
  r[3] = e4m3x2_to_f16x2<true>(c[2 * HALF + 1]);
  return __builtin_bit_cast(h8_t, r);
}

// (b.lo16, a.lo16) and (b.hi16, a.hi16) as one dword.
__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(a, b, 0x05040100u);
}
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(a, b, 0x07060302u);
}

__device__ __forceinline__ u4_t load16(const uint8_t* ptr) {
  return *reinterpret_cast<const u4_t*>(ptr);
}

// K/V row load.  With NT the load carries the non-temporal hint: a decode call
// reads every K/V byte exactly once, and streaming it past the caches without
// normal retention measured 11% faster on the long-context batch (and 12% on
// the steady-state streaming rate).  Sparse prefill rows share one pool and
// re-read it through the caches, so they load normally.
template <bool NT>
__device__ __forceinline__ u4_t load_kv(const uint8_t* ptr) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u4_t*>(ptr));
  return *reinterpret_cast<const u4_t*>(ptr);
}

__device__ __forceinline__ uint16_t f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

// t / P and t % P for 0 <= t < 2^22 via a float reciprocal and one
// branch-free correction (the float quotient is off by at most one).
__device__ __forceinline__ int div_page(int t, int P, float invP, int& slot) {
  int qt = static_cast<int>(static_cast<float>(t) * invP);
  int rem = t - qt * P;
  const int adj = rem < 0 ? -1 : (rem >= P ? 1 : 0);
  qt += adj;
  slot = rem - adj * P;
  return qt;
}

template <bool FP8>
struct Geo;
template <>
struct Geo<true> {
  static constexpr int kK = 4;  // 16-byte K pieces per lane per tile
  static constexpr int kV = 1;  // 16-byte V pieces per lane per token
};
template <>
struct Geo<false> {
  static constexpr int kK = 8;
  static constexpr int kV = 2;
};

template <bool FP8>
struct TileRegs {
  u4_t k[Geo<FP8>::kK];
  u4_t v[4][Geo<FP8>::kV];
};

// RW (row per wave): the wave walks every tile of its own row; otherwise
// wave w of NW takes tiles w, w + NW, ... of the workgroup's range.
template <bool FP8, int NW, bool NT, bool RW>
struct Wave {
  static constexpr int kTileStride = RW ? 1 : NW;
  // constant per wave
  const AttnParams& p;
  const int32_t* tab;
  int64_t head_off;  // g * head_stride (bytes)
  int64_t fallback;  // row offset read by lanes whose token is not live
  int s0, s1, wave, r, qd;
  h8_t qop[8];
  // running state
  f4_t acc[16];
  float m_run, l_run;
  bool bad;

  __device__ __forceinline__ int tile_start(int k) const {
    return s0 + ((RW ? 0 : wave) + kTileStride * k) * kTile;
  }

  // q^T operand of sequence b, kv head g: head r of the group (zero past the
  // group), the head-dim pieces in the same permuted order as the K operand.
  __device__ __forceinline__ void load_q(int b, int g) {
    const int head = g * p.group + r;
    const uint8_t* qrow = reinterpret_cast<const uint8_t*>(
        p.q + (static_cast<int64_t>(b) * p.hq + (r < p.group ? head : 0)) * kHeadDim);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const int d0 = FP8 ? 16 * (qd + 4 * (st >> 1)) + 8 * (st & 1) : 8 * (qd + 4 * st);
      u4_t v = load16(qrow + 2 * d0);
      if (r >= p.group) v = u4_t{0u, 0u, 0u, 0u};
      qop[st] = __builtin_bit_cast(h8_t, v);
    }
  }

  // Page-table entry (and slot) for this lane's K token of tile k.  The token
  // is clamped to [0, max_len) only, so the load does not wait for the
  // sequence length; entries of tokens past the live length are read but
  // never used (issue() masks those lanes).
  __device__ __forceinline__ int fetch_page(int k, int& slot) const {
    int t = max(0, min(tile_start(k) + r, p.max_len - 1));
    int idx = div_page(t, p.page_size, p.inv_page_size, slot);
    return tab[idx];
  }

  // Byte offset of a lane's row given its page-table entry (page 0 stands
  // in for an out-of-range entry, so the address is always inside the pool).
  __device__ __forceinline__ int64_t row_offset(int page, int slot) const {
    const bool ok = (page >= 0) & (page < p.num_pages);
    return static_cast<int64_t>(ok ? page : 0) * p.page_stride +
           static_cast<int64_t>(slot) * p.token_stride + head_off;
  }

  // Issue the K and V loads of tile k.  Lanes whose token is not live read
  // the fallback row (the wave's first live row: cached, finite); an
  // out-of-range page id of a live token marks the wave's result bad.
  __device__ __forceinline__ void issue(TileRegs<FP8>& R, int page, int slot, int k) {
    const bool live = tile_start(k) + r < s1;
    const bool ok = (page >= 0) & (page < p.num_pages);
    bad |= live & !ok;
    const int64_t off = live ? row_offset(page, slot) : fallback;
    const uint8_t* krow = p.k_base + off;
#pragma unroll
    for (int i = 0; i < Geo<FP8>::kK; ++i) R.k[i] = load_kv<NT>(krow + 16 * (qd + 4 * i));
    // V rows of tokens 4qd .. 4qd+3: their offsets come from the lanes that
    // computed them for K.
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      int64_t voff = __shfl(off, 4 * qd + e);
      const uint8_t* vrow = p.v_base + voff + 16 * r;
#pragma unroll
      for (int c = 0; c < Geo<FP8>::kV; ++c) R.v[e][c] = load_kv<NT>(vrow + 256 * c);
    }
  }

  __device__ __forceinline__ void process(const TileRegs<FP8>& R, int k) {
    const int t0 = tile_start(k);
    // ---- logits: S^T[token][head] on MFMA
    f4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      h8_t kop;
      if constexpr (FP8) {
        kop = (st & 1) ? e4m3x8_to_h8<1>(R.k[st >> 1]) : e4m3x8_to_h8<0>(R.k[st >> 1]);
      } else {
        kop = __builtin_bit_cast(h8_t, R.k[st]);
      }
      s = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[st], s, 0, 0, 0);
    }
    // ---- online softmax, log2 domain
    float z[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int t = t0 + 4 * qd + i;
      z[i] = (t < s1) ? s[i] * p.qk_scale_log2 : -__builtin_huge_valf();
    }
    float mt = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);  // finite: the tile has a live token
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float pz[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pz[i] = __builtin_amdgcn_exp2f(z[i] - m_new);
    l_run = l_run * alpha + ((pz[0] + pz[1]) + (pz[2] + pz[3]));
    m_run = m_new;
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[j] *= alpha;
    }
    h4_t pop;
    pop[0] = static_cast<_Float16>(pz[0]);
    pop[1] = static_cast<_Float16>(pz[1]);
    pop[2] = static_cast<_Float16>(pz[2]);
    pop[3] = static_cast<_Float16>(pz[3]);
    // ---- PV on MFMA
    if constexpr (FP8) {
      uint32_t hv[4][8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          hv[e][2 * w] = e4m3x2_to_f16x2<false>(R.v[e][0][w]);
          hv[e][2 * w + 1] = e4m3x2_to_f16x2<true>(R.v[e][0][w]);
        }
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int pw = j >> 1;
        u2_t a;
        if (j & 1) {
          a[0] = hi_pair(hv[1][pw], hv[0][pw]);
          a[1] = hi_pair(hv[3][pw], hv[2][pw]);
        } else {
          a[0] = lo_pair(hv[1][pw], hv[0][pw]);
          a[1] = lo_pair(hv[3][pw], hv[2][pw]);
        }
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h4_t, a), pop,
                                                       acc[j], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int c = j >> 3;
        const int w = (j & 7) >> 1;
        u2_t a;
        if (j & 1) {
          a[0] = hi_pair(R.v[1][c][w], R.v[0][c][w]);
          a[1] = hi_pair(R.v[3][c][w], R.v[2][c][w]);
        } else {
          a[0] = lo_pair(R.v[1][c][w], R.v[0][c][w]);
          a[1] = lo_pair(R.v[3][c][w], R.v[2][c][w]);
        }
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h4_t, a), pop,
                                                       acc[j], 0, 0, 0);
      }
    }
  }

  // Head-dim index held by acc[j][i] of this lane.
  __device__ __forceinline__ int out_dim(int j, int i) const {
    const int m = 4 * qd + i;
    if constexpr (FP8) return 16 * m + j;
    return 128 * (j >> 3) + 8 * m + (j & 7);
  }
};

constexpr int gcd_const(int a, int b) { return b == 0 ? a : gcd_const(b, a % b); }

// The leading scalar arguments are what the first page-table and length loads
// depend on (bal_n = n selects the balanced plan, 0 the static one); the
// library is built with kernel-argument preloading, so they arrive in SGPRs at
// wave launch and those loads do not wait for the parameter block (which is
// fetched from memory in parallel).
template <bool FP8, int NW, int PD, int PL, bool NT, bool RW>
__global__ __launch_bounds__(64 * NW) void attention_kernel(
    const int32_t* table, const int32_t* lens, int32_t max_pages, int32_t max_len, int32_t chunk,
    int32_t splits, int32_t hkv, int32_t page_size, float inv_page_size, int32_t bal_n,
    AttnParams p) {
  p.table = table;
  p.lens = lens;
  p.max_pages = max_pages;
  p.max_len = max_len;
  p.chunk = chunk;
  p.splits = splits;
  p.hkv = hkv;
  p.page_size = page_size;
  p.inv_page_size = inv_page_size;
  constexpr int kNT = 64 * NW;
  extern __shared__ float smem[];
  const int lane = threadIdx.x & 63;
  // The wave index is uniform across the wave; saying so keeps the tile loop
  // on scalar branches.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wg = blockIdx.x;
  // Row per wave (one split only): wave w of workgroup wg owns (sequence,
  // kv head) NW * wg + w.
  const int split = RW ? 0 : wg % p.splits;
  const int bg = RW ? NW * wg + wave : wg / p.splits;
  if (RW && bg >= p.n * p.hkv) return;  // past the last row (whole wave)
  int b = bg / p.hkv;
  const int g = bg - b * p.hkv;

  // The static plan: split `split` of sequence b.  Its page-table entries are
  // fetched before the lengths arrive; a balanced plan (bal_n = n > 0) that
  // moves this workgroup elsewhere fetches them again.
  int Lraw = p.lens[b];  // its load overlaps the page-table prefetch below
  int s0 = split * p.chunk;
  int chunk_len = p.chunk;
  // Partial slot (split partials only): (b, split) here, and in a balanced
  // plan too, where this workgroup's chunk index is J = b*S + split.
  const int slot_row = b, slot_col = split;
  // Every sequence's length, for the balanced plan: issued first, so that
  // waiting for them does not also wait for the page-table prefetch.
  int raw[kBalancePer];
  if (bal_n > 0) balance_load(raw, p.lens, bal_n, lane);

  Wave<FP8, NW, NT, RW> W{p};
  W.tab = p.table + static_cast<int64_t>(b) * p.max_pages;
  W.head_off = static_cast<int64_t>(g) * p.head_stride;
  W.s0 = s0;
  W.wave = wave;
  W.r = lane & 15;
  W.qd = lane >> 4;

  // Software pipeline over a ring of PD tile buffers: while tile k is
  // computed, the K/V loads of tiles k+1 .. k+PD-1 are in flight.  Page-table
  // entries run PL tiles further ahead, and each iteration loads them before
  // its K/V loads (loads complete in issue order, so waiting for a page id
  // never drains K/V loads issued after it).  The first entries are loaded
  // before the sequence length is known, so they share its memory latency.
  // Page-entry ring: the first PD - 1 + PL entries are loaded before the first
  // K/V loads are issued, so it holds that many (PL + 1 would do after that).
  constexpr int RP = PD - 1 + PL;
  constexpr int U = PD * RP / gcd_const(PD, RP);  // unroll: ring indices are constants
  int pg[RP], ps[RP];  // page-table entry and slot-in-page, per ring position
#pragma unroll
  for (int t = 0; t <= PD - 2 + PL; ++t) pg[t % RP] = W.fetch_page(t, ps[t % RP]);

  if (bal_n > 0) {
    const Balance B = balance_finish(raw, bal_n, p.max_len, __builtin_ctz(kTile * NW), lane);
    if (!B.full) {
      const int J = b * p.splits + split;
      const int m = balance_units(B, bal_n * p.splits);
      int seq, k, L;
      if (m == 0 || !balance_locate(B, m, J, seq, k, L)) return;  // a slot with no chunk
      chunk_len = m * kTile * NW;
      const int s0n = k * chunk_len;
      if (seq != b) W.tab = p.table + static_cast<int64_t>(seq) * p.max_pages;
      if (seq != b || s0n != s0) {
        W.s0 = s0n;
#pragma unroll
        for (int t = 0; t <= PD - 2 + PL; ++t) pg[t % RP] = W.fetch_page(t, ps[t % RP]);
      }
      b = seq;
      s0 = s0n;
      Lraw = L;
    }
  }
  // Loaded once the sequence is settled; the first tile waits for its K/V
  // loads, issued after these, so this latency is hidden behind theirs.
  W.load_q(b, g);

  const int L = min(Lraw, p.max_len);
  const int s1 = min(s0 + chunk_len, L);
  if (p.partials && s0 >= L) {
    // A split with no live token: its partial is empty (lse = -inf).
    if (threadIdx.x < p.group) {
      const int64_t oh = static_cast<int64_t>(slot_row) * p.hq + g * p.group + threadIdx.x;
      p.ws_lse[oh * p.splits + slot_col] = -__builtin_huge_valf();
    }
    return;
  }
  W.s1 = s1;
  W.m_run = -__builtin_huge_valf();
  W.l_run = 0.f;
  W.bad = false;
#pragma unroll
  for (int j = 0; j < 16; ++j) W.acc[j] = f4_t{0.f, 0.f, 0.f, 0.f};

  constexpr int kStep = Wave<FP8, NW, NT, RW>::kTileStride * kTile;  // tokens between own tiles
  const int span = s1 - s0 - (RW ? 0 : wave) * kTile;
  const int ntiles = span > 0 ? (span + kStep - 1) / kStep : 0;

  // The loop body is straight-line so the wait counts are exact; it runs to a
  // multiple of U tiles.  Tiles past the wave's range load only the cached
  // fallback row and are not computed.
  if (ntiles > 0) {
    // Lane 0's token of tile 0 is live (ntiles > 0): its row is the fallback.
    W.fallback = __shfl(W.row_offset(pg[0], ps[0]), 0);
    TileRegs<FP8> R[PD];
#pragma unroll
    for (int t = 0; t + 1 < PD; ++t) W.issue(R[t], pg[t % RP], ps[t % RP], t);
    for (int k = 0; k < ntiles; k += U) {
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int tf = j + PD - 1 + PL;  // tile whose page entry is loaded now
        const int ti = j + PD - 1;       // tile whose K/V loads are issued now
        pg[tf % RP] = W.fetch_page(k + tf, ps[tf % RP]);
        W.issue(R[ti % PD], pg[ti % RP], ps[ti % RP], k + ti);
        if (k + j < ntiles) W.process(R[j % PD], k + j);
      }
    }
  }

  if constexpr (RW) {
    // The wave holds its whole row: normalise and store from registers.
    float l_tot = W.l_run + __shfl_xor(W.l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    const bool bad = __ballot(W.bad) != 0;
    if (W.r < p.group) {
      // v_scale applied; an empty row (l = 0) gives zeros; a bad page NaNs.
      const float scale = bad ? __builtin_nanf("") : (l_tot > 0.f ? p.v_scale / l_tot : 0.f);
      uint16_t* orow =
          p.out + (static_cast<int64_t>(b) * p.hq + g * p.group + W.r) * kHeadDim;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          u2_t packed;
          packed[0] = f16_bits(W.acc[4 * jj][i] * scale) |
                      (static_cast<uint32_t>(f16_bits(W.acc[4 * jj + 1][i] * scale)) << 16);
          packed[1] = f16_bits(W.acc[4 * jj + 2][i] * scale) |
                      (static_cast<uint32_t>(f16_bits(W.acc[4 * jj + 3][i] * scale)) << 16);
          *reinterpret_cast<u2_t*>(orow + W.out_dim(4 * jj, i)) = packed;
        }
      }
    }
    return;
  }

  // ---- merge the waves of the workgroup through LDS
  const int group = p.group;
  float* so = smem;                           // [NW][group][kLdsRow]
  float* sm = so + NW * group * kLdsRow;      // [NW][16]
  float* sl = sm + NW * 16;                   // [NW][16]
  float* swt = sl + NW * 16;                  // [16][NW] merge weights (scale folded in)
  int* sflags = reinterpret_cast<int*>(swt + NW * 16);  // [NW] bad-page flags
  float l_tot = W.l_run + __shfl_xor(W.l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const bool wave_bad = __ballot(W.bad) != 0;
  if (W.r < group) {
    float* row = so + (wave * group + W.r) * kLdsRow;
    // acc[j][i] for j = 4jj .. 4jj+3 hold four consecutive head dims.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        float4 v = make_float4(W.acc[4 * jj][i], W.acc[4 * jj + 1][i], W.acc[4 * jj + 2][i],
                               W.acc[4 * jj + 3][i]);
        *reinterpret_cast<float4*>(row + W.out_dim(4 * jj, i)) = v;
      }
    }
    if (W.qd == 0) {
      sm[wave * 16 + W.r] = W.m_run;
      sl[wave * 16 + W.r] = l_tot;
    }
  }
  if (lane == 0) sflags[wave] = wave_bad ? 1 : 0;
  __syncthreads();

  // Per head: the waves' weights 2^(m_w - M) times the output scale, once;
  // the items below only read them.
  if (threadIdx.x < group) {
    const int h = threadIdx.x;
    bool any_bad = false;
#pragma unroll
    for (int w = 0; w < NW; ++w) any_bad |= sflags[w] != 0;
    float M = -__builtin_huge_valf();
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm[w * 16 + h]);
    float e[NW];
    float den = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = sm[w * 16 + h];
      e[w] = mw != -__builtin_huge_valf() ? __builtin_amdgcn_exp2f(mw - M) : 0.f;
      den += e[w] * sl[w * 16 + h];
    }
    // v_scale applied; an empty range (den = 0) gives zeros; a bad page NaNs.
    const float scale = any_bad ? __builtin_nanf("") : (den > 0.f ? p.v_scale / den : 0.f);
#pragma unroll
    for (int w = 0; w < NW; ++w) swt[h * NW + w] = e[w] * scale;
    if (p.partials) {
      const int64_t oh = static_cast<int64_t>(slot_row) * p.hq + g * group + h;
      p.ws_lse[oh * p.splits + slot_col] = den > 0.f ? M + __log2f(den) : -__builtin_huge_valf();
    }
  }
  __syncthreads();
  // One item = (head h, four consecutive dims).
  for (int item = threadIdx.x; item < group * (kHeadDim / 4); item += kNT) {
    const int h = item / (kHeadDim / 4);
    const int d = 4 * (item % (kHeadDim / 4));
    float wt[NW];
#pragma unroll
    for (int w = 0; w < NW; w += 4) {
      const float4 v = *reinterpret_cast<const float4*>(swt + h * NW + w);
      wt[w] = v.x;
      wt[w + 1] = v.y;
      wt[w + 2] = v.z;
      wt[w + 3] = v.w;
    }
    float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if (wt[w] != 0.f || wt[w] != wt[w]) {  // a zero weight adds nothing; NaN propagates
        const float4 o = *reinterpret_cast<const float4*>(so + (w * group + h) * kLdsRow + d);
        num.x += wt[w] * o.x;
        num.y += wt[w] * o.y;
        num.z += wt[w] * o.z;
        num.w += wt[w] * o.w;
      }
    }
    if (!p.partials) {
      const int64_t oh = static_cast<int64_t>(b) * p.hq + g * group + h;
      u2_t packed;
      packed[0] = f16_bits(num.x) | (static_cast<uint32_t>(f16_bits(num.y)) << 16);
      packed[1] = f16_bits(num.z) | (static_cast<uint32_t>(f16_bits(num.w)) << 16);
      *reinterpret_cast<u2_t*>(p.out + oh * kHeadDim + d) = packed;
    } else {
      const int64_t oh = static_cast<int64_t>(slot_row) * p.hq + g * group + h;
      *reinterpret_cast<float4*>(p.ws_o + (oh * p.splits + slot_col) * kHeadDim + d) = num;
    }
  }
}

// Merge the split partials of one (row, query head), each lane owning 4
// consecutive head dims.  Split s is weighted by 2^(lse_s - max lse); a split
// with lse = -inf (no live token) has weight 0 and its stored output is not
// used.  The lse values and the partial outputs of a chunk of 32 splits are
// loaded together, so a chunk costs about one memory round trip.  W = 1: one
// wave takes the row's chunks in turn; its first chunk holds FIRST entries
// (16 when there are at most 16 splits, so no load re-reads a slot for
// nothing), later ones 32.  W > 1 (more than 32 splits): W waves
// take chunks w, w + W, ... at once, each merging its own into (max, sum,
// outputs, two chunks' loads in flight at once), and wave 0 combines the W
// results in wave order through LDS, so a row of 256 splits costs one round
// trip, not eight.
//
// Static layout (lens = nullptr): row r's partials are slots r*S .. r*S+S-1.
// Balanced layout (a whole decode call, rows = (sequence b, query head h)):
// the row's chunk indices J come from the plan above and live in slots
// ((J / S) * hq + h) * S + J % S.  The first chunk is loaded at the static
// slots while the lengths are in flight; it is loaded again only if the plan
// is not the static one.
template <int W, int FIRST>
__global__ __launch_bounds__(64 * W) void merge_kernel(const float* lse_base, const float* o_base,
                                                       int32_t splits, const int32_t* lens,
                                                       int32_t n, int32_t hq_in, MergeParams p) {
  p.lse = lse_base;  // leading arguments: preloaded into SGPRs
  p.o = o_base;
  p.splits = splits;
  p.lens = lens;
  p.n = n;
  p.hq = hq_in;
  constexpr int kChunk = 32;
  const int S = p.splits;
  const int lane = threadIdx.x & 63;
  const int hq = p.lens ? p.hq : 1;
  const int row = blockIdx.x;
  const int b = row / hq;
  const int h = row - b * hq;
  const float4* po = reinterpret_cast<const float4*>(p.o) + lane;

  // Chunk indices j0 .. j0+count-1 (1 <= count <= N, the size of vv) into
  // vv, and this lane's lse into lv (-inf past count).  BF (branch-free):
  // entries past count re-read the last slot and are never used (their
  // weight is 0), so a wait for loads issued before these does not wait for
  // them too.
  auto load_chunk = [&](auto& vv, float& lv, int j0, int count, auto bf) {
    constexpr bool BF = decltype(bf)::value;
    constexpr int N = sizeof(vv) / sizeof(vv[0]);
    int q = j0 / S, r = j0 - q * S;
    if (r + count <= S) {  // one run of consecutive slots
      const int64_t base = (static_cast<int64_t>(q) * hq + h) * S + r;
#pragma unroll
      for (int u = 0; u < N; ++u) {
        if (BF) vv[u] = po[(base + min(u, count - 1)) * (kHeadDim / 4)];
        else if (u < count) vv[u] = po[(base + u) * (kHeadDim / 4)];
      }
      const float x = p.lse[base + min(lane, count - 1)];
      lv = lane < count ? x : -__builtin_huge_valf();
    } else {
      int64_t slot = 0;
#pragma unroll
      for (int u = 0; u < N; ++u) {
        if (u < count) slot = (static_cast<int64_t>(q) * hq + h) * S + r;
        if (BF || u < count) vv[u] = po[slot * (kHeadDim / 4)];
        if (++r == S) {
          r = 0;
          ++q;
        }
      }
      const int jl = j0 + min(lane, count - 1);
      const int ql = jl / S;
      const float x = p.lse[(static_cast<int64_t>(ql) * hq + h) * S + (jl - ql * S)];
      lv = lane < count ? x : -__builtin_huge_valf();
    }
  };

  float M = -__builtin_huge_valf(), den = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  // Online log-sum-exp merge of one chunk into (M, den, acc).
  auto combine = [&](const auto& vv, float lv) {
    constexpr int N = sizeof(vv) / sizeof(vv[0]);
    float mc = lv;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mc = fmaxf(mc, __shfl_xor(mc, o));
    const float m_new = fmaxf(M, mc);
    if (m_new == -__builtin_huge_valf()) return;  // nothing live so far
    const float alpha = __builtin_amdgcn_exp2f(M - m_new);  // 0 when M = -inf
    const float wl = lv == -__builtin_huge_valf() ? 0.f : __builtin_amdgcn_exp2f(lv - m_new);
    float ws = wl;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ws += __shfl_xor(ws, o);
    den = den * alpha + ws;
    acc.x *= alpha;
    acc.y *= alpha;
    acc.z *= alpha;
    acc.w *= alpha;
#pragma unroll
    for (int u = 0; u < N; ++u) {
      const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), u));
      if (w != 0.f) {
        acc.x += w * vv[u].x;
        acc.y += w * vv[u].y;
        acc.z += w * vv[u].z;
        acc.w += w * vv[u].w;
      }
    }
    M = m_new;
  };

  int raw[kBalancePer];
  if (p.lens) balance_load(raw, p.lens, p.n, lane);
  int start = b * S, cnt = S;
  if constexpr (W > 1) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (p.lens) {
      const Balance B = balance_finish(raw, p.n, p.max_len, p.a_shift, lane);
      if (!B.full) {
        const int m = balance_units(B, p.n * S);
        int st = 0, c = 0;
        if (m > 0) balance_range(B, m, b, st, c);
        start = st;
        cnt = c;
      }
    }
    // This wave's chunks c0, c0 + 32W, ..., two at a time: both chunks'
    // loads are issued before either is merged, so a pair costs one round
    // trip (with at most 4 waves a row of up to 256 splits is one pair).
    for (int c0 = kChunk * wave; c0 < cnt; c0 += 2 * kChunk * W) {
      const int c1 = c0 + kChunk * W;
      float4 va[kChunk], vb[kChunk];
      float la, lb = -__builtin_huge_valf();
      load_chunk(va, la, start + c0, min(cnt - c0, kChunk), std::true_type{});
      if (c1 < cnt) load_chunk(vb, lb, start + c1, min(cnt - c1, kChunk), std::true_type{});
      combine(va, la);
      if (c1 < cnt) combine(vb, lb);
    }
    __shared__ float4 s_acc[W][64];
    __shared__ float s_m[W], s_den[W];
    s_acc[wave][lane] = acc;
    if (lane == 0) {
      s_m[wave] = M;
      s_den[wave] = den;
    }
    __syncthreads();
    if (wave != 0) return;
    float mt = -__builtin_huge_valf();
#pragma unroll
    for (int w = 0; w < W; ++w) mt = fmaxf(mt, s_m[w]);
    float dt = 0.f;
    float4 at = make_float4(0.f, 0.f, 0.f, 0.f);
    if (mt != -__builtin_huge_valf()) {
#pragma unroll
      for (int w = 0; w < W; ++w) {
        if (s_m[w] == -__builtin_huge_valf()) continue;  // no live split in this wave
        const float a = __builtin_amdgcn_exp2f(s_m[w] - mt);
        const float4 x = s_acc[w][lane];
        dt += a * s_den[w];
        at.x += a * x.x;
        at.y += a * x.y;
        at.z += a * x.z;
        at.w += a * x.w;
      }
    }
    acc = at;
    den = dt;
  } else {
  // The first chunk, at the static slots: FIRST (>= S) entries.
  float4 v[FIRST];
  float l;
  load_chunk(v, l, start, min(cnt, FIRST), std::true_type{});
  bool reload = false;
  if (p.lens) {
    const Balance B = balance_finish(raw, p.n, p.max_len, p.a_shift, lane);
    if (!B.full) {
      const int m = balance_units(B, p.n * S);
      int st = 0, c = 0;
      if (m > 0) balance_range(B, m, b, st, c);
      reload = st != start || c > S;
      if (!reload && c < cnt) l = lane < c ? l : -__builtin_huge_valf();
      start = st;
      cnt = c;
    }
  }

  int c0 = 0;
  if (!reload) {  // the first chunk is the one already loaded
    if (cnt > 0) combine(v, l);
    c0 = FIRST;
  }
  for (; c0 < cnt; c0 += kChunk) {
    float4 w4[kChunk];
    float lw;
    load_chunk(w4, lw, start + c0, min(cnt - c0, kChunk), std::false_type{});
    combine(w4, lw);
  }
  }
  const float scale = den > 0.f ? 1.f / den : 0.f;
  uint16_t* op = p.out + static_cast<int64_t>(row) * kHeadDim + 4 * lane;
  u2_t packed;
  packed[0] = f16_bits(acc.x * scale) | (static_cast<uint32_t>(f16_bits(acc.y * scale)) << 16);
  packed[1] = f16_bits(acc.z * scale) | (static_cast<uint32_t>(f16_bits(acc.w * scale)) << 16);
  *reinterpret_cast<u2_t*>(op) = packed;
}

__global__ void e4m3_table_kernel(float* out) {
  const int c = threadIdx.x;
  const uint32_t h = e4m3x2_to_f16x2<false>(static_cast<uint32_t>(c));
  out[c] = static_cast<float>(__builtin_bit_cast(h2_t, h)[0]);
}

template <bool FP8, int NW, bool NT, bool RW>
hipError_t launch(const AttnParams& p, hipStream_t stream) {
  constexpr int PD = kPipelineDepth;
  constexpr int PL = kPageLookahead;
  const size_t lds = RW ? 0 : attention_lds_bytes(p.group, NW);
  if (lds > 65536) {
    // Merge buffers beyond the default 64 KiB dynamic LDS limit need the
    // limit raised (once per process and kernel).
    static const hipError_t raised = hipFuncSetAttribute(
        reinterpret_cast<const void*>(attention_kernel<FP8, NW, PD, PL, NT, RW>),
        hipFuncAttributeMaxDynamicSharedMemorySize,
        static_cast<int>(attention_lds_bytes(kMaxGroup, NW)));
    if (raised != hipSuccess) return raised;
  }
  const int64_t rows = static_cast<int64_t>(p.n) * p.hkv;
  const dim3 grid(static_cast<unsigned>(RW ? (rows + NW - 1) / NW : p.splits * rows));
  return pgqa_launch::launch(attention_kernel<FP8, NW, PD, PL, NT, RW>, grid, dim3(64 * NW), lds,
                             stream, p.table, p.lens, p.max_pages, p.max_len, p.chunk, p.splits,
                             p.hkv, p.page_size, p.inv_page_size, p.balance_n, p);
}

template <bool FP8, int NW, bool NT>
hipError_t launch_rw(const AttnParams& p, hipStream_t stream) {
  return p.row_per_wave ? launch<FP8, NW, NT, true>(p, stream)
                        : launch<FP8, NW, NT, false>(p, stream);
}

}  // namespace

size_t attention_lds_bytes(int group, int waves) {
  return sizeof(float) * (static_cast<size_t>(waves) * group * kLdsRow + 3 * waves * 16) +
         sizeof(int) * waves;
}

hipError_t launch_attention(const AttnParams& p, bool fp8, hipStream_t stream) {
  constexpr int NW = kWavesPerWg;
  if (p.stream_kv)
    return fp8 ? launch_rw<true, NW, true>(p, stream) : launch_rw<false, NW, true>(p, stream);
  return fp8 ? launch_rw<true, NW, false>(p, stream) : launch_rw<false, NW, false>(p, stream);
}

template <int W, int FIRST = 32>
hipError_t launch_merge_w(const MergeParams& p, hipStream_t stream) {
  return pgqa_launch::launch(merge_kernel<W, FIRST>, dim3(static_cast<unsigned>(p.rows)), dim3(64 * W), 0,
                             stream, p.lse, p.o, p.splits, p.lens, p.n, p.hq, p);
}

hipError_t launch_merge(const MergeParams& p, hipStream_t stream) {
  // Waves per row: one up to 32 splits, then one per 32 splits, at most 4
  // (with 8 the 512-thread workgroup caps a wave at 256 VGPRs and the chunk
  // registers spill; past 128 splits a wave takes two or more chunks).
  // With up to 16 splits the first chunk holds 16 entries, not 32 (half the
  // loads of the static plan's one round trip).
  if (p.splits <= 16) return launch_merge_w<1, 16>(p, stream);
  if (p.splits <= 32) return launch_merge_w<1>(p, stream);
  if (p.splits <= 64) return launch_merge_w<2>(p, stream);
  return launch_merge_w<4>(p, stream);
}

hipError_t launch_e4m3_table(float* out256, hipStream_t stream) {
  return pgqa_launch::launch(e4m3_table_kernel, dim3(1), dim3(256), 0, stream, out256);
}

}  // namespace pgqa
