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
// One workgroup of 1024 threads owns one row.  Thread t holds elements
// j = 4096 i + 4 t + c (register slot i, component c) as keys in VGPRs, so a
// row of up to 65,536 blocks is read from HBM exactly once.  The steps:
//   1. T, a lower bound for the pivot: the k-th largest per-thread maximum
//      (each of k threads owns a key >= T, so at least k keys are >= T).
//      Skipped (T = 0) for rows that fit the candidate buffer.
//   2. Keys >= T are appended to an LDS candidate buffer (about 1% of a row
//      of independent scores when k is 1/128 of the row).
//   3. Pivot P: four 8-bit MSB-first histogram passes over the candidates
//      give the k-th largest key P and `need`, how many keys equal to P are
//      kept.  If the candidates overflow the buffer the passes run over the
//      register keys instead (same result, slower).
//   4. Ordered output: per slot, wave ballots of (key > P) and (key == P)
//      give each element its rank among greater-than and tied elements in
//      index order; element j is kept if key > P or it is one of the first
//      `need` ties, and lands at position (#greater before j) + min(#ties
//      before j, need).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pgqa_internal.h"

namespace pgqa {
namespace {

constexpr int kThreads = kTopkThreads;
constexpr int kWaves = kThreads / 64;
constexpr int kSlotElems = 4 * kThreads;    // elements one register slot covers
constexpr int kMaxItems = kTopkMaxBlocks / kSlotElems;
constexpr int kCandCap = 8192;              // LDS candidate keys

struct TopkShared {
  uint32_t cand[kCandCap];
  uint32_t tmax[kThreads];
  uint32_t hist[2][256];
  uint32_t gt_base[kMaxItems * kWaves];
  uint32_t tie_base[kMaxItems * kWaves];
  uint32_t n_cand;
  uint32_t digit;
  uint32_t cbefore;
};

__device__ __forceinline__ uint32_t key_of(float x) {
  const uint32_t u = __float_as_uint(x);
  return u ^ (static_cast<uint32_t>(static_cast<int32_t>(u) >> 31) | 0x80000000u);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// A copy of x the compiler cannot see through.  Each phase re-derives its
// per-element compare masks from such a copy instead of keeping dozens of
// 64-bit masks from an earlier phase alive across barriers.
__device__ __forceinline__ int32_t fresh_v(int32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}
__device__ __forceinline__ uint32_t fresh_s(uint32_t x) {
  asm volatile("" : "+s"(x));
  return x;
}

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  const int lane = lane_id();
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  return x;
}

// Number of set bits of `mask` in lanes below this one.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

// hist[d] += 1 for every active lane; one atomic per wave when all active
// lanes share the digit (common in the first pass, where many scores share
// an exponent).  Must be reached by the whole wave.
__device__ __forceinline__ void hist_add(uint32_t* hist, bool act, uint32_t d) {
  const uint64_t am = __ballot(act);
  if (am == 0) return;
  const int first = __ffsll(static_cast<unsigned long long>(am)) - 1;
  const uint32_t d0 = __builtin_amdgcn_readlane(d, first);
  const uint64_t same = __ballot(act && d == d0);
  if (same == am) {
    if (lane_id() == first) atomicAdd(&hist[d0], static_cast<uint32_t>(__popcll(am)));
  } else if (act) {
    atomicAdd(&hist[d], 1u);
  }
}

// Wave 0: the digit whose bin holds the rem-th largest key (bins scanned from
// 255 down), and the count of keys in higher bins.  Also clears the other
// histogram buffer for the next pass.
__device__ __forceinline__ void find_digit(TopkShared& sh, int buf, uint32_t rem) {
  const int lane = lane_id();
  uint32_t h[4];
  uint32_t s = 0;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    h[m] = sh.hist[buf][255 - 4 * lane - m];
    s += h[m];
  }
  uint32_t c = wave_incl_scan(s) - s;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    if (c < rem && rem <= c + h[m]) {
      sh.digit = 255 - 4 * lane - m;
      sh.cbefore = c;
    }
    c += h[m];
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) sh.hist[buf ^ 1][4 * lane + m] = 0;
}

// k-th largest key (k >= 1) of the multiset the visitor enumerates, and how
// many keys equal to it rank within the first k (returned in *need).
// Requires sh.hist[0] zeroed and a barrier since; leaves it zeroed again.
template <class Visit>
__device__ __forceinline__ uint32_t pivot_search(TopkShared& sh, uint32_t k, uint32_t* need,
                                                 Visit visit) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t prefix = 0, rem = k;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    const uint32_t hi_mask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
    uint32_t* hist = sh.hist[pass & 1];
    visit([&](bool act, uint32_t key) {
      hist_add(hist, act && ((key ^ prefix) & hi_mask) == 0, (key >> shift) & 255u);
    });
    __syncthreads();
    if (wave == 0) find_digit(sh, pass & 1, rem);
    __syncthreads();
    prefix |= __builtin_amdgcn_readfirstlane(sh.digit) << shift;
    rem -= __builtin_amdgcn_readfirstlane(sh.cbefore);
  }
  *need = rem;
  return prefix;
}

template <int ITEMS, bool VEC>
__global__ __launch_bounds__(kThreads) void topk_kernel(TopkParams p) {
  __shared__ TopkShared sh;
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t k = p.k;
  int32_t nv = p.n_valid ? p.n_valid[row] : p.n_blocks;
  nv = nv < 0 ? 0 : (nv > p.n_blocks ? p.n_blocks : nv);
  int32_t* out = p.out_idx + static_cast<int64_t>(row) * k;

  if (nv <= k) {  // every eligible block is kept
    for (int j = tid; j < k; j += kThreads) out[j] = j < nv ? j : -1;
    if (tid == 0 && p.out_count) p.out_count[row] = nv;
    return;
  }
  if (k == 0) {
    if (tid == 0 && p.out_count) p.out_count[row] = 0;
    return;
  }

  // ---- load the row's keys: element (i, c) of this thread is j = 4096 i + 4 tid + c,
  // valid when 4096 i + c < lim.
  const float* src = p.scores + static_cast<int64_t>(row) * p.row_stride;
  const int32_t lim = nv - 4 * tid;
  uint32_t key[ITEMS][4];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
#pragma unroll
    for (int c = 0; c < 4; ++c) key[i][c] = 0;
    if (i * kSlotElems < nv) {
      if (VEC) {
        if (i * kSlotElems < lim) {
          const float4 v =
              *reinterpret_cast<const float4*>(src + i * kSlotElems + 4 * tid);
          // Components past the row's length keep key 0: the per-thread
          // maximum below must only see eligible blocks.
          key[i][0] = key_of(v.x);
          key[i][1] = i * kSlotElems + 1 < lim ? key_of(v.y) : 0u;
          key[i][2] = i * kSlotElems + 2 < lim ? key_of(v.z) : 0u;
          key[i][3] = i * kSlotElems + 3 < lim ? key_of(v.w) : 0u;
        }
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (i * kSlotElems + c < lim) key[i][c] = key_of(src[i * kSlotElems + 4 * tid + c]);
      }
    }
  }

  // ---- 1. lower bound T from the per-thread maxima.  Rows longer than the
  // candidate buffer give every thread at least one valid key (slot 0 is full).
  const bool thresh = nv > kCandCap && k <= kThreads;
  if (thresh) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) m = key[i][c] > m ? key[i][c] : m;  // invalid keys are 0
    sh.tmax[tid] = m;
  }
  if (tid < 256) sh.hist[0][tid] = 0;
  if (tid == 0) sh.n_cand = 0;
  __syncthreads();
  uint32_t T = 0;
  if (thresh) {
    uint32_t unused;
    T = pivot_search(sh, static_cast<uint32_t>(k), &unused, [&](auto f) {
      f(true, sh.tmax[tid]);
    });
  }

  // ---- 2. candidates (keys >= T) into LDS, wave-aggregated append.
  uint32_t cnt = 0;
  {
    const int32_t l = fresh_v(lim);
    const uint32_t t = fresh_s(T);
#pragma unroll
    for (int i = 0; i < ITEMS; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) cnt += (i * kSlotElems + c < l && key[i][c] >= t) ? 1u : 0u;
  }
  const uint32_t incl = wave_incl_scan(cnt);
  uint32_t base = 0;
  if (lane == 63) base = atomicAdd(&sh.n_cand, incl);
  base = __builtin_amdgcn_readlane(base, 63);
  {
    uint32_t pos = base + incl - cnt;
    const int32_t l = fresh_v(lim);
    const uint32_t t = fresh_s(T);
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      if (i * kSlotElems >= nv) break;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (i * kSlotElems + c < l && key[i][c] >= t) {
          if (pos < kCandCap) sh.cand[pos] = key[i][c];
          ++pos;
        }
      }
    }
  }
  __syncthreads();
  const uint32_t nc = __builtin_amdgcn_readfirstlane(sh.n_cand);

  // ---- 3. the pivot.
  uint32_t need = 0;
  uint32_t P;
  if (nc <= kCandCap) {
    P = pivot_search(sh, static_cast<uint32_t>(k), &need, [&](auto f) {
      for (uint32_t b = 0; b < nc; b += kThreads) {
        const uint32_t e = b + tid;
        f(e < nc, e < nc ? sh.cand[e] : 0u);
      }
    });
  } else {
    P = pivot_search(sh, static_cast<uint32_t>(k), &need, [&](auto f) {
      const int32_t l = fresh_v(lim);
      const uint32_t t = fresh_s(T);
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        if (i * kSlotElems >= nv) break;
#pragma unroll
        for (int c = 0; c < 4; ++c) f(i * kSlotElems + c < l && key[i][c] >= t, key[i][c]);
      }
    });
  }

  // ---- 4. ordered output.  Per (slot, wave) counts of greater and tied keys.
  {
    const int32_t lim4 = fresh_v(lim);
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      uint32_t g = 0, q = 0;
      if (i * kSlotElems < nv) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const bool v = i * kSlotElems + c < lim4;
          g += __popcll(__ballot(v && key[i][c] > P));
          q += __popcll(__ballot(v && key[i][c] == P));
        }
      }
      if (lane == 0) {
        sh.gt_base[i * kWaves + wave] = g;
        sh.tie_base[i * kWaves + wave] = q;
      }
    }
  }
  __syncthreads();
  if (wave == 0) {  // exclusive scan over (slot, wave) in index order
    constexpr int E = ITEMS * kWaves;
    constexpr int PER = (E + 63) / 64;
    uint32_t gv[PER], tv[PER], gs = 0, ts = 0;
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int e = lane * PER + m;
      gv[m] = e < E ? sh.gt_base[e] : 0u;
      tv[m] = e < E ? sh.tie_base[e] : 0u;
      gs += gv[m];
      ts += tv[m];
    }
    uint32_t ge = wave_incl_scan(gs) - gs;
    uint32_t te = wave_incl_scan(ts) - ts;
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int e = lane * PER + m;
      if (e < E) {
        sh.gt_base[e] = ge;
        sh.tie_base[e] = te;
      }
      ge += gv[m];
      te += tv[m];
    }
  }
  __syncthreads();
  const int32_t lim5 = fresh_v(lim);
  const uint32_t P5 = fresh_s(P);
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    if (i * kSlotElems >= nv) break;
    bool gt[4], eq[4];
    uint64_t gm[4], tm[4];
    uint64_t any = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bool v = i * kSlotElems + c < lim5;
      gt[c] = v && key[i][c] > P5;
      eq[c] = v && key[i][c] == P5;
      gm[c] = __ballot(gt[c]);
      tm[c] = __ballot(eq[c]);
      any |= gm[c] | tm[c];
    }
    if (any == 0) continue;
    uint32_t gb = sh.gt_base[i * kWaves + wave];
    uint32_t tb = sh.tie_base[i * kWaves + wave];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      gb += lanes_below(gm[c]);
      tb += lanes_below(tm[c]);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t at = gb + (tb < need ? tb : need);
      if ((gt[c] || (eq[c] && tb < need)) && at < static_cast<uint32_t>(k))
        out[at] = i * kSlotElems + 4 * tid + c;
      gb += gt[c] ? 1u : 0u;
      tb += eq[c] ? 1u : 0u;
    }
  }
  if (tid == 0 && p.out_count) p.out_count[row] = k;
}

template <int ITEMS>
hipError_t launch_items(const TopkParams& p, bool vec, hipStream_t stream) {
  if (vec)
    hipLaunchKernelGGL((topk_kernel<ITEMS, true>), dim3(p.rows), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((topk_kernel<ITEMS, false>), dim3(p.rows), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
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

}  // namespace pgqa
