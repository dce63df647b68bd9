// gfx950 kernels for combined top-k / top-p masking of sampler logits.
//
// Source: "[Kernel][SM70] Scale NVFP4 E4M3 decode batches", Purpose (combined
// top-k/top-p masking for B8/B16 x 248,320 logits) and Performance contract
// (sampler top-k 20, top-p 0.95).  The operation, per row of V logits with
// top-k k and top-p p:
//   order the tokens by (logit descending, index ascending), logits ranked by
//   their IEEE 754 totalOrder keys; the first n = min(k, V) form the top-k
//   set; in that order token i stays iff i is first or the softmax mass of
//   the tokens before it (over the top-k set) is below p (p >= 1 keeps all
//   n); kept tokens keep their logit, every other token becomes -inf.
//
// A token is represented by the 64-bit value (key << 32) | ~index: larger
// means earlier in the order, and all such values are distinct, and the key
// gives back the logit's fp32 bits exactly.  The kept tokens are a prefix
// of the order, at most k <= 256 of them.
//
// Two launches:
//   1. chunk_top_kernel, one 256-thread workgroup per (chunk of <= 8192
//      logits, row): the chunk's top min(k, chunk) tokens in order.  A
//      threshold T from the lane maxima (each of the four waves contributes
//      ceil(k/4) lanes whose maximum is >= T, so at least k keys are >= T)
//      leaves a few candidates; one wave sorts up to 512 of them in
//      registers, more (ties, large k) go through an LDS bitonic sort.  The
//      same workgroup writes -inf over its chunk of the output once its
//      logits are in registers (or copies the chunk for an invalid row), so
//      the logits are read once and every output element written once.
//   2. cut_kernel, one wave per row: the top-k set in order from the <= 64
//      sorted chunk lists (the list prefixes at or above the k-th largest
//      list head, sorted in registers; a tournament over the list heads when
//      there are too many); then the softmax masses in fp32 (exp2 with
//      log2(e) folded in), a wave prefix sum, the kept count, and the kept
//      tokens' logits written back over the -inf.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch_util.h"
#include "sampler_internal.h"

namespace sampler {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ uint32_t key_of(float x) {
  const uint32_t u = __float_as_uint(x);
  return u ^ (static_cast<uint32_t>(static_cast<int32_t>(u) >> 31) | 0x80000000u);
}
__device__ __forceinline__ float value_of(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}
__device__ __forceinline__ uint64_t token(uint32_t key, int32_t index) {
  return (static_cast<uint64_t>(key) << 32) | static_cast<uint32_t>(~index);
}

__device__ __forceinline__ bool row_valid(const MaskParams& p, int row, int32_t& k, float& pp) {
  k = p.k[row];
  pp = p.p[row];
  return k >= 1 && k <= p.k_max && !__builtin_isnan(pp);
}

// The m-th largest (1 <= m <= 64) of the wave's 64 lane values, by bisection
// on the bits from the top; with LOW > 0 the bisection stops there, and the
// result is the m-th largest with its bits below LOW cleared (a lower bound
// that at least m lanes reach).
template <int LOW = 0>
__device__ __forceinline__ uint32_t wave_mth_largest_bits(uint32_t x, uint32_t m) {
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

// x combined with the lane the DPP control CTRL names, in the rows ROWS
// enables (lanes without a source see 0).
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, ROWS, 0xf, false));
}

// Maximum over the wave's 64 lanes: row shifts 1, 2, 4, 8 fold each row of 16
// lanes into its lane 15, the row broadcasts 15 and 31 fold the rows into
// lane 63.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, dpp_u32<0x111, 0xf>(x));
  x = max(x, dpp_u32<0x112, 0xf>(x));
  x = max(x, dpp_u32<0x114, 0xf>(x));
  x = max(x, dpp_u32<0x118, 0xf>(x));
  x = max(x, dpp_u32<0x142, 0xa>(x));
  x = max(x, dpp_u32<0x143, 0xc>(x));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), 63));
}

// The same m-th largest by repeated maxima: each round takes the largest
// value left and sets the lanes holding it to 0 (the smallest key, so they
// matter only when the answer is 0).  At most m rounds; cheaper than the 32
// bisection steps for small m.
template <int LOW = 0>
__device__ __forceinline__ uint32_t wave_mth_largest(uint32_t x, uint32_t m) {
  if (m > 8) return wave_mth_largest_bits<LOW>(x, m);
  for (;;) {
    const uint32_t mx = wave_max_u32(x);
    const uint32_t c = static_cast<uint32_t>(__popcll(__ballot(x == mx)));
    if (c >= m || mx == 0) return mx;
    m -= c;
    x = x == mx ? 0u : x;
  }
}

// Inclusive prefix sum over the wave's 64 lanes, the same DPP pattern.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += dpp_u32<0x111, 0xf>(x);
  x += dpp_u32<0x112, 0xf>(x);
  x += dpp_u32<0x114, 0xf>(x);
  x += dpp_u32<0x118, 0xf>(x);
  x += dpp_u32<0x142, 0xa>(x);
  x += dpp_u32<0x143, 0xc>(x);
  return x;
}

// x from lane (lane ^ M): quad permutes for M = 1, 2, row shifts within 16
// lanes for M = 4, 8 (lanes with bit M clear read lane + M, the others
// lane - M), gfx950's lane-swap instructions for 16 and 32 (the value as
// both operands: the partner's value is the first result in the lanes with
// bit M set, the second in the others).
template <int M>
__device__ __forceinline__ uint32_t xor_lane(uint32_t x) {
  if constexpr (M == 1 || M == 2) {
    return __builtin_amdgcn_update_dpp(0u, x, M == 1 ? 0xB1 : 0x4E, 0xF, 0xF, false);
  } else if constexpr (M == 4 || M == 8) {
    const uint32_t up = __builtin_amdgcn_update_dpp(0u, x, 0x100 + M, 0xF, 0xF, false);
    const uint32_t down = __builtin_amdgcn_update_dpp(0u, x, 0x110 + M, 0xF, 0xF, false);
    return (threadIdx.x & M) ? down : up;
  } else {
    static_assert(M == 16 || M == 32, "lane distances within a wave");
    const auto r = M == 16 ? __builtin_amdgcn_permlane16_swap(x, x, false, false)
                           : __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (threadIdx.x & M) ? r[0] : r[1];
  }
}

template <int M>
__device__ __forceinline__ uint64_t xor_lane_u64(uint64_t x) {
  const uint32_t hi = xor_lane<M>(static_cast<uint32_t>(x >> 32));
  const uint32_t lo = xor_lane<M>(static_cast<uint32_t>(x));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Stages J, J/2, .., 1 of merge level K of a descending bitonic sort of the
// wave's 64*E values, lane l holding elements l*E .. l*E + E-1.  Element i
// keeps the larger of its pair when ((i & J) == 0) == ((i & K) == 0).
template <int E, int K, int J>
__device__ __forceinline__ void desc_stages(uint64_t (&x)[E]) {
  if constexpr (J >= 1) {
    const int lane = threadIdx.x & 63;
    if constexpr (J < E) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int f = e ^ J;
        if (f > e) {
          const bool desc = ((lane * E + e) & K) == 0;
          const uint64_t a = x[e], b = x[f];
          const bool swap = desc ? (a < b) : (a > b);
          x[e] = swap ? b : a;
          x[f] = swap ? a : b;
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int i = lane * E + e;
        const uint64_t y = xor_lane_u64<J / E>(x[e]);
        const bool keep_large = (((i & J) == 0) == ((i & K) == 0));
        x[e] = keep_large ? (x[e] > y ? x[e] : y) : (x[e] < y ? x[e] : y);
      }
    }
    desc_stages<E, K, J / 2>(x);
  }
}

template <int E, int K>
__device__ __forceinline__ void desc_levels(uint64_t (&x)[E]) {
  if constexpr (K <= 64 * E) {
    desc_stages<E, K, K / 2>(x);
    desc_levels<E, 2 * K>(x);
  }
}

template <int E>
__device__ __forceinline__ void wave_sort_desc(uint64_t (&x)[E]) {
  desc_levels<E, 2>(x);
}

// Descending sort of lanes 0..31 (one value each); lanes 32..63 end in some
// other order.  The merge levels stop at 32: 15 stages instead of 21.
__device__ __forceinline__ void wave_sort_desc32(uint64_t& x) {
  uint64_t a[1] = {x};
  desc_stages<1, 2, 1>(a);
  desc_stages<1, 4, 2>(a);
  desc_stages<1, 8, 4>(a);
  desc_stages<1, 16, 8>(a);
  desc_stages<1, 32, 16>(a);
  x = a[0];
}

constexpr int kWaveSortE = 8;  // one wave sorts up to 512 candidates in registers

// One wave's sort of the n_c <= 64 E candidates and the chunk's list: its top
// kc tokens in order, then zeros up to k.
template <int E>
__device__ __forceinline__ void sort_and_write(const uint64_t* cand, uint32_t n_c, int32_t kc,
                                               int32_t k, uint64_t* dst, int32_t n_chunks) {
  const int lane = threadIdx.x & 63;
  uint64_t x[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t i = lane * E + e;
    x[e] = i < n_c ? cand[i] : 0;
  }
  wave_sort_desc<E>(x);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int32_t i = lane * E + e;
    if (i < k) dst[static_cast<int64_t>(i) * n_chunks] = i < kc ? x[e] : 0;
  }
  for (int32_t i = 64 * E + lane; i < k; i += 64) dst[static_cast<int64_t>(i) * n_chunks] = 0;
}

// PER entries per thread: chunks of up to 256 PER logits (16 for the usual
// 4096, 32 for the largest); the work per thread scales with PER.
template <int PER>
__global__ __launch_bounds__(kThreads) void chunk_top_kernel(MaskParams p) {
  extern __shared__ uint64_t cand[];  // [pow2 >= chunk] candidates, then padding
  __shared__ uint32_t wval[kWaves];
  const int chunk = blockIdx.x;
  const int row = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int32_t start = chunk * p.chunk;
  const int32_t len = min(p.chunk, p.vocab - start);
  const float* src = p.logits + static_cast<int64_t>(row) * p.row_stride + start;

  // Thread t holds entries t + 256 i; key 0 (never a logit's key but the
  // negative NaN 0xFFFFFFFF's) marks entries past the chunk.  The loads are
  // issued before the row's k and p are known.
  uint32_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int32_t e = tid + kThreads * i;
    key[i] = e < len ? __float_as_uint(src[e]) : 0xFFFFFFFFu;
  }
  float* out = p.out + static_cast<int64_t>(row) * p.out_stride + start;
  const bool in_place = p.out == p.logits;  // then the strides are equal
  int32_t k;
  float pp;
  if (!row_valid(p, row, k, pp)) {
    // An invalid row is copied unchanged (in place it already is).
    if (!in_place) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int32_t e = tid + kThreads * i;
        if (e < len) out[e] = __uint_as_float(key[i]);
      }
    }
    return;
  }
  const int32_t kc = min(k, len);
  uint32_t lmax = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    key[i] = key_of(__uint_as_float(key[i]));  // 0xFFFFFFFF (past the chunk) -> key 0
    lmax = max(lmax, key[i]);
  }
  // -inf over the chunk: each thread overwrites only the entries it has
  // already read into registers, so this is safe in place too.  The kept
  // logits are written back by cut_kernel, after this launch has finished.
  // (Issuing it before the loads return, into a separate output, measured
  // no faster.)
  const float ninf = -__builtin_huge_valf();
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int32_t e = tid + kThreads * i;
    if (e < len) __builtin_nontemporal_store(ninf, out + e);
  }

  // Threshold: each wave's ceil(kc/4)-th largest lane maximum; T = their
  // minimum.  kc > 256 takes every entry.
  uint32_t T = 0;
  if (kc <= 4 * 64) {
    const uint32_t tw = wave_mth_largest(lmax, static_cast<uint32_t>((kc + 3) / 4));
    if (lane == 0) wval[wave] = tw;
    __syncthreads();
    T = wval[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) T = min(T, wval[w]);
    __syncthreads();  // wval is reused below
  }

  // Candidates (entries with key >= T) to LDS, compacted in thread order.
  uint32_t cnt = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) cnt += (tid + kThreads * i < len && key[i] >= T) ? 1u : 0u;
  const uint32_t incl = wave_incl_scan(cnt);
  if (lane == 63) wval[wave] = incl;
  __syncthreads();
  uint32_t pos = incl - cnt, n_c = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    pos += w < wave ? wval[w] : 0u;
    n_c += wval[w];
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int32_t e = tid + kThreads * i;
    if (e < len && key[i] >= T) cand[pos++] = token(key[i], start + e);
  }
  // The chunk's list, rank-major: rank i at dst[i * n_chunks].
  uint64_t* dst = p.cand + static_cast<int64_t>(row) * p.n_chunks * p.k_max + chunk;
  if (n_c <= 64 * kWaveSortE) {
    // Few candidates (the usual case): one wave sorts them in registers and
    // writes the chunk's list, its top kc tokens in order, then zeros up to k.
    __syncthreads();
    if (wave != 0) return;
    if (n_c <= 32) {
      // Up to 32 candidates: the 32-wide network; lanes 32.. write only
      // zeros (kc <= n_c <= 32).
      uint64_t x = lane < static_cast<int>(n_c) ? cand[lane] : 0;
      wave_sort_desc32(x);
      if (lane < k) dst[static_cast<int64_t>(lane) * p.n_chunks] = lane < kc ? x : 0;
      for (int32_t i = 64 + lane; i < k; i += 64) dst[static_cast<int64_t>(i) * p.n_chunks] = 0;
    } else if (n_c <= 64)
      sort_and_write<1>(cand, n_c, kc, k, dst, p.n_chunks);
    else if (n_c <= 128)
      sort_and_write<2>(cand, n_c, kc, k, dst, p.n_chunks);
    else if (n_c <= 256)
      sort_and_write<4>(cand, n_c, kc, k, dst, p.n_chunks);
    else
      sort_and_write<8>(cand, n_c, kc, k, dst, p.n_chunks);
    return;
  }
  uint32_t n2 = 64;
  while (n2 < n_c) n2 <<= 1;
  for (uint32_t i = n_c + tid; i < n2; i += kThreads) cand[i] = 0;
  __syncthreads();

  // Bitonic sort of cand[0 .. n2), descending.
  for (uint32_t kk = 2; kk <= n2; kk <<= 1) {
    for (uint32_t j = kk >> 1; j > 0; j >>= 1) {
      for (uint32_t t = tid; t < n2 / 2; t += kThreads) {
        const uint32_t i = 2 * j * (t / j) + (t % j);
        const uint64_t a = cand[i], b = cand[i + j];
        const bool desc = (i & kk) == 0;
        if (desc ? (a < b) : (a > b)) {
          cand[i] = b;
          cand[i + j] = a;
        }
      }
      __syncthreads();
    }
  }

  // The chunk's list: its top kc tokens in order, then zeros up to k.
  for (int32_t i = tid; i < k; i += kThreads)
    dst[static_cast<int64_t>(i) * p.n_chunks] = i < kc ? cand[i] : 0;
}

// Sorts buf[0 .. cnt) descending in place (one wave, cnt <= 64 E).
template <int E>
__device__ __forceinline__ void sort_top(uint64_t* buf, uint32_t cnt) {
  const int lane = threadIdx.x & 63;
  uint64_t x[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t i = lane * E + e;
    x[e] = i < cnt ? buf[i] : 0;
  }
  wave_sort_desc<E>(x);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t i = lane * E + e;
    if (i < cnt) buf[i] = x[e];
  }
}

// Sorts buf[0 .. cnt) descending in place (one wave, cnt <= 32).
__device__ __forceinline__ void sort_top32(uint64_t* buf, uint32_t cnt) {
  const uint32_t lane = threadIdx.x & 63;
  uint64_t x = lane < cnt ? buf[lane] : 0;
  wave_sort_desc32(x);
  if (lane < cnt) buf[lane] = x;
}

// Step of the wave maximum: combine with the lane DPP control `ctrl` names
// (lanes without a source see 0, the minimum).
template <int CTRL, int ROWS>
__device__ __forceinline__ void max_step(uint32_t& hi, uint32_t& lo) {
  const uint32_t h2 = __builtin_amdgcn_update_dpp(0u, hi, CTRL, ROWS, 0xF, false);
  const uint32_t l2 = __builtin_amdgcn_update_dpp(0u, lo, CTRL, ROWS, 0xF, false);
  const bool take = h2 > hi || (h2 == hi && l2 > lo);
  hi = take ? h2 : hi;
  lo = take ? l2 : lo;
}

// Maximum over the wave's 64 lanes, on every lane: row shifts fold each row
// of 16 lanes into its lane 15, row broadcasts fold the rows into lane 63.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
  uint32_t hi = static_cast<uint32_t>(x >> 32), lo = static_cast<uint32_t>(x);
  max_step<0x111, 0xF>(hi, lo);  // row_shr:1
  max_step<0x112, 0xF>(hi, lo);  // row_shr:2
  max_step<0x114, 0xF>(hi, lo);  // row_shr:4
  max_step<0x118, 0xF>(hi, lo);  // row_shr:8
  max_step<0x142, 0xA>(hi, lo);  // row_bcast:15 into rows 1 and 3
  max_step<0x143, 0xC>(hi, lo);  // row_bcast:31 into rows 2 and 3
  hi = __builtin_amdgcn_readlane(hi, 63);
  lo = __builtin_amdgcn_readlane(lo, 63);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__global__ __launch_bounds__(64) void cut_kernel(MaskParams p) {
  extern __shared__ uint64_t lists[];  // [k][n_chunks], rank-major
  __shared__ uint64_t top[64 * kWaveSortE];
  const int row = blockIdx.x;
  const int lane = threadIdx.x;
  // The chunk lists of the row, rank-major (list j's rank r at r * n_chunks
  // + j): the first kSpec ranks of every list are one flat coalesced read,
  // issued before k is known; ranks at or past k hold stale data and are
  // zeroed once it is.  Deeper ranks are read only if a list needs them.
  constexpr int kSpec = 8;
  const uint64_t* src = p.cand + static_cast<int64_t>(row) * p.n_chunks * p.k_max;
  const int32_t spec_total = min(kSpec, p.k_max) * p.n_chunks;  // <= 64 kSpec
  uint64_t sv[kSpec];
#pragma unroll
  for (int u = 0; u < kSpec; ++u) {
    const int32_t e = 64 * u + lane;
    sv[u] = e < spec_total ? src[e] : 0;
  }
  int32_t k;
  float pp;
  if (!row_valid(p, row, k, pp)) {  // copied by chunk_top_kernel
    if (lane == 0 && p.status)
      p.status[row] = (k >= 1 && k <= p.k_max ? 0 : kBadK) | (__builtin_isnan(pp) ? kBadP : 0);
    return;
  }
  const int32_t n = min(k, p.vocab);
  const int32_t total = k * p.n_chunks;
#pragma unroll
  for (int u = 0; u < kSpec; ++u) {
    const int32_t e = 64 * u + lane;
    if (e < spec_total) lists[e] = e < total ? sv[u] : 0;
  }
  // Ranks kSpec .. k-1 of every list (one flat read).
  int32_t loaded = min(spec_total, total);
  auto load_rest = [&]() {
    constexpr int kBatch = 16;
    for (int32_t e0 = loaded; e0 < total; e0 += 64 * kBatch) {
      uint64_t v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int32_t e = e0 + 64 * u + lane;
        v[u] = e < total ? src[e] : 0;
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int32_t e = e0 + 64 * u + lane;
        if (e < total) lists[e] = v[u];
      }
    }
    loaded = total;
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);

  // The top-n tokens in order.  The n-th largest list-head key is a lower
  // bound for the n-th largest key of the row (n heads reach it), and so is
  // T, that key with its low 16 bits cleared (the bisection stops there; a
  // few more heads may reach T); the list prefixes with keys >= T hold the
  // top n.  Usually a few dozen: one wave sorts them in registers.  More
  // than 512 (many equal keys) take a tournament instead: lane j holds list
  // j's head; the wave maximum is the next token.
  // Ranks 0 .. lim-1 of list j in lane j's registers, read in one round.
  const int32_t lim = loaded / p.n_chunks;
  uint64_t r[kSpec];
#pragma unroll
  for (int u = 0; u < kSpec; ++u)
    r[u] = (lane < p.n_chunks && u < lim) ? lists[u * p.n_chunks + lane] : 0;
  const uint64_t head = r[0];
  uint32_t T = 0;
  if (n <= p.n_chunks) T = wave_mth_largest<16>(static_cast<uint32_t>(head >> 32), n);
  // c = list j's entries with keys >= T (lane j): a prefix, as a list is in
  // descending order; first within the ranks already loaded, and a list that
  // fills them continues after the rest is read.
  int32_t c = 0;
  if (lane < p.n_chunks) {
#pragma unroll
    for (int u = 0; u < kSpec; ++u)
      c += (u < lim && static_cast<uint32_t>(r[u] >> 32) >= T) ? 1 : 0;
  }
  if (__ballot(lane < p.n_chunks && c == lim && lim < k) != 0) {
    load_rest();
    if (lane < p.n_chunks && c == lim)
      while (c < k && static_cast<uint32_t>(lists[c * p.n_chunks + lane] >> 32) >= T) ++c;
  }
  const uint32_t cincl = wave_incl_scan(static_cast<uint32_t>(c));
  const uint32_t total_c = __builtin_amdgcn_readlane(cincl, 63);
  if (total_c <= 64 * kWaveSortE) {
    const int32_t pos = static_cast<int32_t>(cincl) - c;
#pragma unroll
    for (int u = 0; u < kSpec; ++u)
      if (u < c) top[pos + u] = r[u];
    for (int32_t i = kSpec; i < c; ++i) top[pos + i] = lists[i * p.n_chunks + lane];
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (total_c <= 32)
      sort_top32(top, total_c);
    else if (total_c <= 64)
      sort_top<1>(top, total_c);
    else if (total_c <= 128)
      sort_top<2>(top, total_c);
    else if (total_c <= 256)
      sort_top<4>(top, total_c);
    else
      sort_top<8>(top, total_c);
  } else {
    if (loaded < total) load_rest();
    int32_t at = 0;
    uint64_t h = head;
    for (int32_t s = 0; s < n; ++s) {
      const uint64_t best = wave_max_u64(h);
      if (lane == 0) top[s] = best;
      if (h == best) {
        ++at;
        h = at < k ? lists[at * p.n_chunks + lane] : 0;
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);

  // Top-p over the n tokens: lane l holds tokens 4l .. 4l+3.
  constexpr float kLog2e = 1.4426950408889634f;
  const float m = value_of(static_cast<uint32_t>(top[0] >> 32));
  float w[4];
  float lsum = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int32_t i = 4 * lane + e;
    w[e] = i < n ? __builtin_amdgcn_exp2f((value_of(static_cast<uint32_t>(top[i] >> 32)) - m) *
                                          kLog2e)
                 : 0.f;
    lsum += w[e];
  }
  // Wave prefix sum of the lane sums (DPP row shifts and broadcasts: a fixed
  // order, so the result is deterministic), then each token's mass before it.
  auto fadd = [](float x, uint32_t y) { return x + __uint_as_float(y); };
  float incl = lsum;
  incl = fadd(incl, dpp_u32<0x111, 0xf>(__float_as_uint(incl)));
  incl = fadd(incl, dpp_u32<0x112, 0xf>(__float_as_uint(incl)));
  incl = fadd(incl, dpp_u32<0x114, 0xf>(__float_as_uint(incl)));
  incl = fadd(incl, dpp_u32<0x118, 0xf>(__float_as_uint(incl)));
  incl = fadd(incl, dpp_u32<0x142, 0xa>(__float_as_uint(incl)));
  incl = fadd(incl, dpp_u32<0x143, 0xc>(__float_as_uint(incl)));
  const float W = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(incl), 63));
  float before = incl - lsum;
  int32_t keep = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int32_t i = 4 * lane + e;
    if (i < n && (i == 0 || pp >= 1.0f || before / W < pp)) keep = i + 1;
    before += w[e];
  }
  // Kept tokens form a prefix of the order: the count is the largest keep.
  keep = static_cast<int32_t>(wave_max_u32(static_cast<uint32_t>(keep)));
  // The kept tokens (a prefix of the order) get their logits back; the
  // rest of the row holds the -inf chunk_top_kernel wrote.
  // Every kept entry is a real token (list padding is the value 0, below all
  // of them, and there are at least n real ones); the range check keeps the
  // store inside the row regardless.
  float* out = p.out + static_cast<int64_t>(row) * p.out_stride;
  for (int32_t i = lane; i < keep; i += 64) {
    const uint64_t t = top[i];
    const uint32_t idx = ~static_cast<uint32_t>(t);
    if (idx < static_cast<uint32_t>(p.vocab)) out[idx] = value_of(static_cast<uint32_t>(t >> 32));
  }
  if (lane == 0 && p.status) p.status[row] = 0;
}

}  // namespace

void plan_chunks(int32_t vocab, int32_t* chunk, int32_t* n_chunks) {
  if (vocab < 1 || vocab > kMaxVocab) {
    *chunk = 0;
    *n_chunks = 0;
    return;
  }
  int32_t c = (vocab + kMaxChunks - 1) / kMaxChunks;
  c = (c + 1023) / 1024 * 1024;
  c = c < kMinChunk ? kMinChunk : c;
  *chunk = c;
  *n_chunks = (vocab + c - 1) / c;
}

size_t workspace_bytes(int32_t rows, int32_t vocab, int32_t k_max) {
  int32_t chunk = 0, n_chunks = 0;
  plan_chunks(vocab, &chunk, &n_chunks);
  return sizeof(uint64_t) * static_cast<size_t>(rows) * n_chunks * k_max;
}

hipError_t launch_mask(const MaskParams& p, hipStream_t stream) {
  if (p.rows <= 0) return hipSuccess;
  // The candidate buffer holds a whole chunk (every entry can be a
  // candidate when many logits tie), padded to the sort's power of two.
  size_t pow2 = 64;
  while (pow2 < static_cast<size_t>(p.chunk)) pow2 <<= 1;
  const size_t lds1 = sizeof(uint64_t) * pow2;
  const dim3 grid1(p.n_chunks, p.rows);
  if (p.chunk <= 16 * kThreads) {
    const hipError_t e1 =
        pgqa_launch::launch(chunk_top_kernel<16>, grid1, dim3(kThreads), lds1, stream, p);
    if (e1 != hipSuccess) return e1;  // the cut kernel would read an unfilled workspace
  } else {
    if (lds1 > 65536 - 64) {
      static const hipError_t raised = hipFuncSetAttribute(
          reinterpret_cast<const void*>(chunk_top_kernel<kMaxChunk / kThreads>),
          hipFuncAttributeMaxDynamicSharedMemorySize,
          static_cast<int>(sizeof(uint64_t) * kMaxChunk));
      if (raised != hipSuccess) return raised;
    }
    const hipError_t e1 = pgqa_launch::launch(chunk_top_kernel<kMaxChunk / kThreads>, grid1,
                                              dim3(kThreads), lds1, stream, p);
    if (e1 != hipSuccess) return e1;
  }
  const size_t lds = sizeof(uint64_t) * static_cast<size_t>(p.n_chunks) * p.k_max;
  if (lds > 65536) {
    static const hipError_t raised = hipFuncSetAttribute(
        reinterpret_cast<const void*>(cut_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
        static_cast<int>(sizeof(uint64_t) * kMaxChunks * kMaxK));
    if (raised != hipSuccess) return raised;
  }
  return pgqa_launch::launch(cut_kernel, dim3(p.rows), dim3(64), lds, stream, p);
}

}  // namespace sampler
