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
// means earlier in the order, and all such values are distinct.  The kept
// tokens are exactly those at or above the last kept token's value (the
// row's "cut"), so the masked row is one comparison per logit.
//
// Three launches:
//   1. chunk_top_kernel, one 256-thread workgroup per (chunk of <= 8192
//      logits, row): the chunk's top min(k, chunk) tokens in order.  A
//      threshold T from the lane maxima (each of the four waves contributes
//      ceil(k/4) lanes whose maximum is >= T, so at least k keys are >= T)
//      leaves a few candidates, which an LDS bitonic sort orders.
//   2. cut_kernel, one wave per row: a tournament over the <= 64 sorted chunk
//      lists (each lane holds one list's head; the wave maximum is the next
//      token) yields the top-k set in order; then the softmax masses in fp32
//      (exp2 with log2(e) folded in), a wave prefix sum, and the cut.
//   3. apply_kernel: out = logit where its value >= cut, else -inf (rows that
//      are invalid are copied).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sampler_internal.h"

namespace sampler {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kPerThread = kMaxChunk / kThreads;  // 32

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
// on the bits from the top.
__device__ __forceinline__ uint32_t wave_mth_largest(uint32_t x, uint32_t m) {
  uint32_t res = 0;
#pragma unroll
  for (int b = 31; b >= 0; --b) {
    const uint32_t trial = res | (1u << b);
    const uint32_t c = static_cast<uint32_t>(__popcll(__ballot((x >> b) == (trial >> b))));
    if (c >= m)
      res = trial;
    else
      m -= c;
  }
  return res;
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = static_cast<uint32_t>(__shfl_up(static_cast<int>(x), d));
    if (lane >= d) x += y;
  }
  return x;
}

__global__ __launch_bounds__(kThreads) void chunk_top_kernel(MaskParams p) {
  extern __shared__ uint64_t cand[];  // [pow2 >= chunk] candidates, then padding
  __shared__ uint32_t wval[kWaves];
  const int chunk = blockIdx.x;
  const int row = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int32_t k;
  float pp;
  if (!row_valid(p, row, k, pp)) return;  // the row is copied by apply_kernel
  const int32_t start = chunk * p.chunk;
  const int32_t len = min(p.chunk, p.vocab - start);
  const int32_t kc = min(k, len);
  const float* src = p.logits + static_cast<int64_t>(row) * p.row_stride + start;

  // Thread t holds entries t + 256 i; key 0 (never a logit's key but the
  // negative NaN 0xFFFFFFFF's) marks entries past the chunk.
  uint32_t key[kPerThread];
  uint32_t lmax = 0;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int32_t e = tid + kThreads * i;
    key[i] = e < len ? key_of(src[e]) : 0u;
    lmax = max(lmax, key[i]);
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
  for (int i = 0; i < kPerThread; ++i) cnt += (tid + kThreads * i < len && key[i] >= T) ? 1u : 0u;
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
  for (int i = 0; i < kPerThread; ++i) {
    const int32_t e = tid + kThreads * i;
    if (e < len && key[i] >= T) cand[pos++] = token(key[i], start + e);
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
  uint64_t* dst = p.cand + (static_cast<int64_t>(row) * p.n_chunks + chunk) * p.k_max;
  for (int32_t i = tid; i < k; i += kThreads) dst[i] = i < kc ? cand[i] : 0;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t hi = static_cast<uint32_t>(__shfl_xor(static_cast<int>(x >> 32), o));
    const uint32_t lo = static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), o));
    const uint64_t y = (static_cast<uint64_t>(hi) << 32) | lo;
    x = x > y ? x : y;
  }
  return x;
}

__global__ __launch_bounds__(64) void cut_kernel(MaskParams p) {
  extern __shared__ uint64_t lists[];  // [n_chunks][k]
  __shared__ uint64_t top[kMaxK];
  const int row = blockIdx.x;
  const int lane = threadIdx.x;
  int32_t k;
  float pp;
  if (!row_valid(p, row, k, pp)) {
    if (lane == 0) {
      p.cut[row] = 0;
      if (p.status) p.status[row] = (k >= 1 && k <= p.k_max ? 0 : kBadK) |
                                    (__builtin_isnan(pp) ? kBadP : 0);
    }
    return;
  }
  const int32_t n = min(k, p.vocab);
  // The chunk lists of the row (list j at lists + j * k), loaded together.
  const uint64_t* src = p.cand + static_cast<int64_t>(row) * p.n_chunks * p.k_max;
  for (int32_t j = 0; j < p.n_chunks; ++j)
    for (int32_t i = lane; i < k; i += 64) lists[j * k + i] = src[j * p.k_max + i];
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);

  // Tournament: lane j holds list j's head; the wave maximum is the next
  // token in the order.
  int32_t at = 0;
  uint64_t head = lane < p.n_chunks ? lists[lane * k] : 0;
  for (int32_t s = 0; s < n; ++s) {
    const uint64_t best = wave_max_u64(head);
    if (lane == 0) top[s] = best;
    if (head == best) {
      ++at;
      head = at < k ? lists[lane * k + at] : 0;
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
  // Wave prefix sum of the lane sums (fixed order: the result is
  // deterministic), then each token's mass before it.
  float incl = lsum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const float y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  const float W = __shfl(incl, 63);
  float before = incl - lsum;
  int32_t keep = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int32_t i = 4 * lane + e;
    if (i < n && (i == 0 || pp >= 1.0f || before / W < pp)) keep = i + 1;
    before += w[e];
  }
  // Kept tokens form a prefix of the order: the count is the largest keep.
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) keep = max(keep, __shfl_xor(keep, o));
  if (lane == 0) {
    p.cut[row] = top[keep - 1];
    if (p.status) p.status[row] = 0;
  }
}

__global__ __launch_bounds__(256) void apply_kernel(MaskParams p) {
  const int row = blockIdx.y;
  const uint64_t cut = p.cut[row];
  const float* src = p.logits + static_cast<int64_t>(row) * p.row_stride;
  float* dst = p.out + static_cast<int64_t>(row) * p.out_stride;
  const int32_t base = blockIdx.x * (256 * 16);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int32_t t = base + 256 * i + static_cast<int32_t>(threadIdx.x);
    if (t < p.vocab) {
      const float z = src[t];
      dst[t] = (cut == 0 || token(key_of(z), t) >= cut) ? z : -__builtin_huge_valf();
    }
  }
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
  const size_t cand = sizeof(uint64_t) * static_cast<size_t>(rows) * n_chunks * k_max;
  return cand + sizeof(uint64_t) * static_cast<size_t>(rows);
}

hipError_t launch_mask(const MaskParams& p, hipStream_t stream) {
  if (p.rows <= 0) return hipSuccess;
  // The candidate buffer holds a whole chunk (every entry can be a
  // candidate when many logits tie), padded to the sort's power of two.
  size_t pow2 = 64;
  while (pow2 < static_cast<size_t>(p.chunk)) pow2 <<= 1;
  const size_t lds1 = sizeof(uint64_t) * pow2;
  if (lds1 > 65536 - 64) {
    static const hipError_t raised = hipFuncSetAttribute(
        reinterpret_cast<const void*>(chunk_top_kernel),
        hipFuncAttributeMaxDynamicSharedMemorySize,
        static_cast<int>(sizeof(uint64_t) * kMaxChunk));
    if (raised != hipSuccess) return raised;
  }
  hipLaunchKernelGGL(chunk_top_kernel, dim3(p.n_chunks, p.rows), dim3(kThreads), lds1, stream, p);
  const size_t lds = sizeof(uint64_t) * static_cast<size_t>(p.n_chunks) * p.k_max;
  if (lds > 65536) {
    static const hipError_t raised = hipFuncSetAttribute(
        reinterpret_cast<const void*>(cut_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
        static_cast<int>(sizeof(uint64_t) * kMaxChunks * kMaxK));
    if (raised != hipSuccess) return raised;
  }
  hipLaunchKernelGGL(cut_kernel, dim3(p.rows), dim3(64), lds, stream, p);
  const unsigned blocks = static_cast<unsigned>((p.vocab + 256 * 16 - 1) / (256 * 16));
  hipLaunchKernelGGL(apply_kernel, dim3(blocks, p.rows), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sampler
