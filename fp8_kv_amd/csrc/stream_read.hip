// Plain streaming read of device memory: a measurement aid that sits beside
// the attention path and is not part of it (its own library, libstream_read.so;
// no attention entry point calls it).
//
// It reads the bytes of two buffers exactly once with 16-byte vector loads,
// either non-temporal (the hint the decode kernels put on K and V loads, which
// also keeps the bytes out of the last-level cache) or ordinary (as sparse
// prefill reads its shared pool, so a warm buffer can be served from that
// cache).  It computes nothing but an XOR checksum per workgroup, so the
// loads cannot be dropped and a test can check that every byte was read.  Its rate is the read
// bandwidth that those bytes can reach on this device with no page-table
// indirection, no dependent round trips and no arithmetic: the ceiling the
// attention kernel's KV rate is compared with (non-temporal, buffers rotated
// for decode; ordinary loads over one warm pool for sparse prefill).
//
// Layout: the two buffers form one range of 16-byte words (all of a, then
// all of b); workgroup w reads the contiguous words [w*C, (w+1)*C) of that
// range, C = ceil(words / blocks) rounded up to 256 words (4 KiB), so each
// wave instruction reads one aligned 1 KiB run.  sink[w] (16 bytes) receives
// the XOR of the words workgroup w read (zero for a workgroup with none).
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "launch_util.h"

namespace {

typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;         // 16-byte loads in flight per thread
constexpr int kMaxBlocks = 1 << 16;

template <bool NT>
__device__ inline u4_t load16(const u4_t* ptr) {
  if constexpr (NT) return __builtin_nontemporal_load(ptr);
  else return *ptr;
}

// XORs the cnt words at base (a uniform start) into acc: lane t reads words
// t, t + 256, ... with kUnroll loads in flight, each at an immediate offset
// from one per-iteration address; a word past cnt re-reads word i and is
// dropped.  (Computing a full 64-bit address per load, with a select between
// the two buffers, read the same bytes about 4% slower.)
template <bool NT>
__device__ __forceinline__ void read_range(const u4_t* __restrict__ base, uint32_t cnt, u4_t& acc) {
  for (uint32_t i = threadIdx.x; i < cnt; i += kThreads * kUnroll) {
    const u4_t* ptr = base + i;
    u4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      v[u] = load16<NT>(i + u * kThreads < cnt ? ptr + u * kThreads : ptr);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      acc ^= i + u * kThreads < cnt ? v[u] : u4_t{0u, 0u, 0u, 0u};
  }
}

template <bool NT>
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u4_t* __restrict__ a,
                                                               size_t na,
                                                               const u4_t* __restrict__ b,
                                                               size_t per_block, size_t n,
                                                               u4_t* __restrict__ sink) {
  const size_t begin = static_cast<size_t>(blockIdx.x) * per_block;
  const size_t end = begin + per_block < n ? begin + per_block : n;
  u4_t acc = {0u, 0u, 0u, 0u};
  // The words [begin, end) of the range a ++ b: the part in a, then the part
  // in b (per_block < 2^32 words, checked on the host).
  if (begin < end) {
    const size_t a_end = end < na ? end : na;
    if (begin < a_end) read_range<NT>(a + begin, static_cast<uint32_t>(a_end - begin), acc);
    const size_t b_begin = begin > na ? begin : na;
    if (b_begin < end) read_range<NT>(b + (b_begin - na), static_cast<uint32_t>(end - b_begin), acc);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    acc.x ^= __shfl_xor(acc.x, off);
    acc.y ^= __shfl_xor(acc.y, off);
    acc.z ^= __shfl_xor(acc.z, off);
    acc.w ^= __shfl_xor(acc.w, off);
  }
  __shared__ u4_t part[kThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    u4_t r = part[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) r ^= part[w];
    sink[blockIdx.x] = r;
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// One wave reads the shader-clock counter (s_memtime) and the constant
// 100 MHz real-time counter (s_memrealtime) at the start and end of a spin of
// about `ticks` real-time ticks; out[0] = real-time ticks elapsed, out[1] =
// shader-clock ticks over the same interval.  The spin ends after at most
// kMaxProbeIters iterations whatever the counters do.
constexpr int kMaxProbeIters = 1 << 22;
__global__ void clock_probe_kernel(uint64_t* out, uint32_t ticks) {
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  uint64_t r1 = r0, t1 = t0;
  for (int i = 0; i < kMaxProbeIters && r1 - r0 < ticks; ++i) {
    r1 = __builtin_amdgcn_s_memrealtime();
    t1 = __builtin_amdgcn_s_memtime();
  }
  if (threadIdx.x == 0) {
    out[0] = r1 - r0;
    out[1] = t1 - t0;
  }
}

}  // namespace

extern "C" {

// Return codes: 0 success, -1 a required pointer is NULL, -2 a size is out
// of range (blocks outside 1..65536, a byte count not a multiple of 16, or
// 2^32 - 2048 or more 16-byte words per workgroup), -3
// a pointer is not 16-byte aligned, -4 the launch failed.  Nothing is
// launched on an error.
//
// a, b: device buffers of a_bytes and b_bytes (multiples of 16; a buffer of
// 0 bytes may be NULL).  blocks: workgroups of 256 threads.  nontemporal:
// nonzero for non-temporal loads, 0 for ordinary ones.  sink: device memory
// of 16*blocks bytes, overwritten.  stream: a hipStream_t (NULL = the
// default stream).  Asynchronous.
int stream_read(const void* a, size_t a_bytes, const void* b, size_t b_bytes, int32_t blocks,
                int32_t nontemporal, void* sink, void* stream) {
  if (!sink || (a_bytes && !a) || (b_bytes && !b)) return -1;
  if (blocks < 1 || blocks > kMaxBlocks || (a_bytes | b_bytes) % 16) return -2;
  if (!aligned16(sink) || (a_bytes && !aligned16(a)) || (b_bytes && !aligned16(b))) return -3;
  const size_t na = a_bytes / 16, n = na + b_bytes / 16;
  size_t per_block = (n + blocks - 1) / blocks;
  per_block = (per_block + kThreads - 1) / kThreads * kThreads;
  if (per_block >= (size_t{1} << 32) - kThreads * kUnroll) return -2;  // 32-bit word counts
  const auto* pa = static_cast<const u4_t*>(a);
  const auto* pb = static_cast<const u4_t*>(b);
  auto* ps = static_cast<u4_t*>(sink);
  const auto st = static_cast<hipStream_t>(stream);
  const hipError_t e =
      nontemporal
          ? pgqa_launch::launch(stream_read_kernel<true>, dim3(blocks), dim3(kThreads), 0, st, pa,
                                na, pb, per_block, n, ps)
          : pgqa_launch::launch(stream_read_kernel<false>, dim3(blocks), dim3(kThreads), 0, st,
                                pa, na, pb, per_block, n, ps);
  return e == hipSuccess ? 0 : -4;
}

// Shader clock over a short spin (benchmark bookkeeping: the clock the
// device ran at right after a timed batch).  out: device memory of two
// uint64 (8-byte aligned): real-time ticks (100 MHz) and shader-clock ticks
// over the same interval, so MHz = 100 * out[1] / out[0].  ticks: spin
// length in real-time ticks, 1..100000 (10 ns each).  Returns 0, -1 (out
// NULL), -2 (ticks out of range), -3 (out not 8-byte aligned) or -4 (launch
// failed).  Asynchronous.
int clock_probe(void* out, int32_t ticks, void* stream) {
  if (!out) return -1;
  if (ticks < 1 || ticks > 100000) return -2;
  if (reinterpret_cast<uintptr_t>(out) & 7) return -3;
  const hipError_t e =
      pgqa_launch::launch(clock_probe_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                          static_cast<uint64_t*>(out), static_cast<uint32_t>(ticks));
  return e == hipSuccess ? 0 : -4;
}

}  // extern "C"
