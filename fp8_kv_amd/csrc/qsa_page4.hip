// gfx950 kernel that turns expanded QSA selections into virtual page-4 tables
// for sparse prefill.
//
// Source: "[Kernel][SM70] Accelerate Qwen3.8 QSA paged prefill", Purpose and
// Changes: every selected 4-token block becomes one zero-copy page of a
// page-4 view of the KV pool, the pages are sorted for locality, the causal
// partial page goes last and is checked against the expanded selection,
// positions past the live length are clamped away and invalid rows are made
// inert.  The operation (per row r, live length L, causal block c = (L-1)/4):
//   S      = the distinct selected positions t with 0 <= t < L;
//   pages  = blocks b < c with all four of 4b..4b+3 in S (any other position
//            of S below 4c makes the row invalid: PARTIAL);
//   tail   = S ∩ [4c, L), which must be 4c .. 4c+n_tail-1 (else TAIL);
//   id(b)  = p * vpages_per_page + (4b mod P)/4 with p = block_table[4b/P]
//            (a missing or out-of-range p: PAGE);
//   output = the pages' ids ascending, then id(c) if n_tail > 0, then -1;
//            length 4 * pages + n_tail.  Invalid rows: all -1, length 0.
//
// One wave (64 lanes) owns one row; nothing needs a workgroup barrier.
//   1. The row's positions are read with coalesced loads, eight per lane in
//      flight, and each live position below 4c is inserted into an LDS hash
//      set of blocks: a slot holds (block << 4) | mask, the mask having bit
//      t & 3 for every position seen (compare-and-swap claims an empty
//      slot, an atomic OR adds bits).  Duplicates and order drop out here.
//      Positions of the causal block only set bits of a per-lane mask.
//   2. A pass over the slots finds the full blocks (mask 0xF) and flags any
//      partial one; the full blocks are compacted by ballot into LDS.
//   3. Each block is mapped through the block table to its view id.
//   4. The ids are sorted in registers: a bitonic network over 64*E values,
//      E per lane (intra-lane stages are compare-exchanges, cross-lane ones
//      a lane shuffle).  Equal ids are equal values, so the result does not
//      depend on the hash layout, which concurrent inserts may vary.
//   5. The row is written with the causal page last and -1 padding.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr uint32_t kEmptySlot = 0xFFFFFFFFu;  // never a (block << 4) | mask with block < 2^24

// Orders this wave's LDS accesses: earlier ones complete before later ones
// start (a single wave needs no barrier for its own LDS traffic).
__device__ __forceinline__ void lds_fence_wave() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ uint32_t wave_or(uint32_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), o));
  return x;
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

// Adds position bit `bit` of block b to the hash set; returns false only if
// every slot was probed without finding b or an empty slot (cannot happen:
// the set has more slots than the row has positions).
__device__ __forceinline__ bool hash_insert(uint32_t* slots, uint32_t mask, int32_t log2,
                                            uint32_t b, uint32_t bit) {
  const uint32_t want = (b << 4) | bit;
  uint32_t h = (b * 0x9E3779B1u) >> (32 - log2);  // multiplicative hash: top bits
  for (uint32_t probe = 0; probe <= mask; ++probe) {
    uint32_t w = __hip_atomic_load(&slots[h], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (w == kEmptySlot) {
      const uint32_t old = atomicCAS(&slots[h], kEmptySlot, want);
      if (old == kEmptySlot) return true;
      w = old;
    }
    if ((w >> 4) == b) {
      atomicOr(&slots[h], bit);
      return true;
    }
    h = (h + 1) & mask;
  }
  return false;
}

// Ascending bitonic sort of the wave's 64*E values, lane l holding elements
// l*E .. l*E + E-1 (blocked order).
template <int E>
__device__ __forceinline__ void wave_sort(int32_t (&x)[E]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 2; k <= 64 * E; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j < E) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int f = e ^ j;
          if (f > e) {
            const bool asc = ((lane * E + e) & k) == 0;
            const int32_t a = x[e], b = x[f];
            const bool swap = asc ? (a > b) : (a < b);
            x[e] = swap ? b : a;
            x[f] = swap ? a : b;
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int i = lane * E + e;
          const int32_t y = __shfl_xor(x[e], j / E);
          const bool keep_min = (((i & j) == 0) == ((i & k) == 0));
          x[e] = keep_min ? min(x[e], y) : max(x[e], y);
        }
      }
    }
  }
}

template <int E>
__global__ __launch_bounds__(64) void page4_kernel(Page4Params p, int32_t hash_log2) {
  extern __shared__ uint32_t lds[];
  const uint32_t hmask = (1u << hash_log2) - 1u;
  uint32_t* slots = lds;                                       // [hmask + 1]
  int32_t* ids = reinterpret_cast<int32_t*>(lds + hmask + 1);  // [64 E + 1]
  const int row = blockIdx.x;
  const int lane = threadIdx.x;
  int32_t* orow = p.out_table + static_cast<int64_t>(row) * p.out_stride;
  const int32_t L = p.live_len[row];

  int32_t status = 0;
  if (L <= 0) status = kPage4Empty;
  if (L > kPage4MaxLive) status = kPage4Long;
  int32_t n_full = 0, n_tail = 0;
  if (status == 0) {
    const int32_t c = (L - 1) >> 2;
    for (uint32_t i = lane; i <= hmask; i += 64) slots[i] = kEmptySlot;
    lds_fence_wave();

    // ---- 1. positions -> hash set of blocks (causal block: lane masks)
    const int32_t* trow = p.tokens + static_cast<int64_t>(row) * p.token_stride;
    uint32_t tmask = 0;
    bool lost = false;
    constexpr int kBatch = 8;
    for (int32_t base = 0; base < p.n_tokens; base += 64 * kBatch) {
      int32_t t[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int32_t i = base + 64 * u + lane;
        t[u] = i < p.n_tokens ? trow[i] : -1;
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (t[u] < 0 || t[u] >= L) continue;
        const uint32_t b = static_cast<uint32_t>(t[u]) >> 2;
        const uint32_t bit = 1u << (t[u] & 3);
        if (b == static_cast<uint32_t>(c))
          tmask |= bit;
        else
          lost |= !hash_insert(slots, hmask, hash_log2, b, bit);
      }
    }
    lds_fence_wave();
    tmask = wave_or(tmask);
    n_tail = __popc(tmask);
    if (n_tail > 0 && tmask != (1u << n_tail) - 1u) status |= kPage4Tail;
    if (__ballot(lost)) status |= kPage4Overflow;

    // ---- 2. full blocks, compacted in slot order; any partial block flags
    bool partial = false;
    for (uint32_t i = lane; i <= hmask; i += 64) {
      const uint32_t w = slots[i];
      const bool used = w != kEmptySlot;
      const bool full = used && (w & 15u) == 15u;
      partial |= used && !full;
      const uint64_t fm = __ballot(full);
      if (full) ids[n_full + static_cast<int32_t>(lanes_below(fm))] = static_cast<int32_t>(w >> 4);
      n_full += static_cast<int32_t>(__popcll(fm));
    }
    if (__ballot(partial)) status |= kPage4Partial;
    const int32_t n_pages = n_full + (n_tail > 0 ? 1 : 0);
    if (n_pages > p.out_stride) status |= kPage4Overflow;
    if (n_tail > 0 && lane == 0) ids[n_full] = c;
    lds_fence_wave();

    // ---- 3. block -> view id through the sequence's block table
    const int32_t seq = p.row_seq ? p.row_seq[row] : 0;
    if (seq < 0 || seq >= p.n_seqs) {
      status |= kPage4Seq;
    } else {
      const int32_t* btab = p.block_table + static_cast<int64_t>(seq) * p.max_pages;
      const int32_t quarter = p.page_size >> 2;  // 4-token groups per physical page
      bool bad = false;
      for (int32_t j = lane; j < n_pages; j += 64) {
        const int32_t b = ids[j];
        const int32_t lp = b / quarter;
        const int32_t pg = lp < p.max_pages ? btab[lp] : -1;
        const bool ok = pg >= 0 && pg < p.num_pages;
        bad |= !ok;
        ids[j] = ok ? pg * p.vpages_per_page + (b - lp * quarter) : -1;
      }
      if (__ballot(bad)) status |= kPage4Page;
    }
    lds_fence_wave();

    // ---- 4. locality order of the full pages
    if (status == 0 && n_full > 1) {
      int32_t x[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int32_t i = lane * E + e;
        x[e] = i < n_full ? ids[i] : INT32_MAX;
      }
      wave_sort<E>(x);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int32_t i = lane * E + e;
        if (i < n_full) ids[i] = x[e];
      }
      lds_fence_wave();
    }
  }

  // ---- 5. the row: pages, causal page last, -1 padding; inert if invalid
  const int32_t n_out = status == 0 ? n_full + (n_tail > 0 ? 1 : 0) : 0;
  for (int32_t i = lane; i < p.out_stride; i += 64) orow[i] = i < n_out ? ids[i] : -1;
  if (lane == 0) {
    p.out_len[row] = status == 0 ? 4 * n_full + n_tail : 0;
    if (p.out_status) p.out_status[row] = status;
  }
}

template <int E>
hipError_t launch_e(const Page4Params& p, int32_t hash_log2, hipStream_t stream) {
  const size_t lds = sizeof(uint32_t) * ((size_t{1} << hash_log2) + 64 * E + 1);
  if (lds > 65536) {
    // Beyond the default 64 KiB of dynamic LDS the limit must be raised
    // (once per process and instance; the largest size this instance uses).
    static const hipError_t raised = hipFuncSetAttribute(
        reinterpret_cast<const void*>(page4_kernel<E>),
        hipFuncAttributeMaxDynamicSharedMemorySize,
        static_cast<int>(sizeof(uint32_t) * (2 * kPage4MaxTokens + 64 * E + 1)));
    if (raised != hipSuccess) return raised;
  }
  hipLaunchKernelGGL(page4_kernel<E>, dim3(static_cast<unsigned>(p.rows)), dim3(64), lds, stream,
                     p, hash_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_page4(const Page4Params& p, hipStream_t stream) {
  if (p.rows <= 0) return hipSuccess;
  // More slots than positions (an empty slot always remains), at least one
  // per lane.
  int32_t hash_log2 = 6;
  while ((1 << hash_log2) <= p.n_tokens) ++hash_log2;
  // Full pages per row are at most n_tokens / 4; the sort holds 64 E.
  const int32_t max_full = p.n_tokens / 4;
  if (max_full <= 64) return launch_e<1>(p, hash_log2, stream);
  if (max_full <= 128) return launch_e<2>(p, hash_log2, stream);
  if (max_full <= 256) return launch_e<4>(p, hash_log2, stream);
  if (max_full <= 512) return launch_e<8>(p, hash_log2, stream);
  if (max_full <= 1024) return launch_e<16>(p, hash_log2, stream);
  return launch_e<32>(p, hash_log2, stream);
}

}  // namespace qsa
