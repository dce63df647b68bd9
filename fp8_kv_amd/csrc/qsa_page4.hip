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
// One wave (64 lanes) owns one row; a workgroup of four waves shares the
// hash set of the general path, which its waves use one at a time.
//   1. Collection of the full blocks and the causal positions, two ways:
//      - Expanded layout (no atomics): the row read as chunks of four entries
//        from its start (one 16-byte load each); a chunk 4b, 4b+1, 4b+2,
//        4b+3 with b < c is that full block (compacted by ballot), a chunk
//        of padding, stale or causal-block positions only adds to the
//        causal mask.  A row
//        with any other chunk takes the general path; so does one whose
//        sorted ids hold two equal neighbours (a block listed twice, or two
//        blocks on one physical page: the general path settles which).
//      - General: the row read with 16-byte loads, twelve per lane in
//        flight; each lane merges a chunk's positions of one block into a
//        4-bit mask and adds (block, mask) to an LDS hash set whose slots hold
//        (block << 4) | mask: a compare-and-swap claims an empty slot, an
//        atomic OR adds bits to a claimed one.  The operation that makes a
//        slot's mask 0xF appends the block to the list of full blocks
//        (exactly one does, since the ORs are atomic); claims are counted,
//        and PARTIAL is "claims != full blocks".  Duplicates and order drop
//        out here.
//   2. Each full block is mapped through the block table to its view id,
//      the table entries of up to 16 blocks per lane loaded together.
//   3. The ids are sorted in registers: a bitonic network over 64*E values,
//      E per lane.  A merge level whose direction depends on the lane runs on
//      complemented values in descending lanes, so every stage is a plain
//      min/max; cross-lane partners arrive by DPP (lane distance 1, 2, 4, 8)
//      or a lane shuffle (16, 32).
//      Equal ids are equal values, so the result does not depend on the
//      order of the full-block list, which concurrent inserts may vary.
//   4. The row is written with the causal page last and -1 padding.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch_util.h"
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

struct Insert {
  bool claimed;    // this call took an empty slot (a new block)
  bool completed;  // this call made the block's mask 0xF
  bool lost;       // every slot probed (cannot happen: more slots than positions)
};

// Adds position mask `bits` of block b to the hash set.  One compare-and-swap
// per probe: it claims an empty slot, or returns the slot's block.
__device__ __forceinline__ Insert hash_insert(uint32_t* slots, uint32_t mask, int32_t log2,
                                              uint32_t b, uint32_t bits) {
  const uint32_t want = (b << 4) | bits;
  uint32_t h = (b * 0x9E3779B1u) >> (32 - log2);  // multiplicative hash: top bits
  for (uint32_t probe = 0; probe <= mask; ++probe) {
    const uint32_t old = atomicCAS(&slots[h], kEmptySlot, want);
    if (old == kEmptySlot) return Insert{true, bits == 15u, false};
    if ((old >> 4) == b) {
      if ((old & bits) == bits) return Insert{false, false, false};  // nothing new
      const uint32_t prev = atomicOr(&slots[h], bits);
      return Insert{false, (prev & 15u) != 15u && ((prev | bits) & 15u) == 15u, false};
    }
    h = (h + 1) & mask;
  }
  return Insert{false, false, true};
}

// One cross-lane compare-exchange of a bitonic stage whose pairs are lane
// distance M apart, every pair ascending: the lane with bit M clear keeps the
// smaller value, its partner the larger.  Distances 1, 2, 4, 8 move the
// partner's value with DPP (quad permutes, or row shifts within 16 lanes);
// 16 and 32 with gfx950's lane-swap instructions (v_permlane16_swap and
// v_permlane32_swap with the value as both operands: the partner's value is
// the first result in the lanes with bit M set, the second in the others).
template <int M>
__device__ __forceinline__ int32_t exchange(int32_t x) {
  const bool upper = (threadIdx.x & M) != 0;
  if constexpr (M == 1 || M == 2) {
    const int32_t y = __builtin_amdgcn_update_dpp(0, x, M == 1 ? 0xB1 : 0x4E, 0xF, 0xF, false);
    return upper ? max(x, y) : min(x, y);
  } else if constexpr (M == 4 || M == 8) {
    const int32_t from_above = __builtin_amdgcn_update_dpp(0, x, 0x100 + M, 0xF, 0xF, false);
    const int32_t from_below = __builtin_amdgcn_update_dpp(0, x, 0x110 + M, 0xF, 0xF, false);
    return upper ? max(x, from_below) : min(x, from_above);
  } else {
    static_assert(M == 16 || M == 32, "lane distances within a wave");
    const auto r = M == 16 ? __builtin_amdgcn_permlane16_swap(x, x, false, false)
                           : __builtin_amdgcn_permlane32_swap(x, x, false, false);
    const int32_t y = static_cast<int32_t>(upper ? r[0] : r[1]);
    return upper ? max(x, y) : min(x, y);
  }
}

// Stages J, J/2, .., 1 of a bitonic merge level whose pairs all ascend
// (element i = lane*E + e; i ^ J lives in the same lane when J < E, in lane
// lane ^ (J / E) otherwise).
template <int E, int J>
__device__ __forceinline__ void ascending_stages(int32_t (&x)[E]) {
  if constexpr (J >= 1) {
    if constexpr (J < E) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if ((e ^ J) > e) {
          const int32_t a = x[e], b = x[e ^ J];
          x[e] = min(a, b);
          x[e ^ J] = max(a, b);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) x[e] = exchange<J / E>(x[e]);
    }
    ascending_stages<E, J / 2>(x);
  }
}

// Merge level K of the bitonic sort: element i ascends when (i & K) == 0.
// For K >= E that direction is a property of the lane; a descending lane
// complements its values (which reverses their order), merges ascending and
// complements back.  For K < E it is a property of e alone.
template <int E, int K>
__device__ __forceinline__ void bitonic_level(int32_t (&x)[E]) {
  if constexpr (K >= E) {
    const int32_t flip = ((threadIdx.x & 63) * E) & K ? -1 : 0;
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] ^= flip;
    ascending_stages<E, K / 2>(x);
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] ^= flip;
  } else {
#pragma unroll
    for (int j = K / 2; j >= 1; j /= 2) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if ((e ^ j) > e) {
          const int32_t a = x[e], b = x[e ^ j];
          const bool asc = (e & K) == 0;
          x[e] = asc ? min(a, b) : max(a, b);
          x[e ^ j] = asc ? max(a, b) : min(a, b);
        }
      }
    }
  }
}

template <int E, int K>
__device__ __forceinline__ void bitonic_levels(int32_t (&x)[E]) {
  if constexpr (K <= 64 * E) {
    bitonic_level<E, K>(x);
    bitonic_levels<E, 2 * K>(x);
  }
}

// Ascending bitonic sort of the wave's 64*E values, lane l holding elements
// l*E .. l*E + E-1 (blocked order).
template <int E>
__device__ __forceinline__ void wave_sort(int32_t (&x)[E]) {
  bitonic_levels<E, 2>(x);
}

// What the collection of a row's selection yields.
struct Collected {
  int32_t n_full;     // full blocks appended to ids[0 .. n_full)
  int32_t n_claimed;  // distinct blocks below the causal block
  uint32_t tmask;     // this lane's causal-block positions (bit t & 3)
  bool lost;          // a hash insert found no slot (cannot happen)
};

// The general collection: every position through the LDS hash set.
__device__ __forceinline__ Collected collect_hash(const Page4Params& p, const int32_t* trow,
                                                  int32_t L, int32_t c, uint32_t* slots,
                                                  uint32_t hmask, int32_t hash_log2,
                                                  int32_t* ids) {
  const int lane = threadIdx.x & 63;
  int32_t n_full = 0;
  {
    uint4* s4 = reinterpret_cast<uint4*>(slots);
    const uint4 e4 = make_uint4(kEmptySlot, kEmptySlot, kEmptySlot, kEmptySlot);
    for (uint32_t i = lane; i <= (hmask >> 2); i += 64) s4[i] = e4;
  }
  lds_fence_wave();

  // The row is read as 16-byte chunks of the aligned span that covers it:
  // chunk i holds entries 4i - lead .. 4i - lead + 3 of the row; chunks
  // that stick out of the row (at most the first and the last) are read
  // entry by entry, so nothing outside the row is touched.
  const int32_t lead = static_cast<int32_t>((reinterpret_cast<uintptr_t>(trow) & 15u) >> 2);
  const int32_t n_chunks = (lead + p.n_tokens + 3) >> 2;
  uint32_t tmask = 0;
  int32_t n_claimed = 0;
  bool lost = false;
  constexpr int kChunks = 12;  // 16-byte loads per lane in flight
  for (int32_t c0 = 0; c0 < n_chunks; c0 += 64 * kChunks) {
    int4 v[kChunks];
#pragma unroll
    for (int u = 0; u < kChunks; ++u) {
      const int32_t ci = c0 + 64 * u + lane;
      const int32_t first = 4 * ci - lead;
      if (ci < n_chunks && first >= 0 && first + 4 <= p.n_tokens) {
        v[u] = *reinterpret_cast<const int4*>(trow + first);  // 16-byte aligned
      } else {
        const bool in = ci < n_chunks;
        v[u].x = in && first >= 0 && first < p.n_tokens ? trow[first] : -1;
        v[u].y = in && first + 1 >= 0 && first + 1 < p.n_tokens ? trow[first + 1] : -1;
        v[u].z = in && first + 2 >= 0 && first + 2 < p.n_tokens ? trow[first + 2] : -1;
        v[u].w = in && first + 3 >= 0 && first + 3 < p.n_tokens ? trow[first + 3] : -1;
      }
    }
#pragma unroll
    for (int u = 0; u < kChunks; ++u) {
      if (c0 + 64 * u >= n_chunks) break;  // wave-uniform: no chunk of this slot in range
      // The chunk's live positions below the causal block, as up to four
      // (block, mask) groups of consecutive equal blocks: a group starts at
      // entry e unless e continues the block of entry e - 1.
      const int32_t tv[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      bool elig[4], cont[4];
      uint32_t blk[4], bit[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int32_t t = tv[e];
        const bool live = t >= 0 && t < L;
        blk[e] = static_cast<uint32_t>(t) >> 2;
        bit[e] = 1u << (t & 3);
        if (live && blk[e] == static_cast<uint32_t>(c)) tmask |= bit[e];
        elig[e] = live && blk[e] != static_cast<uint32_t>(c);
        cont[e] = e > 0 && elig[e] && elig[e - 1] && blk[e] == blk[e - 1];
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const bool starts = elig[g] && !cont[g];
        if (!__ballot(starts)) continue;  // wave-uniform
        uint32_t m = bit[g];
        bool run = true;
#pragma unroll
        for (int e = g + 1; e < 4; ++e) {
          run = run && cont[e];
          m |= run ? bit[e] : 0u;
        }
        Insert r{false, false, false};
        if (starts) r = hash_insert(slots, hmask, hash_log2, blk[g], m);
        lost |= r.lost;
        n_claimed += static_cast<int32_t>(__popcll(__ballot(r.claimed)));
        const uint64_t cm = __ballot(r.completed);
        if (r.completed)
          ids[n_full + static_cast<int32_t>(lanes_below(cm))] = static_cast<int32_t>(blk[g]);
        n_full += static_cast<int32_t>(__popcll(cm));
      }
    }
  }
  return Collected{n_full, n_claimed, tmask, lost};
}

// The expanded layout, without atomics: the row read as chunks of four
// entries from its start.  A chunk 4b, 4b+1, 4b+2, 4b+3 with b < c is that
// full block; a chunk of padding, stale positions and causal-block positions
// only adds to the causal mask.  Any other chunk
// makes the row take the general path (returns false, wave-uniform).  A
// block listed twice is caught after the sort (adjacent equal ids).
// WIDE (rows of at least 4 entries): one 16-byte load per chunk (rows are
// 4-byte aligned, which these loads need).  The 4-entry window a lane reads
// starts at its chunk, or at the row's last four entries for the partial
// last chunk and for chunks past the row, so every load stays inside the
// row; entries past the row are -1.  All of a pass's loads are issued before
// any window is inspected.
template <bool WIDE>
__device__ __forceinline__ bool collect_fast(const Page4Params& p, const int32_t* trow, int32_t L,
                                             int32_t c, int32_t* ids, Collected& out) {
  const int lane = threadIdx.x & 63;
  const int32_t nt = p.n_tokens;
  const int32_t n_chunks = (nt + 3) >> 2;
  int32_t n_full = 0;
  uint32_t tmask = 0;
  bool ok = true;
  constexpr int kChunks = 12;
  for (int32_t c0 = 0; c0 < n_chunks; c0 += 64 * kChunks) {
    int32_t t[kChunks][4];
#pragma unroll
    for (int u = 0; u < kChunks; ++u) {
      if constexpr (WIDE) {
        const int32_t first = 4 * (c0 + 64 * u + lane);
        typedef int i4u __attribute__((ext_vector_type(4), aligned(4)));
        const i4u wv = __builtin_nontemporal_load(
            reinterpret_cast<const i4u*>(trow + min(first, nt - 4)));
        int4 w = make_int4(wv.x, wv.y, wv.z, wv.w);
        t[u][0] = w.x;
        t[u][1] = w.y;
        t[u][2] = w.z;
        t[u][3] = w.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int32_t i = 4 * (c0 + 64 * u + lane) + e;
          t[u][e] = i < nt ? trow[i] : -1;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kChunks; ++u) {
      if (c0 + 64 * u >= n_chunks) break;  // wave-uniform
      if constexpr (WIDE) {
        if (4 * (c0 + 64 * u + 64) > nt) {  // wave-uniform: the slot reaches past the row
          // Realign the last chunk's window (shift sh = 1..3) and blank
          // the entries past the row.
          const int32_t first = 4 * (c0 + 64 * u + lane);
          const int32_t sh = first - min(first, nt - 4);
          const int32_t win[4] = {t[u][0], t[u][1], t[u][2], t[u][3]};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int32_t j = sh + e;
            const int32_t v = j == 0 ? win[0] : j == 1 ? win[1] : j == 2 ? win[2] : win[3];
            t[u][e] = first + e < nt ? v : -1;
          }
        }
      }
      // A full block in expanded form: 4b, 4b+1, 4b+2, 4b+3 with b < c.
      const int32_t t0 = t[u][0];
      const uint32_t b0 = static_cast<uint32_t>(t0) >> 2;
      const bool full = t0 >= 0 && (t0 & 3) == 0 && t[u][1] == t0 + 1 && t[u][2] == t0 + 2 &&
                        t[u][3] == t0 + 3 && b0 < static_cast<uint32_t>(c);
      if (__ballot(!full)) {
        // Padding, stale positions and causal-block positions only.
        bool side = true;
        uint32_t tm = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int32_t v = t[u][e];
          const bool live = v >= 0 && v < L;
          const bool causal = live && (static_cast<uint32_t>(v) >> 2) == static_cast<uint32_t>(c);
          side = side && (!live || causal);
          tm |= causal ? 1u << (v & 3) : 0u;
        }
        ok = ok && (full || side);
        if (!full && side) tmask |= tm;
      }
      const uint64_t fm = __ballot(full);
      if (full) ids[n_full + static_cast<int32_t>(lanes_below(fm))] = static_cast<int32_t>(b0);
      n_full += static_cast<int32_t>(__popcll(fm));
    }
    if (__ballot(!ok)) return false;
  }
  out = Collected{n_full, n_full, tmask, false};
  return true;
}

// Adjacent equal values anywhere in the wave's sorted blocked sequence.
template <int E>
__device__ __forceinline__ bool has_adjacent_equal(const int32_t (&x)[E], int32_t n) {
  const int lane = threadIdx.x & 63;
  bool eq = false;
#pragma unroll
  for (int e = 0; e + 1 < E; ++e) eq |= (lane * E + e + 1 < n) && x[e] == x[e + 1];
  const int32_t next_first = __shfl_down(x[0], 1);  // lane + 1's first element
  eq |= (lane < 63) && (lane * E + E < n) && x[E - 1] == next_first;
  return __ballot(eq) != 0;
}

// Result of building one row's table (ids hold the row: full pages, then
// the causal page).
struct RowState {
  int32_t status, n_full, n_tail;
  bool retry;  // the expanded-layout attempt could not settle the row
};

// One attempt at a row with live length L (1 <= L <= kPage4MaxLive): the
// expanded-layout collection when !general (which may ask for a retry), else
// the general one through the hash set.
template <int E>
__device__ __forceinline__ RowState attempt(const Page4Params& p, int row, int32_t L, bool general,
                                            uint32_t* slots, uint32_t hmask, int32_t hash_log2,
                                            int32_t* ids) {
  const int lane = threadIdx.x & 63;
  const int32_t c = (L - 1) >> 2;
  const int32_t* trow = p.tokens + static_cast<int64_t>(row) * p.token_stride;
  int32_t status = 0;

  // ---- 1. the full blocks and the causal positions
  Collected col;
  if (general)
    col = collect_hash(p, trow, L, c, slots, hmask, hash_log2, ids);
  else if (!(p.n_tokens >= 4 ? collect_fast<true>(p, trow, L, c, ids, col)
                              : collect_fast<false>(p, trow, L, c, ids, col)))
    return RowState{0, 0, 0, true};
  const int32_t n_full = col.n_full;
  const uint32_t tmask = wave_or(col.tmask);
  const int32_t n_tail = __popc(tmask);
  if (n_tail > 0 && tmask != (1u << n_tail) - 1u) status |= kPage4Tail;
  if (__ballot(col.lost)) status |= kPage4Overflow;
  if (col.n_claimed != n_full) status |= kPage4Partial;
  const int32_t n_pages = n_full + (n_tail > 0 ? 1 : 0);
  if (n_pages > p.out_stride) status |= kPage4Overflow;
  if (n_tail > 0 && lane == 0) ids[n_full] = c;
  lds_fence_wave();

  // ---- 2. block -> view id through the sequence's block table; the table
  // entries of a batch of 16 ids per lane are loaded together.
  const int32_t seq = p.row_seq ? p.row_seq[row] : 0;
  if (seq < 0 || seq >= p.n_seqs) {
    status |= kPage4Seq;
  } else {
    const int32_t* btab = p.block_table + static_cast<int64_t>(seq) * p.max_pages;
    const int32_t quarter = p.page_size >> 2;  // 4-token groups per physical page
    const bool pow2 = (quarter & (quarter - 1)) == 0;
    const int32_t qshift = __ffs(quarter) - 1;
    bool bad = false;
    constexpr int kLook = 16;
    for (int32_t j0 = 0; j0 < n_pages; j0 += 64 * kLook) {
      int32_t b[kLook], lp[kLook], pg[kLook];
#pragma unroll
      for (int u = 0; u < kLook; ++u) {
        const int32_t j = j0 + 64 * u + lane;
        b[u] = j < n_pages ? ids[j] : 0;
        lp[u] = pow2 ? (b[u] >> qshift) : b[u] / quarter;
      }
      // Every entry is loaded (an index past the table reads its last entry)
      // and judged only once all are issued, so the loads are in flight
      // together rather than one after another.
#pragma unroll
      for (int u = 0; u < kLook; ++u) pg[u] = btab[min(lp[u], p.max_pages - 1)];
#pragma unroll
      for (int u = 0; u < kLook; ++u) {
        const int32_t j = j0 + 64 * u + lane;
        if (lp[u] >= p.max_pages) pg[u] = -1;
        if (j < n_pages) {
          const bool ok = pg[u] >= 0 && pg[u] < p.num_pages;
          bad |= !ok;
          ids[j] = ok ? pg[u] * p.vpages_per_page + (b[u] - lp[u] * quarter) : -1;
        }
      }
    }
    if (__ballot(bad)) status |= kPage4Page;
  }
  lds_fence_wave();

  // ---- 3. locality order of the full pages
  if (status == 0 && n_full > 1) {
    int32_t x[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int32_t i = lane * E + e;
      x[e] = i < n_full ? ids[i] : INT32_MAX;
    }
    wave_sort<E>(x);
    // Two equal neighbours: the fast path may have listed a block twice.
    if (!general && has_adjacent_equal<E>(x, n_full)) return RowState{0, 0, 0, true};
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int32_t i = lane * E + e;
      if (i < n_full) ids[i] = x[e];
    }
    lds_fence_wave();
  }
  return RowState{status, n_full, n_tail, false};
}

// W waves, one row each; the hash set of the general path is shared by the
// workgroup and used by one wave at a time (rows that need it are rare).
template <int E, int W>
__global__ __launch_bounds__(64 * W) void page4_kernel(Page4Params p, int32_t hash_log2) {
  extern __shared__ uint32_t lds[];
  constexpr int kIds = 64 * E + 4;  // per-wave id list (the causal page included)
  const uint32_t hmask = (1u << hash_log2) - 1u;
  uint32_t* slots = lds;            // [hmask + 1]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  int32_t* ids = reinterpret_cast<int32_t*>(lds + hmask + 1) + wave * kIds;
  const int row = blockIdx.x * W + wave;
  const bool active = row < p.rows;

  RowState st{0, 0, 0, false};
  int32_t L = 0;
  if (active) {
    L = p.live_len[row];
    if (L <= 0)
      st.status = kPage4Empty;
    else if (L > kPage4MaxLive)
      st.status = kPage4Long;
    else
      st = attempt<E>(p, row, L, false, slots, hmask, hash_log2, ids);
  }
  // The general path, one wave at a time (every wave reaches every barrier).
  for (int w = 0; w < W; ++w) {
    __syncthreads();
    if (wave == w && active && st.retry)
      st = attempt<E>(p, row, L, true, slots, hmask, hash_log2, ids);
  }
  if (!active) return;

  // ---- 4. the row: pages, causal page last, -1 padding; inert if invalid
  int32_t* orow = p.out_table + static_cast<int64_t>(row) * p.out_stride;
  const int32_t n_out = st.status == 0 ? st.n_full + (st.n_tail > 0 ? 1 : 0) : 0;
  for (int32_t i = lane; i < p.out_stride; i += 64)
    __builtin_nontemporal_store(i < n_out ? ids[i] : -1, orow + i);
  if (lane == 0) {
    p.out_len[row] = st.status == 0 ? 4 * st.n_full + st.n_tail : 0;
    if (p.out_status) p.out_status[row] = st.status;
  }
}

constexpr int kRowsPerGroup = 4;

template <int E>
hipError_t launch_e(const Page4Params& p, int32_t hash_log2, hipStream_t stream) {
  constexpr int W = kRowsPerGroup;
  const auto bytes = [](size_t slots) {
    return sizeof(uint32_t) * (slots + static_cast<size_t>(W) * (64 * E + 4));
  };
  const size_t lds = bytes(size_t{1} << hash_log2);
  if (lds > 65536) {
    // Beyond the default 64 KiB of dynamic LDS the limit must be raised
    // (once per process and instance; the largest size this instance uses).
    static const hipError_t raised = hipFuncSetAttribute(
        reinterpret_cast<const void*>(page4_kernel<E, W>),
        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes(2 * kPage4MaxTokens)));
    if (raised != hipSuccess) return raised;
  }
  const unsigned groups = static_cast<unsigned>((p.rows + W - 1) / W);
  return pgqa_launch::launch(page4_kernel<E, W>, dim3(groups), dim3(64 * W), lds, stream, p,
                             hash_log2);
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
