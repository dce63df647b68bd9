// Internal interface between the C-ABI host layer of the QSA selection
// operations (qsa_api.hip) and their gfx950 kernels (qsa_topk.hip,
// qsa_page4.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

// Top-k block selection (qsa_topk.hip): one workgroup per row.
constexpr int kTopkThreads = 1024;
constexpr int kTopkMaxBlocks = 65536;   // blocks per row held in registers

struct TopkParams {
  const float* scores;     // [rows][row_stride]
  int64_t row_stride;      // elements
  const int32_t* n_valid;  // [rows] or nullptr (= n_blocks)
  int32_t rows;
  int32_t n_blocks;        // <= kTopkMaxBlocks
  int32_t k;
  int32_t* out_idx;        // [rows][k]
  int32_t* out_count;      // [rows] or nullptr
  int32_t grid;            // workgroups (>= 1): each takes every grid-th row
};

// vec: scores 16-byte aligned, row_stride and n_blocks multiples of 4.
hipError_t launch_topk(const TopkParams& p, bool vec, hipStream_t stream);

// Virtual page-4 table of expanded QSA selections (qsa_page4.hip): one wave
// per row.
constexpr int kPage4MaxTokens = 8192;      // selection entries per row
constexpr int32_t kPage4MaxLive = 1 << 26; // longest live length a row may have

// Row status bits (the same values as PGQA_PAGE4_* in pgqa.h).
constexpr int32_t kPage4Empty = 1;
constexpr int32_t kPage4Partial = 2;
constexpr int32_t kPage4Tail = 4;
constexpr int32_t kPage4Page = 8;
constexpr int32_t kPage4Overflow = 16;
constexpr int32_t kPage4Seq = 32;
constexpr int32_t kPage4Long = 64;

struct Page4Params {
  const int32_t* tokens;      // [rows][token_stride], -1 = padding
  int64_t token_stride;       // elements
  int32_t n_tokens;           // 0 .. kPage4MaxTokens
  const int32_t* live_len;    // [rows]
  const int32_t* block_table; // [n_seqs][max_pages]
  int32_t max_pages;
  const int32_t* row_seq;     // [rows] or nullptr (all rows in sequence 0)
  int32_t n_seqs;
  int32_t num_pages;          // physical pages
  int32_t page_size;          // multiple of 4
  int32_t vpages_per_page;    // >= page_size / 4; num_pages * it fits int32
  int32_t rows;
  int32_t* out_table;         // [rows][out_stride]
  int32_t out_stride;
  int32_t* out_len;           // [rows]
  int32_t* out_status;        // [rows] or nullptr
};

hipError_t launch_page4(const Page4Params& p, hipStream_t stream);

}  // namespace qsa
