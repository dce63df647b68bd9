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
};

// vec: scores 16-byte aligned, row_stride and n_blocks multiples of 4.
hipError_t launch_topk(const TopkParams& p, bool vec, hipStream_t stream);

}  // namespace qsa
