// Internal interface between the C-ABI host layer of the sampler masking
// operation (sampler_api.hip) and its gfx950 kernels (sampler_mask.hip).
// Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sampler {

constexpr int kMaxK = 256;          // largest per-row top-k
constexpr int kMaxChunks = 64;      // chunk lists merged by one wave
constexpr int kMinChunk = 4096;     // logits per chunk workgroup, at least
constexpr int kMaxChunk = 8192;     // and at most (32 per thread)
constexpr int kMaxVocab = kMaxChunks * kMaxChunk;

// Row status bits (the same values as SAMPLER_MASK_* in pgqa.h).
constexpr int32_t kBadK = 1;
constexpr int32_t kBadP = 2;

struct MaskParams {
  const float* logits;     // [rows][row_stride]
  int64_t row_stride;      // elements
  int32_t rows;
  int32_t vocab;
  const int32_t* k;        // [rows]
  const float* p;          // [rows]
  int32_t k_max;           // 1 .. kMaxK
  float* out;              // [rows][out_stride]; may be logits
  int64_t out_stride;
  int32_t* status;         // [rows] or nullptr
  int32_t chunk;           // logits per chunk (multiple of 1024)
  int32_t n_chunks;        // <= kMaxChunks
  uint64_t* cand;          // workspace [rows][k_max][n_chunks] chunk top lists, rank-major
};

// Chunk size and count for a vocabulary; chunk = 0 when it is too large.
void plan_chunks(int32_t vocab, int32_t* chunk, int32_t* n_chunks);
size_t workspace_bytes(int32_t rows, int32_t vocab, int32_t k_max);
hipError_t launch_mask(const MaskParams& p, hipStream_t stream);

}  // namespace sampler
