// C-ABI host layer of the QSA selection operations in libpgqa: argument
// validation and launches on the caller's stream.  Declared in
// include/pgqa.h.  As in the attention entry points, validation runs before
// any HIP call: an argument error launches nothing and writes nothing.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pgqa.h"
#include "qsa_internal.h"

namespace {

bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0; }

}  // namespace

extern "C" {

int qsa_topk_select(const float* scores, int64_t row_stride, const int32_t* n_valid,
                    int32_t rows, int32_t n_blocks, int32_t k, int32_t* out_idx,
                    int32_t* out_count, void* stream) {
  static_assert(PGQA_QSA_MAX_BLOCKS == qsa::kTopkMaxBlocks, "block limit mismatch");
  if (rows < 0 || k < 0 || n_blocks < 0 || n_blocks > PGQA_QSA_MAX_BLOCKS ||
      k > PGQA_QSA_MAX_BLOCKS)
    return PGQA_ERR_SHAPE;
  if (rows == 0) return PGQA_OK;
  if (!scores || (k > 0 && !out_idx)) return PGQA_ERR_NULL;
  if (row_stride < n_blocks || row_stride < 0) return PGQA_ERR_LAYOUT;
  const auto misaligned4 = [](const void* ptr) {
    return (reinterpret_cast<uintptr_t>(ptr) & 3u) != 0;
  };
  if (misaligned4(scores) || misaligned4(out_idx) || misaligned4(n_valid) ||
      misaligned4(out_count))
    return PGQA_ERR_LAYOUT;
  qsa::TopkParams p;
  p.scores = scores;
  p.row_stride = row_stride;
  p.n_valid = n_valid;
  p.rows = rows;
  p.n_blocks = n_blocks;
  p.k = k;
  p.out_idx = out_idx;
  p.out_count = out_count;
  const bool vec = aligned(scores, 16) && row_stride % 4 == 0 && n_blocks % 4 == 0;
  if (qsa::launch_topk(p, vec, static_cast<hipStream_t>(stream)) != hipSuccess)
    return PGQA_ERR_HIP;
  return PGQA_OK;
}

}  // extern "C"
