// C-ABI host layer of the sampler masking operation in libpgqa: argument
// validation and launches on the caller's stream.  Declared in
// include/pgqa.h.  Validation runs before any HIP call: an argument error
// launches nothing and writes nothing.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pgqa.h"
#include "sampler_internal.h"

namespace {

bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0; }

}  // namespace

extern "C" {

size_t sampler_topk_topp_workspace_bytes(int32_t rows, int32_t vocab, int32_t k_max) {
  if (rows < 0 || vocab < 1 || vocab > SAMPLER_MAX_VOCAB || k_max < 1 || k_max > SAMPLER_MAX_K)
    return SIZE_MAX;
  return sampler::workspace_bytes(rows, vocab, k_max);
}

int sampler_topk_topp_mask(const float* logits, int64_t row_stride, int32_t rows, int32_t vocab,
                           const int32_t* k, const float* p, int32_t k_max, float* out,
                           int64_t out_stride, int32_t* status, void* workspace,
                           size_t workspace_bytes, void* stream) {
  static_assert(SAMPLER_MAX_K == sampler::kMaxK && SAMPLER_MAX_VOCAB == sampler::kMaxVocab,
                "limits mismatch");
  static_assert(SAMPLER_MASK_BAD_K == sampler::kBadK && SAMPLER_MASK_BAD_P == sampler::kBadP,
                "status codes mismatch");
  if (rows < 0 || vocab < 1 || vocab > SAMPLER_MAX_VOCAB || k_max < 1 || k_max > SAMPLER_MAX_K)
    return PGQA_ERR_SHAPE;
  if (rows == 0) return PGQA_OK;
  if (!logits || !k || !p || !out) return PGQA_ERR_NULL;
  if (row_stride < vocab || out_stride < vocab) return PGQA_ERR_LAYOUT;
  // In place needs equal strides; otherwise the two row ranges may not meet.
  const uintptr_t z0 = reinterpret_cast<uintptr_t>(logits), o0 = reinterpret_cast<uintptr_t>(out);
  const uintptr_t z1 = z0 + ((rows - 1) * static_cast<uint64_t>(row_stride) + vocab) * 4;
  const uintptr_t o1 = o0 + ((rows - 1) * static_cast<uint64_t>(out_stride) + vocab) * 4;
  if (z0 == o0 ? out_stride != row_stride : (z0 < o1 && o0 < z1)) return PGQA_ERR_LAYOUT;
  if (!aligned(logits, 4) || !aligned(k, 4) || !aligned(p, 4) || !aligned(out, 4) ||
      !aligned(status, 4))
    return PGQA_ERR_LAYOUT;
  const size_t need = sampler::workspace_bytes(rows, vocab, k_max);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 8)) return PGQA_ERR_WORKSPACE;
  sampler::MaskParams m;
  m.logits = logits;
  m.row_stride = row_stride;
  m.rows = rows;
  m.vocab = vocab;
  m.k = k;
  m.p = p;
  m.k_max = k_max;
  m.out = out;
  m.out_stride = out_stride;
  m.status = status;
  sampler::plan_chunks(vocab, &m.chunk, &m.n_chunks);
  m.cand = static_cast<uint64_t*>(workspace);
  if (sampler::launch_mask(m, static_cast<hipStream_t>(stream)) != hipSuccess)
    return PGQA_ERR_HIP;
  return PGQA_OK;
}

}  // extern "C"
