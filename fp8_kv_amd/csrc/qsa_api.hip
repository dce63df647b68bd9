// C-ABI host layer of the QSA selection operations in libpgqa: argument
// validation and launches on the caller's stream.  Declared in
// include/pgqa.h.  As in the attention entry points, validation runs before
// any HIP call: an argument error launches nothing and writes nothing.
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cstdint>

#include "pgqa.h"
#include "qsa_internal.h"

namespace {

bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0; }

constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

// Compute units of the current device (cached per device), or -1 if HIP
// cannot say.
int current_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  if (dev < kMaxDevices) {
    const int cached = g_cus[dev].load(std::memory_order_relaxed);
    if (cached > 0) return cached;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return -1;
  if (dev < kMaxDevices) g_cus[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

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
  if (!aligned(scores, 4) || !aligned(out_idx, 4) || !aligned(n_valid, 4) ||
      !aligned(out_count, 4))
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
  p.grid = current_cus();
  if (p.grid <= 0) return PGQA_ERR_HIP;
  const bool vec = aligned(scores, 16) && row_stride % 4 == 0 && n_blocks % 4 == 0;
  if (qsa::launch_topk(p, vec, static_cast<hipStream_t>(stream)) != hipSuccess)
    return PGQA_ERR_HIP;
  return PGQA_OK;
}

int qsa_build_page4_table(const int32_t* tokens, int64_t token_stride, int32_t n_tokens,
                          const int32_t* live_len, const int32_t* block_table,
                          int32_t max_pages, const int32_t* row_seq, int32_t n_seqs,
                          int32_t num_pages, int32_t page_size, int32_t vpages_per_page,
                          int32_t rows, int32_t* out_table, int32_t out_stride,
                          int32_t* out_len, int32_t* out_status, void* stream) {
  static_assert(PGQA_QSA_MAX_SEL_TOKENS == qsa::kPage4MaxTokens, "token limit mismatch");
  static_assert(PGQA_PAGE4_EMPTY == qsa::kPage4Empty && PGQA_PAGE4_PARTIAL == qsa::kPage4Partial &&
                    PGQA_PAGE4_TAIL == qsa::kPage4Tail && PGQA_PAGE4_PAGE == qsa::kPage4Page &&
                    PGQA_PAGE4_OVERFLOW == qsa::kPage4Overflow &&
                    PGQA_PAGE4_SEQ == qsa::kPage4Seq && PGQA_PAGE4_LONG == qsa::kPage4Long &&
                    PGQA_PAGE4_MAX_LIVE == qsa::kPage4MaxLive,
                "status codes mismatch");
  if (rows < 0 || n_tokens < 0 || n_tokens > PGQA_QSA_MAX_SEL_TOKENS || max_pages < 1 ||
      n_seqs < 1 || num_pages < 0 || page_size < 4 || page_size % 4 != 0 || out_stride < 1 ||
      vpages_per_page < page_size / 4 ||
      static_cast<int64_t>(num_pages) * vpages_per_page > INT32_MAX)
    return PGQA_ERR_SHAPE;
  if (rows == 0) return PGQA_OK;
  if ((!tokens && n_tokens > 0) || !live_len || !block_table || !out_table || !out_len)
    return PGQA_ERR_NULL;
  if (token_stride < n_tokens) return PGQA_ERR_LAYOUT;
  if (!aligned(tokens, 4) || !aligned(live_len, 4) || !aligned(block_table, 4) ||
      !aligned(row_seq, 4) || !aligned(out_table, 4) || !aligned(out_len, 4) ||
      !aligned(out_status, 4))
    return PGQA_ERR_LAYOUT;
  qsa::Page4Params p;
  p.tokens = tokens;
  p.token_stride = token_stride;
  p.n_tokens = n_tokens;
  p.live_len = live_len;
  p.block_table = block_table;
  p.max_pages = max_pages;
  p.row_seq = row_seq;
  p.n_seqs = n_seqs;
  p.num_pages = num_pages;
  p.page_size = page_size;
  p.vpages_per_page = vpages_per_page;
  p.rows = rows;
  p.out_table = out_table;
  p.out_stride = out_stride;
  p.out_len = out_len;
  p.out_status = out_status;
  if (qsa::launch_page4(p, static_cast<hipStream_t>(stream)) != hipSuccess) return PGQA_ERR_HIP;
  return PGQA_OK;
}

}  // extern "C"
