// C-ABI host layer of libpgqa: argument validation, split planning and
// launches on the caller's stream.  Declared in include/pgqa.h.
//
// Validation runs before any HIP call, so every argument error is reported
// without touching a device: nothing is launched and nothing is written.
// The only HIP queries are the current device and its compute
// unit count (cached per device), needed for the automatic split count.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "pgqa.h"
#include "pgqa_internal.h"

namespace {

using pgqa::kHeadDim;
using pgqa::kMaxGroup;
using pgqa::kTile;

// Split planning: waves per workgroup (fixed by the kernels) and resident
// waves per compute unit the automatic split count aims for.
constexpr int kWaves = pgqa::kWavesPerWg;
constexpr int kWavesPerCu = 4;
// Upper bound on splits (the merge reads every partial of a head).
constexpr int64_t kMaxSplits = 256;
// Upper bound on the automatic choice: past it the merge's reads of the
// partials cost more than the extra workgroups save (one 16K-token sequence,
// E4M3: 11.5 us per call at 128 splits, 14.0 at 256).
constexpr int64_t kAutoMaxSplits = 128;
constexpr int kChunkAlign = kTile * kWaves;  // split length granularity
constexpr int kChunkAlignShift = 6;
static_assert(kChunkAlign == 1 << kChunkAlignShift, "granularity is a power of two");
// Rows up to this length, when there are enough of them to give every compute
// unit a workgroup of kWaves rows, run one row per wave.
constexpr int kRowPerWaveMaxLen = 4096;

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

// Split partials of paged_gqa_decode_noalloc.  Each device holds its own copy
// at its own address; host code uses only the address hipGetSymbolAddress
// returns for the current device (the array's name on the host is a
// stand-in, not a device address).
static __device__ __align__(256) unsigned char scratch[PGQA_NOALLOC_SCRATCH_BYTES];
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

// Device address of the current device's scratch, looked up once per device
// with that device current.
hipError_t current_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255u) != 0) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// Compute units of the current device, or -1 if HIP cannot say.
int current_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  if (dev < kMaxDevices) {
    int cached = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cached > 0) return cached;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return -1;
  if (dev < kMaxDevices) g_cu_count[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

struct SplitPlan {
  int32_t splits;
  int32_t chunk;
};

// Key-range splits: aim for kWavesPerCu resident waves per compute
// unit, never fewer than kChunkAlign tokens (one tile per wave) per split.
SplitPlan plan_splits(int64_t groups, int32_t max_len, int32_t requested, int cus) {
  const int64_t len = max_len > 0 ? max_len : 1;
  const int64_t max_splits = ceil_div(len, kChunkAlign);
  int64_t s;
  if (requested > 0) {
    s = requested;
  } else {
    const int64_t target_wgs =
        static_cast<int64_t>(cus > 0 ? cus : 256) * kWavesPerCu / kWaves;
    s = ceil_div(target_wgs, groups > 0 ? groups : 1);
    if (s > kAutoMaxSplits) s = kAutoMaxSplits;
  }
  if (s > max_splits) s = max_splits;
  if (s > kMaxSplits) s = kMaxSplits;
  if (s < 1) s = 1;
  const int64_t chunk = ceil_div(ceil_div(len, s), kChunkAlign) * kChunkAlign;
  return SplitPlan{static_cast<int32_t>(ceil_div(len, chunk)), static_cast<int32_t>(chunk)};
}

// Workspace: the fp32 split outputs [n*hq][splits][256], then their
// log-sum-exps [n*hq][splits].
size_t workspace_need(int32_t n, int32_t hq, int32_t hkv, int32_t splits) {
  (void)hkv;
  if (splits <= 1) return 0;
  return static_cast<size_t>(n) * hq * splits * (kHeadDim + 1) * sizeof(float);
}

// Checks that need no HIP call.  Returns PGQA_OK or an error code.
int validate_sizes(int32_t n, int32_t hq, int32_t hkv, int32_t head_dim, int32_t max_len,
                   int32_t num_splits) {
  if (head_dim != kHeadDim) return PGQA_ERR_SHAPE;
  if (n < 0 || hkv < 1 || hq < 1 || hq % hkv != 0) return PGQA_ERR_SHAPE;
  const int32_t group = hq / hkv;
  if (group > kMaxGroup) return PGQA_ERR_SHAPE;
  if (max_len < 0 || max_len > PGQA_MAX_SEQ_LEN) return PGQA_ERR_SHAPE;
  if (num_splits < 0) return PGQA_ERR_ARG;
  // The grid is splits * n * hkv workgroups in one dimension.
  const int64_t max_splits = ceil_div(max_len > 0 ? max_len : 1, kChunkAlign);
  if (static_cast<int64_t>(n) * hkv * max_splits > INT32_MAX) return PGQA_ERR_SHAPE;
  return PGQA_OK;
}

int validate_call(const void* q, const pgqa_kv_pool* kv, const int32_t* table,
                  int32_t max_pages, const int32_t* lens, int32_t max_len, int32_t n,
                  int32_t hq, int32_t hkv, int32_t head_dim, float sm_scale,
                  int32_t num_splits, const void* out) {
  int rc = validate_sizes(n, hq, hkv, head_dim, max_len, num_splits);
  if (rc != PGQA_OK) return rc;
  if (!kv) return PGQA_ERR_NULL;
  if (kv->kv_dtype != PGQA_KV_FP16 && kv->kv_dtype != PGQA_KV_E4M3) return PGQA_ERR_DTYPE;
  if (!std::isfinite(sm_scale)) return PGQA_ERR_ARG;
  if (kv->kv_dtype == PGQA_KV_E4M3 && (!std::isfinite(kv->k_scale) || !std::isfinite(kv->v_scale)))
    return PGQA_ERR_ARG;
  if (n == 0) return PGQA_OK;
  if (!q || !out || !table || !lens || !kv->k_base || !kv->v_base) return PGQA_ERR_NULL;
  if (kv->page_size < 1 || kv->num_pages < 1 || max_pages < 1) return PGQA_ERR_SHAPE;
  if (static_cast<int64_t>(max_len) > static_cast<int64_t>(max_pages) * kv->page_size)
    return PGQA_ERR_SHAPE;
  const int64_t es = kv->kv_dtype == PGQA_KV_FP16 ? 2 : 1;
  if (kv->page_stride < 0 || kv->token_stride < 0 || kv->head_stride < 0) return PGQA_ERR_LAYOUT;
  if ((kv->page_stride * es) % 16 || (kv->token_stride * es) % 16 || (kv->head_stride * es) % 16)
    return PGQA_ERR_LAYOUT;
  if (!aligned16(kv->k_base) || !aligned16(kv->v_base) || !aligned16(q) || !aligned16(out))
    return PGQA_ERR_LAYOUT;
  return PGQA_OK;
}

// Fills the launch parameters shared by every attention call.
pgqa::AttnParams make_params(const void* q, const pgqa_kv_pool* kv, const int32_t* table,
                             int32_t max_pages, const int32_t* lens, int32_t max_len, int32_t n,
                             int32_t hq, int32_t hkv, float sm_scale, const SplitPlan& plan) {
  const bool fp8 = kv->kv_dtype == PGQA_KV_E4M3;
  const int64_t es = fp8 ? 1 : 2;
  pgqa::AttnParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k_base = static_cast<const uint8_t*>(kv->k_base);
  p.v_base = static_cast<const uint8_t*>(kv->v_base);
  p.page_stride = kv->page_stride * es;
  p.token_stride = kv->token_stride * es;
  p.head_stride = kv->head_stride * es;
  p.num_pages = kv->num_pages;
  p.page_size = kv->page_size;
  p.inv_page_size = 1.0f / static_cast<float>(kv->page_size);
  p.table = table;
  p.max_pages = max_pages;
  p.lens = lens;
  p.max_len = max_len;
  p.n = n;
  p.hq = hq;
  p.hkv = hkv;
  p.group = hq / hkv;
  const double log2e = 1.4426950408889634;
  p.qk_scale_log2 =
      static_cast<float>(static_cast<double>(sm_scale) * (fp8 ? kv->k_scale : 1.0) * log2e);
  p.v_scale = fp8 ? kv->v_scale : 1.0f;
  p.splits = plan.splits;
  p.chunk = plan.chunk;
  return p;
}

// The split plan of a validated call (queries the device only for num_splits = 0).
int plan_call(int32_t n, int32_t hkv, int32_t max_len, int32_t num_splits, SplitPlan* plan) {
  int cus = 0;
  if (num_splits == 0) {
    cus = current_cu_count();
    if (cus <= 0) return PGQA_ERR_HIP;
  }
  *plan = plan_splits(static_cast<int64_t>(n) * hkv, max_len, num_splits, cus);
  return PGQA_OK;
}

int run_attention(const void* q, const pgqa_kv_pool* kv, const int32_t* table, int32_t max_pages,
                  const int32_t* lens, int32_t max_len, int32_t n, int32_t hq, int32_t hkv,
                  int32_t head_dim, float sm_scale, int32_t num_splits, void* out,
                  void* workspace, size_t workspace_bytes, void* stream, bool stream_kv) {
  int rc = validate_call(q, kv, table, max_pages, lens, max_len, n, hq, hkv, head_dim, sm_scale,
                         num_splits, out);
  if (rc != PGQA_OK || n == 0) return rc;
  SplitPlan plan;
  rc = plan_call(n, hkv, max_len, num_splits, &plan);
  if (rc != PGQA_OK) return rc;
  const size_t need = workspace_need(n, hq, hkv, plan.splits);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return PGQA_ERR_WORKSPACE;

  const bool fp8 = kv->kv_dtype == PGQA_KV_E4M3;
  pgqa::AttnParams p = make_params(q, kv, table, max_pages, lens, max_len, n, hq, hkv, sm_scale,
                                   plan);
  p.out = static_cast<uint16_t*>(out);
  p.partials = plan.splits > 1;
  p.stream_kv = stream_kv;
  if (p.partials) {
    p.ws_o = static_cast<float*>(workspace);
    p.ws_lse = p.ws_o + static_cast<size_t>(n) * hq * plan.splits * kHeadDim;
    // Unequal lengths: the kernels spread the live tokens over all n*S
    // workgroup slots of a kv head (the partial layout stays internal).
    if (n <= pgqa::kBalanceMaxSeqs) p.balance_n = n;
  } else if (max_len <= kRowPerWaveMaxLen) {
    // One split and many rows: a workgroup of kWaves rows pays its launch
    // and ramp once for all of them.
    const int cus = current_cu_count();
    p.row_per_wave = cus > 0 && static_cast<int64_t>(n) * hkv >= static_cast<int64_t>(kWaves) * cus;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (pgqa::launch_attention(p, fp8, s) != hipSuccess) return PGQA_ERR_HIP;
  if (!p.partials) return PGQA_OK;
  pgqa::MergeParams m{p.ws_o, p.ws_lse, static_cast<int64_t>(n) * hq, plan.splits, p.out};
  if (p.balance_n > 0) {
    m.lens = lens;
    m.n = n;
    m.hq = hq;
    m.max_len = max_len;
    m.a_shift = kChunkAlignShift;
  }
  return pgqa::launch_merge(m, s) == hipSuccess ? PGQA_OK : PGQA_ERR_HIP;
}

}  // namespace

extern "C" {

int32_t paged_gqa_num_splits(int32_t n, int32_t num_kv_heads, int32_t max_seq_len,
                             int32_t num_splits) {
  if (n < 0 || num_kv_heads < 1 || max_seq_len < 0 || max_seq_len > PGQA_MAX_SEQ_LEN ||
      num_splits < 0)
    return PGQA_ERR_ARG;
  int cus = 0;
  if (num_splits == 0) {
    cus = current_cu_count();
    if (cus <= 0) return PGQA_ERR_HIP;
  }
  return plan_splits(static_cast<int64_t>(n) * num_kv_heads, max_seq_len, num_splits, cus).splits;
}

size_t paged_gqa_workspace_bytes(int32_t n, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_seq_len, int32_t num_splits) {
  if (validate_sizes(n, num_q_heads, num_kv_heads, head_dim, max_seq_len, num_splits) != PGQA_OK)
    return SIZE_MAX;
  const int32_t splits = paged_gqa_num_splits(n, num_kv_heads, max_seq_len, num_splits);
  if (splits < 1) return SIZE_MAX;
  return workspace_need(n, num_q_heads, num_kv_heads, splits);
}

int paged_gqa_decode(const void* q, const pgqa_kv_pool* kv, const int32_t* page_table,
                     int32_t max_pages, const int32_t* seq_lens, int32_t max_seq_len,
                     int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, float sm_scale, int32_t num_splits, void* out,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return run_attention(q, kv, page_table, max_pages, seq_lens, max_seq_len, batch, num_q_heads,
                       num_kv_heads, head_dim, sm_scale, num_splits, out, workspace,
                       workspace_bytes, stream,
                       // Each K/V byte is read once per call: non-temporal loads.
                       /*stream_kv=*/true);
}

int paged_gqa_decode_noalloc(const void* q, const pgqa_kv_pool* kv, const int32_t* page_table,
                             int32_t max_pages, const int32_t* seq_lens, int32_t max_seq_len,
                             int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, float sm_scale, int32_t num_splits, void* out,
                             void* stream) {
  // The size check comes before the scratch lookup, so an oversized call is
  // rejected without any HIP call when num_splits is explicit.
  int rc = validate_call(q, kv, page_table, max_pages, seq_lens, max_seq_len, batch, num_q_heads,
                         num_kv_heads, head_dim, sm_scale, num_splits, out);
  if (rc != PGQA_OK || batch == 0) return rc;
  SplitPlan plan;
  rc = plan_call(batch, num_kv_heads, max_seq_len, num_splits, &plan);
  if (rc != PGQA_OK) return rc;
  const size_t need = workspace_need(batch, num_q_heads, num_kv_heads, plan.splits);
  if (need > PGQA_NOALLOC_SCRATCH_BYTES) return PGQA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0 && current_scratch(&ws) != hipSuccess) return PGQA_ERR_HIP;
  return run_attention(q, kv, page_table, max_pages, seq_lens, max_seq_len, batch, num_q_heads,
                       num_kv_heads, head_dim, sm_scale, num_splits, out, ws,
                       need > 0 ? PGQA_NOALLOC_SCRATCH_BYTES : 0, stream, /*stream_kv=*/true);
}

int paged_gqa_prefill_sparse(const void* q, const pgqa_kv_pool* kv, const int32_t* row_tables,
                             int32_t max_pages, const int32_t* row_lens, int32_t max_row_len,
                             int32_t rows, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, float sm_scale, int32_t num_splits, void* out,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return run_attention(q, kv, row_tables, max_pages, row_lens, max_row_len, rows, num_q_heads,
                       num_kv_heads, head_dim, sm_scale, num_splits, out, workspace,
                       workspace_bytes, stream,
                       // Rows share one pool and re-read it through the caches: normal
                       // loads (non-temporal ones measured 23% slower on 4096 rows).
                       /*stream_kv=*/false);
}

int paged_gqa_decode_partial(const void* q, const pgqa_kv_pool* kv, const int32_t* page_table,
                             int32_t max_pages, const int32_t* seq_lens, int32_t max_seq_len,
                             int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, float sm_scale, int32_t num_splits,
                             float* part_o, float* part_lse, void* stream) {
  // `out` is not written here; pass part_o to the shared checks in its place.
  int rc = validate_call(q, kv, page_table, max_pages, seq_lens, max_seq_len, batch, num_q_heads,
                         num_kv_heads, head_dim, sm_scale, num_splits, part_o);
  if (rc != PGQA_OK || batch == 0) return rc;
  if (!part_lse) return PGQA_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(part_lse) & 3u) return PGQA_ERR_LAYOUT;
  SplitPlan plan;
  rc = plan_call(batch, num_kv_heads, max_seq_len, num_splits, &plan);
  if (rc != PGQA_OK) return rc;
  pgqa::AttnParams p = make_params(q, kv, page_table, max_pages, seq_lens, max_seq_len, batch,
                                   num_q_heads, num_kv_heads, sm_scale, plan);
  p.partials = true;
  p.stream_kv = true;
  p.ws_o = part_o;
  p.ws_lse = part_lse;
  return pgqa::launch_attention(p, kv->kv_dtype == PGQA_KV_E4M3,
                                static_cast<hipStream_t>(stream)) == hipSuccess
             ? PGQA_OK
             : PGQA_ERR_HIP;
}

int paged_gqa_merge_partials(const float* part_o, const float* part_lse, int32_t rows,
                             int32_t splits, int32_t head_dim, void* out, void* stream) {
  if (head_dim != kHeadDim || rows < 0 || splits < 1) return PGQA_ERR_SHAPE;
  if (rows == 0) return PGQA_OK;
  if (!part_o || !part_lse || !out) return PGQA_ERR_NULL;
  if (!aligned16(part_o) || !aligned16(out) || (reinterpret_cast<uintptr_t>(part_lse) & 3u))
    return PGQA_ERR_LAYOUT;
  pgqa::MergeParams m{part_o, part_lse, rows, splits, static_cast<uint16_t*>(out)};
  return pgqa::launch_merge(m, static_cast<hipStream_t>(stream)) == hipSuccess ? PGQA_OK
                                                                                : PGQA_ERR_HIP;
}

int e4m3_decode_table(float* out256, void* stream) {
  if (!out256) return PGQA_ERR_NULL;
  if (!aligned16(out256)) return PGQA_ERR_LAYOUT;
  return pgqa::launch_e4m3_table(out256, static_cast<hipStream_t>(stream)) == hipSuccess
             ? PGQA_OK
             : PGQA_ERR_HIP;
}

const char* pgqa_error_string(int code) {
  switch (code) {
    case PGQA_OK: return "ok";
    case PGQA_ERR_NULL: return "a required pointer is NULL";
    case PGQA_ERR_SHAPE: return "unsupported or inconsistent sizes";
    case PGQA_ERR_LAYOUT: return "pointer or stride not 16-byte aligned, or negative stride";
    case PGQA_ERR_DTYPE: return "unknown kv_dtype";
    case PGQA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case PGQA_ERR_HIP: return "HIP runtime error";
    case PGQA_ERR_ARG: return "invalid scalar argument";
    default: return "unknown error code";
  }
}

}  // extern "C"
