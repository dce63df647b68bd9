// Internal interface between the C-ABI host layer (pgqa_api.hip) and the
// gfx950 kernels (pgqa_kernels.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pgqa {

constexpr int kHeadDim = 256;   // head dimension the kernels are built for
constexpr int kTile = 16;       // tokens per wave tile (one MFMA M/K block)
constexpr int kWavesPerWg = 4;  // waves per attention workgroup, each on its own tiles
constexpr int kMaxGroup = 16;   // query heads per kv head (MFMA N = 16)
constexpr int kBalanceMaxSeqs = 512;  // sequences a balanced (ragged) plan covers

// Everything a launch needs; strides already converted to bytes.
struct AttnParams {
  const uint16_t* q;       // fp16 bits [n][hq][256]
  const uint8_t* k_base;   // byte address of K(page 0, slot 0, head 0, dim 0)
  const uint8_t* v_base;
  int64_t page_stride;     // bytes
  int64_t token_stride;    // bytes
  int64_t head_stride;     // bytes
  int32_t num_pages;
  int32_t page_size;
  float inv_page_size;     // 1.0f / page_size, for the in-kernel division
  const int32_t* table;    // [n][max_pages]
  int32_t max_pages;
  const int32_t* lens;     // [n]
  int32_t max_len;         // lengths are clamped to this
  int32_t n;               // sequences or rows
  int32_t hq;
  int32_t hkv;
  int32_t group;           // hq / hkv, 1..16
  float qk_scale_log2;     // sm_scale * k_scale * log2(e) (k_scale = 1 for FP16)
  float v_scale;           // 1 for FP16
  int32_t splits;          // key-range splits per (sequence, kv head)
  int32_t chunk;           // tokens per split, multiple of kTile * waves
  int32_t balance_n;       // n > 0: spread unequal lengths over the n*splits slots
                           // (split partials only, n <= kBalanceMaxSeqs); 0: static
  bool partials;           // write split partials (ws_o, ws_lse) instead of out
  bool row_per_wave;       // one split: each wave owns a whole (row, kv head)
  bool stream_kv;          // non-temporal K/V loads (each byte read once per call)
  uint16_t* out;           // fp16 bits [n][hq][256]
  float* ws_o;             // [n*hq][splits][256] split outputs (v_scale applied)
  float* ws_lse;           // [n*hq][splits] base-2 log-sum-exp, -inf if empty
};

// Merge of split partials into fp16 rows.
struct MergeParams {
  const float* o;          // [rows][splits][256]
  const float* lse;        // [rows][splits]
  int64_t rows;
  int32_t splits;
  uint16_t* out;           // fp16 bits [rows][256]
  // Balanced layout of a whole decode call (see attention): the lengths the
  // attention launch planned with, else nullptr for the static layout.
  const int32_t* lens;     // [n]
  int32_t n;               // sequences (rows = n * hq)
  int32_t hq;
  int32_t max_len;
  int32_t a_shift;         // log2 of the split granularity
};

hipError_t launch_attention(const AttnParams& p, bool fp8, hipStream_t stream);
hipError_t launch_merge(const MergeParams& p, hipStream_t stream);
hipError_t launch_e4m3_table(float* out256, hipStream_t stream);
size_t attention_lds_bytes(int group, int waves);

}  // namespace pgqa
