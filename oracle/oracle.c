/*
 * oracle.c -- plain CPU oracle for paged grouped-query attention (fp64), for
 * QSA top-k block selection, for virtual page-4 tables of QSA selections
 * (exact integer/ordering work) and for combined top-k/top-p masking of
 * sampler logits.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or constant with the
 * GPU library: every value below is derived here from the format definitions.
 *
 * What it computes (sources, by page title and section):
 *   - "[Kernel][SM70] Scale NVFP4 E4M3 decode batches", Purpose: FP8-E4M3,
 *     GQA-6, D256 paged decode for batches of sequences, K/V read through a
 *     page table.
 *   - "[Kernel][SM70] Accelerate Qwen3.8 QSA paged prefill", Changes: each
 *     query row attends to a selected token set exposed as a virtual page-4
 *     table (the same paged attention with rows in place of sequences), with
 *     contiguous or interleaved K/V strides and rows clamped to their live
 *     length; invalid (empty) rows are inert.
 * The method reaches an exact result (softmax attention), so the oracle is
 * that definition written out:
 *   1. decode every input exactly (IEEE binary16 for q and FP16 KV, the OCP
 *      E4M3FN definition for FP8 KV; real value = per-tensor scale * code),
 *   2. de-page the sequence's K and V into contiguous fp64 rows,
 *   3. z_t = sm_scale * <q_h, K_t>,  w_t = exp(z_t - max z),
 *      o_h = sum_t w_t V_t / sum_t w_t,  and o_h = 0 for an empty sequence.
 * No blocking, fusion or reordering beyond that.  Parallelism: one OpenMP
 * task per (sequence, kv head) pair; each pair is computed serially.
 *
 * QSA top-k selection ("[Kernel][SM70] Accelerate exact Qwen3.8 decode",
 * Implementation) is exact as well, so the oracle is its definition: a full
 * sort of each row by (score descending, index ascending), the first k kept,
 * reported in increasing index order.  Pinned by numpy's stable argsort,
 * brute-force rank counting, the IEEE totalOrder spot list
 * (tests/golden/fp32_total_order.txt), closed forms and invariants.
 *
 * The virtual page-4 table of a QSA selection ("[Kernel][SM70] Accelerate
 * Qwen3.8 QSA paged prefill", Purpose and Changes) is integer work defined
 * by set operations; the oracle writes them out (sort, dedupe, walk the
 * blocks, look up pages, sort the ids).  Pinned by hand-worked examples
 * (tests/golden/page4_table_examples.txt), enumeration over blocks on tiny
 * inputs, invariants, and attention through the built table against dense
 * attention over the selected positions.
 *
 * Combined top-k / top-p masking of sampler logits ("[Kernel][SM70] Scale
 * NVFP4 E4M3 decode batches", Purpose) is the sort order of the top-k
 * selection followed by a cumulative-probability cut in fp64.  Pinned by
 * hand-worked rows (tests/golden/topk_topp_examples.txt), a numpy float64
 * formulation (lexsort, cumsum), closed forms (p = 1, k = 1, p = 0, flat
 * rows) and invariants.
 *
 * Every function here is pinned by the CPU test suite (closed forms,
 * invariants, and library routines: torch's float8_e4m3fn cast, numpy's
 * binary16 decode, torch scaled_dot_product_attention in float64).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Error codes returned by oracle_paged_gqa. */
#define ORACLE_OK 0
#define ORACLE_ERR_ARG (-1)      /* bad sizes / null pointers                 */
#define ORACLE_ERR_PAGE (-2)     /* a page id outside [0, num_pages)          */
#define ORACLE_ERR_TABLE (-3)    /* a length needs more pages than the table  */
#define ORACLE_ERR_NOMEM (-4)

/* OCP 8-bit floating point, E4M3FN variant (bias 7, no infinities, the two
 * codes S.1111.111 are NaN, largest finite magnitude 448).  The pages name
 * the KV format "FP8-E4M3"; this is the variant whose maximum is 448. */
double oracle_e4m3_value(uint8_t code) {
  int s = code >> 7;
  int e = (code >> 3) & 15;
  int m = code & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m, -9);               /* subnormal: m/8 * 2^(1-7) */
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);  /* normal */
  return s ? -mag : mag;
}

/* IEEE 754 binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double oracle_f16_value(uint16_t bits) {
  int s = bits >> 15;
  int e = (bits >> 10) & 31;
  int m = bits & 1023;
  double mag;
  if (e == 31) {
    if (m != 0) return NAN;
    mag = INFINITY;
  } else if (e == 0) {
    mag = ldexp((double)m, -24);
  } else {
    mag = ldexp(1.0 + (double)m / 1024.0, e - 15);
  }
  return s ? -mag : mag;
}

void oracle_e4m3_table(double* out256) {
  for (int c = 0; c < 256; ++c) out256[c] = oracle_e4m3_value((uint8_t)c);
}

void oracle_f16_decode(const uint16_t* in, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_value(in[i]);
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Read one KV element as a real number.  kv_dtype 0 = FP16 (scale ignored),
 * 1 = FP8-E4M3 (real value = scale * decoded code). */
static double kv_element(const uint8_t* base, int64_t elem_index, int kv_dtype,
                         double scale) {
  if (kv_dtype == 0) {
    uint16_t bits;
    memcpy(&bits, base + 2 * elem_index, 2);
    return oracle_f16_value(bits);
  }
  return scale * oracle_e4m3_value(base[elem_index]);
}

/*
 * Paged GQA attention for a subset of sequences (decode) or query rows
 * (sparse prefill, where each row's "sequence" is its virtual page table).
 *
 * q        : fp16 bits, [n_seq][Hq][D], contiguous.
 * k_base, v_base : host byte pointers to element (page 0, slot 0, head 0,
 *            dim 0) of the K and V pools.  Element (p, t, g, d) sits at
 *            element offset p*page_stride + t*token_stride + g*head_stride + d.
 * table    : int32 [n_seq][max_pages]; logical token i of sequence b lives in
 *            physical page table[b][i / page_size], slot i % page_size.
 * lens     : int32 [n_seq]; length <= 0 means an empty (inert) sequence.
 * seq_ids  : which sequences to compute (n_ids of them); NULL = all n_seq.
 * out      : fp64 [n_ids][Hq][D].
 */
int oracle_paged_gqa(const uint16_t* q, int32_t n_seq, int32_t Hq, int32_t Hkv,
                     int32_t D, const uint8_t* k_base, const uint8_t* v_base,
                     int64_t page_stride, int64_t token_stride,
                     int64_t head_stride, int32_t num_pages, int32_t page_size,
                     int32_t kv_dtype, double k_scale, double v_scale,
                     const int32_t* table, int32_t max_pages,
                     const int32_t* lens, double sm_scale,
                     const int32_t* seq_ids, int32_t n_ids, double* out) {
  if (!q || !k_base || !v_base || !table || !lens || !out) return ORACLE_ERR_ARG;
  if (n_seq < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0 ||
      page_size <= 0 || num_pages < 0 || max_pages < 0 ||
      (kv_dtype != 0 && kv_dtype != 1))
    return ORACLE_ERR_ARG;
  if (!seq_ids) n_ids = n_seq;
  const int32_t group = Hq / Hkv;

  /* Validate every table entry that will be read before computing. */
  for (int32_t i = 0; i < n_ids; ++i) {
    int32_t b = seq_ids ? seq_ids[i] : i;
    if (b < 0 || b >= n_seq) return ORACLE_ERR_ARG;
    int32_t L = lens[b];
    if (L <= 0) continue;
    int64_t pages_needed = ((int64_t)L + page_size - 1) / page_size;
    if (pages_needed > max_pages) return ORACLE_ERR_TABLE;
    for (int64_t j = 0; j < pages_needed; ++j) {
      int32_t p = table[(int64_t)b * max_pages + j];
      if (p < 0 || p >= num_pages) return ORACLE_ERR_PAGE;
    }
  }

  int failed = 0;
  int64_t n_items = (int64_t)n_ids * Hkv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t item = 0; item < n_items; ++item) {
    int32_t i = (int32_t)(item / Hkv);
    int32_t g = (int32_t)(item % Hkv);
    int32_t b = seq_ids ? seq_ids[i] : i;
    int32_t L = lens[b];
    double* o_group = out + ((int64_t)i * Hq + (int64_t)g * group) * D;
    if (L <= 0) {
      memset(o_group, 0, sizeof(double) * (size_t)group * D);
      continue;
    }
    /* Step 2: de-page this sequence's K and V rows for kv head g. */
    double* Kd = (double*)malloc(sizeof(double) * (size_t)L * D);
    double* Vd = (double*)malloc(sizeof(double) * (size_t)L * D);
    double* z = (double*)malloc(sizeof(double) * (size_t)L);
    double* qd = (double*)malloc(sizeof(double) * (size_t)D);
    if (!Kd || !Vd || !z || !qd) {
      free(Kd); free(Vd); free(z); free(qd);
#pragma omp atomic write
      failed = 1;
      continue;
    }
    for (int32_t t = 0; t < L; ++t) {
      int64_t page = table[(int64_t)b * max_pages + t / page_size];
      int64_t slot = t % page_size;
      int64_t row = page * page_stride + slot * token_stride + (int64_t)g * head_stride;
      for (int32_t d = 0; d < D; ++d) {
        Kd[(int64_t)t * D + d] = kv_element(k_base, row + d, kv_dtype, k_scale);
        Vd[(int64_t)t * D + d] = kv_element(v_base, row + d, kv_dtype, v_scale);
      }
    }
    /* Step 3: softmax attention for every query head of the group. */
    for (int32_t hh = 0; hh < group; ++hh) {
      int32_t h = g * group + hh;
      const uint16_t* qrow = q + ((int64_t)b * Hq + h) * D;
      for (int32_t d = 0; d < D; ++d) qd[d] = oracle_f16_value(qrow[d]);
      double zmax = -INFINITY;
      for (int32_t t = 0; t < L; ++t) {
        double acc = 0.0;
        for (int32_t d = 0; d < D; ++d) acc += qd[d] * Kd[(int64_t)t * D + d];
        z[t] = sm_scale * acc;
        if (z[t] > zmax) zmax = z[t];
      }
      double wsum = 0.0;
      for (int32_t t = 0; t < L; ++t) {
        z[t] = exp(z[t] - zmax); /* z now holds the unnormalised weight */
        wsum += z[t];
      }
      double* o = o_group + (int64_t)hh * D;
      for (int32_t d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int32_t t = 0; t < L; ++t) acc += z[t] * Vd[(int64_t)t * D + d];
        o[d] = acc / wsum;
      }
    }
    free(Kd); free(Vd); free(z); free(qd);
  }
  return failed ? ORACLE_ERR_NOMEM : ORACLE_OK;
}

/* ------------------------------------------------------------------------
 * Top-k block selection ("[Kernel][SM70] Accelerate exact Qwen3.8 decode",
 * Implementation: QSA selection by score with increasing-index tie order at
 * the pivot).  Definition: order the row's eligible blocks j < n_valid by
 * (score descending, index ascending), keep the first min(k, n_valid), and
 * report the kept indices in increasing order.  Scores are ranked by their
 * IEEE-754 bit patterns mapped to an order-preserving unsigned key (so -0.0
 * ranks just below +0.0; two scores tie only when their bits are equal).
 */
static uint32_t score_key(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

typedef struct {
  uint32_t key;
  int32_t idx;
} keyed_t;

static int cmp_rank(const void* a, const void* b) {
  const keyed_t* x = (const keyed_t*)a;
  const keyed_t* y = (const keyed_t*)b;
  if (x->key != y->key) return x->key > y->key ? -1 : 1; /* larger score first */
  return x->idx < y->idx ? -1 : (x->idx > y->idx ? 1 : 0); /* then lower index */
}

static int cmp_int(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return x < y ? -1 : (x > y ? 1 : 0);
}

/* scores: [rows][row_stride] fp32; n_valid: [rows] eligible prefix lengths
 * (NULL = all n_blocks); out_idx: [rows][k] (kept indices ascending, then -1);
 * out_count: [rows] number kept. */
int oracle_topk_select(const float* scores, int64_t row_stride, const int32_t* n_valid,
                       int32_t rows, int32_t n_blocks, int32_t k, int32_t* out_idx,
                       int32_t* out_count) {
  if (!scores || !out_idx || !out_count || rows < 0 || n_blocks < 0 || k < 0 ||
      row_stride < n_blocks)
    return ORACLE_ERR_ARG;
  int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t r = 0; r < rows; ++r) {
    int32_t m = n_valid ? n_valid[r] : n_blocks;
    if (m < 0) m = 0;
    if (m > n_blocks) m = n_blocks;
    keyed_t* items = (keyed_t*)malloc(sizeof(keyed_t) * (size_t)(m > 0 ? m : 1));
    if (!items) {
#pragma omp atomic write
      failed = 1;
      continue;
    }
    const float* row = scores + (int64_t)r * row_stride;
    for (int32_t j = 0; j < m; ++j) {
      items[j].key = score_key(row[j]);
      items[j].idx = j;
    }
    qsort(items, (size_t)m, sizeof(keyed_t), cmp_rank);
    int32_t t = m < k ? m : k;
    int32_t* o = out_idx + (int64_t)r * k;
    for (int32_t i = 0; i < t; ++i) o[i] = items[i].idx;
    qsort(o, (size_t)t, sizeof(int32_t), cmp_int);
    for (int32_t i = t; i < k; ++i) o[i] = -1;
    out_count[r] = t;
    free(items);
  }
  return failed ? ORACLE_ERR_NOMEM : ORACLE_OK;
}

/* ---------------------------------------------------------------------------
 * Virtual page-4 table of a QSA selection ("[Kernel][SM70] Accelerate Qwen3.8
 * QSA paged prefill", Purpose and Changes: each four-token selection becomes
 * a zero-copy page of a page-4 view of the KV pool; the page-4 pages are
 * sorted for locality; the causal partial page goes last and is checked
 * against the expanded selection; positions past the live length are clamped
 * away and invalid rows are made inert).
 *
 * Definition, per row r (L = live_len[r], s = row_seq ? row_seq[r] : 0):
 *   L <= 0: the row is inert (status EMPTY); L > 2^26: inert (status LONG).
 *   s outside [0, n_seqs): no block table to read (status SEQ).
 *   S = { t in tokens[r] : 0 <= t < L } as a set (duplicates and stale or
 *       padded positions drop out).
 *   c = (L - 1) / 4, the 4-token block holding the row's own position.
 *   Full pages: blocks b < c with all of 4b .. 4b+3 in S.  Any other token
 *       of S below 4c makes the row PARTIAL.
 *   Causal page: T = S ∩ [4c, L), n_tail = |T|; T must be 4c .. 4c+n_tail-1
 *       (else TAIL).
 *   The virtual page-4 id of block b: the physical page
 *       p = block_table[s][4b / P] must exist (4b / P < max_pages) and lie in
 *       [0, num_pages) (else PAGE); id = p * vpages_per_page + (4b mod P) / 4.
 *   More than out_stride pages: OVERFLOW.
 *   Output row: the full pages' ids ascending, then the causal page's id if
 *       n_tail > 0, then -1; out_len = 4 * n_full + n_tail.  A row with any
 *       status bit set is inert: all -1 and out_len 0.
 * Status bits are ORed (EMPTY or LONG alone when L is out of range).
 * --------------------------------------------------------------------------- */
#define PAGE4_EMPTY 1
#define PAGE4_PARTIAL 2
#define PAGE4_TAIL 4
#define PAGE4_PAGE 8
#define PAGE4_OVERFLOW 16
#define PAGE4_SEQ 32
#define PAGE4_LONG 64
#define PAGE4_MAX_LIVE (1 << 26)

int oracle_qsa_page4_table(const int32_t* tokens, int64_t token_stride, int32_t n_tokens,
                           const int32_t* live_len, const int32_t* block_table,
                           int32_t max_pages, const int32_t* row_seq, int32_t n_seqs,
                           int32_t num_pages,
                           int32_t page_size, int32_t vpages_per_page, int32_t rows,
                           int32_t* out_table, int32_t out_stride, int32_t* out_len,
                           int32_t* out_status) {
  if (!tokens || !live_len || !block_table || !out_table || !out_len || !out_status ||
      rows < 0 || n_tokens < 0 || token_stride < n_tokens || max_pages < 1 ||
      page_size < 4 || page_size % 4 != 0 || vpages_per_page < page_size / 4 ||
      out_stride < 1 || num_pages < 0 || n_seqs < 1)
    return ORACLE_ERR_ARG;
  int failed = 0;
#pragma omp parallel for schedule(dynamic, 16)
  for (int32_t r = 0; r < rows; ++r) {
    int32_t* orow = out_table + (int64_t)r * out_stride;
    for (int32_t i = 0; i < out_stride; ++i) orow[i] = -1;
    out_len[r] = 0;
    const int32_t L = live_len[r];
    if (L <= 0 || L > PAGE4_MAX_LIVE) {
      out_status[r] = L <= 0 ? PAGE4_EMPTY : PAGE4_LONG;
      continue;
    }
    /* S: the live selected positions, sorted, duplicates removed. */
    int32_t* set = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n_tokens > 0 ? n_tokens : 1));
    int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n_tokens / 4 + 1));
    if (!set || !ids) {
      free(set);
      free(ids);
#pragma omp atomic write
      failed = 1;
      continue;
    }
    const int32_t* trow = tokens + (int64_t)r * token_stride;
    int32_t m = 0;
    for (int32_t i = 0; i < n_tokens; ++i)
      if (trow[i] >= 0 && trow[i] < L) set[m++] = trow[i];
    qsort(set, (size_t)m, sizeof(int32_t), cmp_int);
    int32_t u = 0;
    for (int32_t i = 0; i < m; ++i)
      if (u == 0 || set[i] != set[u - 1]) set[u++] = set[i];
    m = u;

    const int32_t c = (L - 1) / 4;
    const int32_t seq = row_seq ? row_seq[r] : 0;
    const int seq_ok = seq >= 0 && seq < n_seqs;
    const int32_t* btab = block_table + (int64_t)(seq_ok ? seq : 0) * max_pages;
    int status = seq_ok ? 0 : PAGE4_SEQ, n_full = 0, below = 0, n_tail = 0;
    /* Walk S in order: whole blocks below c become pages. */
    int32_t i = 0;
    while (i < m && set[i] < 4 * c) {
      const int32_t b = set[i] / 4;
      int32_t j = i;
      while (j < m && set[j] / 4 == b) ++j;
      if (j - i == 4) ids[n_full++] = b; /* four distinct tokens of one block: all of it */
      below += j - i;
      i = j;
    }
    if (below != 4 * n_full) status |= PAGE4_PARTIAL;
    n_tail = m - i; /* the tokens of S in [4c, L) */
    if (n_tail > 0 && set[m - 1] != 4 * c + n_tail - 1) status |= PAGE4_TAIL;
    const int32_t n_pages = n_full + (n_tail > 0 ? 1 : 0);
    if (n_pages > out_stride) status |= PAGE4_OVERFLOW;
    if (n_tail > 0) ids[n_full] = c;
    /* Logical block -> virtual page-4 id through the physical block table. */
    for (int32_t k = 0; seq_ok && k < n_pages; ++k) {
      const int32_t b = ids[k];
      const int64_t lp = (int64_t)b * 4 / page_size;
      const int32_t p = lp < max_pages ? btab[lp] : -1;
      if (p < 0 || p >= num_pages) {
        status |= PAGE4_PAGE;
        ids[k] = -1;
      } else {
        ids[k] = p * vpages_per_page + (int32_t)(((int64_t)b * 4 % page_size) / 4);
      }
    }
    out_status[r] = status;
    if (status == 0) {
      qsort(ids, (size_t)n_full, sizeof(int32_t), cmp_int); /* locality order */
      for (int32_t k = 0; k < n_pages; ++k) orow[k] = ids[k];
      out_len[r] = 4 * n_full + n_tail;
    }
    free(set);
    free(ids);
  }
  return failed ? ORACLE_ERR_NOMEM : ORACLE_OK;
}

/* ---------------------------------------------------------------------------
 * Combined top-k / top-p masking of sampler logits ("[Kernel][SM70] Scale
 * NVFP4 E4M3 decode batches", Purpose: combined top-k/top-p masking for B8/B16
 * x 248,320 logits; Performance contract: sampler top-k 20, top-p 0.95).
 *
 * Definition, per row r of V logits (k = k_row[r], p = p_row[r]):
 *   k < 1 or k > k_max, or p NaN: the row is invalid (status bit 1 or 2)
 *       and copied unchanged.
 *   Order the V tokens by (logit descending, index ascending), logits ranked
 *   by their IEEE 754 totalOrder keys.  The top-k set is the first
 *   n = min(k, V) tokens of that order.
 *   Top-p over them, in that order: with m the first logit, w_i = exp(z_i -
 *   m) and W = sum of w_i, token i (1-based) stays iff i == 1 or
 *   (w_1 + .. + w_{i-1}) / W < p.  p >= 1 keeps all n.
 *   out[t] = logit[t] for kept tokens, -inf for every other token.
 * Sums and exponentials in fp64.
 * --------------------------------------------------------------------------- */
#define MASK_BAD_K 1
#define MASK_BAD_P 2

int oracle_topk_topp_mask(const float* logits, int64_t row_stride, int32_t rows, int32_t V,
                          const int32_t* k_row, const float* p_row, int32_t k_max,
                          float* out, int64_t out_stride, int32_t* status, int32_t* n_kept) {
  if (!logits || !k_row || !p_row || !out || !status || !n_kept || rows < 0 || V < 1 ||
      row_stride < V || out_stride < V || k_max < 1)
    return ORACLE_ERR_ARG;
  int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t r = 0; r < rows; ++r) {
    const float* z = logits + (int64_t)r * row_stride;
    float* o = out + (int64_t)r * out_stride;
    const int32_t k = k_row[r];
    const float p = p_row[r];
    int st = 0;
    if (k < 1 || k > k_max) st |= MASK_BAD_K;
    if (isnan(p)) st |= MASK_BAD_P;
    status[r] = st;
    if (st) {
      for (int32_t t = 0; t < V; ++t) o[t] = z[t];
      n_kept[r] = V;
      continue;
    }
    keyed_t* items = (keyed_t*)malloc(sizeof(keyed_t) * (size_t)V);
    if (!items) {
#pragma omp atomic write
      failed = 1;
      continue;
    }
    for (int32_t t = 0; t < V; ++t) {
      items[t].key = score_key(z[t]);
      items[t].idx = t;
    }
    qsort(items, (size_t)V, sizeof(keyed_t), cmp_rank); /* logit desc, index asc */
    const int32_t n = k < V ? k : V;
    int32_t keep = n;
    if (p < 1.0f) {
      const double m = (double)z[items[0].idx];
      double W = 0.0;
      for (int32_t i = 0; i < n; ++i) W += exp((double)z[items[i].idx] - m);
      double before = 0.0;
      keep = 1;
      for (int32_t i = 1; i < n; ++i) {
        before += exp((double)z[items[i - 1].idx] - m);
        if (before / W < (double)p)
          keep = i + 1;
        else
          break;
      }
    }
    for (int32_t t = 0; t < V; ++t) o[t] = -INFINITY;
    for (int32_t i = 0; i < keep; ++i) o[items[i].idx] = z[items[i].idx];
    n_kept[r] = keep;
    free(items);
  }
  return failed ? ORACLE_ERR_NOMEM : ORACLE_OK;
}
