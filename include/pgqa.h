/*
 * pgqa.h -- C ABI of libpgqa, paged grouped-query attention for MI355X (gfx950).
 *
 * The operation (by page title and section):
 *   - "[Kernel][SM70] Scale NVFP4 E4M3 decode batches", Purpose: decode
 *     attention for batches of sequences where a group of 6 query heads shares
 *     one KV head of dimension 256, K/V gathered through a page table from a
 *     paged pool stored as FP8-E4M3, including long contexts.
 *   - "[Kernel][SM70] Accelerate Qwen3.8 QSA paged prefill", Changes: sparse
 *     prefill, where each query row attends to its selected tokens exposed as
 *     a virtual page table of 4-token pages into a shared FP16 pool; K/V may
 *     use contiguous or interleaved strides; rows are clamped to their live
 *     length and empty rows are inert.
 * For every sequence (or row) b, query head h and kv head g = h / (Hq/Hkv):
 *     z_t = sm_scale * <q[b][h], K_t>,   t = 0 .. L_b - 1
 *     out[b][h] = sum_t exp(z_t - max z) V_t / sum_t exp(z_t - max z)
 * where logical token t lives in physical page page_table[b][t / page_size],
 * slot t % page_size, and K_t, V_t are the pool rows there for kv head g.  For
 * FP8 pools the real value of a stored code c is k_scale * E4M3(c) (K) and
 * v_scale * E4M3(c) (V), E4M3 being the OCP E4M3FN format.  L_b <= 0 gives a
 * zero output row and reads no KV.
 *
 * Conventions shared by every entry point:
 *   - All array pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or retains them.  `stream` is a hipStream_t (NULL
 *     = the default stream).  Work is enqueued asynchronously: a return of
 *     PGQA_OK means the launch was accepted, and device faults surface at the
 *     caller's next synchronisation, as usual in HIP.
 *   - On an argument error code nothing is launched and no output is written.
 *     PGQA_ERR_HIP means the HIP runtime refused a query or a launch (the
 *     status of that call itself, not an error left over from earlier HIP
 *     calls).  A call that launches two kernels never launches the second
 *     after the first was refused; if the second is refused, the first has
 *     run into the workspace only and the output is not written.
 *   - Thread-safe and stateless apart from a per-device cache of the compute
 *     unit count.  Calls may be captured into HIP graphs (no allocation, no
 *     synchronisation, no memset inside).
 */
#ifndef PGQA_H
#define PGQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define PGQA_OK 0
#define PGQA_ERR_NULL (-1)      /* a required pointer is NULL                        */
#define PGQA_ERR_SHAPE (-2)     /* head_dim != 256, Hq not 1..16 x Hkv, bad sizes     */
#define PGQA_ERR_LAYOUT (-3)    /* pointer or stride not 16-byte aligned, bad strides */
#define PGQA_ERR_DTYPE (-4)     /* kv_dtype is neither PGQA_KV_FP16 nor PGQA_KV_E4M3  */
#define PGQA_ERR_WORKSPACE (-5) /* workspace missing or smaller than required         */
#define PGQA_ERR_HIP (-6)       /* the HIP runtime refused a query or a launch        */
#define PGQA_ERR_ARG (-7)       /* non-finite scale, negative split count, ...        */

/* KV element formats. */
#define PGQA_KV_FP16 0 /* IEEE binary16; k_scale / v_scale are ignored           */
#define PGQA_KV_E4M3 1 /* OCP FP8 E4M3FN codes (uint8); real = scale * E4M3(c)  */

#define PGQA_HEAD_DIM 256
#define PGQA_MAX_GROUP 16         /* query heads per kv head                 */
#define PGQA_MAX_SEQ_LEN 4194304  /* tokens per sequence or row (2^22)       */

/*
 * A paged KV pool.  Element (page p, slot t, kv head g, dim d) of K is at
 *     (elem*)k_base + p*page_stride + t*token_stride + g*head_stride + d
 * and likewise for V from v_base; strides are in elements and d is unit
 * stride.  This covers, for a pool [num_pages][P][Hkv][256]:
 *   contiguous  (separate K and V arrays): page_stride = P*Hkv*256,
 *               token_stride = Hkv*256, head_stride = 256;
 *   interleaved (one array [num_pages][2][P][Hkv][256], K block then V block
 *               in every page): v_base = k_base + P*Hkv*256 elements,
 *               page_stride = 2*P*Hkv*256;
 *   head-major  ([num_pages][Hkv][P][256]): token_stride = 256,
 *               head_stride = P*256.
 * k_base, v_base and every stride in bytes must be multiples of 16.
 */
typedef struct pgqa_kv_pool {
  const void* k_base;
  const void* v_base;
  int64_t page_stride;
  int64_t token_stride;
  int64_t head_stride;
  int32_t num_pages;  /* valid page ids are 0 .. num_pages-1 (>= 1)       */
  int32_t page_size;  /* tokens per page, >= 1                            */
  int32_t kv_dtype;   /* PGQA_KV_FP16 or PGQA_KV_E4M3                     */
  float k_scale;      /* per-tensor multipliers, FP8 only, must be finite */
  float v_scale;
} pgqa_kv_pool;

/*
 * Bytes of workspace a decode or prefill call needs for `n` sequences/rows,
 * `num_q_heads` heads and `max_seq_len`, with `num_splits` (0 = the automatic
 * choice for the current device).  Returns 0 when no workspace is needed
 * (a single split) and SIZE_MAX on invalid arguments or a HIP query failure.
 * The workspace holds the fp32 split partials only; it needs no
 * initialisation.
 */
size_t paged_gqa_workspace_bytes(int32_t n, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_seq_len, int32_t num_splits);

/*
 * Split count a call with these arguments would use (num_splits = 0 means the
 * automatic choice for the current device).  Returns < 0 on invalid arguments.
 */
int32_t paged_gqa_num_splits(int32_t n, int32_t num_kv_heads, int32_t max_seq_len,
                             int32_t num_splits);

/*
 * Paged GQA decode (source: "[Kernel][SM70] Scale NVFP4 E4M3 decode batches",
 * Purpose -- batched paged decode with FP8-E4M3 KV and long-context routes).
 *
 * q          : fp16 [batch][num_q_heads][256], contiguous, 16-byte aligned.
 * kv         : host pointer to the pool description (read during the call only).
 * page_table : int32 [batch][max_pages], row-major; only the first
 *              ceil(min(L_b, max_seq_len) / page_size) entries of row b are
 *              used (entries up to ceil(max_seq_len / page_size) may be read
 *              ahead and ignored, so they need not hold valid page ids).
 *              An entry outside [0, num_pages) is never dereferenced: the
 *              affected output row becomes NaN instead.
 * seq_lens   : int32 [batch]; L_b <= 0 gives zeros; L_b is clamped to max_seq_len.
 * max_seq_len: host-side bound on the lengths (sizes the grid and the split
 *              plan); must satisfy max_seq_len <= max_pages * page_size and
 *              max_seq_len <= PGQA_MAX_SEQ_LEN.
 * num_q_heads: group * num_kv_heads with 1 <= group <= 16 (6 in the pages).
 * head_dim   : must be 256.
 * sm_scale   : softmax scale applied to q.K (finite).
 * num_splits : number of key-range splits per (sequence, kv head), 0 = auto
 *              (about one workgroup per compute unit, at most 128 splits);
 *              capped at 256 and at one split per 64 tokens (query the
 *              effective count with paged_gqa_num_splits).
 *              With more than one split the call writes split partials into
 *              `workspace` and merges them (two launches on `stream`).  When
 *              every L_b >= max_seq_len (or batch > 512) the splits are those
 *              of paged_gqa_decode_partial and the result equals it followed
 *              by paged_gqa_merge_partials bit for bit.  Otherwise the
 *              batch * S workgroup slots of each kv head are shared out by
 *              length: one chunk length C (a multiple of 64) for all
 *              sequences, the smallest with sum_b ceil(L_b / C) <= batch * S,
 *              sequence b taking ceil(L_b / C) chunks, so that unequal
 *              lengths keep every workgroup equally busy.
 * out        : fp16 [batch][num_q_heads][256], contiguous, 16-byte aligned;
 *              must not alias q.
 * workspace  : device scratch of at least paged_gqa_workspace_bytes(...) bytes
 *              (may be NULL when that is 0), 16-byte aligned, not shared
 *              with a concurrently running call.
 */
int paged_gqa_decode(const void* q, const pgqa_kv_pool* kv, const int32_t* page_table,
                     int32_t max_pages, const int32_t* seq_lens, int32_t max_seq_len,
                     int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, float sm_scale, int32_t num_splits, void* out,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Sparse paged prefill (source: "[Kernel][SM70] Accelerate Qwen3.8 QSA paged
 * prefill", Changes -- every query row attends to the tokens its virtual
 * page-4 table selects, with no KV copy).
 *
 * Same contract as paged_gqa_decode with query rows in place of sequences:
 * q and out are [rows][num_q_heads][256]; row_tables is int32
 * [rows][max_pages], each row listing the physical pages (normally page_size 4:
 * the selected 4-token blocks in increasing order, then the causal partial
 * page) whose first row_lens[r] tokens the row attends to; max_row_len bounds
 * row_lens.  The result for a row equals paged_gqa_decode on the same table
 * and length.
 */
int paged_gqa_prefill_sparse(const void* q, const pgqa_kv_pool* kv, const int32_t* row_tables,
                             int32_t max_pages, const int32_t* row_lens, int32_t max_row_len,
                             int32_t rows, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, float sm_scale, int32_t num_splits, void* out,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_gqa_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments without the workspace, the same result bit for bit.
 * The split partials go to a scratch array inside the library, one per GPU
 * (PGQA_NOALLOC_SCRATCH_BYTES bytes, held by every GPU the call runs on until
 * the process ends).  The call allocates nothing, takes no workspace and
 * needs none cleared: every scratch byte it reads it has written itself.
 * Calls that overlap on one GPU (two streams, two threads) share that GPU's
 * scratch and race; serialise them.  The first call on a device looks up
 * that device's scratch address (a HIP symbol query, no allocation).
 * Errors: those of paged_gqa_decode; PGQA_ERR_WORKSPACE when
 * paged_gqa_workspace_bytes(...) for the call exceeds
 * PGQA_NOALLOC_SCRATCH_BYTES (nothing is launched); PGQA_ERR_HIP when the
 * scratch address cannot be obtained or a launch is refused.
 */
#define PGQA_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int paged_gqa_decode_noalloc(const void* q, const pgqa_kv_pool* kv, const int32_t* page_table,
                             int32_t max_pages, const int32_t* seq_lens, int32_t max_seq_len,
                             int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, float sm_scale, int32_t num_splits, void* out,
                             void* stream);

/*
 * First stage of paged_gqa_decode alone: per-split partial results, for
 * callers that merge them themselves (e.g. shards of one sequence computed on
 * different devices).  Same arguments as paged_gqa_decode up to num_splits.
 * With S = paged_gqa_num_splits(batch, num_kv_heads, max_seq_len, num_splits),
 * split s of sequence b covers the tokens [s*C, min((s+1)*C, L_b)) for a
 * chunk C = ceil(max_seq_len / S) rounded up to a multiple of 64, and writes
 *   part_o  : fp32 [batch][num_q_heads][S][256], 16-byte aligned: the
 *             split's softmax-weighted mean of V (v_scale applied);
 *   part_lse: fp32 [batch][num_q_heads][S], 4-byte aligned:
 *             log2(sum_t exp(z_t)) over the split's tokens, or -inf for a
 *             split with no live token (its part_o is then not written).
 * Both buffers are caller-allocated device memory of at least the sizes above.
 */
int paged_gqa_decode_partial(const void* q, const pgqa_kv_pool* kv, const int32_t* page_table,
                             int32_t max_pages, const int32_t* seq_lens, int32_t max_seq_len,
                             int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, float sm_scale, int32_t num_splits,
                             float* part_o, float* part_lse, void* stream);

/*
 * Second stage: merge `splits` partials per row by their log-sum-exp
 * (source: "[Kernel][SM70] Scale NVFP4 E4M3 decode batches", Purpose -- the
 * long-context decode routes).  For each of `rows` rows (a row is one
 * (sequence, query head)): out[r] = sum_s 2^(lse_s - M) o_s / sum_s
 * 2^(lse_s - M), M = max_s lse_s; splits with lse = -inf are skipped and a
 * row whose splits are all -inf is zero.  part_o fp32 [rows][splits][256]
 * and out fp16 [rows][256] are 16-byte aligned; part_lse is fp32
 * [rows][splits], 4-byte aligned; head_dim must be 256.
 */
int paged_gqa_merge_partials(const float* part_o, const float* part_lse, int32_t rows,
                             int32_t splits, int32_t head_dim, void* out, void* stream);

/*
 * Writes to out256[c] (device, fp32 [256]) the value the attention kernels'
 * E4M3 dequantisation gives code c with a unit scale (source: "[Kernel][SM70]
 * Scale NVFP4 E4M3 decode batches", Audit fixes -- the E4M3 converter is
 * part of the decode path).  The two NaN codes yield NaN.
 */
int e4m3_decode_table(float* out256, void* stream);

/*
 * QSA top-k block selection (source: "[Kernel][SM70] Accelerate exact Qwen3.8
 * decode", Implementation -- the QSA selection takes the top-k block scores
 * with score radix passes and keeps ties at the pivot in increasing index
 * order).  For each row r, the eligible blocks are j = 0 .. m_r - 1 with
 * m_r = clamp(n_valid[r], 0, n_blocks) (n_valid NULL: m_r = n_blocks).  The
 * kept set is the first min(k, m_r) blocks in the order (score descending,
 * index ascending), where scores are ranked by IEEE 754 totalOrder of their
 * fp32 bit patterns (-NaN < -inf < ... < -0 < +0 < ... < +inf < +NaN; two
 * scores tie only when their bits are equal).
 *
 *   scores     fp32 [rows][row_stride] (device), row r at scores + r*row_stride;
 *              only columns < n_blocks are read, and of row r only < m_r.
 *              4-byte aligned; 16-byte alignment with row_stride and n_blocks
 *              multiples of 4 takes the vector-load path.
 *   row_stride elements, >= n_blocks.
 *   n_valid    int32 [rows] (device) or NULL.
 *   rows       >= 0 (0: nothing is launched).
 *   n_blocks   0 .. PGQA_QSA_MAX_BLOCKS.
 *   k          0 .. PGQA_QSA_MAX_BLOCKS.
 *   out_idx    int32 [rows][k] (device): row r's kept block indices in
 *              increasing order, then -1 in the remaining k - min(k, m_r)
 *              entries.  May be NULL only when k == 0.
 *   out_count  int32 [rows] (device) or NULL: min(k, m_r).
 * Errors: PGQA_ERR_NULL (scores, or out_idx with k > 0, missing while
 * rows > 0), PGQA_ERR_SHAPE (negative rows/k, n_blocks or k out of range),
 * PGQA_ERR_LAYOUT (row_stride < n_blocks or misaligned pointers),
 * PGQA_ERR_HIP (the compute-unit count query or the launch refused).
 */
#define PGQA_QSA_MAX_BLOCKS 65536 /* 262,144 tokens in 4-token blocks */
int qsa_topk_select(const float* scores, int64_t row_stride, const int32_t* n_valid,
                    int32_t rows, int32_t n_blocks, int32_t k, int32_t* out_idx,
                    int32_t* out_count, void* stream);

/*
 * Virtual page-4 table of expanded QSA selections (source: "[Kernel][SM70]
 * Accelerate Qwen3.8 QSA paged prefill", Purpose and Changes -- each selected
 * four-token block is exposed as a zero-copy page of a page-4 view of the KV
 * pool, the pages are locality-sorted, the causal partial page is kept last
 * and checked against the expanded selection, positions past the live length
 * are clamped away and invalid requests are inert).  The result is what
 * paged_gqa_prefill_sparse takes as row_tables / row_lens with page_size 4
 * over the view: k_base and v_base unchanged, page_stride = 4 * token_stride,
 * num_pages = the view pages whose K and V rows both lie in the pool:
 * num_pages * vpages_per_page for separate K and V arrays; an interleaved
 * pool (each page's V rows after its K rows) loses the last few views of its
 * final page, which lie over V rows and are never emitted here.
 *
 * Per row r, with L = live_len[r] and c = (L - 1) / 4 (the 4-token block that
 * holds the row's own position):
 *   S     = the distinct positions t listed in row r with 0 <= t < L
 *           (order, duplicates, padding < 0 and positions >= L do not matter);
 *   pages = the blocks b < c with all of 4b .. 4b+3 in S; any other position
 *           of S below 4c makes the row invalid (PARTIAL);
 *   tail  = S ∩ [4c, L), which must be 4c .. 4c + n_tail - 1 (else TAIL);
 *   id(b) = p * vpages_per_page + (4b mod page_size) / 4 where
 *           p = block_table[seq][4b / page_size] must exist (4b / page_size <
 *           max_pages) and lie in [0, num_pages) (else PAGE);
 *   row   = the pages' ids ascending, then id(c) if n_tail > 0, then -1 up
 *           to out_stride; out_len = 4 * |pages| + n_tail.
 * A row with any status bit set is inert: all -1, out_len 0.
 *
 *   tokens          int32 [rows][token_stride] (device): the expanded
 *                   selection, n_tokens entries per row, logical positions in
 *                   the row's sequence, -1 (any negative) = padding.  May be
 *                   NULL when n_tokens is 0.
 *   n_tokens        0 .. PGQA_QSA_MAX_SEL_TOKENS.
 *   live_len        int32 [rows] (device): tokens 0 .. L-1 exist for the row
 *                   (its position + 1).  L <= 0: EMPTY; L above
 *                   PGQA_PAGE4_MAX_LIVE: LONG (the row is inert).
 *   block_table     int32 [n_seqs][max_pages] (device): physical page of each
 *                   logical page of page_size tokens.
 *   row_seq         int32 [rows] (device) or NULL (every row in sequence 0):
 *                   a value outside [0, n_seqs) gives SEQ.
 *   num_pages       physical pages of the pool (page ids are checked).
 *   page_size       tokens per physical page, a multiple of 4.
 *   vpages_per_page page-4 views per physical page: page_stride /
 *                   (4 * token_stride) of the pool (page_size / 4 for separate
 *                   K and V arrays, page_size / 2 for interleaved K/V pages);
 *                   >= page_size / 4, num_pages * vpages_per_page <= INT32_MAX.
 *   out_table       int32 [rows][out_stride] (device), every entry written.
 *   out_len         int32 [rows] (device).
 *   out_status      int32 [rows] (device) or NULL: OR of PGQA_PAGE4_* bits.
 * Caller-owned device memory; nothing is allocated; runs on `stream`.
 * Errors: PGQA_ERR_SHAPE (sizes out of range), PGQA_ERR_NULL (a required
 * pointer missing while rows > 0), PGQA_ERR_LAYOUT (token_stride < n_tokens or
 * a pointer not 4-byte aligned), PGQA_ERR_HIP (launch refused).  Values inside
 * the device arrays are checked per row and reported in out_status.
 */
#define PGQA_QSA_MAX_SEL_TOKENS 8192
#define PGQA_PAGE4_MAX_LIVE (1 << 26)
#define PGQA_PAGE4_EMPTY 1      /* live_len <= 0 */
#define PGQA_PAGE4_PARTIAL 2    /* a block below the causal one partly selected */
#define PGQA_PAGE4_TAIL 4       /* causal-block positions not a prefix of it */
#define PGQA_PAGE4_PAGE 8       /* a needed page missing from the table or out of range */
#define PGQA_PAGE4_OVERFLOW 16  /* more pages than out_stride */
#define PGQA_PAGE4_SEQ 32       /* row_seq outside [0, n_seqs) */
#define PGQA_PAGE4_LONG 64      /* live_len above PGQA_PAGE4_MAX_LIVE */
int qsa_build_page4_table(const int32_t* tokens, int64_t token_stride, int32_t n_tokens,
                          const int32_t* live_len, const int32_t* block_table,
                          int32_t max_pages, const int32_t* row_seq, int32_t n_seqs,
                          int32_t num_pages, int32_t page_size, int32_t vpages_per_page,
                          int32_t rows, int32_t* out_table, int32_t out_stride,
                          int32_t* out_len, int32_t* out_status, void* stream);

/*
 * Combined top-k / top-p masking of sampler logits (source: "[Kernel][SM70]
 * Scale NVFP4 E4M3 decode batches", Purpose -- combined top-k/top-p masking
 * for B8/B16 x 248,320 logits -- and Performance contract, whose sampler uses
 * top-k 20 and top-p 0.95).  Per row r of `vocab` logits with k = k[r] and
 * p = p[r]:
 *   order the tokens by (logit descending, index ascending), logits ranked by
 *   IEEE 754 totalOrder of their fp32 bit patterns; the first min(k, vocab)
 *   form the top-k set; in that order token i stays iff it is the first or
 *   the softmax mass (over the top-k set, computed in fp32) of the tokens
 *   before it is below p; p >= 1 keeps the whole top-k set; p <= 0 keeps the
 *   first token only.  out[r][t] = logits[r][t] for kept tokens, -inf for
 *   every other token.  Logits are finite or -inf (NaN and +inf give
 *   unspecified masks).
 *
 *   logits       fp32 [rows][row_stride] (device), 4-byte aligned.
 *   rows         >= 0 (0: nothing is launched).
 *   vocab        1 .. SAMPLER_MAX_VOCAB.
 *   k, p         int32 [rows] and fp32 [rows] (device).  A row with k outside
 *                [1, k_max] (status SAMPLER_MASK_BAD_K) or p NaN
 *                (SAMPLER_MASK_BAD_P) is copied to out unchanged.
 *   k_max        1 .. SAMPLER_MAX_K: the largest k the call accepts; sizes
 *                the workspace.
 *   out          fp32 [rows][out_stride] (device); may be `logits` itself
 *                (in place, with out_stride == row_stride); must not
 *                otherwise overlap it.
 *   status       int32 [rows] (device) or NULL: OR of SAMPLER_MASK_* bits.
 *   workspace    device memory, 8-byte aligned, at least
 *                sampler_topk_topp_workspace_bytes(rows, vocab, k_max)
 *                bytes; caller-owned, contents need no initialisation.
 * Runs two kernels on `stream`; nothing is allocated.
 * Errors: PGQA_ERR_SHAPE (rows, vocab or k_max out of range), PGQA_ERR_NULL,
 * PGQA_ERR_LAYOUT (a stride below vocab, a misaligned pointer, out equal
 * to logits with another stride, or out overlapping logits otherwise),
 * PGQA_ERR_WORKSPACE, PGQA_ERR_HIP.
 */
#define SAMPLER_MAX_K 256
#define SAMPLER_MAX_VOCAB 524288
#define SAMPLER_MASK_BAD_K 1
#define SAMPLER_MASK_BAD_P 2
size_t sampler_topk_topp_workspace_bytes(int32_t rows, int32_t vocab, int32_t k_max);
int sampler_topk_topp_mask(const float* logits, int64_t row_stride, int32_t rows, int32_t vocab,
                           const int32_t* k, const float* p, int32_t k_max, float* out,
                           int64_t out_stride, int32_t* status, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Static description of a return code. */
const char* pgqa_error_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* PGQA_H */
