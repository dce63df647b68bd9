"""Seeded synthetic inputs for paged GQA decode and sparse prefill.

This module only draws random numbers and arranges them in memory; it holds
none of the attention arithmetic.  The fp64 oracle and the GPU library both
consume what it returns, so it imports neither of them.

Recipes (page sections cited by title):
  - Decode ("[Kernel][SM70] Scale NVFP4 E4M3 decode batches", Purpose and
    Performance contract): 6 query heads per KV head, head dim 256, batches of
    1-16 sequences with 1K-16K context, FP8-E4M3 KV.  q, K and V are drawn
    from N(0, 1); FP8 KV holds the round-to-nearest-even E4M3 codes of those
    draws (torch's CPU float8_e4m3fn cast), FP16 the binary16 rounding.
  - Sparse prefill ("[Kernel][SM70] Accelerate Qwen3.8 QSA paged prefill",
    Changes): each row selects 4-aligned blocks of a shared KV pool; its
    virtual page-4 table lists the selected blocks in increasing order
    (locality-sorted) followed by the causal partial page.
Seeds: ``numpy.random.SeedSequence(seed).spawn(6)`` children are used, in this
order, for q, K, V, the page tables, the scales and the lengths.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

KV_FP16 = 0
KV_E4M3 = 1
LAYOUTS = ("contiguous", "interleaved", "head_major")


def quantize_e4m3(x: np.ndarray) -> np.ndarray:
    """Round float32 values to OCP E4M3FN codes (uint8) with torch's CPU cast
    (round to nearest, ties to even).  Callers keep |x| < 448."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@dataclass
class PagedCase:
    """One paged-attention problem held in host memory."""

    q: np.ndarray                 # float16 [n][Hq][D]
    k_store: np.ndarray           # pool storage holding K (uint8 codes or float16)
    v_store: np.ndarray           # pool storage holding V (may be k_store itself)
    k_offset: int                 # element offset of K(page 0, slot 0, head 0, dim 0)
    v_offset: int
    page_stride: int              # strides in elements
    token_stride: int
    head_stride: int
    num_pages: int
    page_size: int
    kv_dtype: int                 # KV_FP16 or KV_E4M3
    k_scale: float
    v_scale: float
    table: np.ndarray             # int32 [n][max_pages]
    lens: np.ndarray              # int32 [n]
    max_seq_len: int
    sm_scale: float
    num_kv_heads: int
    layout: str
    meta: dict = field(default_factory=dict)

    @property
    def n(self) -> int:
        return self.q.shape[0]

    @property
    def num_q_heads(self) -> int:
        return self.q.shape[1]

    @property
    def head_dim(self) -> int:
        return self.q.shape[2]

    @property
    def kv_elem_bytes(self) -> int:
        return 2 if self.kv_dtype == KV_FP16 else 1

    def kv_bytes_read(self) -> int:
        """Algorithmic KV bytes one call must read: every live token's K and V
        row for every KV head, read once."""
        live = np.clip(self.lens.astype(np.int64), 0, self.max_seq_len).sum()
        return int(live) * self.num_kv_heads * self.head_dim * self.kv_elem_bytes * 2

    def oracle_kwargs(self) -> dict:
        return dict(q=self.q, k_store=self.k_store, v_store=self.v_store,
                    k_offset=self.k_offset, v_offset=self.v_offset,
                    page_stride=self.page_stride, token_stride=self.token_stride,
                    head_stride=self.head_stride, num_pages=self.num_pages,
                    page_size=self.page_size, kv_dtype=self.kv_dtype,
                    k_scale=self.k_scale, v_scale=self.v_scale, table=self.table,
                    lens=self.lens, sm_scale=self.sm_scale,
                    num_kv_heads=self.num_kv_heads)


def _values(rng: np.random.Generator, shape, kv_dtype: int) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if kv_dtype == KV_E4M3:
        return quantize_e4m3(x)
    return x.astype(np.float16)


def build_pool(kvals: np.ndarray, vvals: np.ndarray, layout: str) -> dict:
    """Lay out K and V page contents ([num_pages][P][Hkv][D] each) as a pool.

    contiguous : separate K and V arrays [num_pages][P][Hkv][D]
    interleaved: one array [num_pages][2][P][Hkv][D] (K block, then V block)
    head_major : separate arrays [num_pages][Hkv][P][D]
    """
    npg, P, hkv, d = kvals.shape
    if layout == "contiguous":
        return dict(k_store=np.ascontiguousarray(kvals), v_store=np.ascontiguousarray(vvals),
                    k_offset=0, v_offset=0, page_stride=P * hkv * d,
                    token_stride=hkv * d, head_stride=d)
    if layout == "interleaved":
        store = np.empty((npg, 2, P, hkv, d), dtype=kvals.dtype)
        store[:, 0] = kvals
        store[:, 1] = vvals
        return dict(k_store=store, v_store=store, k_offset=0, v_offset=P * hkv * d,
                    page_stride=2 * P * hkv * d, token_stride=hkv * d, head_stride=d)
    if layout == "head_major":
        return dict(k_store=np.ascontiguousarray(kvals.transpose(0, 2, 1, 3)),
                    v_store=np.ascontiguousarray(vvals.transpose(0, 2, 1, 3)),
                    k_offset=0, v_offset=0, page_stride=P * hkv * d,
                    token_stride=d, head_stride=P * d)
    raise ValueError(f"unknown layout {layout!r}")


def decode_case(*, batch: int, lens, page_size: int, kv_dtype: int,
                layout: str = "contiguous", seed: int = 0, num_q_heads: int = 6,
                num_kv_heads: int = 1, head_dim: int = 256, scales="unit",
                table: str = "perm", num_pages: int | None = None,
                max_seq_len: int | None = None, sm_scale: float | None = None) -> PagedCase:
    """Paged decode problem.

    lens   : int (all sequences) or a sequence of ints, or ("uniform", lo, hi)
             for lengths drawn uniformly on [lo, hi] from the lengths stream.
    scales : "unit" (1.0, 1.0), "uniform" (each ~ U[0.5, 2]) or a (k, v) pair.
    table  : "perm"  - the pool holds exactly batch*max_pages pages and the
                       tables are a random permutation of them, reshaped;
             "identity" - sequence b owns pages b*max_pages .. in order.
    """
    ss = np.random.SeedSequence(seed).spawn(6)
    rq, rk, rv, rt, rs, rl = (np.random.default_rng(s) for s in ss)
    if isinstance(lens, tuple) and lens and lens[0] == "uniform":
        lens_arr = rl.integers(lens[1], lens[2], size=batch, endpoint=True).astype(np.int32)
    elif np.isscalar(lens):
        lens_arr = np.full(batch, int(lens), dtype=np.int32)
    else:
        lens_arr = np.asarray(lens, dtype=np.int32)
        assert lens_arr.shape == (batch,)
    if max_seq_len is None:
        max_seq_len = max(1, int(lens_arr.max(initial=0)))
    max_pages = -(-max_seq_len // page_size)
    if num_pages is None:
        num_pages = batch * max_pages
    if table == "perm":
        assert num_pages >= batch * max_pages
        tab = rt.permutation(num_pages)[: batch * max_pages].reshape(batch, max_pages)
    elif table == "identity":
        assert num_pages >= batch * max_pages
        tab = np.arange(batch * max_pages).reshape(batch, max_pages)
    else:
        raise ValueError(table)
    if scales == "unit":
        k_scale, v_scale = 1.0, 1.0
    elif scales == "uniform":
        k_scale, v_scale = (float(s) for s in rs.uniform(0.5, 2.0, size=2))
    else:
        k_scale, v_scale = (float(s) for s in scales)
    q = rq.standard_normal((batch, num_q_heads, head_dim), dtype=np.float32).astype(np.float16)
    shape = (num_pages, page_size, num_kv_heads, head_dim)
    pool = build_pool(_values(rk, shape, kv_dtype), _values(rv, shape, kv_dtype), layout)
    return PagedCase(q=q, **pool, num_pages=num_pages, page_size=page_size,
                     kv_dtype=kv_dtype, k_scale=k_scale, v_scale=v_scale,
                     table=np.ascontiguousarray(tab, dtype=np.int32), lens=lens_arr,
                     max_seq_len=int(max_seq_len),
                     sm_scale=(1.0 / np.sqrt(head_dim)) if sm_scale is None else sm_scale,
                     num_kv_heads=num_kv_heads, layout=layout)


def sparse_prefill_case(*, rows: int, selected_blocks: int, tail: int, pool_blocks: int,
                        layout: str = "interleaved", seed: int = 0, num_q_heads: int = 6,
                        num_kv_heads: int = 1, head_dim: int = 256,
                        kv_dtype: int = KV_FP16, scales="unit", page_size: int = 4,
                        share_rows: int = 1) -> PagedCase:
    """Sparse prefill through virtual page tables (page-4 by default).

    Row r owns block c_r = pool_blocks - rows + r (its causal block).  It
    selects `selected_blocks` distinct blocks uniformly from [0, c_r), sorted
    increasingly (locality order), then the partial page: the first `tail`
    tokens of block c_r (tail = 0 means no partial page).  Row length is
    page_size*selected_blocks + tail.  With share_rows = G > 1, each group of
    G consecutive rows shares one selection, drawn below the causal block of
    the group's first row (a stand-in for the overlap of neighbouring query
    rows' selections; the pages do not describe it).  share_rows = 1 draws
    exactly as before.
    """
    P = page_size
    assert 0 <= tail < P and pool_blocks - rows >= selected_blocks
    ss = np.random.SeedSequence(seed).spawn(6)
    rq, rk, rv, rt, rs, _ = (np.random.default_rng(s) for s in ss)
    n_entries = selected_blocks + (1 if tail else 0)
    tab = np.empty((rows, n_entries), dtype=np.int32)
    for r in range(rows):
        c_r = pool_blocks - rows + r
        if r % share_rows == 0:
            sel = np.sort(rt.choice(c_r, size=selected_blocks, replace=False, shuffle=False))
        tab[r, :selected_blocks] = sel
        if tail:
            tab[r, selected_blocks] = c_r
    L = P * selected_blocks + tail
    if scales == "unit":
        k_scale, v_scale = 1.0, 1.0
    elif scales == "uniform":
        k_scale, v_scale = (float(s) for s in rs.uniform(0.5, 2.0, size=2))
    else:
        k_scale, v_scale = (float(s) for s in scales)
    q = rq.standard_normal((rows, num_q_heads, head_dim), dtype=np.float32).astype(np.float16)
    shape = (pool_blocks, P, num_kv_heads, head_dim)
    pool = build_pool(_values(rk, shape, kv_dtype), _values(rv, shape, kv_dtype), layout)
    return PagedCase(q=q, **pool, num_pages=pool_blocks, page_size=P, kv_dtype=kv_dtype,
                     k_scale=k_scale, v_scale=v_scale, table=tab,
                     lens=np.full(rows, L, dtype=np.int32), max_seq_len=L,
                     sm_scale=1.0 / np.sqrt(head_dim), num_kv_heads=num_kv_heads,
                     layout=layout, meta=dict(selected_blocks=selected_blocks, tail=tail,
                                              share_rows=share_rows))


# The five workloads, by what they are.
WORKLOADS = {
    "decode_b1_1k_fp16_p16": dict(kind="decode", batch=1, lens=1024, page_size=16,
                                   kv_dtype=KV_FP16, layout="contiguous", seed=0,
                                   sm_scale=1.0 / 16),
    "decode_b8_1k_e4m3_p64": dict(kind="decode", batch=8, lens=1024, page_size=64,
                                   kv_dtype=KV_E4M3, layout="contiguous", seed=0),
    "decode_b16_16k_e4m3_p128": dict(kind="decode", batch=16, lens=16384, page_size=128,
                                      kv_dtype=KV_E4M3, layout="contiguous", seed=0,
                                      scales="uniform"),
    # The rest of the pages' batch-scaling grid (B1/B8/B16 x 1K/16K), in the
    # benchmark's format (E4M3, page 128, scales ~ U[0.5, 2]).
    "decode_b1_1k_e4m3_p128": dict(kind="decode", batch=1, lens=1024, page_size=128,
                                    kv_dtype=KV_E4M3, layout="contiguous", seed=0,
                                    scales="uniform"),
    "decode_b8_1k_e4m3_p128": dict(kind="decode", batch=8, lens=1024, page_size=128,
                                    kv_dtype=KV_E4M3, layout="contiguous", seed=0,
                                    scales="uniform"),
    "decode_b16_1k_e4m3_p128": dict(kind="decode", batch=16, lens=1024, page_size=128,
                                     kv_dtype=KV_E4M3, layout="contiguous", seed=0,
                                     scales="uniform"),
    "decode_b1_16k_e4m3_p128": dict(kind="decode", batch=1, lens=16384, page_size=128,
                                     kv_dtype=KV_E4M3, layout="contiguous", seed=0,
                                     scales="uniform"),
    "decode_b8_16k_e4m3_p128": dict(kind="decode", batch=8, lens=16384, page_size=128,
                                     kv_dtype=KV_E4M3, layout="contiguous", seed=0,
                                     scales="uniform"),
    "decode_ragged_b16_16k_p256": dict(kind="decode", batch=16, lens=("uniform", 1, 16384),
                                        page_size=256, max_seq_len=16384, seed=0),
    # The other three ragged variants: {FP8, FP16} x {contiguous, interleaved}.
    "decode_ragged_b16_16k_p256_interleaved": dict(kind="decode", batch=16,
                                                    lens=("uniform", 1, 16384), page_size=256,
                                                    max_seq_len=16384, seed=0,
                                                    layout="interleaved"),
    "decode_ragged_b16_16k_p256_fp16": dict(kind="decode", batch=16, lens=("uniform", 1, 16384),
                                             page_size=256, max_seq_len=16384, seed=0,
                                             kv_dtype=KV_FP16),
    "decode_ragged_b16_16k_p256_fp16_interleaved": dict(kind="decode", batch=16,
                                                         lens=("uniform", 1, 16384),
                                                         page_size=256, max_seq_len=16384,
                                                         seed=0, kv_dtype=KV_FP16,
                                                         layout="interleaved"),
    "prefill_sparse_4096x2051_p4": dict(kind="prefill", rows=4096, selected_blocks=512,
                                         tail=3, pool_blocks=65536, layout="interleaved",
                                         seed=0),
    # The same shape over an FP8-E4M3 pool (scales ~ U[0.5, 2]).
    "prefill_sparse_4096x2051_p4_e4m3": dict(kind="prefill", rows=4096, selected_blocks=512,
                                              tail=3, pool_blocks=65536, layout="interleaved",
                                              seed=0, kv_dtype=KV_E4M3, scales="uniform"),
    # The same shape with groups of 32 consecutive rows sharing a selection.
    "prefill_sparse_4096x2051_p4_shared32": dict(kind="prefill", rows=4096,
                                                  selected_blocks=512, tail=3,
                                                  pool_blocks=65536, layout="interleaved",
                                                  seed=0, share_rows=32),
    # The page-16 selected-context sweep at 4096 rows (64, 512, 2048 tokens).
    "prefill_sparse_4096x64_p16": dict(kind="prefill", rows=4096, selected_blocks=4, tail=0,
                                        pool_blocks=16384, page_size=16,
                                        layout="interleaved", seed=0),
    "prefill_sparse_4096x512_p16": dict(kind="prefill", rows=4096, selected_blocks=32, tail=0,
                                         pool_blocks=16384, page_size=16,
                                         layout="interleaved", seed=0),
    "prefill_sparse_4096x2048_p16": dict(kind="prefill", rows=4096, selected_blocks=128,
                                          tail=0, pool_blocks=16384, page_size=16,
                                          layout="interleaved", seed=0),
}


def hybrid_784_16_case(*, batch: int, blocks_per_seq: int, lens, kv_dtype: int = KV_FP16,
                       seed: int = 0, layout: str = "contiguous") -> PagedCase:
    """The hybrid 784/16 geometry: the allocator hands out blocks of 784
    tokens, which the kernel reads as 49 pages of 16 tokens; a sequence's
    page-16 table lists, for each of its allocator blocks (taken in a random,
    nonmonotonic order), that block's 49 kernel pages in order (physical page
    ids in kernel-page units)."""
    sub = 784 // 16
    n_blocks = batch * blocks_per_seq
    case = decode_case(batch=batch, lens=lens, page_size=16, kv_dtype=kv_dtype, seed=seed,
                       layout=layout, num_pages=n_blocks * sub, table="identity",
                       max_seq_len=blocks_per_seq * 784)
    rng = np.random.default_rng(np.random.SeedSequence(seed).spawn(7)[6])
    blocks = rng.permutation(n_blocks).reshape(batch, blocks_per_seq)
    tab = (blocks[:, :, None] * sub + np.arange(sub)[None, None, :]).reshape(batch, -1)
    case.table = np.ascontiguousarray(tab, dtype=np.int32)
    case.meta = dict(allocator_block=784, kernel_page=16)
    return case


def workload_case(name: str, **overrides) -> PagedCase:
    spec = dict(WORKLOADS[name])
    spec.update(overrides)
    kind = spec.pop("kind")
    if kind == "decode":
        spec.setdefault("kv_dtype", KV_E4M3)
        return decode_case(**spec)
    return sparse_prefill_case(**spec)


# ---------------------------------------------------------------- QSA top-k
@dataclass
class TopkCase:
    """Block scores for QSA top-k selection ("[Kernel][SM70] Accelerate exact
    Qwen3.8 decode", Implementation): fp32 scores [rows][row_stride], of which
    row r's first n_valid[r] blocks are eligible; k blocks are kept per row."""
    scores: np.ndarray          # float32 [rows][row_stride]
    n_valid: np.ndarray         # int32 [rows]
    n_blocks: int               # columns the selection may look at (<= row_stride)
    k: int
    meta: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        return int(self.scores.shape[0])

    def score_bytes(self) -> int:
        """Bytes of scores a selection must read: the eligible prefixes."""
        nv = np.clip(self.n_valid.astype(np.int64), 0, self.n_blocks)
        return int(nv.sum()) * 4


def topk_case(*, rows: int, n_blocks: int, k: int, seed: int, dist: str = "normal",
              n_valid="full", row_stride: int | None = None) -> TopkCase:
    """Seeded block scores.

    dist: "normal" (N(0,1) fp32), "ties" (N(0,1) rounded to multiples of 1/4,
    so many blocks share a score), "constant" (every score 0.5), "special"
    (normal draws with +-inf, +-0 and NaNs of both signs mixed in), "ramp"
    (score j = j, increasing with the block index).
    n_valid: "full" (every row sees n_blocks), "causal" (row r sees
    n_blocks - rows + r blocks, the last rows of a prefill chunk), "random"
    (uniform in [0, n_blocks], with 0, 1 and n_blocks forced into the first
    rows), an int, or an explicit per-row sequence.
    Seeds: SeedSequence(seed).spawn(2) children draw the scores and the
    lengths, in that order.
    """
    stride = n_blocks if row_stride is None else int(row_stride)
    assert stride >= n_blocks
    s_rng, l_rng = (np.random.default_rng(c) for c in np.random.SeedSequence(seed).spawn(2))
    shape = (rows, stride)
    if dist == "normal":
        sc = s_rng.standard_normal(shape, dtype=np.float32)
    elif dist == "ties":
        sc = np.round(s_rng.standard_normal(shape, dtype=np.float32) * 4) / 4
    elif dist == "constant":
        sc = np.full(shape, 0.5, dtype=np.float32)
    elif dist == "special":
        sc = s_rng.standard_normal(shape, dtype=np.float32)
        specials = np.array([np.inf, -np.inf, 0.0, -0.0, np.nan, -np.nan], dtype=np.float32)
        specials_bits = specials.view(np.uint32).copy()
        specials_bits[5] |= 0x80000000     # a negative NaN
        specials = specials_bits.view(np.float32)
        pick = s_rng.random(shape) < 0.05
        sc[pick] = specials[s_rng.integers(0, len(specials), size=int(pick.sum()))]
    elif dist == "ramp":
        sc = np.broadcast_to(np.arange(stride, dtype=np.float32), shape).copy()
    else:
        raise ValueError(dist)
    sc = np.ascontiguousarray(sc.astype(np.float32))
    if isinstance(n_valid, str):
        if n_valid == "full":
            nv = np.full(rows, n_blocks, dtype=np.int32)
        elif n_valid == "causal":
            nv = (n_blocks - rows + np.arange(rows)).astype(np.int32)
            assert nv.min() >= 0
        elif n_valid == "random":
            nv = l_rng.integers(0, n_blocks + 1, size=rows).astype(np.int32)
            nv[:3] = [0, 1, n_blocks][:min(3, rows)]
        else:
            raise ValueError(n_valid)
    elif np.isscalar(n_valid):
        nv = np.full(rows, int(n_valid), dtype=np.int32)
    else:
        nv = np.asarray(n_valid, dtype=np.int32)
        assert nv.shape == (rows,)
    return TopkCase(scores=sc, n_valid=np.ascontiguousarray(nv), n_blocks=n_blocks, k=k,
                    meta=dict(seed=seed, dist=dist))


# The QSA selection keeps 512 four-token blocks per query (the 2051-token
# selection layout of "[Kernel][SM70] Accelerate Qwen3.8 QSA paged prefill",
# Changes).  Decode: one sequence at 8,192 input + 512 output tokens (the speed
# gate of "[Kernel][SM70] Accelerate exact Qwen3.8 decode", Scope and
# contract) has 2,176 blocks.  Prefill: the 4096 rows of the sparse-prefill
# workload, row r with 61,440 + r complete blocks behind it (262,144-token
# maximum length, page-4 blocks).
TOPK_WORKLOADS = {
    "qsa_topk_decode_1x2176_k512": dict(rows=1, n_blocks=2176, k=512, seed=71),
    "qsa_topk_prefill_4096x65536_k512": dict(rows=4096, n_blocks=65536, k=512, seed=72,
                                             n_valid="causal"),
}


def topk_workload_case(name: str, **overrides) -> TopkCase:
    kw = dict(TOPK_WORKLOADS[name])
    kw.update(overrides)
    return topk_case(**kw)


@dataclass
class Page4Case:
    """Expanded QSA selections of query rows ("[Kernel][SM70] Accelerate
    Qwen3.8 QSA paged prefill", Changes): row r's selection lists logical token
    positions of its sequence, four per selected 4-token block plus the
    selected tokens of its own (causal) block; the sequence's tokens live in
    physical pages of `page_size` tokens named by a block table."""
    tokens: np.ndarray            # int32 [rows][n_tokens], -1 = padding
    live_len: np.ndarray          # int32 [rows]
    block_table: np.ndarray       # int32 [n_seqs][max_pages]
    row_seq: np.ndarray | None    # int32 [rows] or None (every row in sequence 0)
    num_pages: int                # physical pages in the pool
    page_size: int                # tokens per physical page (a multiple of 4)
    vpages_per_page: int          # page-4 views per physical page: page_stride / (4 token_stride)
    out_stride: int               # entries per output table row
    kv: PagedCase | None = None   # q and the physical pool (with_kv only)
    meta: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        return int(self.tokens.shape[0])

    @property
    def n_tokens(self) -> int:
        return int(self.tokens.shape[1])

    def builder_kwargs(self) -> dict:
        return dict(num_pages=self.num_pages, page_size=self.page_size,
                    vpages_per_page=self.vpages_per_page, out_stride=self.out_stride,
                    row_seq=self.row_seq)


def page4_selection_case(*, rows: int, selected_blocks: int, tail: int, seq_blocks: int,
                         page_size: int = 16, live_tail: int | None = None,
                         order: str = "expanded", layout: str = "interleaved", seed: int = 0,
                         pad: int = 0, out_stride: int | None = None, with_kv: bool = False,
                         kv_dtype: int = KV_FP16, num_q_heads: int = 6, num_kv_heads: int = 1,
                         head_dim: int = 256) -> Page4Case:
    """Selections of `rows` query rows of one sequence of 4*seq_blocks tokens.

    Row r's causal block is c_r = seq_blocks - rows + r and its live length
    4*c_r + live_tail (live_tail in 1..4, default max(tail, 1)).  It selects
    `selected_blocks` distinct blocks drawn uniformly from [0, c_r) plus the
    first `tail` (0..live_tail) tokens of block c_r.
    order: "expanded" (blocks ascending, each as 4b..4b+3, then the causal
    tokens), "blocks" (the blocks in random order, each expanded), or
    "shuffled" (every token position in random order).  `pad` entries of -1
    follow.  The block table is a random permutation of the sequence's
    physical pages (nonmonotonic).  Seeds: SeedSequence(seed).spawn(6) children
    for q, K, V, the block table, the selections and the orders.
    """
    P = page_size
    live_tail = max(tail, 1) if live_tail is None else live_tail
    assert P % 4 == 0 and (4 * seq_blocks) % P == 0
    assert 1 <= live_tail <= 4 and 0 <= tail <= live_tail
    assert seq_blocks - rows >= selected_blocks and rows >= 1
    num_pages = 4 * seq_blocks // P
    ss = np.random.SeedSequence(seed).spawn(6)
    rq, rk, rv, rt, rsel, rord = (np.random.default_rng(s) for s in ss)
    btab = rt.permutation(num_pages).astype(np.int32)[None, :]
    n_tok = 4 * selected_blocks + tail + pad
    tokens = np.full((rows, n_tok), -1, dtype=np.int32)
    live = np.empty(rows, dtype=np.int32)
    quad = np.arange(4, dtype=np.int64)
    for r in range(rows):
        c_r = seq_blocks - rows + r
        live[r] = 4 * c_r + live_tail
        blocks = rsel.choice(c_r, size=selected_blocks, replace=False, shuffle=False)
        if order == "expanded":
            blocks = np.sort(blocks)
        elif order in ("blocks", "shuffled"):
            blocks = rord.permutation(blocks)
        else:
            raise ValueError(order)
        toks = np.concatenate([(4 * blocks.astype(np.int64)[:, None] + quad).reshape(-1),
                               4 * c_r + np.arange(tail, dtype=np.int64)])
        if order == "shuffled":
            toks = rord.permutation(toks)
        tokens[r, :toks.size] = toks
    if out_stride is None:
        out_stride = selected_blocks + 1
    ts = num_kv_heads * head_dim
    kv = None
    if with_kv:
        q = rq.standard_normal((rows, num_q_heads, head_dim), dtype=np.float32).astype(np.float16)
        shape = (num_pages, P, num_kv_heads, head_dim)
        pool = build_pool(_values(rk, shape, kv_dtype), _values(rv, shape, kv_dtype), layout)
        ts = pool["token_stride"]
        kv = PagedCase(q=q, **pool, num_pages=num_pages, page_size=P, kv_dtype=kv_dtype,
                       k_scale=1.0, v_scale=1.0, table=btab, lens=live.copy(),
                       max_seq_len=int(live.max()), sm_scale=1.0 / np.sqrt(head_dim),
                       num_kv_heads=num_kv_heads, layout=layout)
        page_stride = pool["page_stride"]
    else:
        page_stride = (2 if layout == "interleaved" else 1) * P * ts
    assert page_stride % (4 * ts) == 0
    return Page4Case(tokens=tokens, live_len=live, block_table=btab, row_seq=None,
                     num_pages=num_pages, page_size=P,
                     vpages_per_page=page_stride // (4 * ts), out_stride=out_stride, kv=kv,
                     meta=dict(selected_blocks=selected_blocks, tail=tail, order=order,
                               seed=seed, layout=layout))


def page4_view(kv: PagedCase, table: np.ndarray, lens: np.ndarray) -> PagedCase:
    """The same physical pool read as pages of 4 tokens: page i of the view
    starts at element i * 4 * token_stride of the pool (so a view id is
    physical page * page_stride / (4 token_stride) + slot / 4), with the
    given per-row tables and lengths."""
    ts = kv.token_stride
    assert kv.page_stride % (4 * ts) == 0
    # As many view pages as keep both K and V of the last one inside their
    # storage (interleaved pools: the views over a page's V half have no V
    # rows of their own, so the final few ids are left out).
    last = 3 * ts + (kv.num_kv_heads - 1) * kv.head_stride + kv.head_dim  # one page's reach
    room = min(kv.k_store.size - kv.k_offset, kv.v_store.size - kv.v_offset)
    num_pages = (room - last) // (4 * ts) + 1
    return PagedCase(q=kv.q, k_store=kv.k_store, v_store=kv.v_store, k_offset=kv.k_offset,
                     v_offset=kv.v_offset, page_stride=4 * ts, token_stride=ts,
                     head_stride=kv.head_stride, num_pages=num_pages, page_size=4,
                     kv_dtype=kv.kv_dtype, k_scale=kv.k_scale, v_scale=kv.v_scale,
                     table=np.ascontiguousarray(table, dtype=np.int32),
                     lens=np.ascontiguousarray(lens, dtype=np.int32),
                     max_seq_len=max(1, int(np.max(lens, initial=0))), sm_scale=kv.sm_scale,
                     num_kv_heads=kv.num_kv_heads, layout=kv.layout + "/page4-view")


# Page-4 table building for the sparse-prefill workload's shape: 4096 rows,
# 512 selected blocks plus 3 causal tokens each (2051 tokens), one sequence of
# 262,144 tokens in physical pages of 16 tokens, interleaved K/V.
PAGE4_WORKLOADS = {
    "qsa_page4_table_4096x2051_p16": dict(rows=4096, selected_blocks=512, tail=3,
                                          seq_blocks=65536, page_size=16, order="blocks",
                                          layout="interleaved", seed=81),
}


def page4_workload_case(name: str, **overrides) -> Page4Case:
    kw = dict(PAGE4_WORKLOADS[name])
    kw.update(overrides)
    return page4_selection_case(**kw)


@dataclass
class SamplerCase:
    """Sampler logits for combined top-k/top-p masking ("[Kernel][SM70] Scale
    NVFP4 E4M3 decode batches", Purpose and Performance contract: B8/B16 x
    248,320 logits, top-k 20, top-p 0.95)."""
    logits: np.ndarray          # float32 [rows][V]
    k: np.ndarray               # int32 [rows]
    p: np.ndarray               # float32 [rows]
    k_max: int
    meta: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        return int(self.logits.shape[0])

    @property
    def vocab(self) -> int:
        return int(self.logits.shape[1])


def sampler_case(*, rows: int, vocab: int, k=20, p=0.95, seed: int = 0, scale: float = 3.0,
                 dist: str = "normal", k_max: int = 256) -> SamplerCase:
    """Seeded logits.  dist: "normal" (N(0, scale^2) fp32), "ties" (normal
    rounded to multiples of 1/2, so many tokens share a logit), "flat" (every
    logit 0), "peaked" (normal plus a few tokens raised by 10*scale).  k and p:
    scalars or per-row sequences.  Seeds: SeedSequence(seed).spawn(2)
    children draw the logits and the peaks, in that order."""
    z_rng, x_rng = (np.random.default_rng(c) for c in np.random.SeedSequence(seed).spawn(2))
    if dist in ("normal", "ties", "peaked"):
        z = z_rng.standard_normal((rows, vocab), dtype=np.float32) * np.float32(scale)
        if dist == "ties":
            z = np.round(z * 2) / 2
        if dist == "peaked":
            for r in range(rows):
                idx = x_rng.choice(vocab, size=min(5, vocab), replace=False)
                z[r, idx] += np.float32(10 * scale)
    elif dist == "flat":
        z = np.zeros((rows, vocab), dtype=np.float32)
    else:
        raise ValueError(dist)
    kk = np.ascontiguousarray(np.broadcast_to(np.asarray(k, dtype=np.int32), (rows,)))
    pp = np.ascontiguousarray(np.broadcast_to(np.asarray(p, dtype=np.float32), (rows,)))
    return SamplerCase(logits=np.ascontiguousarray(z.astype(np.float32)), k=kk, p=pp,
                       k_max=k_max, meta=dict(seed=seed, dist=dist, scale=scale))


# The pages' sampler workload: B8 and B16 rows of 248,320 logits with top-k 20
# and top-p 0.95; logits ~ N(0, 3^2).
SAMPLER_WORKLOADS = {
    "sampler_topk_topp_b16_248320": dict(rows=16, vocab=248320, k=20, p=0.95, seed=91),
    "sampler_topk_topp_b8_248320": dict(rows=8, vocab=248320, k=20, p=0.95, seed=92),
}


def sampler_workload_case(name: str, **overrides) -> SamplerCase:
    kw = dict(SAMPLER_WORKLOADS[name])
    kw.update(overrides)
    return sampler_case(**kw)
