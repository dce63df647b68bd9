"""The C ABI on the CPU: the library loads, exports every symbol pgqa.h
declares, and rejects bad arguments before any HIP call (no GPU needed)."""
from __future__ import annotations

import ctypes
import math
import os
import re

import pytest

from fp8_kv_amd import pgqa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pgqa.h")


@pytest.fixture(scope="module")
def lib():
    return pgqa.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_0-9]+)\s*\(", text)) - {"defined"})


def test_header_and_binding_agree():
    assert sorted(pgqa.EXPORTS) == declared_functions()


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_header_constants_match_binding():
    text = open(HEADER).read()
    for name in ("PGQA_OK", "PGQA_ERR_NULL", "PGQA_ERR_SHAPE", "PGQA_ERR_LAYOUT",
                 "PGQA_ERR_DTYPE", "PGQA_ERR_WORKSPACE", "PGQA_ERR_HIP", "PGQA_ERR_ARG",
                 "PGQA_KV_FP16", "PGQA_KV_E4M3"):
        m = re.search(rf"#define {name} \(?(-?\d+)\)?", text)
        assert m and int(m.group(1)) == getattr(pgqa, name), name


def test_struct_layout():
    # pgqa_kv_pool: 2 pointers, 3 int64, 3 int32, 2 float, padded to 8 bytes.
    C = pgqa.KVPoolC
    assert [C.page_stride.offset, C.num_pages.offset, C.kv_dtype.offset, C.v_scale.offset] == \
        [16, 40, 48, 56]
    assert ctypes.sizeof(C) == 64


# Fake, aligned, never-dereferenced device addresses: validation must reject
# the call before touching them.
FAKE = 1 << 20


def pool(**kw):
    base = dict(k_base=FAKE, v_base=FAKE + 4096, page_stride=16 * 256, token_stride=256,
                head_stride=256, num_pages=8, page_size=16, kv_dtype=pgqa.PGQA_KV_E4M3,
                k_scale=1.0, v_scale=1.0)
    base.update(kw)
    return pgqa.KVPoolC(**base)


def call(lib, fn="paged_gqa_decode", q=FAKE, kv=None, table=FAKE, max_pages=64, lens=FAKE,
         max_len=1024, n=2, hq=6, hkv=1, d=256, sm=0.0625, splits=0, out=FAKE * 2, ws=None,
         ws_bytes=0):
    kv = pool() if kv is None else kv
    return getattr(lib, fn)(q, ctypes.byref(kv), table, max_pages, lens, max_len, n, hq, hkv, d,
                            sm, splits, out, ws, ws_bytes, None)


@pytest.mark.parametrize("fn", ["paged_gqa_decode", "paged_gqa_prefill_sparse"])
def test_validation_errors(lib, fn):
    E = pgqa
    c = lambda **kw: call(lib, fn, **kw)  # noqa: E731
    assert c(q=None) == E.PGQA_ERR_NULL
    assert c(out=None) == E.PGQA_ERR_NULL
    assert c(table=None) == E.PGQA_ERR_NULL
    assert c(lens=None) == E.PGQA_ERR_NULL
    assert c(kv=pool(k_base=None)) == E.PGQA_ERR_NULL
    assert getattr(lib, fn)(FAKE, None, FAKE, 64, FAKE, 1024, 2, 6, 1, 256, 0.0625, 0, FAKE,
                            None, 0, None) == E.PGQA_ERR_NULL
    assert c(d=128) == E.PGQA_ERR_SHAPE
    assert c(hq=17, hkv=1) == E.PGQA_ERR_SHAPE
    assert c(hq=6, hkv=4) == E.PGQA_ERR_SHAPE
    assert c(hkv=0) == E.PGQA_ERR_SHAPE
    assert c(n=-1) == E.PGQA_ERR_SHAPE
    assert c(max_len=1025) == E.PGQA_ERR_SHAPE        # > max_pages * page_size
    assert c(max_len=1 << 23, max_pages=1 << 20) == E.PGQA_ERR_SHAPE  # > PGQA_MAX_SEQ_LEN
    assert c(max_len=-1) == E.PGQA_ERR_SHAPE
    assert c(kv=pool(page_size=0)) == E.PGQA_ERR_SHAPE
    assert c(kv=pool(num_pages=0)) == E.PGQA_ERR_SHAPE
    assert c(kv=pool(kv_dtype=2)) == E.PGQA_ERR_DTYPE
    assert c(kv=pool(k_base=FAKE + 8)) == E.PGQA_ERR_LAYOUT
    assert c(kv=pool(token_stride=264)) == E.PGQA_ERR_LAYOUT   # 264 B, not 16-aligned
    assert c(kv=pool(page_stride=-4096)) == E.PGQA_ERR_LAYOUT
    assert c(q=FAKE + 2) == E.PGQA_ERR_LAYOUT
    assert c(splits=-1) == E.PGQA_ERR_ARG
    assert c(sm=math.nan) == E.PGQA_ERR_ARG
    assert c(kv=pool(k_scale=math.inf)) == E.PGQA_ERR_ARG
    # FP16 ignores the scales, so a non-finite one is accepted there: the
    # call then fails only for want of a workspace.
    assert c(kv=pool(kv_dtype=pgqa.PGQA_KV_FP16, k_scale=math.inf, token_stride=256),
             splits=4) == E.PGQA_ERR_WORKSPACE
    # Explicit splits need no device query; the workspace is checked.
    assert c(splits=4) == E.PGQA_ERR_WORKSPACE
    need = lib.paged_gqa_workspace_bytes(2, 6, 1, 256, 1024, 4)
    assert need == 2 * 6 * 4 * 257 * 4
    assert c(splits=4, ws=FAKE * 4, ws_bytes=need - 1) == E.PGQA_ERR_WORKSPACE
    assert c(splits=4, ws=FAKE * 4 + 8, ws_bytes=need) == E.PGQA_ERR_WORKSPACE
    # Nothing to do: accepted without any HIP call.
    assert c(n=0, q=None, out=None, table=None, lens=None) == E.PGQA_OK


def test_noalloc_rejects_before_any_hip_call(lib):
    """The no-allocation decode validates like paged_gqa_decode and rejects a
    call whose partials exceed its scratch (explicit splits: no device
    query, nothing launched)."""
    text = open(os.path.join(ROOT, "include", "pgqa.h")).read()
    m = re.search(r"#define PGQA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == pgqa.NOALLOC_SCRATCH_BYTES

    def c(q=FAKE, kv=None, n=2, hq=6, hkv=1, d=256, max_len=1024, max_pages=64, splits=4):
        kv = pool() if kv is None else kv
        return lib.paged_gqa_decode_noalloc(q, ctypes.byref(kv), FAKE, max_pages, FAKE, max_len,
                                            n, hq, hkv, d, 0.0625, splits, FAKE * 2, None)
    assert c(q=None) == pgqa.PGQA_ERR_NULL
    assert c(d=128) == pgqa.PGQA_ERR_SHAPE
    assert c(splits=-1) == pgqa.PGQA_ERR_ARG
    assert c(n=0) == pgqa.PGQA_OK  # nothing to do
    # 64 sequences x 16 heads x 8 splits of (256 + 1) floats: just over 8 MiB.
    big = lib.paged_gqa_workspace_bytes(64, 16, 1, 256, 1024, 8)
    assert big == 64 * 16 * 8 * 257 * 4 > pgqa.NOALLOC_SCRATCH_BYTES
    assert c(n=64, hq=16, splits=8) == pgqa.PGQA_ERR_WORKSPACE
    assert lib.paged_gqa_workspace_bytes(64, 16, 1, 256, 1024, 7) <= pgqa.NOALLOC_SCRATCH_BYTES


def test_workspace_bytes(lib):
    ws = lib.paged_gqa_workspace_bytes
    assert ws(16, 6, 1, 256, 16384, 32) == 16 * 6 * 32 * 257 * 4
    assert ws(16, 6, 1, 256, 16384, 1) == 0
    assert ws(16, 6, 1, 128, 16384, 4) == pgqa.SIZE_MAX
    assert ws(16, 6, 1, 256, -5, 4) == pgqa.SIZE_MAX
    # More splits than 64-token chunks are capped.
    assert lib.paged_gqa_num_splits(1, 1, 100, 50) == 2
    assert lib.paged_gqa_num_splits(1, 1, 16384, 32) == 32
    assert lib.paged_gqa_num_splits(1, 1, 16384, 7) == 7
    assert lib.paged_gqa_num_splits(1, 1, 0, 3) == 1
    assert lib.paged_gqa_num_splits(1, 1, 1 << 22, 100000) == 256
    assert lib.paged_gqa_num_splits(1, 0, 10, 3) < 0


def test_partial_and_merge_validation(lib):
    E = pgqa
    kv = pool()
    args = lambda **kw: [kw.get("q", FAKE), ctypes.byref(kw.get("kv", kv)), FAKE, 64, FAKE,  # noqa: E731
                         1024, 2, 6, 1, kw.get("d", 256), 0.0625, 4, kw.get("po", FAKE * 4),
                         kw.get("pl", FAKE * 8), None]
    assert lib.paged_gqa_decode_partial(*args(q=None)) == E.PGQA_ERR_NULL
    assert lib.paged_gqa_decode_partial(*args(po=None)) == E.PGQA_ERR_NULL
    assert lib.paged_gqa_decode_partial(*args(pl=None)) == E.PGQA_ERR_NULL
    # part_lse takes 4-byte alignment only (the kernels store and load it as
    # single floats).
    assert lib.paged_gqa_decode_partial(*args(pl=FAKE * 8 + 2)) == E.PGQA_ERR_LAYOUT
    assert lib.paged_gqa_decode_partial(*args(d=64)) == E.PGQA_ERR_SHAPE
    m = lib.paged_gqa_merge_partials
    assert m(FAKE, FAKE, 10, 4, 128, FAKE, None) == E.PGQA_ERR_SHAPE
    assert m(FAKE, FAKE, 10, 0, 256, FAKE, None) == E.PGQA_ERR_SHAPE
    assert m(FAKE, FAKE, -1, 4, 256, FAKE, None) == E.PGQA_ERR_SHAPE
    assert m(None, FAKE, 10, 4, 256, FAKE, None) == E.PGQA_ERR_NULL
    assert m(FAKE, FAKE, 10, 4, 256, None, None) == E.PGQA_ERR_NULL
    assert m(FAKE + 8, FAKE, 10, 4, 256, FAKE, None) == E.PGQA_ERR_LAYOUT
    assert m(FAKE, FAKE + 2, 10, 4, 256, FAKE, None) == E.PGQA_ERR_LAYOUT
    assert m(None, None, 0, 4, 256, None, None) == E.PGQA_OK  # nothing to do


def test_e4m3_table_rejects_null(lib):
    assert lib.e4m3_decode_table(None, None) == pgqa.PGQA_ERR_NULL
    assert lib.e4m3_decode_table(FAKE + 4, None) == pgqa.PGQA_ERR_LAYOUT


def test_error_strings(lib):
    for code in range(-7, 1):
        assert lib.pgqa_error_string(code)
    assert lib.pgqa_error_string(-99) == b"unknown error code"


def test_topk_validation(lib):
    """qsa_topk_select: every rejected call returns before any HIP call."""
    f = lib.qsa_topk_select
    ok = dict(scores=FAKE, stride=64, nv=None, rows=2, nb=64, k=8, out=FAKE, cnt=None)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["scores"], a["stride"], a["nv"], a["rows"], a["nb"], a["k"], a["out"],
                 a["cnt"], None)

    assert call(rows=0) == pgqa.PGQA_OK                      # nothing to do, nothing launched
    assert call(rows=-1) == pgqa.PGQA_ERR_SHAPE
    assert call(k=-1) == pgqa.PGQA_ERR_SHAPE
    assert call(nb=-1) == pgqa.PGQA_ERR_SHAPE
    assert call(nb=pgqa.QSA_MAX_BLOCKS + 1, stride=pgqa.QSA_MAX_BLOCKS + 4) == pgqa.PGQA_ERR_SHAPE
    assert call(k=pgqa.QSA_MAX_BLOCKS + 1) == pgqa.PGQA_ERR_SHAPE
    assert call(scores=None) == pgqa.PGQA_ERR_NULL
    assert call(out=None) == pgqa.PGQA_ERR_NULL
    assert call(stride=63) == pgqa.PGQA_ERR_LAYOUT
    assert call(scores=FAKE + 2) == pgqa.PGQA_ERR_LAYOUT
    assert call(out=FAKE + 1) == pgqa.PGQA_ERR_LAYOUT
    assert call(nv=FAKE + 3) == pgqa.PGQA_ERR_LAYOUT
    assert call(cnt=FAKE + 2) == pgqa.PGQA_ERR_LAYOUT


def test_topk_limit_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define PGQA_QSA_MAX_BLOCKS (\d+)", text)
    assert m and int(m.group(1)) == pgqa.QSA_MAX_BLOCKS


def test_page4_validation(lib):
    """qsa_build_page4_table: every rejected call returns before any HIP call."""
    f = lib.qsa_build_page4_table
    ok = dict(tok=FAKE, stride=64, n=64, live=FAKE, bt=FAKE, mp=16, seq=None, ns=1, npg=16, P=16,
              V=4, rows=2, out=FAKE, ostride=17, ln=FAKE, st=None)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["tok"], a["stride"], a["n"], a["live"], a["bt"], a["mp"], a["seq"], a["ns"],
                 a["npg"], a["P"], a["V"], a["rows"], a["out"], a["ostride"], a["ln"], a["st"],
                 None)

    assert call(rows=0) == pgqa.PGQA_OK
    for bad in (dict(rows=-1), dict(n=-1), dict(n=pgqa.QSA_MAX_SEL_TOKENS + 1,
                                                 stride=pgqa.QSA_MAX_SEL_TOKENS + 1),
                dict(mp=0), dict(ns=0), dict(npg=-1), dict(P=6), dict(P=0), dict(ostride=0),
                dict(V=3), dict(npg=1 << 30, V=4)):
        assert call(**bad) == pgqa.PGQA_ERR_SHAPE, bad
    for name in ("tok", "live", "bt", "out", "ln"):
        assert call(**{name: None}) == pgqa.PGQA_ERR_NULL, name
    assert call(tok=None, n=0, rows=0) == pgqa.PGQA_OK
    assert call(stride=63) == pgqa.PGQA_ERR_LAYOUT
    for name in ("tok", "live", "bt", "seq", "out", "ln", "st"):
        assert call(**{name: FAKE + 2}) == pgqa.PGQA_ERR_LAYOUT, name


def test_page4_constants_match_header():
    text = open(HEADER).read()
    for name, val in (("PGQA_QSA_MAX_SEL_TOKENS", pgqa.QSA_MAX_SEL_TOKENS),
                      ("PGQA_PAGE4_EMPTY", pgqa.PAGE4_EMPTY),
                      ("PGQA_PAGE4_PARTIAL", pgqa.PAGE4_PARTIAL),
                      ("PGQA_PAGE4_TAIL", pgqa.PAGE4_TAIL), ("PGQA_PAGE4_PAGE", pgqa.PAGE4_PAGE),
                      ("PGQA_PAGE4_OVERFLOW", pgqa.PAGE4_OVERFLOW),
                      ("PGQA_PAGE4_SEQ", pgqa.PAGE4_SEQ), ("PGQA_PAGE4_LONG", pgqa.PAGE4_LONG)):
        m = re.search(rf"#define {name} (\d+)", text)
        assert m and int(m.group(1)) == val, name
    m = re.search(r"#define PGQA_PAGE4_MAX_LIVE \(1 << (\d+)\)", text)
    assert m and (1 << int(m.group(1))) == pgqa.PAGE4_MAX_LIVE
    import oracle
    # The oracle uses the same bit values (it shares no code with the library).
    assert (oracle.PAGE4_EMPTY, oracle.PAGE4_PARTIAL, oracle.PAGE4_TAIL, oracle.PAGE4_PAGE,
            oracle.PAGE4_OVERFLOW, oracle.PAGE4_SEQ, oracle.PAGE4_LONG) == \
        (pgqa.PAGE4_EMPTY, pgqa.PAGE4_PARTIAL, pgqa.PAGE4_TAIL, pgqa.PAGE4_PAGE,
         pgqa.PAGE4_OVERFLOW, pgqa.PAGE4_SEQ, pgqa.PAGE4_LONG)


def test_sampler_validation(lib):
    """sampler_topk_topp_mask: every rejected call returns before any HIP call."""
    f = lib.sampler_topk_topp_mask
    need = lib.sampler_topk_topp_workspace_bytes(4, 1000, 20)
    assert need < (1 << 40)
    ok = dict(z=FAKE, stride=1000, rows=4, V=1000, k=FAKE, p=FAKE, kmax=20, out=FAKE,
              ostride=1000, st=None, ws=FAKE, wsb=need)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["z"], a["stride"], a["rows"], a["V"], a["k"], a["p"], a["kmax"], a["out"],
                 a["ostride"], a["st"], a["ws"], a["wsb"], None)

    assert call(rows=0) == pgqa.PGQA_OK
    for bad in (dict(rows=-1), dict(V=0), dict(V=pgqa.SAMPLER_MAX_VOCAB + 1,
                                              stride=pgqa.SAMPLER_MAX_VOCAB + 1,
                                              ostride=pgqa.SAMPLER_MAX_VOCAB + 1),
                dict(kmax=0), dict(kmax=pgqa.SAMPLER_MAX_K + 1)):
        assert call(**bad) == pgqa.PGQA_ERR_SHAPE, bad
    for name in ("z", "k", "p", "out"):
        assert call(**{name: None}) == pgqa.PGQA_ERR_NULL, name
    assert call(stride=999) == pgqa.PGQA_ERR_LAYOUT
    assert call(ostride=999) == pgqa.PGQA_ERR_LAYOUT
    assert call(ostride=1004) == pgqa.PGQA_ERR_LAYOUT       # in place, other stride
    assert call(out=FAKE + 4 * 16) == pgqa.PGQA_ERR_LAYOUT  # partial overlap
    assert call(out=FAKE - 4 * 3996) == pgqa.PGQA_ERR_LAYOUT  # ends inside logits
    for name in ("z", "k", "p", "out", "st"):
        assert call(**{name: FAKE + 2}) == pgqa.PGQA_ERR_LAYOUT, name
    assert call(ws=None) == pgqa.PGQA_ERR_WORKSPACE
    assert call(wsb=need - 1) == pgqa.PGQA_ERR_WORKSPACE
    assert call(ws=FAKE + 4) == pgqa.PGQA_ERR_WORKSPACE
    assert lib.sampler_topk_topp_workspace_bytes(4, 0, 20) == ctypes.c_size_t(-1).value
    assert lib.sampler_topk_topp_workspace_bytes(4, 1000, 257) == ctypes.c_size_t(-1).value


def test_sampler_constants_match_header():
    text = open(HEADER).read()
    for name, val in (("SAMPLER_MAX_K", pgqa.SAMPLER_MAX_K),
                      ("SAMPLER_MAX_VOCAB", pgqa.SAMPLER_MAX_VOCAB),
                      ("SAMPLER_MASK_BAD_K", pgqa.SAMPLER_MASK_BAD_K),
                      ("SAMPLER_MASK_BAD_P", pgqa.SAMPLER_MASK_BAD_P)):
        m = re.search(rf"#define {name} (\d+)", text)
        assert m and int(m.group(1)) == val, name
    import oracle
    assert (oracle.MASK_BAD_K, oracle.MASK_BAD_P) == (pgqa.SAMPLER_MASK_BAD_K,
                                                      pgqa.SAMPLER_MASK_BAD_P)


def test_stream_read_library_validation():
    """The streaming-read measurement library loads and rejects bad arguments
    before launching anything."""
    from fp8_kv_amd import stream_read as sr
    lib = sr.load()
    f = lib.stream_read
    assert f(FAKE, 64, None, 0, 4, 1, None, None) == -1          # no sink
    assert f(None, 64, None, 0, 4, 1, FAKE, None) == -1          # a missing
    assert f(FAKE, 64, None, 16, 4, 1, FAKE, None) == -1         # b missing
    assert f(FAKE, 64, None, 0, 0, 1, FAKE, None) == -2          # blocks
    assert f(FAKE, 64, None, 0, sr.MAX_BLOCKS + 1, 1, FAKE, None) == -2
    assert f(FAKE, 65, None, 0, 4, 1, FAKE, None) == -2          # not whole words
    assert f(FAKE + 8, 64, None, 0, 4, 1, FAKE, None) == -3      # alignment
    assert f(FAKE, 64, FAKE + 4, 16, 4, 1, FAKE, None) == -3
    assert f(FAKE, 64, None, 0, 4, 1, FAKE + 8, None) == -3
    p = lib.clock_probe
    assert p(None, 100, None) == -1
    assert p(FAKE, 0, None) == -2
    assert p(FAKE, 100001, None) == -2
    assert p(FAKE + 4, 100, None) == -3


def test_explicit_split_counts(lib):
    """A requested split count becomes a chunk length rounded up to a
    multiple of 64 tokens, then the count that chunk gives; at most 256 and
    one split per 64 tokens (no device query for explicit counts)."""
    f = lib.paged_gqa_num_splits
    assert f(2, 1, 16384, 300) == 256
    assert f(2, 1, 16384, 200) == 128
    assert f(2, 1, 16384, 45) == 43
    assert f(2, 1, 16384, 100) == 86
    assert f(2, 1, 12000, 190) == 188
    assert f(1, 1, 64, 5) == 1
    assert f(1, 1, 100, 50) == 2
