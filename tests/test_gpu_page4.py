"""Virtual page-4 tables: the gfx950 builder against the oracle, bit-exact.

Every case compares the whole output table, the lengths and the status bits
element by element with oracle.qsa_page4_table on the same seeded
selections.  Cases: the 4096-row sparse-prefill shape (512 blocks + 3 causal
tokens per row, one 262,144-token sequence in page-16 pages), every token
order, duplicates, stale positions and padding, each sort width (64 .. 2048
pages per row, including the 8192-token selection that needs more than the
default 64 KiB of LDS), every status bit, several sequences, empty rows and
an empty selection; then the built table driving sparse prefill end to end.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from fp8_kv_amd import inputs
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp8_kv_amd import pgqa
    pgqa.load()
    return torch.device("cuda:0")


def run_gpu(tokens, live, btab, dev, *, row_seq=None, **kw):
    from fp8_kv_amd import pgqa
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    rows = tokens.shape[0]
    out_stride = kw["out_stride"]
    # Poison the outputs so unwritten entries show up.
    t = torch.full((rows, out_stride), -7, dtype=torch.int32, device=dev)
    ln = torch.full((rows,), -7, dtype=torch.int32, device=dev)
    st = torch.full((rows,), -7, dtype=torch.int32, device=dev)
    print(f"page4 rows={rows} n_tokens={tokens.shape[1]} P={kw['page_size']} "
          f"V={kw['vpages_per_page']} out_stride={out_stride}", flush=True)
    pgqa.qsa_build_page4_table(
        torch.from_numpy(tokens).to(dev), torch.from_numpy(np.asarray(live, np.int32)).to(dev),
        torch.from_numpy(np.ascontiguousarray(btab, dtype=np.int32)).to(dev),
        row_seq=None if row_seq is None else torch.from_numpy(np.asarray(row_seq, np.int32)).to(dev),
        out_table=t, out_len=ln, out_status=st, **kw)
    torch.cuda.synchronize()
    return t.cpu().numpy(), ln.cpu().numpy(), st.cpu().numpy()


def check(tokens, live, btab, dev, *, row_seq=None, **kw):
    got = run_gpu(tokens, live, btab, dev, row_seq=row_seq, **kw)
    ref = oracle.qsa_page4_table(tokens, live, btab, row_seq=row_seq, **kw)
    for name, g, r in zip(("table", "len", "status"), got, ref):
        bad = np.flatnonzero((g != r).reshape(g.shape[0], -1).any(axis=1))
        assert bad.size == 0, (f"{name}: rows {bad[:8]} differ; first: got "
                               f"{g[bad[0]][:12]} want {r[bad[0]][:12]}")
    return got


def check_case(case: inputs.Page4Case, dev):
    return check(case.tokens, case.live_len, case.block_table, dev, **case.builder_kwargs())


def test_sparse_prefill_shape(dev):
    """4096 rows x 2051 tokens (the sparse-prefill workload's selections)."""
    case = inputs.page4_workload_case("qsa_page4_table_4096x2051_p16")
    t, ln, st = check_case(case, dev)
    assert np.all(st == 0) and np.all(ln == 2051)


@pytest.mark.parametrize("order", ["expanded", "blocks", "shuffled"])
@pytest.mark.parametrize("layout", ["interleaved", "contiguous"])
def test_orders_and_layouts(dev, order, layout):
    case = inputs.page4_selection_case(rows=300, selected_blocks=100, tail=2, seq_blocks=4096,
                                       page_size=32, order=order, layout=layout, seed=5, pad=37)
    check_case(case, dev)


@pytest.mark.parametrize("blocks,tail", [(10, 1), (60, 3), (100, 0), (250, 2), (500, 4),
                                         (1000, 3), (2040, 4), (2048, 0)])
def test_sort_widths(dev, blocks, tail):
    """Selections of 40 .. 8192 tokens: every sort width of the kernel, and
    the hash sizes up to 16384 slots (more than 64 KiB of LDS)."""
    case = inputs.page4_selection_case(rows=40, selected_blocks=blocks, tail=tail,
                                       seq_blocks=4 * ((blocks + 2003) // 4), page_size=16,
                                       order="shuffled",
                                       seed=blocks, live_tail=max(tail, 1))
    t, ln, st = check_case(case, dev)
    assert np.all(st == 0) and np.all(ln == 4 * blocks + tail)


def defect_rows(rng, rows, P, n_lp, num_pages, n_tokens):
    """Rows of random selections with every kind of defect: partial blocks,
    stale positions, duplicates, padding, non-prefix causal tokens, empty and
    too-long rows.  Returns tokens [rows][n_tokens] and live lengths."""
    tokens = np.full((rows, n_tokens), -1, dtype=np.int32)
    live = np.empty(rows, dtype=np.int32)
    for r in range(rows):
        L = int(rng.integers(-3, P * n_lp + 1))
        if r % 50 == 0:
            L = -(r % 3)                                  # empty rows: 0, -1, -2
        if r % 97 == 5:
            L = (1 << 26) + int(rng.integers(1, 50))
        toks = []
        for b in range(max(0, min(L, P * n_lp) + 3) // 4):
            u = rng.random()
            if u < 0.5:
                toks += [4 * b + i for i in range(4)]
            elif u < 0.53:
                toks += [4 * b + i for i in range(4) if rng.random() < 0.6]
        toks += [int(x) for x in rng.integers(-5, max(L, 1) + 9, size=int(rng.integers(0, 4)))]
        toks = rng.permutation(np.array(toks, dtype=np.int64))[:n_tokens]
        dup = rng.integers(0, 3)
        if dup and toks.size:
            extra = toks[rng.integers(0, toks.size, dup)]
            toks = np.concatenate([toks, extra])[:n_tokens]
        tokens[r, :toks.size] = toks
        live[r] = L
    return tokens, live


@pytest.mark.parametrize("P,V", [(4, 1), (4, 2), (16, 4), (16, 8), (64, 16), (128, 64)])
def test_defects(dev, P, V):
    rng = np.random.default_rng(P * 100 + V)
    n_lp, num_pages = 24, 30
    btab = rng.permutation(num_pages)[:n_lp].astype(np.int32)
    btab[rng.integers(0, n_lp)] = num_pages + 3          # one out-of-range page
    tokens, live = defect_rows(rng, 500, P, n_lp, num_pages, n_tokens=int(P * n_lp * 0.8) + 16)
    _, _, st = check(tokens, live, btab[None], dev, num_pages=num_pages, page_size=P,
                     vpages_per_page=V, out_stride=int(rng.integers(4, P * n_lp // 4 + 2)))
    seen = np.bitwise_or.reduce(st)
    assert seen & oracle.PAGE4_PARTIAL and seen & oracle.PAGE4_EMPTY, seen


def test_every_status(dev):
    """The hand-worked examples (tests/golden/page4_table_examples.txt), one
    launch each."""
    from tests.oracle_pins import _page4_golden
    for c in _page4_golden():
        check(np.array([c["tokens"]], np.int32), [c["L"]], np.array([c["btab"]], np.int32),
              dev, num_pages=c["num_pages"], page_size=c["P"], vpages_per_page=c["V"],
              out_stride=c["out_stride"])


def test_sequences_and_overflow(dev):
    """Rows spread over three sequences (and two invalid sequence ids), and an
    output row too short for some of them."""
    case = inputs.page4_selection_case(rows=200, selected_blocks=30, tail=3, seq_blocks=1024,
                                       page_size=16, order="blocks", seed=12)
    rng = np.random.default_rng(3)
    bts = np.stack([case.block_table[0], rng.permutation(case.num_pages),
                    rng.permutation(case.num_pages)]).astype(np.int32)
    row_seq = rng.integers(-1, 4, size=case.rows).astype(np.int32)
    kw = case.builder_kwargs()
    kw.pop("row_seq")
    _, _, st = check(case.tokens, case.live_len, bts, dev, row_seq=row_seq, **kw)
    assert np.all((st == oracle.PAGE4_SEQ) == ((row_seq < 0) | (row_seq > 2)))
    kw["out_stride"] = 30                                   # 31 pages needed
    _, _, st = check(case.tokens, case.live_len, bts, dev, row_seq=row_seq, **kw)
    assert np.all(st & oracle.PAGE4_OVERFLOW)


@pytest.mark.parametrize("n_tokens", [1, 2, 3, 4, 5, 6, 7])
def test_short_rows(dev, n_tokens):
    """Selections of 1 .. 7 entries: rows shorter than one 16-byte window
    (read entry by entry) and rows whose last chunk is partial (its window
    realigned inside the row).  Causal-only rows, a full block with and
    without causal positions, padding, a stale position and a broken block
    (general path), each against the oracle bit for bit."""
    L = 42                                  # causal block c = 10: positions 40, 41
    rows = [
        [40, 41],                           # causal only
        [41, 40],                           # causal, out of order
        [8, 9, 10, 11, 40, 41],             # full block 2, then causal
        [8, 9, 10, 11, -1, -1, -1],         # full block, padding
        [40, 99, 41],                       # a stale position past L
        [8, 9, 11, 10],                     # block 2 out of order (general path)
        [-1, -1, -1, -1, 40],               # padding, then causal
    ]
    tokens = np.full((len(rows), n_tokens), -1, dtype=np.int32)
    for r, tok in enumerate(rows):
        tok = tok[:n_tokens]
        tokens[r, :len(tok)] = tok
    btab = np.random.default_rng(n_tokens).permutation(16).astype(np.int32)[None]
    check(tokens, [L] * len(rows), btab, dev, num_pages=16, page_size=16, vpages_per_page=4,
          out_stride=4)


def test_empty_selection_and_rows(dev):
    tokens = np.zeros((3, 0), np.int32)
    bt = np.arange(4, dtype=np.int32)[None]
    t, ln, st = check(tokens, [5, 0, -2], bt, dev, num_pages=4, page_size=16, vpages_per_page=4,
                      out_stride=3)
    assert ln.tolist() == [0, 0, 0] and st.tolist() == [0, 1, 1] and np.all(t == -1)


def test_repeat_is_bitwise_identical(dev):
    """The hash layout may differ between runs; the table may not."""
    case = inputs.page4_selection_case(rows=1024, selected_blocks=512, tail=3, seq_blocks=8192,
                                       page_size=16, order="shuffled", seed=21)
    kw = case.builder_kwargs()
    a = run_gpu(case.tokens, case.live_len, case.block_table, dev, **kw)
    b = run_gpu(case.tokens, case.live_len, case.block_table, dev, **kw)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("layout,tail", [("interleaved", 3), ("contiguous", 1),
                                         ("interleaved", 0)])
def test_prefill_through_built_table(dev, layout, tail):
    """Selections -> GPU page-4 table -> GPU sparse prefill over the view,
    against the fp64 oracle's attention over the oracle-built table."""
    from fp8_kv_amd import pgqa
    case = inputs.page4_selection_case(rows=64, selected_blocks=40, tail=tail, seq_blocks=512,
                                       page_size=16, order="shuffled", layout=layout, seed=7,
                                       with_kv=True)
    kw = case.builder_kwargs()
    t, ln, st = check_case(case, dev)
    assert np.all(st == 0)
    view = inputs.page4_view(case.kv, t, ln)
    q, pool, _, _ = pgqa.device_case(view, dev)
    d_t, d_ln, _ = pgqa.qsa_build_page4_table(
        torch.from_numpy(case.tokens).to(dev), torch.from_numpy(case.live_len).to(dev),
        torch.from_numpy(case.block_table).to(dev), **kw)
    out = torch.empty_like(q)
    max_len = int(ln.max())
    wsb = pgqa.paged_gqa_workspace_bytes(q.shape[0], q.shape[1], 1, max_len)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    pgqa.paged_gqa_prefill_sparse(q, pool, d_t, d_ln, max_len, view.sm_scale, out,
                                  num_kv_heads=1, workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.paged_gqa(**view.oracle_kwargs())
    assert_parity(out.cpu().numpy(), ref, f"page4 prefill {layout} tail {tail}")


def test_graph_replay_with_new_selections(dev):
    """One captured build replayed after the selections and live lengths
    change in place: each replay equals the oracle on the new inputs."""
    from fp8_kv_amd import pgqa
    cases = [inputs.page4_selection_case(rows=256, selected_blocks=120, tail=3, seq_blocks=2048,
                                         page_size=16, order=o, seed=sd)
             for o, sd in (("shuffled", 40), ("expanded", 41), ("blocks", 42))]
    kw = cases[0].builder_kwargs()
    tok = torch.from_numpy(cases[0].tokens).to(dev)
    live = torch.from_numpy(cases[0].live_len).to(dev)
    bt = torch.from_numpy(cases[0].block_table).to(dev)
    rows = tok.shape[0]
    t = torch.empty((rows, kw["out_stride"]), dtype=torch.int32, device=dev)
    ln = torch.empty(rows, dtype=torch.int32, device=dev)
    st = torch.empty(rows, dtype=torch.int32, device=dev)

    def build(stream=None):
        pgqa.qsa_build_page4_table(tok, live, bt, out_table=t, out_len=ln, out_status=st,
                                   stream=stream, **kw)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        build(s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        build(s)
    for c in cases[1:] + cases[:1]:
        assert c.tokens.shape == cases[0].tokens.shape and c.builder_kwargs() == kw
        print(f"page4 graph replay tokens {c.tokens.shape} live {c.live_len[:2]}", flush=True)
        tok.copy_(torch.from_numpy(c.tokens))
        live.copy_(torch.from_numpy(c.live_len))
        bt.copy_(torch.from_numpy(c.block_table))
        for x in (t, ln, st):
            x.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = oracle.qsa_page4_table(c.tokens, c.live_len, c.block_table, **kw)
        for name, gv, rv in zip(("table", "len", "status"), (t, ln, st), ref):
            assert np.array_equal(gv.cpu().numpy(), rv), name
