"""QSA top-k block selection: the gfx950 kernel against the oracle, bit-exact.

Every case compares the kept indices and the counts element by element with
oracle.topk_select on the same seeded scores.  The cases reach each path of
the kernel: rows no longer than k (everything kept), rows that fit the LDS
candidate buffer (8192 keys), longer rows through the per-thread-maximum
threshold, rows whose candidates overflow the buffer (ties, constant rows, or
k above 1024), the vector-load and scalar-load variants, and every register
slot count (rows of 1..65,536 blocks).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from fp8_kv_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp8_kv_amd import pgqa
    pgqa.load()
    return torch.device("cuda:0")


def run_gpu(case: inputs.TopkCase, dev, *, misalign: bool = False):
    from fp8_kv_amd import pgqa
    sc = torch.from_numpy(case.scores)
    if misalign:  # shift the data by one float: 4-byte but not 16-byte aligned rows
        buf = torch.empty(sc.numel() + 1, dtype=torch.float32, device=dev)
        buf[1:] = sc.reshape(-1).to(dev)
        d_sc = buf[1:].view(sc.shape)
    else:
        d_sc = sc.to(dev)
    nv = torch.from_numpy(case.n_valid).to(dev)
    rows = case.rows
    # Poison the outputs so unwritten entries show up.
    idx = torch.full((rows, case.k), -7, dtype=torch.int32, device=dev)
    cnt = torch.full((rows,), -7, dtype=torch.int32, device=dev)
    print(f"topk rows={rows} n_blocks={case.n_blocks} stride={case.scores.shape[1]} "
          f"k={case.k} meta={case.meta} misalign={misalign}", flush=True)
    pgqa.qsa_topk_select(d_sc, case.k, nv, n_blocks=case.n_blocks, out_idx=idx, out_count=cnt)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), cnt.cpu().numpy()


def check(case: inputs.TopkCase, dev, **kw):
    got_i, got_c = run_gpu(case, dev, **kw)
    ref_i, ref_c = oracle.topk_select(case.scores, case.k, case.n_valid, n_blocks=case.n_blocks)
    assert np.array_equal(got_c, ref_c), np.flatnonzero(got_c != ref_c)[:8]
    bad = np.flatnonzero((got_i != ref_i).any(axis=1))
    assert bad.size == 0, f"rows {bad[:8]} differ; first: got {got_i[bad[0]][:16]} " \
                          f"want {ref_i[bad[0]][:16]}"
    return got_i, got_c


# n_blocks values reach register slot counts 1, 2, 4, 8 and 16 and the
# buffer boundary (8192); odd sizes take the scalar-load path.
SIZES = [1, 3, 100, 2176, 4096, 4097, 8192, 8193, 12000, 16385, 32768, 40001, 65536]


@pytest.mark.parametrize("n_blocks", SIZES)
@pytest.mark.parametrize("k", [1, 37, 512])
def test_topk_normal(dev, n_blocks, k):
    rows = 24 if n_blocks <= 16385 else 8
    check(inputs.topk_case(rows=rows, n_blocks=n_blocks, k=k, seed=n_blocks * 7 + k,
                           n_valid="random"), dev)


@pytest.mark.parametrize("dist", ["ties", "constant", "special", "ramp"])
@pytest.mark.parametrize("n_blocks", [777, 8192, 20000, 65536])
def test_topk_distributions(dev, dist, n_blocks):
    """Ties at the pivot, constant rows (every candidate overflows the
    buffer), signed zeros / infinities / NaNs, and monotone rows."""
    for k in (1, 300, 1024):
        seed = 1000 * ["ties", "constant", "special", "ramp"].index(dist) + k + n_blocks
        check(inputs.topk_case(rows=6, n_blocks=n_blocks, k=k, seed=seed,
                               dist=dist, n_valid="random"), dev)


@pytest.mark.parametrize("k", [1025, 4096, 60000])
def test_topk_large_k(dev, k):
    """k above 1024 skips the threshold; long rows go through the slow path."""
    check(inputs.topk_case(rows=4, n_blocks=65536, k=k, seed=k, n_valid="random"), dev)


def test_topk_scalar_layouts(dev):
    """Row stride not a multiple of 4, and 4-byte (not 16-byte) aligned rows."""
    c = inputs.topk_case(rows=9, n_blocks=9000, k=100, seed=3, row_stride=9003,
                         n_valid="random")
    check(c, dev)
    c = inputs.topk_case(rows=5, n_blocks=16384, k=256, seed=4, n_valid="random")
    check(c, dev, misalign=True)
    # Columns past n_blocks hold +inf and must never be picked.
    c = inputs.topk_case(rows=5, n_blocks=10000, k=64, seed=5, row_stride=10016)
    c.scores[:, 10000:] = np.inf
    check(c, dev)


def test_topk_edges(dev):
    # k = 0; every row empty; k larger than every row.
    check(inputs.topk_case(rows=3, n_blocks=500, k=0, seed=1), dev)
    check(inputs.topk_case(rows=3, n_blocks=500, k=10, seed=2, n_valid=0), dev)
    check(inputs.topk_case(rows=3, n_blocks=500, k=600, seed=3, n_valid="random"), dev)
    # Lengths outside [0, n_blocks] are clamped.
    check(inputs.topk_case(rows=4, n_blocks=9000, k=20, seed=6,
                           n_valid=[-5, 0, 9000, 1 << 30]), dev)
    # Exactly k + 1 eligible blocks, and k = n - 1 on a long row.
    check(inputs.topk_case(rows=2, n_blocks=65536, k=65535, seed=7), dev)
    check(inputs.topk_case(rows=2, n_blocks=9000, k=8999, seed=8, dist="ties"), dev)


def test_topk_zero_rows(dev):
    from fp8_kv_amd import pgqa
    sc = torch.zeros((0, 16), dtype=torch.float32, device=dev)
    idx, cnt = pgqa.qsa_topk_select(sc, 4)
    assert idx.shape == (0, 4) and cnt.shape == (0,)


@pytest.mark.parametrize("n_blocks", [65536, 20000, 12000])
@pytest.mark.parametrize("k", [37, 512])
def test_topk_rows_per_workgroup_mixed_lengths(dev, n_blocks, k):
    """More rows than workgroups, so each workgroup walks several rows and
    loads the next row's first half while the current row is selected.  The
    lengths mix empty, partial and whole register slots and rows at or below
    k, so the next row's slots are loaded every way: during the candidate
    pass (wholly eligible), with their masks after it (partial or past the
    row), and after a row that selects everything."""
    marks = [0, 1, k - 1, k, k + 1, 4095, 4096, 4097, 8191, 8192, 8193, 16385,
             32767, 32768, 32769, 45000, n_blocks - 1, n_blocks]
    marks = sorted({m for m in marks if 0 <= m <= n_blocks})
    rng = np.random.default_rng(n_blocks + k)
    nv = rng.choice(marks, size=600).astype(np.int32)
    check(inputs.topk_case(rows=600, n_blocks=n_blocks, k=k, seed=n_blocks + 3 * k,
                           n_valid=nv), dev)


@pytest.mark.parametrize("name", sorted(inputs.TOPK_WORKLOADS))
def test_topk_workloads(dev, name):
    """The decode (1 x 2,176) and prefill (4096 rows x 61,440..65,535 blocks)
    selections, every row compared."""
    check(inputs.topk_workload_case(name), dev)


def test_topk_deterministic_and_graph(dev):
    """Identical results across eager calls and HIP graph replays."""
    from fp8_kv_amd import pgqa
    case = inputs.topk_case(rows=64, n_blocks=65536, k=512, seed=9, n_valid="causal")
    sc = torch.from_numpy(case.scores).to(dev)
    nv = torch.from_numpy(case.n_valid).to(dev)
    i0, c0 = pgqa.qsa_topk_select(sc, 512, nv)
    torch.cuda.synchronize()
    ref = i0.clone()
    s = torch.cuda.Stream()
    idx = torch.full_like(i0, -7)
    cnt = torch.full_like(c0, -7)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        pgqa.qsa_topk_select(sc, 512, nv, out_idx=idx, out_count=cnt, stream=s)
    for rep in range(3):
        idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref), rep
        assert torch.equal(cnt, c0), rep
