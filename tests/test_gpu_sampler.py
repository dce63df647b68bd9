"""Combined top-k/top-p masking: the gfx950 kernels against the oracle.

The top-k part is exact integer/ordering work and must match bit for bit:
every kept token is one of the first min(k, V) tokens of the (logit
descending, index ascending) order, kept tokens carry their logit exactly,
all others are -inf, and the kept tokens form a prefix of that order.  The
top-p cut is a floating-point decision (the GPU sums fp32 masses, the oracle
fp64): the kept count must equal the oracle's, except where the oracle's mass
before the boundary token lies within EPS of p, where one token more or less
is also correct.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from fp8_kv_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

EPS = 3e-5  # fp32 sums of <= 256 masses against fp64


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp8_kv_amd import pgqa
    pgqa.load()
    return torch.device("cuda:0")


def run_gpu(z, k, p, dev, *, k_max=256, in_place=False, pad=0):
    from fp8_kv_amd import pgqa
    rows, V = z.shape
    print(f"mask rows={rows} V={V} k={np.unique(k)[:4]} p={np.unique(p)[:4]} k_max={k_max} "
          f"in_place={in_place} pad={pad}", flush=True)
    buf = torch.zeros((rows, V + pad), dtype=torch.float32, device=dev)
    buf[:, :V] = torch.from_numpy(z).to(dev)
    d_z = buf[:, :V]
    out = d_z if in_place else torch.full((rows, V), 7.0, dtype=torch.float32, device=dev)
    st = torch.full((rows,), -7, dtype=torch.int32, device=dev)
    pgqa.sampler_topk_topp_mask(d_z, torch.from_numpy(np.asarray(k, np.int32)).to(dev),
                                torch.from_numpy(np.asarray(p, np.float32)).to(dev),
                                k_max=k_max, out=out, status=st)
    torch.cuda.synchronize()
    return out.cpu().numpy(), st.cpu().numpy()


def order_of(z_row: np.ndarray) -> np.ndarray:
    """(logit descending, index ascending) by totalOrder keys of the fp32 bits."""
    u = z_row.view(np.uint32).astype(np.uint64)
    key = np.where(u & 0x80000000, (~u) & 0xFFFFFFFF, u | 0x80000000)
    return np.lexsort((np.arange(z_row.size), -key.astype(np.int64)))


def check(z, k, p, dev, **kw):
    k = np.broadcast_to(np.asarray(k, np.int32), (z.shape[0],)).copy()
    p = np.broadcast_to(np.asarray(p, np.float32), (z.shape[0],)).copy()
    got, st = run_gpu(z, k, p, dev, **kw)
    ref, rst, rkept = oracle.topk_topp_mask(z, k, p, k_max=kw.get("k_max", 256))
    assert np.array_equal(st, rst), (st, rst)
    loose = 0
    for r in range(z.shape[0]):
        if rst[r]:
            assert np.array_equal(got[r].view(np.uint32), z[r].view(np.uint32)), r
            continue
        order = order_of(z[r])
        n = min(int(k[r]), z.shape[1])
        kept = np.flatnonzero(got[r] != -np.inf) if np.isfinite(z[r]).all() else None
        if kept is None:  # rows with -inf logits: compare with the oracle exactly
            assert np.array_equal(got[r], ref[r]), r
            continue
        ng = kept.size
        # A prefix of the order, inside the top-k set, values unchanged.
        assert np.array_equal(np.sort(order[:ng]), kept) and 1 <= ng <= n, (r, ng, n)
        assert np.array_equal(got[r, kept].view(np.uint32), z[r, kept].view(np.uint32)), r
        no = int(rkept[r])
        if ng != no:
            top = z[r, order[:n]].astype(np.float64)
            w = np.exp(top - top[0])
            before = np.concatenate([[0.0], np.cumsum(w)[:-1]]) / w.sum()
            edge = before[max(ng, no) - 1]   # the mass deciding the token in dispute
            assert abs(ng - no) == 1 and abs(edge - float(p[r])) < EPS, (r, ng, no, edge, p[r])
            loose += 1
    return got, st, loose


@pytest.mark.parametrize("name", sorted(inputs.SAMPLER_WORKLOADS))
def test_workloads(dev, name):
    case = inputs.sampler_workload_case(name)
    _, _, loose = check(case.logits, case.k, case.p, dev)
    assert loose == 0


@pytest.mark.parametrize("k", [1, 2, 20, 64, 65, 200, 255, 256])
@pytest.mark.parametrize("p", [0.0, 0.3, 0.95, 1.0])
def test_k_and_p(dev, k, p):
    case = inputs.sampler_case(rows=6, vocab=50_000, k=k, p=p, seed=k * 10 + int(p * 100))
    check(case.logits, case.k, case.p, dev)


@pytest.mark.parametrize("dist", ["ties", "peaked", "flat"])
def test_distributions(dev, dist):
    case = inputs.sampler_case(rows=5, vocab=100_003, k=[1, 20, 100, 256, 37],
                               p=[0.9, 0.95, 0.5, 1.0, 0.99], seed=3, dist=dist)
    check(case.logits, case.k, case.p, dev)


@pytest.mark.parametrize("V", [1, 7, 100, 4095, 4096, 4097, 65_536, 262_145, 524_288])
def test_vocab_sizes(dev, V):
    """Every chunk plan: one partial chunk, exact multiples, the largest
    vocabulary (64 chunks of 8192)."""
    case = inputs.sampler_case(rows=3, vocab=V, k=[20, 256, 3], p=[0.95, 0.8, 1.0], seed=V % 97)
    check(case.logits, case.k, case.p, dev)


def test_invalid_rows_copied(dev):
    case = inputs.sampler_case(rows=6, vocab=10_000, k=20, p=0.9, seed=8)
    k = np.array([0, -3, 257, 20, 20, 300], np.int32)
    p = np.array([0.9, 0.9, 0.9, np.nan, 0.5, np.nan], np.float32)
    _, st, _ = check(case.logits, k, p, dev)
    assert st.tolist() == [1, 1, 1, 2, 0, 3]
    # A smaller k_max rejects larger k.
    _, st, _ = check(case.logits, [20, 21, 1, 5, 21, 20], 0.9, dev, k_max=20)
    assert st.tolist() == [0, 1, 0, 0, 1, 0]


def test_in_place_and_strides(dev):
    case = inputs.sampler_case(rows=4, vocab=30_001, k=[5, 50, 250, 1], p=0.9, seed=9)
    a, _, _ = check(case.logits, case.k, case.p, dev, in_place=True, pad=3)
    b, _, _ = check(case.logits, case.k, case.p, dev)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_neg_inf_logits(dev):
    """-inf logits rank last; with fewer finite logits than k they fill the set."""
    z = np.full((3, 5000), -np.inf, np.float32)
    rng = np.random.default_rng(2)
    z[0, rng.choice(5000, 3, replace=False)] = [1.0, 2.0, 3.0]
    z[1, :] = rng.standard_normal(5000).astype(np.float32)
    z[1, ::2] = -np.inf
    z[2, 4999] = 0.0
    check(z, [10, 100, 256], [1.0, 0.9, 0.5], dev)


def test_repeat_is_bitwise_identical(dev):
    case = inputs.sampler_workload_case("sampler_topk_topp_b16_248320")
    a, _ = run_gpu(case.logits, case.k, case.p, dev)
    b, _ = run_gpu(case.logits, case.k, case.p, dev)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_graph_replay_with_new_logits(dev):
    """One captured masking call replayed after the logits, k and p change in
    place: each replay equals an eager call on the new inputs bit for bit."""
    from fp8_kv_amd import pgqa
    rows, V = 8, 248_320
    cases = [inputs.sampler_case(rows=rows, vocab=V, k=k, p=p, seed=s)
             for k, p, s in ((20, 0.95, 31), ([1, 256, 64, 20, 5, 100, 200, 2], 0.5, 32),
                             (256, 1.0, 33))]
    z = torch.from_numpy(cases[0].logits).to(dev)
    kk = torch.from_numpy(np.array(cases[0].k, np.int32)).to(dev)
    pp = torch.from_numpy(np.array(cases[0].p, np.float32)).to(dev)
    out = torch.empty_like(z)
    st = torch.empty(rows, dtype=torch.int32, device=dev)
    ws = torch.empty(pgqa.sampler_topk_topp_workspace_bytes(rows, V), dtype=torch.uint8,
                     device=dev)

    def mask(o, so, stream=None):
        pgqa.sampler_topk_topp_mask(z, kk, pp, out=o, status=so, workspace=ws, stream=stream)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        mask(out, st, s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        mask(out, st, s)
    for c in cases[1:] + cases[:1]:
        print(f"sampler graph replay k={np.unique(c.k)[:3]} p={np.unique(c.p)[:3]}", flush=True)
        z.copy_(torch.from_numpy(c.logits))
        kk.copy_(torch.from_numpy(np.array(c.k, np.int32)))
        pp.copy_(torch.from_numpy(np.array(c.p, np.float32)))
        eo = torch.empty_like(z)
        es = torch.empty_like(st)
        mask(eo, es)
        out.fill_(3.0)
        st.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), eo.view(torch.int32))
        assert torch.equal(st, es)
