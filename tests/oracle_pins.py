"""Checks that pin the fp64 oracle to facts other than itself.

Each ``pin_*`` function takes the path of an oracle library build and raises
AssertionError when the oracle disagrees with:
  - a library routine that implements the same definition independently
    (torch's float8_e4m3fn cast, numpy's binary16 decode, torch's
    scaled_dot_product_attention in float64 with a boolean mask for the
    selected-token case),
  - a closed form (context length 1, uniform keys, zero query, two tokens,
    one dominating key),
  - an invariant of the definition (physical page permutation, K/V layout,
    logical token order, scale factoring, linearity in the V scale),
  - the E4M3 spot values worked out from the format definition
    (tests/golden/e4m3_spot_values.txt).
The same functions run against deliberately broken oracle builds in
test_oracle_mutants.py, which shows that each planted mistake fails a pin.
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch

import oracle
from fp8_kv_amd import inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------- helpers
def logical_kv(case: inputs.PagedCase, b: int):
    """K, V of sequence b as float64 [L][Hkv][D] for an identity-table,
    contiguous-layout case (pages b*max_pages.. in order: a plain reshape)."""
    assert case.layout == "contiguous"
    mp = case.table.shape[1]
    assert np.array_equal(case.table[b], np.arange(b * mp, (b + 1) * mp))
    L = int(case.lens[b])
    P, hkv, d = case.page_size, case.num_kv_heads, case.head_dim
    ks = case.k_store.reshape(case.num_pages, P, hkv, d)[b * mp:(b + 1) * mp]
    vs = case.v_store.reshape(case.num_pages, P, hkv, d)[b * mp:(b + 1) * mp]
    ks = ks.reshape(mp * P, hkv, d)[:L]
    vs = vs.reshape(mp * P, hkv, d)[:L]
    return decode_kv(ks, case.kv_dtype, case.k_scale), decode_kv(vs, case.kv_dtype, case.v_scale)


def decode_kv(arr: np.ndarray, kv_dtype: int, scale: float) -> np.ndarray:
    """Library decode of pool values: numpy binary16, torch float8_e4m3fn."""
    if kv_dtype == inputs.KV_FP16:
        return arr.astype(np.float64)
    t = torch.from_numpy(np.ascontiguousarray(arr)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy() * scale


def sdpa(q: np.ndarray, k: np.ndarray, v: np.ndarray, sm_scale: float,
         mask: np.ndarray | None = None) -> np.ndarray:
    """torch scaled_dot_product_attention in float64 on the CPU.
    q [Hq][D]; k, v [L][Hkv][D]; returns [Hq][D]."""
    tq = torch.from_numpy(q.astype(np.float64))[None, :, None, :]
    tk = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))[None]
    tv = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))[None]
    m = None if mask is None else torch.from_numpy(mask)[None, None, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=m, scale=sm_scale, enable_gqa=True)
    return o[0, :, 0, :].numpy()


def run(case: inputs.PagedCase, lib: str, **kw) -> np.ndarray:
    return oracle.paged_gqa(**case.oracle_kwargs(), lib_path=lib, **kw)


def close(a, b, rtol=1e-12, atol=1e-13, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = np.abs(a - b)
    bound = atol + rtol * np.abs(b)
    assert np.all(err <= bound), f"{what}: max err {err.max():.3e}"


def _with_kv(case: inputs.PagedCase, kfun=None, vfun=None) -> inputs.PagedCase:
    """Copy of a contiguous case with K and/or V storage rewritten."""
    import dataclasses
    ks = case.k_store.copy() if kfun is None else kfun(case.k_store.copy())
    vs = case.v_store.copy() if vfun is None else vfun(case.v_store.copy())
    return dataclasses.replace(case, k_store=ks, v_store=vs)


# -------------------------------------------------------------- the pins
def pin_e4m3_vs_torch(lib: str) -> None:
    """All 256 codes against torch's float8_e4m3fn -> float64 (NaN == NaN)."""
    ours = oracle.e4m3_table(lib)
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(
        torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.flatnonzero(np.isnan(ours)).tolist() == [0x7F, 0xFF]
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))
    assert np.nanmax(ours) == 448.0 and np.nanmin(ours) == -448.0


def pin_e4m3_golden(lib: str) -> None:
    ours = oracle.e4m3_table(lib)
    n = 0
    with open(os.path.join(GOLDEN, "e4m3_spot_values.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            code_s, val_s = line.split()[:2]
            code, val = int(code_s, 16), float(val_s)
            if math.isnan(val):
                assert math.isnan(ours[code]), hex(code)
            else:
                assert ours[code] == val and math.copysign(1, ours[code]) == math.copysign(1, val), hex(code)
            n += 1
    assert n >= 15


def pin_f16_vs_numpy(lib: str) -> None:
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_decode(bits, lib)
    ref = bits.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))


def pin_sdpa(lib: str) -> None:
    """Identity tables, contiguous layout: the paged result equals torch's
    float64 attention on the logical K/V (GQA groups of consecutive heads)."""
    cases = [
        dict(batch=3, lens=[37, 16, 50], page_size=16, kv_dtype=inputs.KV_FP16),
        dict(batch=2, lens=[64, 29], page_size=8, kv_dtype=inputs.KV_E4M3, scales=(0.75, 1.5)),
        dict(batch=2, lens=[33, 7], page_size=4, kv_dtype=inputs.KV_E4M3, scales="uniform",
             num_q_heads=12, num_kv_heads=2),
        dict(batch=1, lens=[20], page_size=5, kv_dtype=inputs.KV_FP16, num_q_heads=8,
             num_kv_heads=4, head_dim=64),
    ]
    for i, kw in enumerate(cases):
        case = inputs.decode_case(table="identity", seed=100 + i, **kw)
        got = run(case, lib)
        for b in range(case.n):
            k, v = logical_kv(case, b)
            ref = sdpa(case.q[b].astype(np.float64), k, v, case.sm_scale)
            close(got[b], ref, rtol=1e-11, atol=1e-13, what=f"sdpa case {i} seq {b}")


def pin_sparse_vs_masked_sdpa(lib: str) -> None:
    """Sparse prefill: each row equals dense attention over the whole (tiny)
    pool, masked to exactly the tokens its virtual page-4 table selects.  Tail
    counts 1, 2, 3 and 0."""
    for tail in (1, 2, 3, 0):
        case = inputs.sparse_prefill_case(rows=5, selected_blocks=6, tail=tail, pool_blocks=16,
                                          layout="contiguous", seed=7 + tail,
                                          kv_dtype=inputs.KV_E4M3, scales="uniform")
        got = run(case, lib)
        P, hkv, d = 4, case.num_kv_heads, case.head_dim
        kall = decode_kv(case.k_store.reshape(-1, hkv, d), case.kv_dtype, case.k_scale)
        vall = decode_kv(case.v_store.reshape(-1, hkv, d), case.kv_dtype, case.v_scale)
        for r in range(case.n):
            mask = np.zeros(kall.shape[0], dtype=bool)
            nsel = case.meta["selected_blocks"]
            for blk in case.table[r, :nsel]:
                mask[P * blk:P * blk + P] = True
            if tail:
                c = case.table[r, nsel]
                mask[P * c:P * c + tail] = True
            assert mask.sum() == case.lens[r]
            ref = sdpa(case.q[r].astype(np.float64), kall, vall, case.sm_scale, mask)
            close(got[r], ref, rtol=1e-11, atol=1e-13, what=f"tail {tail} row {r}")


def pin_closed_forms(lib: str) -> None:
    base = inputs.decode_case(batch=1, lens=1, page_size=4, kv_dtype=inputs.KV_E4M3,
                              table="identity", scales=(1.25, 0.625), seed=3)
    # Context length 1: output = V_0 (times the V scale), exactly.
    got = run(base, lib)
    v0 = decode_kv(base.v_store.reshape(-1, 1, 256)[0], base.kv_dtype, base.v_scale)
    for h in range(6):
        assert np.array_equal(got[0, h], v0[0]), "L=1"

    # Uniform keys (every K row identical): output = mean of V.
    L = 23
    case = inputs.decode_case(batch=1, lens=L, page_size=4, kv_dtype=inputs.KV_E4M3,
                              table="identity", scales=(1.5, 0.75), seed=4)

    def same_rows(ks):
        ks = ks.reshape(-1, 256)
        ks[:] = ks[0]
        return ks.reshape(case.k_store.shape)
    uni = _with_kv(case, kfun=same_rows)
    got = run(uni, lib)
    _, v = logical_kv(uni, 0)
    for h in range(6):
        close(got[0, h], v[:, 0].mean(axis=0), rtol=1e-13, atol=1e-15, what="uniform keys")

    # Zero query: output = mean of V whatever the keys.
    import dataclasses
    zq = dataclasses.replace(case, q=np.zeros_like(case.q))
    got = run(zq, lib)
    _, v = logical_kv(zq, 0)
    close(got[0, 0], v[:, 0].mean(axis=0), rtol=1e-13, atol=1e-15, what="zero q")

    # Two tokens: o = s*V1 + (1-s)*V0, s = sigmoid(z1 - z0), K0 = 0, K1 = e_0.
    two = inputs.decode_case(batch=1, lens=2, page_size=2, kv_dtype=inputs.KV_E4M3,
                             table="identity", scales=(1.75, 1.25), seed=5, sm_scale=0.3)

    def keys(ks):
        ks = ks.reshape(-1, 256)
        ks[:] = 0
        ks[1, 0] = 0x38  # 1.0
        return ks.reshape(two.k_store.shape)
    two = _with_kv(two, kfun=keys)
    qv = np.zeros_like(two.q)
    qv[0, :, 0] = np.array([1.0, -2.0, 3.5, 0.0, 0.5, -0.25], dtype=np.float16)
    two = dataclasses.replace(two, q=qv)
    got = run(two, lib)
    _, v = logical_kv(two, 0)
    for h in range(6):
        dz = 0.3 * 1.75 * float(qv[0, h, 0])
        s = 1.0 / (1.0 + math.exp(-dz))
        close(got[0, h], s * v[1, 0] + (1 - s) * v[0, 0], rtol=1e-13, atol=1e-15,
              what=f"two tokens h{h}")

    # One key dominating by a logit gap >= 40: output = that key's V to e^-40.
    dom = inputs.decode_case(batch=1, lens=9, page_size=4, kv_dtype=inputs.KV_FP16,
                             table="identity", seed=6, sm_scale=1.0)

    def domkeys(ks):
        ks = ks.reshape(-1, 256)
        ks[:] = 0
        ks[5, 3] = 64.0
        return ks.reshape(dom.k_store.shape)
    dom = _with_kv(dom, kfun=domkeys)
    qd = np.zeros_like(dom.q)
    qd[0, :, 3] = 1.0
    dom = dataclasses.replace(dom, q=qd)
    got = run(dom, lib)
    _, v = logical_kv(dom, 0)
    close(got[0, 0], v[5, 0], rtol=1e-15, atol=1e-16 + 9 * math.exp(-64) * np.abs(v).max(),
          what="dominant key")


def pin_invariants(lib: str) -> None:
    import dataclasses
    case = inputs.decode_case(batch=3, lens=[45, 64, 17], page_size=8, kv_dtype=inputs.KV_E4M3,
                              scales=(0.8, 1.7), seed=11)
    ref = run(case, lib)

    # Physical page permutation with the table remapped: bitwise identical.
    rng = np.random.default_rng(12)
    perm = rng.permutation(case.num_pages)           # page p moves to perm[p]
    ks = np.empty_like(case.k_store)
    vs = np.empty_like(case.v_store)
    ks[perm] = case.k_store
    vs[perm] = case.v_store
    moved = dataclasses.replace(case, k_store=ks, v_store=vs,
                                table=perm[case.table].astype(np.int32))
    assert np.array_equal(run(moved, lib), ref), "page permutation"

    # K/V layout: contiguous, interleaved and head-major give identical results.
    for layout in ("interleaved", "head_major"):
        other = inputs.decode_case(batch=3, lens=[45, 64, 17], page_size=8,
                                   kv_dtype=inputs.KV_E4M3, scales=(0.8, 1.7), seed=11,
                                   layout=layout)
        assert np.array_equal(run(other, lib), ref), layout

    # Scale factoring: (k_scale * c, sm_scale / c) leaves the logits unchanged.
    f = dataclasses.replace(case, k_scale=case.k_scale * 4.0, sm_scale=case.sm_scale / 4.0)
    close(run(f, lib), ref, rtol=1e-12, atol=1e-14, what="scale factoring")

    # Linearity in the V scale (a power of two: exact).
    lin = dataclasses.replace(case, v_scale=case.v_scale * 2.0)
    assert np.array_equal(run(lin, lib), 2.0 * ref), "v scale"

    # Logical token order: permuting the full pages a sequence lists (a
    # length that is a multiple of the page size) changes only rounding.
    b = 1
    t2 = case.table.copy()
    t2[b, :8] = t2[b, :8][rng.permutation(8)]
    shuf = dataclasses.replace(case, table=t2)
    close(run(shuf, lib)[b], ref[b], rtol=1e-12, atol=1e-14, what="token order")

    # Table entries past ceil(L / P) are never read.
    t3 = case.table.copy()
    for i, L in enumerate(case.lens):
        t3[i, -(-int(L) // 8):] = -12345
    assert np.array_equal(run(dataclasses.replace(case, table=t3), lib), ref), "unread entries"

    # Empty sequences are inert: zeros, and their table is not read.
    e = dataclasses.replace(case, lens=np.array([0, 64, -3], dtype=np.int32),
                            table=np.where(np.arange(3)[:, None] == 1, case.table, -1).astype(np.int32))
    got = run(e, lib)
    assert np.all(got[0] == 0) and np.all(got[2] == 0)
    assert np.array_equal(got[1], ref[1])

    # Subset evaluation equals the full evaluation.
    assert np.array_equal(run(case, lib, seq_ids=[2, 0]), ref[[2, 0]])


def pin_errors(lib: str) -> None:
    import dataclasses
    case = inputs.decode_case(batch=2, lens=[10, 12], page_size=4, kv_dtype=inputs.KV_FP16,
                              seed=13)
    bad = case.table.copy()
    bad[1, 2] = case.num_pages
    try:
        run(dataclasses.replace(case, table=bad), lib)
        raise AssertionError("out-of-range page id accepted")
    except oracle.OracleError as e:
        assert e.code == oracle.ORACLE_ERR_PAGE
    try:
        run(dataclasses.replace(case, lens=np.array([10, 13], dtype=np.int32)), lib)
        raise AssertionError("over-long sequence accepted")
    except oracle.OracleError as e:
        assert e.code == oracle.ORACLE_ERR_TABLE


# ------------------------------------------------------ QSA top-k selection
def _check_topk_layout(idx, cnt, k, nv):
    """Shape facts every selection result has: count = min(k, nv), the kept
    indices strictly increasing inside [0, nv), then -1 padding."""
    for r in range(idx.shape[0]):
        want = min(k, max(0, int(nv[r])))
        assert cnt[r] == want, (r, cnt[r], want)
        kept = idx[r, :want]
        assert np.all(np.diff(kept) > 0), r
        assert want == 0 or (kept[0] >= 0 and kept[-1] < nv[r]), r
        assert np.all(idx[r, want:] == -1), r


def pin_topk_vs_stable_sort(lib: str) -> None:
    """Against numpy's stable argsort of the negated scores: the first k of
    that order are the top-k with ties broken by increasing index.  -0.0 is
    folded into +0.0 first, since float comparison ties them."""
    for dist, k in (("normal", 7), ("ties", 16), ("ties", 1), ("constant", 5), ("normal", 300)):
        case = inputs.topk_case(rows=24, n_blocks=257, k=k, seed=31 + k, dist=dist,
                                n_valid="random")
        sc = case.scores + np.float32(0.0)
        idx, cnt = oracle.topk_select(sc, k, case.n_valid, lib_path=lib)
        _check_topk_layout(idx, cnt, k, case.n_valid)
        for r in range(case.rows):
            nv = int(case.n_valid[r])
            order = np.argsort(-sc[r, :nv].astype(np.float64), kind="stable")
            want = np.sort(order[:k])
            assert np.array_equal(idx[r, :len(want)], want), (dist, k, r)


def pin_topk_brute_force(lib: str) -> None:
    """Every length-5 score vector over {-inf, -1, 0, 1, +inf} and every k:
    block j is kept iff fewer than k blocks outrank it, where i outranks j when
    s_i > s_j, or s_i == s_j and i < j (Python float comparison)."""
    import itertools
    vals = [-math.inf, -1.0, 0.0, 1.0, math.inf]
    rows = np.array(list(itertools.product(vals, repeat=5)), dtype=np.float32)
    n = rows.shape[1]
    for k in range(0, n + 2):
        idx, cnt = oracle.topk_select(rows, k, lib_path=lib)
        for r, sv in enumerate(rows.tolist()):
            kept = [j for j in range(n)
                    if sum(1 for i in range(n)
                           if sv[i] > sv[j] or (sv[i] == sv[j] and i < j)) < k]
            assert cnt[r] == len(kept) and idx[r, :len(kept)].tolist() == kept, (k, sv)
            assert np.all(idx[r, len(kept):] == -1)


def pin_topk_total_order(lib: str) -> None:
    """Special values (tests/golden/fp32_total_order.txt, IEEE 754 totalOrder)
    shuffled into a row: the k kept blocks are always the k highest in the
    golden order."""
    bits = []
    with open(os.path.join(GOLDEN, "fp32_total_order.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                bits.append(int(line.split()[0], 16))
    assert len(bits) >= 19
    rng = np.random.default_rng(5)
    for trial in range(4):
        perm = rng.permutation(len(bits))
        row = np.array([bits[p] for p in perm], dtype=np.uint32).view(np.float32)[None, :]
        rank_of_pos = perm                      # position j holds golden rank perm[j]
        for k in range(len(bits) + 1):
            idx, cnt = oracle.topk_select(row, k, lib_path=lib)
            want = sorted(j for j in range(len(bits)) if rank_of_pos[j] >= len(bits) - k)
            assert idx[0, :cnt[0]].tolist() == want, (trial, k)


def pin_topk_closed_forms(lib: str) -> None:
    n = 100
    ramp = np.arange(n, dtype=np.float32)[None, :]
    idx, cnt = oracle.topk_select(ramp, 10, lib_path=lib)
    assert idx[0].tolist() == list(range(90, 100))            # increasing: last k
    idx, _ = oracle.topk_select(ramp[:, ::-1].copy(), 10, lib_path=lib)
    assert idx[0].tolist() == list(range(10))                  # decreasing: first k
    idx, _ = oracle.topk_select(np.full((1, n), 3.0, np.float32), 10, lib_path=lib)
    assert idx[0].tolist() == list(range(10))                  # all tied: lowest indices
    neg = -np.arange(1, n + 1, dtype=np.float32)[None, :]      # -1, -2, ...: first k
    idx, _ = oracle.topk_select(neg, 4, lib_path=lib)
    assert idx[0].tolist() == [0, 1, 2, 3]
    # One block above a sea of ties: it plus the lowest tied indices.
    row = np.zeros((1, n), np.float32)
    row[0, 77] = 1.0
    idx, _ = oracle.topk_select(row, 3, lib_path=lib)
    assert idx[0].tolist() == [0, 1, 77]
    # Fewer eligible blocks than k: all of them, then padding.
    idx, cnt = oracle.topk_select(ramp, 10, n_valid=[6], lib_path=lib)
    assert cnt[0] == 6 and idx[0].tolist() == list(range(6)) + [-1] * 4
    # k = 0, an empty row, a negative length, a length past n_blocks.
    idx, cnt = oracle.topk_select(ramp, 0, lib_path=lib)
    assert idx.shape == (1, 0) and cnt[0] == 0
    idx, cnt = oracle.topk_select(np.repeat(ramp, 3, 0), 2, n_valid=[0, -5, 10**6], lib_path=lib)
    assert cnt.tolist() == [0, 0, 2] and idx[:2].tolist() == [[-1, -1], [-1, -1]]
    assert idx[2].tolist() == [98, 99]
    # Columns past n_blocks are never looked at.
    wide = np.concatenate([ramp, np.full((1, 28), np.inf, np.float32)], axis=1)
    idx, _ = oracle.topk_select(wide, 3, n_blocks=n, lib_path=lib)
    assert idx[0].tolist() == [97, 98, 99]


def pin_topk_invariants(lib: str) -> None:
    case = inputs.topk_case(rows=16, n_blocks=1000, k=64, seed=44, dist="ties",
                            n_valid="random")
    sc = case.scores + np.float32(0.0)
    idx, cnt = oracle.topk_select(sc, case.k, case.n_valid, lib_path=lib)
    _check_topk_layout(idx, cnt, case.k, case.n_valid)
    for r in range(case.rows):
        nv = int(case.n_valid[r])
        kept = idx[r, :cnt[r]]
        mask = np.zeros(nv, bool)
        mask[kept] = True
        if mask.all() or not mask.any():
            continue
        lo, hi = sc[r, :nv][mask].min(), sc[r, :nv][~mask].max()
        assert lo >= hi, r                              # kept outrank dropped
        if lo == hi:                                    # ties at the pivot: low indices first
            tied = np.flatnonzero(sc[r, :nv] == lo)
            assert mask[tied].tolist() == sorted(mask[tied].tolist(), reverse=True), r
    # Rows are independent: one row at a time gives the same answer.
    for r in (0, 5, 11):
        i1, c1 = oracle.topk_select(sc[r:r + 1], case.k, case.n_valid[r:r + 1], lib_path=lib)
        assert np.array_equal(i1[0], idx[r]) and c1[0] == cnt[r]
    # Moving distinct scores around moves the kept set with them.
    row = inputs.topk_case(rows=1, n_blocks=500, k=40, seed=45).scores
    assert len(np.unique(row)) == row.size
    perm = np.random.default_rng(9).permutation(row.shape[1])
    i0, _ = oracle.topk_select(row, 40, lib_path=lib)
    i1, _ = oracle.topk_select(row[:, perm], 40, lib_path=lib)
    inv = np.argsort(perm)
    assert np.array_equal(np.sort(inv[i0[0]]), i1[0])


def pin_topk_errors(lib: str) -> None:
    """Negative sizes and a row stride shorter than the row are rejected."""
    c = oracle.load(lib)
    sc = np.zeros((2, 4), np.float32)
    out = np.zeros(16, np.int32)
    cnt = np.zeros(2, np.int32)
    args = lambda stride, rows, nb, k: (sc.ctypes.data, stride, None, rows, nb, k,  # noqa: E731
                                        out.ctypes.data, cnt.ctypes.data)
    assert c.oracle_topk_select(*args(4, 2, 4, 2)) == 0
    for bad in (args(4, 2, 4, -1), args(4, -1, 4, 2), args(3, 2, 4, 2), args(4, 2, -2, 2)):
        assert c.oracle_topk_select(*bad) == oracle.ORACLE_ERR_ARG, bad[1:6]



# ------------------------------------------------- virtual page-4 tables
def _page4_golden():
    cases = []
    with open(os.path.join(GOLDEN, "page4_table_examples.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            lhs, rhs = line.split("=>")
            name, P, V, npg, stride, btab, L, toks = lhs.split()
            table, ln, st = rhs.split()
            ints = lambda t: [int(x) for x in t.split(",")]  # noqa: E731
            cases.append(dict(name=name, P=int(P), V=int(V), num_pages=int(npg),
                              out_stride=int(stride), btab=ints(btab), L=int(L),
                              tokens=ints(toks), table=ints(table), len=int(ln),
                              status=int(st)))
    return cases


def pin_page4_golden(lib: str) -> None:
    """The hand-worked examples of tests/golden/page4_table_examples.txt."""
    cases = _page4_golden()
    assert len(cases) >= 12
    for c in cases:
        t, ln, st = oracle.qsa_page4_table(
            np.array([c["tokens"]], np.int32), [c["L"]], np.array([c["btab"]], np.int32),
            num_pages=c["num_pages"], page_size=c["P"], vpages_per_page=c["V"],
            out_stride=c["out_stride"], lib_path=lib)
        assert t[0].tolist() == c["table"] and ln[0] == c["len"] and st[0] == c["status"], (
            c["name"], t[0].tolist(), int(ln[0]), int(st[0]))


def _page4_brute(tokens, L, btab, num_pages, P, V, out_stride):
    """The definition by enumeration over blocks (tiny inputs only): which of
    blocks 0 .. c are fully, partly or not selected, then the view ids."""
    if L <= 0:
        return [-1] * out_stride, 0, 1
    if L > (1 << 26):
        return [-1] * out_stride, 0, 64
    S = {t for t in tokens if 0 <= t < L}
    c = (L - 1) // 4
    status, full = 0, []
    for b in range(c):
        n = sum((4 * b + i) in S for i in range(4))
        if n == 4:
            full.append(b)
        elif n:
            status |= 2
    tail = [4 * c + i for i in range(4) if (4 * c + i) in S]
    if tail and tail != list(range(4 * c, 4 * c + len(tail))):
        status |= 4
    pages = full + ([c] if tail else [])
    if len(pages) > out_stride:
        status |= 16
    ids = []
    for b in pages:
        lp = 4 * b // P
        p = btab[lp] if lp < len(btab) else -1
        if not 0 <= p < num_pages:
            status |= 8
        ids.append(p * V + (4 * b % P) // 4)
    if status:
        return [-1] * out_stride, 0, status
    ids = sorted(ids[:len(full)]) + ids[len(full):]
    return ids + [-1] * (out_stride - len(ids)), 4 * len(full) + len(tail), 0


def pin_page4_brute_force(lib: str) -> None:
    """Random small rows with every kind of defect against the enumeration."""
    rng = np.random.default_rng(17)
    for trial in range(400):
        P = int(rng.choice([4, 8, 16]))
        V = P // 4 * int(rng.choice([1, 2]))
        n_lp = int(rng.integers(1, 7))
        num_pages = n_lp + int(rng.integers(0, 3))
        btab = rng.permutation(num_pages)[:n_lp].astype(np.int32)
        if trial % 7 == 0:
            btab[rng.integers(0, n_lp)] = int(rng.choice([-1, num_pages, num_pages + 5]))
        L = int(rng.integers(-2, P * n_lp + 6))
        toks = []
        for b in range(max(0, (L + 3) // 4)):
            u = rng.random()
            if u < 0.35:
                toks += [4 * b + i for i in range(4)]
            elif u < 0.40:
                toks += [4 * b + i for i in range(4) if rng.random() < 0.7]
        toks += [int(x) for x in rng.integers(-3, L + 8, size=int(rng.integers(0, 3)))]
        toks = [int(x) for x in rng.permutation(np.array(toks, dtype=np.int64))]
        if not toks:
            toks = [-1]
        stride = int(rng.integers(1, 12))
        t, ln, st = oracle.qsa_page4_table(np.array([toks], np.int32), [L],
                                           np.array([btab], np.int32), num_pages=num_pages,
                                           page_size=P, vpages_per_page=V, out_stride=stride,
                                           lib_path=lib)
        want = _page4_brute(toks, L, btab.tolist(), num_pages, P, V, stride)
        assert (t[0].tolist(), int(ln[0]), int(st[0])) == want, (trial, toks, L, btab, want)


def _sequence_kv(kv: inputs.PagedCase, btab: np.ndarray):
    """K, V (float64 [tokens][Hkv][D]) of the sequence whose logical page i is
    physical page btab[i], read element by element through the pool strides."""
    P, hkv, d = kv.page_size, kv.num_kv_heads, kv.head_dim
    n = btab.size * P
    t = np.arange(n)
    base = (btab[t // P].astype(np.int64) * kv.page_stride + (t % P) * kv.token_stride)
    idx = (base[:, None, None] + np.arange(hkv)[None, :, None] * kv.head_stride
           + np.arange(d)[None, None, :])
    ks = kv.k_store.reshape(-1)[kv.k_offset + idx]
    vs = kv.v_store.reshape(-1)[kv.v_offset + idx]
    return decode_kv(ks, kv.kv_dtype, kv.k_scale), decode_kv(vs, kv.kv_dtype, kv.v_scale)


def pin_page4_attention(lib: str) -> None:
    """End to end: paged attention through the built page-4 view equals dense
    attention (torch, float64) over exactly the selected token positions, for
    interleaved and contiguous pools, tails 0-3 and every token order."""
    for layout, tail, order in (("interleaved", 3, "shuffled"), ("contiguous", 1, "blocks"),
                                ("interleaved", 0, "expanded"), ("contiguous", 2, "shuffled")):
        case = inputs.page4_selection_case(rows=5, selected_blocks=6, tail=tail, seq_blocks=32,
                                           page_size=8, order=order, layout=layout, seed=3,
                                           with_kv=True, head_dim=32, num_q_heads=2)
        t, ln, st = oracle.qsa_page4_table(case.tokens, case.live_len, case.block_table,
                                           **case.builder_kwargs(), lib_path=lib)
        assert np.all(st == 0) and np.all(ln == 4 * 6 + tail)
        got = run(inputs.page4_view(case.kv, t, ln), lib)
        kv = case.kv
        K, V = _sequence_kv(kv, case.block_table[0])     # logical token order
        for r in range(case.rows):
            sel = sorted({int(x) for x in case.tokens[r] if 0 <= x < case.live_len[r]})
            want = sdpa(kv.q[r], K[sel], V[sel], kv.sm_scale)
            close(got[r], want, rtol=1e-10, atol=1e-12, what=(layout, tail, order, r))


def pin_page4_invariants(lib: str) -> None:
    case = inputs.page4_selection_case(rows=64, selected_blocks=20, tail=2, seq_blocks=256,
                                       page_size=16, order="blocks", seed=8)
    kw = case.builder_kwargs()
    t0, l0, s0 = oracle.qsa_page4_table(case.tokens, case.live_len, case.block_table, **kw,
                                        lib_path=lib)
    assert np.all(s0 == 0)
    rng = np.random.default_rng(2)
    # Token order, duplicates, stale positions past the live length and
    # padding do not matter.
    noisy = []
    for r in range(case.rows):
        row = case.tokens[r]
        extra = np.concatenate([row[rng.integers(0, row.size, 9)],
                                case.live_len[r] + rng.integers(0, 50, 5), [-1, -7]])
        noisy.append(rng.permutation(np.concatenate([row, extra])))
    t1, l1, s1 = oracle.qsa_page4_table(np.array(noisy, np.int32), case.live_len,
                                        case.block_table, **kw, lib_path=lib)
    assert np.array_equal(t0, t1) and np.array_equal(l0, l1) and np.array_equal(s0, s1)
    # Rows are independent.
    for r in (0, 31, 63):
        t2, l2, _ = oracle.qsa_page4_table(case.tokens[r:r + 1], case.live_len[r:r + 1],
                                           case.block_table, **kw, lib_path=lib)
        assert np.array_equal(t2[0], t0[r]) and l2[0] == l0[r]
    # Renaming physical pages renames the ids and keeps the full part sorted.
    perm = rng.permutation(case.num_pages).astype(np.int32)
    t3, l3, _ = oracle.qsa_page4_table(case.tokens, case.live_len, perm[case.block_table],
                                       **kw, lib_path=lib)
    V = case.vpages_per_page
    nf = (l0 - 2) // 4
    for r in range(case.rows):
        mapped = [perm[i // V] * V + i % V for i in t0[r, :nf[r] + 1]]
        assert sorted(mapped[:-1]) == t3[r, :nf[r]].tolist() and mapped[-1] == t3[r, nf[r]]
        assert np.all(np.diff(t3[r, :nf[r]]) >= 0) and np.all(t3[r, nf[r] + 1:] == -1)
    # The rows of a second sequence use that sequence's table.
    bt2 = np.stack([case.block_table[0], perm[case.block_table[0]]])
    t4, _, _ = oracle.qsa_page4_table(case.tokens, case.live_len, bt2,
                                      **{**kw, "row_seq": np.ones(case.rows, np.int32)},
                                      lib_path=lib)
    assert np.array_equal(t4, t3)
    t5, _, s5 = oracle.qsa_page4_table(case.tokens, case.live_len, bt2,
                                       **{**kw, "row_seq": np.full(case.rows, 2, np.int32)},
                                       lib_path=lib)
    assert np.all(s5 == oracle.PAGE4_SEQ) and np.all(t5 == -1)


def pin_page4_errors(lib: str) -> None:
    """Bad sizes are rejected before any row is looked at."""
    c = oracle.load(lib)
    tok = np.zeros((1, 4), np.int32)
    live = np.ones(1, np.int32)
    bt = np.zeros((1, 2), np.int32)
    out = np.zeros(8, np.int32)
    ln = np.zeros(1, np.int32)
    st = np.zeros(1, np.int32)

    def call(n_tok=4, stride=4, max_pages=2, n_seqs=1, num_pages=2, P=16, V=4, rows=1,
             out_stride=4):
        return c.oracle_qsa_page4_table(tok.ctypes.data, stride, n_tok, live.ctypes.data,
                                        bt.ctypes.data, max_pages, None, n_seqs, num_pages, P,
                                        V, rows, out.ctypes.data, out_stride, ln.ctypes.data,
                                        st.ctypes.data)
    assert call() == 0
    for bad in (dict(n_tok=5), dict(rows=-1), dict(P=6), dict(P=0), dict(V=3), dict(max_pages=0),
                dict(out_stride=0), dict(n_seqs=0), dict(num_pages=-1)):
        assert call(**bad) == oracle.ORACLE_ERR_ARG, bad



# ------------------------------------------------ top-k / top-p masking
def _mask_golden():
    cases = []
    with open(os.path.join(GOLDEN, "topk_topp_examples.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            lhs, rhs = line.split("=>")
            name, k, p, z = lhs.split()
            logits = [math.log(float(v[2:])) for v in z.split(",")]
            cases.append(dict(name=name, k=int(k), p=float(p), logits=logits,
                              kept=[int(v) for v in rhs.split(",")]))
    return cases


def pin_mask_golden(lib: str) -> None:
    cases = _mask_golden()
    assert len(cases) >= 10
    for c in cases:
        z = np.array([c["logits"]], np.float32)
        out, st, kept = oracle.topk_topp_mask(z, [c["k"]], [c["p"]], lib_path=lib)
        got = np.flatnonzero(out[0] != -np.inf).tolist()
        assert st[0] == 0 and got == c["kept"] and kept[0] == len(c["kept"]), (c["name"], got)
        assert np.array_equal(out[0, got], z[0, got])


def _mask_numpy(z: np.ndarray, k: int, p: float) -> np.ndarray:
    """The definition with numpy: lexsort by (-logit, index), float64 softmax
    over the first k, cumulative sums, the keep rule.  Returns kept indices."""
    order = np.lexsort((np.arange(z.size), -z.astype(np.float64)))
    top = order[:min(k, z.size)]
    zt = z[top].astype(np.float64)
    w = np.exp(zt - zt[0])
    before = np.concatenate([[0.0], np.cumsum(w)[:-1]]) / w.sum()
    keep = np.ones(top.size, bool) if p >= 1 else (before < p)
    keep[0] = True
    n = int(np.argmin(keep)) if not keep.all() else keep.size
    return np.sort(top[:n])


def pin_mask_vs_numpy(lib: str) -> None:
    for dist, k, p, scale in (("normal", 20, 0.95, 3.0), ("normal", 1000, 0.5, 1.0),
                              ("ties", 50, 0.9, 3.0), ("peaked", 20, 0.95, 3.0),
                              ("normal", 7, 0.3, 0.5)):
        case = inputs.sampler_case(rows=12, vocab=5000, k=k, p=p, seed=k + int(10 * p),
                                   scale=scale, dist=dist)
        z = case.logits + np.float32(0.0)               # -0.0 -> +0.0 (numpy ties them)
        out, st, kept = oracle.topk_topp_mask(z, case.k, case.p, lib_path=lib)
        assert np.all(st == 0)
        for r in range(case.rows):
            want = _mask_numpy(z[r], int(case.k[r]), float(case.p[r]))
            got = np.flatnonzero(out[r] != -np.inf)
            assert np.array_equal(got, want), (dist, k, p, r)
            assert np.array_equal(out[r, got], z[r, got]) and kept[r] == want.size


def pin_mask_closed_forms(lib: str) -> None:
    rng = np.random.default_rng(4)
    z = rng.standard_normal((6, 300)).astype(np.float32)
    # p = 1: exactly the top-k by (logit desc, index asc).
    out, _, _ = oracle.topk_topp_mask(z, 17, 1.0, lib_path=lib)
    for r in range(6):
        want = np.sort(np.argsort(-z[r].astype(np.float64), kind="stable")[:17])
        assert np.array_equal(np.flatnonzero(out[r] != -np.inf), want)
    # k = 1 or p = 0: the argmax alone (first index among equal maxima).
    zz = z.copy()
    zz[:, 10] = zz[:, 200] = 9.0
    for k, p in ((1, 0.95), (40, 0.0)):
        out, _, kept = oracle.topk_topp_mask(zz, k, p, lib_path=lib)
        assert np.all(kept == 1) and np.all(np.flatnonzero(out.reshape(-1) != -np.inf) % 300 == 10)
    # A flat row: n equal logits, masses before token i are i/n: ceil(p n) stay.
    flat = np.zeros((1, 64), np.float32)
    for k, p in ((64, 0.3), (10, 0.55), (33, 0.99), (5, 0.21)):
        out, _, kept = oracle.topk_topp_mask(flat, k, p, lib_path=lib)
        n = math.ceil(p * k)
        assert kept[0] == n and np.flatnonzero(out[0] == 0).tolist() == list(range(n)), (k, p)
    # Invalid rows are copied unchanged.
    out, st, _ = oracle.topk_topp_mask(z[:3], [0, 1025, 5], [0.5, 0.5, np.nan], lib_path=lib)
    assert st.tolist() == [oracle.MASK_BAD_K, oracle.MASK_BAD_K, oracle.MASK_BAD_P]
    assert np.array_equal(out, z[:3])
    _, st, kept = oracle.topk_topp_mask(z[:2], [1024, 1], [1.0, 1.0], lib_path=lib)
    assert st.tolist() == [0, 0] and kept.tolist() == [300, 1]   # k = k_max is valid
    # -inf logits rank last; with fewer finite logits than k they fill the set.
    zi = np.full((1, 8), -np.inf, np.float32)
    zi[0, [2, 5]] = [1.0, 3.0]
    out, _, kept = oracle.topk_topp_mask(zi, 4, 1.0, lib_path=lib)
    assert kept[0] == 4 and out[0, 5] == 3.0 and out[0, 2] == 1.0


def pin_mask_invariants(lib: str) -> None:
    case = inputs.sampler_case(rows=8, vocab=3000, k=64, p=0.9, seed=5, dist="ties")
    z = case.logits
    out, _, kept = oracle.topk_topp_mask(z, case.k, case.p, lib_path=lib)
    # Adding 1 to every logit (exact on the half-integer grid) keeps the mask.
    out1, _, kept1 = oracle.topk_topp_mask(z + np.float32(1.0), case.k, case.p, lib_path=lib)
    assert np.array_equal(out1 == -np.inf, out == -np.inf) and np.array_equal(kept, kept1)
    # Rows are independent.
    for r in (0, 7):
        o, _, _ = oracle.topk_topp_mask(z[r:r + 1], case.k[r:r + 1], case.p[r:r + 1],
                                        lib_path=lib)
        assert np.array_equal(o[0], out[r])
    # Moving distinct logits around moves the mask with them.
    d = inputs.sampler_case(rows=2, vocab=2000, k=30, p=0.8, seed=6).logits
    assert all(len(np.unique(d[r])) == d.shape[1] for r in range(2))
    perm = np.random.default_rng(1).permutation(d.shape[1])
    o0, _, _ = oracle.topk_topp_mask(d, 30, 0.8, lib_path=lib)
    o1, _, _ = oracle.topk_topp_mask(d[:, perm], 30, 0.8, lib_path=lib)
    assert np.array_equal(o0[:, perm], o1)
    # A larger p never keeps fewer tokens; a larger k never fewer either.
    _, _, ka = oracle.topk_topp_mask(z, 64, 0.5, lib_path=lib)
    _, _, kb = oracle.topk_topp_mask(z, 64, 0.7, lib_path=lib)
    _, _, kc = oracle.topk_topp_mask(z, 128, 0.7, lib_path=lib)
    assert np.all(ka <= kb) and np.all(kb <= kc)


def pin_mask_errors(lib: str) -> None:
    c = oracle.load(lib)
    z = np.zeros((2, 8), np.float32)
    o = np.zeros((2, 8), np.float32)
    k = np.ones(2, np.int32)
    p = np.ones(2, np.float32)
    st = np.zeros(2, np.int32)
    kept = np.zeros(2, np.int32)

    def call(rows=2, V=8, stride=8, ostride=8, k_max=1024):
        return c.oracle_topk_topp_mask(z.ctypes.data, stride, rows, V, k.ctypes.data,
                                       p.ctypes.data, k_max, o.ctypes.data, ostride,
                                       st.ctypes.data, kept.ctypes.data)
    assert call() == 0
    for bad in (dict(rows=-1), dict(V=0), dict(stride=7), dict(ostride=7), dict(k_max=0)):
        assert call(**bad) == oracle.ORACLE_ERR_ARG, bad


ALL_PINS = [pin_e4m3_vs_torch, pin_e4m3_golden, pin_f16_vs_numpy, pin_sdpa,
            pin_sparse_vs_masked_sdpa, pin_closed_forms, pin_invariants, pin_errors,
            pin_topk_vs_stable_sort, pin_topk_brute_force, pin_topk_total_order,
            pin_topk_closed_forms, pin_topk_invariants, pin_topk_errors,
            pin_page4_golden, pin_page4_brute_force, pin_page4_attention,
            pin_page4_invariants, pin_page4_errors,
            pin_mask_golden, pin_mask_vs_numpy, pin_mask_closed_forms, pin_mask_invariants,
            pin_mask_errors]
