"""GPU parity: libpgqa's HIP kernels against the fp64 oracle, through the C ABI.

Every case is seeded synthetic data from fp8_kv_amd.inputs; the oracle sees
the same host arrays the GPU receives.  Bar: max abs <= 2e-3 and rel L2 <=
1e-3 on the fp16 output (tests/parity.py).  Integer-exact properties (layout,
page permutation, determinism, graph replay, prefill = decode) are checked
bitwise.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest

import oracle
from fp8_kv_amd import inputs
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu

E4M3, FP16 = inputs.KV_E4M3, inputs.KV_FP16


@pytest.fixture(scope="module")
def pg():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from fp8_kv_amd import pgqa

    pgqa.load()  # raises if libpgqa.so is missing: there is no fallback
    return pgqa


def _run(pg, case, **kw):
    import torch

    out = pg.run_case(case, **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check(pg, case, what, seq_ids=None, **kw):
    got = _run(pg, case, **kw)
    ref = oracle.paged_gqa(**case.oracle_kwargs(), seq_ids=seq_ids)
    if seq_ids is not None:
        got = got[seq_ids]
    assert_parity(got, ref, what)
    return got


# ---------------------------------------------------------------- E4M3 table
def test_e4m3_table_matches_oracle(pg):
    import torch

    out = torch.empty(256, dtype=torch.float32, device="cuda")
    pg.e4m3_decode_table(out)
    got = out.cpu().numpy().astype(np.float64)
    ref = oracle.e4m3_table()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))


# ------------------------------------------------------------ the workloads
@pytest.mark.parametrize("name", ["decode_b1_1k_fp16_p16", "decode_b8_1k_e4m3_p64",
                                  "decode_b16_16k_e4m3_p128"])
def test_workload_decode(pg, name):
    case = inputs.workload_case(name)
    _check(pg, case, name)


@pytest.mark.parametrize("kv_dtype", [E4M3, FP16])
@pytest.mark.parametrize("layout", ["contiguous", "interleaved"])
def test_workload_ragged(pg, kv_dtype, layout):
    case = inputs.workload_case("decode_ragged_b16_16k_p256", kv_dtype=kv_dtype, layout=layout)
    assert not np.all(np.diff(case.table[0]) == 1)  # nonmonotonic tables
    _check(pg, case, f"ragged {kv_dtype} {layout}")


@pytest.mark.parametrize("name", ["prefill_sparse_4096x2051_p4",
                                  "prefill_sparse_4096x2051_p4_e4m3"])
def test_workload_sparse_prefill_all_rows(pg, name):
    """Every one of the 4096 rows against the oracle (about 26 G fp64
    multiply-adds on the host cores)."""
    case = inputs.workload_case(name)
    got = _run(pg, case, prefill=True)
    ref = oracle.paged_gqa(**case.oracle_kwargs())
    assert_parity(got, ref, f"{name} all rows")


# ------------------------------------------------------- large outputs
@pytest.mark.parametrize("kv_dtype,v_mult", [(E4M3, 4.0), (E4M3, 8.0), (FP16, 6.0)])
@pytest.mark.parametrize("page_size", [1, 16])
def test_large_outputs_against_v_magnitude(pg, kv_dtype, v_mult, page_size):
    """Outputs of magnitude up to about 25 (V scale 4 or 8 on E4M3 codes, FP16
    values scaled by 6), where the absolute bar of 2e-3 is finer than fp16's
    own spacing.  Rows of 1 to 16 tokens.  The PV product takes the softmax
    weights in fp16, so the error scales with the V values averaged, not
    with the output: every output lies within one fp16 unit in the last
    place at the largest |V| of the pool of the fp64 oracle, and a row of
    one token returns fp16(v_scale * V) exactly."""
    lens = list(range(1, 17))
    if kv_dtype == E4M3:
        case = inputs.decode_case(batch=16, lens=lens, page_size=page_size, kv_dtype=E4M3,
                                  scales=(1.0, v_mult), seed=40 + int(v_mult) + page_size)
        vals = oracle.e4m3_table()[case.v_store.astype(np.int64)] * v_mult
    else:
        case = inputs.decode_case(batch=16, lens=lens, page_size=page_size, kv_dtype=FP16,
                                  seed=50 + page_size)
        assert case.v_store is not case.k_store
        big_v = (case.v_store.astype(np.float32) * v_mult).astype(np.float16)
        case = dataclasses.replace(case, v_store=big_v)
        vals = big_v.astype(np.float64)
    ref = oracle.paged_gqa(**case.oracle_kwargs())
    assert np.abs(ref).max() > 8.0
    bar = float(np.spacing(np.float16(np.abs(vals).max())))
    for splits in (1, 0):
        got = _run(pg, case, num_splits=splits).astype(np.float64)
        err = np.abs(got - ref)
        print(f"[large] dtype{kv_dtype} x{v_mult} P{page_size} splits{splits}: max err "
              f"{err.max():.2e} = {err.max() / bar:.2f} fp16 ulp at max|V|", flush=True)
        assert err.max() <= bar
        assert np.array_equal(got[0], ref[0].astype(np.float16).astype(np.float64))  # 1 token


# --------------------------------------------------------- shape coverage
@pytest.mark.parametrize("kv_dtype", [E4M3, FP16])
@pytest.mark.parametrize("page_size", [4, 5, 16, 64, 128, 256])
def test_page_sizes_ragged_tails(pg, kv_dtype, page_size):
    # Lengths cover one partial tile, several tiles and a ragged tail.
    lens = [1, 15, 16, 17, 63, 64, 65, 200, 1000, 777]
    case = inputs.decode_case(batch=len(lens), lens=lens, page_size=page_size,
                              kv_dtype=kv_dtype, seed=page_size, scales="uniform")
    for s in (1, 3, 0):
        _check(pg, case, f"P{page_size} dtype{kv_dtype} splits{s}", num_splits=s)


@pytest.mark.parametrize("layout", ["contiguous", "interleaved", "head_major"])
@pytest.mark.parametrize("kv_dtype", [E4M3, FP16])
def test_multi_kv_head_layouts(pg, layout, kv_dtype):
    case = inputs.decode_case(batch=3, lens=[300, 129, 1], page_size=32, kv_dtype=kv_dtype,
                              layout=layout, num_q_heads=12, num_kv_heads=2, seed=21,
                              scales="uniform")
    _check(pg, case, f"hkv2 {layout} {kv_dtype}")


@pytest.mark.parametrize("group", [1, 2, 8, 16])
def test_group_sizes(pg, group):
    case = inputs.decode_case(batch=2, lens=[333, 70], page_size=16, kv_dtype=E4M3,
                              num_q_heads=group * 2, num_kv_heads=2, seed=30 + group,
                              scales="uniform")
    _check(pg, case, f"group {group}", num_splits=2)


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 0])
def test_split_counts_long_context(pg, splits):
    case = inputs.decode_case(batch=2, lens=[5000, 4097], page_size=128, kv_dtype=E4M3,
                              seed=40, scales="uniform")
    _check(pg, case, f"splits {splits}", num_splits=splits)


@pytest.mark.parametrize("batch", [2, 16])
@pytest.mark.parametrize("page_size", [64, 128, 256])
def test_decode_batch_page_matrix(pg, batch, page_size):
    """B2/B16 at pages 64/128/256 with E4M3 KV, as in the decode operator checks."""
    case = inputs.decode_case(batch=batch, lens=("uniform", 1, 4096), page_size=page_size,
                              kv_dtype=E4M3, seed=80 + page_size + batch, scales="uniform",
                              max_seq_len=4096)
    _check(pg, case, f"B{batch} P{page_size}")


@pytest.mark.parametrize("kv_dtype", [FP16, E4M3])
def test_page_784(pg, kv_dtype):
    case = inputs.decode_case(batch=3, lens=[2000, 784, 785], page_size=784, kv_dtype=kv_dtype,
                              seed=90, scales="uniform")
    for s in (1, 0):
        _check(pg, case, f"P784 dtype{kv_dtype} splits{s}", num_splits=s)


def test_hybrid_784_16_geometry(pg):
    """784-token allocator blocks read as page-16 kernel pages, with a
    nonmonotonic 128-entry page-16 table per sequence."""
    case = inputs.hybrid_784_16_case(batch=4, blocks_per_seq=3, lens=[2048, 2048, 1500, 31],
                                     seed=91)
    assert case.table.shape[1] >= 128
    assert not np.all(np.diff(case.table[0, :128]) == 1)
    # Sequence 0's first 128 entries cover its 2048 tokens.
    _check(pg, case, "hybrid 784/16")
    # Same tokens through page-784 kernel pages give the same attention.
    case784 = dataclasses.replace(
        case, page_size=784, num_pages=case.num_pages // 49,
        page_stride=case.page_stride * 49,
        table=np.ascontiguousarray(case.table[:, ::49] // 49, dtype=np.int32))
    # Same tokens in the same 16-token tiles: the results are bitwise equal.
    for s in (1, 4):
        assert np.array_equal(_run(pg, case, num_splits=s), _run(pg, case784, num_splits=s))


def test_sparse_prefill_page16(pg):
    case = inputs.sparse_prefill_case(rows=40, selected_blocks=32, tail=0, pool_blocks=300,
                                      page_size=16, seed=92)
    _check(pg, case, "prefill page 16", prefill=True)


def test_sparse_prefill_tails(pg):
    for tail in (1, 2, 3, 0):
        case = inputs.sparse_prefill_case(rows=64, selected_blocks=40, tail=tail,
                                          pool_blocks=512, seed=50 + tail)
        _check(pg, case, f"prefill tail {tail}", prefill=True)


def test_sparse_prefill_fp8_contiguous(pg):
    case = inputs.sparse_prefill_case(rows=48, selected_blocks=100, tail=3, pool_blocks=400,
                                      layout="contiguous", kv_dtype=E4M3, scales="uniform",
                                      seed=55)
    _check(pg, case, "prefill fp8 contiguous", prefill=True)


def test_sparse_prefill_unequal_rows_balanced(pg):
    """Rows cut to unequal live lengths (one empty) with several splits: the
    balanced split plan in prefill mode."""
    case = inputs.sparse_prefill_case(rows=64, selected_blocks=40, tail=2, pool_blocks=512,
                                      seed=57)
    rng = np.random.default_rng(57)
    lens = case.lens.copy()
    cut = rng.choice(case.n, 24, replace=False)
    lens[cut] = rng.integers(1, int(lens.max()), size=cut.size)
    lens[5] = 0
    case = dataclasses.replace(case, lens=lens.astype(np.int32))
    for s in (0, 3):
        got = _check(pg, case, f"prefill unequal rows splits {s}", prefill=True, num_splits=s)
        assert np.all(got[5] == 0)


# ------------------------------------------- one row per wave (many rows)
@pytest.mark.parametrize("kv_dtype,layout", [(E4M3, "contiguous"), (FP16, "interleaved")])
def test_row_per_wave_many_short_rows(pg, kv_dtype, layout):
    """1100 sequences with one split: each wave owns a whole sequence (ragged
    lengths from empty to several hundred tokens, one bad page id).  Unit
    scales: rows of a few tokens output values of V itself, and above 4 in
    magnitude half an fp16 ULP alone exceeds the 2e-3 bar."""
    rng = np.random.default_rng(101)
    lens = rng.integers(-2, 300, size=1100)
    lens[:3] = [0, 1, 299]
    case = inputs.decode_case(batch=1100, lens=lens, page_size=16, kv_dtype=kv_dtype,
                              layout=layout, seed=101, scales="unit", max_seq_len=300)
    t = case.table.copy()
    t[7, 0] = case.num_pages + 1                      # row 7 reads a bad page
    bad = dataclasses.replace(case, table=t)
    got = _run(pg, bad, num_splits=1)
    assert np.isnan(got[7]).all() if lens[7] > 0 else np.all(got[7] == 0)
    ids = np.array([i for i in range(case.n) if i != 7], dtype=np.int32)
    ref = oracle.paged_gqa(**case.oracle_kwargs(), seq_ids=ids)
    assert_parity(got[ids], ref, f"row per wave {kv_dtype} {layout}")
    assert np.all(got[lens <= 0] == 0)


def test_row_per_wave_multi_kv_head_and_prefill(pg):
    """Rows x kv heads = 1200 (Hkv = 2), and a 1024-row sparse prefill: the
    row-per-wave kernel against the oracle and, bitwise, prefill = decode."""
    case = inputs.decode_case(batch=600, lens=("uniform", 1, 200), page_size=32, kv_dtype=E4M3,
                              num_q_heads=12, num_kv_heads=2, seed=102, scales="uniform")
    _check(pg, case, "row per wave hkv2", num_splits=1)
    case = inputs.sparse_prefill_case(rows=1024, selected_blocks=16, tail=3, pool_blocks=1400,
                                      seed=103)
    a = _check(pg, case, "row per wave prefill", prefill=True)
    b = _run(pg, case, prefill=False)
    assert np.array_equal(a, b)


# ----------------------------------------------------------- special cases
def test_length_one_is_v(pg):
    case = inputs.decode_case(batch=4, lens=1, page_size=16, kv_dtype=E4M3, seed=60,
                              scales=(1.25, 0.5))
    got = _run(pg, case)
    ref = oracle.paged_gqa(**case.oracle_kwargs())
    # o = V_0 * v_scale exactly, rounded once to fp16.
    assert np.array_equal(got, ref.astype(np.float16))


def test_empty_and_negative_lengths_are_zero(pg):
    case = inputs.decode_case(batch=4, lens=[0, 50, -7, 0], page_size=16, kv_dtype=FP16,
                              seed=61, max_seq_len=64)
    t = case.table.copy()
    t[[0, 2, 3]] = -1  # never read
    case = dataclasses.replace(case, table=t)
    for s in (1, 2, 0):
        got = _run(pg, case, num_splits=s)
        assert np.all(got[[0, 2, 3]] == 0)
        ref = oracle.paged_gqa(**case.oracle_kwargs(), seq_ids=[1])
        assert_parity(got[[1]], ref, f"empty rows splits {s}")


def test_lengths_clamped_to_max_seq_len(pg):
    case = inputs.decode_case(batch=2, lens=[100, 40], page_size=16, kv_dtype=FP16, seed=62)
    clamped = dataclasses.replace(case, max_seq_len=64)
    got = _run(pg, clamped)
    ref = oracle.paged_gqa(**dataclasses.replace(
        case, lens=np.minimum(case.lens, 64).astype(np.int32)).oracle_kwargs())
    assert_parity(got, ref, "clamp")


def test_bad_page_id_poisons_only_its_row(pg):
    case = inputs.decode_case(batch=3, lens=[40, 40, 40], page_size=16, kv_dtype=E4M3, seed=63)
    t = case.table.copy()
    t[1, 1] = case.num_pages + 5
    got = _run(pg, dataclasses.replace(case, table=t))
    assert np.isnan(got[1]).all()
    ref = oracle.paged_gqa(**case.oracle_kwargs(), seq_ids=[0, 2])
    assert_parity(got[[0, 2]], ref, "rows next to a bad page id")


# ------------------------------------------------------- bitwise invariants
def test_page_permutation_bitwise(pg):
    case = inputs.decode_case(batch=4, lens=[700, 333, 64, 1], page_size=16, kv_dtype=E4M3,
                              seed=70, scales="uniform")
    rng = np.random.default_rng(71)
    perm = rng.permutation(case.num_pages)
    ks = np.empty_like(case.k_store)
    vs = np.empty_like(case.v_store)
    ks[perm] = case.k_store
    vs[perm] = case.v_store
    moved = dataclasses.replace(case, k_store=ks, v_store=vs,
                                table=perm[case.table].astype(np.int32))
    for s in (1, 4):
        assert np.array_equal(_run(pg, case, num_splits=s), _run(pg, moved, num_splits=s))


@pytest.mark.parametrize("kv_dtype", [E4M3, FP16])
def test_layouts_bitwise_equal(pg, kv_dtype):
    outs = []
    for layout in ("contiguous", "interleaved", "head_major"):
        case = inputs.decode_case(batch=3, lens=[500, 77, 256], page_size=64, kv_dtype=kv_dtype,
                                  layout=layout, seed=72, num_q_heads=12, num_kv_heads=2)
        outs.append(_run(pg, case))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_deterministic_repeat(pg):
    case = inputs.workload_case("decode_b8_1k_e4m3_p64")
    a = _run(pg, case)
    b = _run(pg, case)
    assert np.array_equal(a, b)


def test_prefill_equals_decode_bitwise(pg):
    case = inputs.sparse_prefill_case(rows=32, selected_blocks=64, tail=2, pool_blocks=256,
                                      seed=73)
    for s in (1, 2):
        a = _run(pg, case, prefill=True, num_splits=s)
        b = _run(pg, case, prefill=False, num_splits=s)
        assert np.array_equal(a, b)


def test_one_workspace_across_shapes(pg):
    """One workspace, never cleared, serves calls of different shapes in
    turn: equal lengths (bit for bit equal to decode_partial +
    merge_partials), ragged batches re-dealt by length (including one
    sequence with 128 chunks, so its merge takes four 32-chunk rounds, and
    empty sequences), a batch of empty sequences only, 71 splits (a four-wave
    merge) and FP16.  Every call matches the oracle and a repeat matches bit
    for bit."""
    import torch

    cases = [
        (dict(batch=16, lens=[4096] * 16, page_size=128, kv_dtype=E4M3, seed=401), 16),
        (dict(batch=3, lens=[4000, 1, 2500], page_size=128, kv_dtype=E4M3, seed=402), 0),
        (dict(batch=16, lens=[16384] + [64] * 15, page_size=128, kv_dtype=E4M3, seed=403), 16),
        (dict(batch=5, lens=[3000, 0, 1, 2049, 64], page_size=64, kv_dtype=E4M3, seed=404), 6),
        (dict(batch=3, lens=[0, 0, 0], page_size=64, kv_dtype=E4M3, seed=405,
              max_seq_len=2048), 4),
        (dict(batch=2, lens=[9000, 9000], page_size=128, kv_dtype=E4M3, seed=406), 71),
        (dict(batch=2, lens=[3000, 3000], page_size=16, kv_dtype=FP16, seed=407), 12),
    ]
    built = [(inputs.decode_case(scales="uniform", **kw), kw, splits) for kw, splits in cases]
    wsb = max(pg.paged_gqa_workspace_bytes(c.lens.shape[0], 6, 1, c.max_seq_len, s)
              for c, _, s in built)
    ws = torch.full((wsb,), 0x7F, dtype=torch.uint8, device="cuda")  # garbage, not zero
    first = []
    for rep in range(2):
        for i, (case, kw, splits) in enumerate(built):
            q, pool, table, lens = pg.device_case(case)
            out = torch.full_like(q, float("nan"))
            print(f"shapes: rep {rep} case {i} lens {kw['lens'][:4]} splits {splits}", flush=True)
            pg.paged_gqa_decode(q, pool, table, lens, case.max_seq_len, case.sm_scale, out,
                                workspace=ws, num_splits=splits)
            torch.cuda.synchronize()
            got = out.cpu().numpy()
            if rep == 0:
                first.append(got)
                ref = oracle.paged_gqa(**case.oracle_kwargs())
                assert_parity(got, ref, f"case {i}")
                if len(set(case.lens.tolist())) == 1 and case.lens[0] > 0:
                    n, hq, _ = q.shape
                    S = pg.paged_gqa_num_splits(n, 1, case.max_seq_len, splits)
                    po = torch.empty((n, hq, S, 256), dtype=torch.float32, device="cuda")
                    pl = torch.empty((n, hq, S), dtype=torch.float32, device="cuda")
                    pg.paged_gqa_decode_partial(q, pool, table, lens, case.max_seq_len,
                                                case.sm_scale, po, pl, num_splits=splits)
                    merged = torch.empty_like(q)
                    pg.paged_gqa_merge_partials(po, pl, merged)
                    torch.cuda.synchronize()
                    assert np.array_equal(merged.cpu().numpy().view(np.uint16),
                                          got.view(np.uint16)), f"case {i} two-stage"
            else:
                assert np.array_equal(got.view(np.uint16), first[i].view(np.uint16)), f"case {i}"


def test_reused_workspace_and_empty_rows(pg):
    import torch

    case = inputs.decode_case(batch=5, lens=[3000, 0, 1, 2049, 64], page_size=64, kv_dtype=E4M3,
                              seed=75, scales="uniform")
    q, pool, table, lens = pg.device_case(case)
    n, hq, _ = q.shape
    wsb = pg.paged_gqa_workspace_bytes(n, hq, 1, case.max_seq_len, 6)
    ws = torch.full((wsb,), 0x7F, dtype=torch.uint8, device="cuda")  # garbage, not zero
    outs = []
    for _ in range(3):
        out = torch.full_like(q, float("nan"))
        pg.paged_gqa_decode(q, pool, table, lens, case.max_seq_len, case.sm_scale, out,
                            workspace=ws, num_splits=6)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    assert np.all(outs[0][1] == 0)
    ref = oracle.paged_gqa(**case.oracle_kwargs())
    assert_parity(outs[0], ref, "reused workspace")


@pytest.mark.parametrize("batch,length,splits,S", [
    (1, 8256, 17, 17), (1, 8448, 33, 33), (3, 2560, 40, 40), (1, 16384, 128, 128),
    (2, 9000, 0, 71)])
def test_split_counts_against_oracle(pg, batch, length, splits, S):
    """Split counts that are not powers of two, with a partial last split
    (8256 = 16 * 512 + 64 tokens in 17 splits), against the oracle and
    repeated bit for bit on the same workspace."""
    import torch

    case = inputs.decode_case(batch=batch, lens=[length] * batch, page_size=128,
                              kv_dtype=E4M3, seed=300 + splits, scales="uniform")
    q, pool, table, lens = pg.device_case(case)
    n, hq, _ = q.shape
    assert pg.paged_gqa_num_splits(n, 1, case.max_seq_len, splits) == S
    wsb = pg.paged_gqa_workspace_bytes(n, hq, 1, case.max_seq_len, splits)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
    ref = oracle.paged_gqa(**case.oracle_kwargs())
    got = []
    for _ in range(2):
        out = torch.empty_like(q)
        pg.paged_gqa_decode(q, pool, table, lens, case.max_seq_len, case.sm_scale, out,
                            workspace=ws, num_splits=splits)
        torch.cuda.synchronize()
        got.append(out.cpu().numpy())
    assert_parity(got[0], ref, f"S={S}")
    assert np.array_equal(got[0].view(np.uint16), got[1].view(np.uint16))


@pytest.mark.parametrize("splits", [2, 5, 0])
def test_partial_then_merge_equals_decode_bitwise(pg, splits):
    """With every length at (or clamped to) max_seq_len a whole call uses the
    static split plan, so it equals decode_partial + merge_partials bit for
    bit; with unequal lengths the two-stage call keeps the static plan (empty
    splits marked -inf) and still matches the oracle."""
    import torch

    for lens, max_len in (([4000, 5000, 4000], 4000), ([4000, 1, 2500], None)):
        case = inputs.decode_case(batch=3, lens=lens, page_size=128, kv_dtype=E4M3,
                                  seed=76, scales="uniform", max_seq_len=max_len)
        q, pool, table, d_lens = pg.device_case(case)
        n, hq, _ = q.shape
        S = pg.paged_gqa_num_splits(n, 1, case.max_seq_len, splits)
        po = torch.empty((n, hq, S, 256), dtype=torch.float32, device="cuda")
        pl = torch.empty((n, hq, S), dtype=torch.float32, device="cuda")
        pg.paged_gqa_decode_partial(q, pool, table, d_lens, case.max_seq_len, case.sm_scale,
                                    po, pl, num_splits=splits)
        merged = torch.empty_like(q)
        pg.paged_gqa_merge_partials(po, pl, merged)
        direct = pg.run_case(case, num_splits=splits)
        torch.cuda.synchronize()
        clamped = dataclasses.replace(
            case, lens=np.minimum(case.lens, case.max_seq_len).astype(np.int32))
        ref = oracle.paged_gqa(**clamped.oracle_kwargs())
        assert_parity(merged.cpu().numpy(), ref, f"two-stage lens {lens}")
        if max_len is not None and S > 1:
            assert torch.equal(merged, direct)
        if max_len is None:
            # Splits past a sequence's end are marked empty.
            lse = pl.cpu().numpy()
            assert np.all(np.isneginf(lse[1, :, 1:]))
            assert np.all(np.isfinite(lse[1, :, 0]))


# ------------------------------------------- unequal lengths (balanced plan)
@pytest.mark.parametrize("lens", [
    [16384] + [0] * 15,          # one sequence takes every slot (> S chunks)
    [1] * 15 + [16384],
    [16384] * 15 + [16000],      # all but one at max_seq_len
    [0, -5, 3, 64, 65, 8191, 16384, 20000] * 2,
])
def test_balanced_extremes(pg, lens):
    case = inputs.decode_case(batch=len(lens), lens=lens, page_size=128, kv_dtype=E4M3,
                              seed=90 + len(set(lens)), scales="uniform", max_seq_len=16384)
    clamped = dataclasses.replace(case, lens=np.minimum(case.lens, 16384).astype(np.int32))
    ref = oracle.paged_gqa(**clamped.oracle_kwargs())
    for s in (0, 3):
        assert_parity(_run(pg, case, num_splits=s), ref, f"balanced {lens[:4]} splits {s}")


@pytest.mark.parametrize("batch,splits", [(100, 0), (300, 4), (512, 2), (513, 2)])
def test_balanced_many_sequences(pg, batch, splits):
    """Plans over 2 .. 8 rows of 64 lengths per wave; 513 sequences keep the
    static plan."""
    rng = np.random.default_rng(batch)
    lens = rng.integers(-2, 700, size=batch)
    lens[rng.integers(0, batch, size=batch // 10)] = 0
    case = inputs.decode_case(batch=batch, lens=lens, page_size=16, kv_dtype=FP16,
                              seed=batch, max_seq_len=700)
    got = _check(pg, case, f"batch {batch} splits {splits}", num_splits=splits)
    assert np.all(got[lens <= 0] == 0)


def test_balanced_multi_kv_head(pg):
    case = inputs.decode_case(batch=5, lens=[3000, 10, 0, 2999, 64], page_size=64,
                              kv_dtype=E4M3, num_q_heads=12, num_kv_heads=2, seed=95,
                              scales="uniform", max_seq_len=4096)
    for s in (0, 2, 7):
        _check(pg, case, f"hkv2 balanced splits {s}", num_splits=s)


def test_balanced_all_empty_and_repeat(pg):
    case = inputs.decode_case(batch=6, lens=[0, 0, -1, 0, 0, 0], page_size=16, kv_dtype=FP16,
                              seed=96, max_seq_len=256)
    assert np.all(_run(pg, case, num_splits=4) == 0)
    case = inputs.workload_case("decode_ragged_b16_16k_p256")
    a = _run(pg, case)
    b = _run(pg, case)
    assert np.array_equal(a, b)


def test_merge_of_shards_equals_whole_sequence(pg):
    """Two shards of each sequence's pages computed separately (one split
    each) and merged by paged_gqa_merge_partials equal attention over the
    whole sequence -- the merge a context-parallel split would use."""
    import torch

    case = inputs.decode_case(batch=4, lens=[2048, 1000, 64, 1536], page_size=64,
                              kv_dtype=E4M3, seed=77, scales="uniform")
    ref = oracle.paged_gqa(**case.oracle_kwargs())
    n = case.n
    cut = np.array([640, 512, 64, 1536])   # shard boundary (multiple of the page size)
    lens_a = np.minimum(case.lens, cut).astype(np.int32)
    lens_b = (case.lens - lens_a).astype(np.int32)
    tab_b = np.zeros_like(case.table)
    for b in range(n):
        k = cut[b] // 64
        tab_b[b, :case.table.shape[1] - k] = case.table[b, k:]
    q, pool, table, _ = pg.device_case(case)
    hq = q.shape[1]
    parts_o = torch.empty((n, hq, 2, 256), dtype=torch.float32, device="cuda")
    parts_l = torch.empty((n, hq, 2), dtype=torch.float32, device="cuda")
    for j, (tab, ln) in enumerate([(case.table, lens_a), (tab_b, lens_b)]):
        po = torch.empty((n, hq, 1, 256), dtype=torch.float32, device="cuda")
        pl = torch.empty((n, hq, 1), dtype=torch.float32, device="cuda")
        pg.paged_gqa_decode_partial(q, pool, torch.from_numpy(tab).cuda(),
                                    torch.from_numpy(ln).cuda(), case.max_seq_len,
                                    case.sm_scale, po, pl, num_splits=1)
        parts_o[:, :, j] = po[:, :, 0]
        parts_l[:, :, j] = pl[:, :, 0]
    out = torch.empty_like(q)
    pg.paged_gqa_merge_partials(parts_o, parts_l, out)
    torch.cuda.synchronize()
    assert_parity(out.cpu().numpy(), ref, "merged shards")


def test_merge_all_empty_rows_are_zero(pg):
    import torch

    po = torch.full((3, 4, 256), float("nan"), dtype=torch.float32, device="cuda")
    pl = torch.full((3, 4), float("-inf"), dtype=torch.float32, device="cuda")
    pl[1, 2] = 0.5
    po[1, 2] = 3.0
    out = torch.empty((3, 256), dtype=torch.float16, device="cuda")
    pg.paged_gqa_merge_partials(po, pl, out)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(o[[0, 2]] == 0) and np.all(o[1] == 3.0)


def test_graph_replay_bitwise(pg):
    import torch

    case = inputs.decode_case(batch=4, lens=[3000, 1500, 999, 4096], page_size=128,
                              kv_dtype=E4M3, seed=74, scales="uniform")
    q, pool, table, lens = pg.device_case(case)
    n, hq, _ = q.shape
    wsb = pg.paged_gqa_workspace_bytes(n, hq, 1, case.max_seq_len, 0)
    ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device="cuda")
    eager = torch.empty_like(q)
    pg.paged_gqa_decode(q, pool, table, lens, case.max_seq_len, case.sm_scale, eager,
                        workspace=ws)
    torch.cuda.synchronize()
    out = torch.empty_like(q)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        pg.paged_gqa_decode(q, pool, table, lens, case.max_seq_len, case.sm_scale, out,
                            workspace=ws)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pg.paged_gqa_decode(q, pool, table, lens, case.max_seq_len, case.sm_scale, out,
                            workspace=ws)
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)


def test_graph_replay_follows_new_lengths(pg):
    """One captured decode call replayed after the device lengths change in
    place: the split plan is made on the device from the lengths, so every
    replay equals an eager call on the same lengths bit for bit, and the
    oracle."""
    import torch

    case = inputs.decode_case(batch=4, lens=[4096] * 4, page_size=128, kv_dtype=E4M3,
                              seed=77, scales="uniform", max_seq_len=4096)
    q, pool, table, lens = pg.device_case(case)
    n, hq, _ = q.shape
    wsb = pg.paged_gqa_workspace_bytes(n, hq, 1, case.max_seq_len, 0)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)

    def call(o, stream=None):
        pg.paged_gqa_decode(q, pool, table, lens, case.max_seq_len, case.sm_scale, o,
                            workspace=ws, stream=stream)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(out, s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(out, s)
    for new in ([4096, 1, 0, 2000], [17, 4096, 4096, 3333], [0, 0, 0, 0], [4096] * 4,
                [-3, 640, 64, 4095]):
        print(f"graph replay lens={new}", flush=True)
        lens.copy_(torch.tensor(new, dtype=torch.int32))
        eager = torch.empty_like(q)
        call(eager)
        out.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), new
        ref = oracle.paged_gqa(**dataclasses.replace(
            case, lens=np.asarray(new, np.int32)).oracle_kwargs())
        assert_parity(out.cpu().numpy(), ref, f"graph replay lens {new}")


# ------------------------------------------------------ seeded random sweep
def _sweep_case(i: int):
    """Configuration i of the sweep: batch, lengths (with empty and negative
    ones), page size, kv heads, group size, dtype, layout, scales and split
    count all drawn from one seeded generator.  The V scale stays <= 1.5 so
    that |o| < 8, where half an fp16 unit in the last place is below the
    2e-3 bar."""
    rng = np.random.default_rng(5000 + i)
    hkv = int(rng.choice([1, 1, 2, 3]))
    group = int(rng.choice([1, 2, 4, 6, 6, 8, 16]))
    P = int(rng.choice([1, 3, 4, 7, 16, 32, 100, 128, 256, 300]))
    batch = int(rng.integers(1, 41))
    lmax = int(rng.choice([1, 40, 700, 3000]))
    lens = rng.integers(-2, lmax + 1, size=batch)
    lens[rng.random(batch) < 0.15] = 0
    kv_dtype = E4M3 if rng.random() < 0.5 else FP16
    layout = str(rng.choice(["contiguous", "interleaved", "head_major"]))
    scales = (float(rng.uniform(0.5, 2.0)), float(rng.uniform(0.5, 1.5)))
    splits = int(rng.choice([0, 0, 1, 2, 5]))
    max_len = max(1, int(lens.max())) + int(rng.choice([0, 0, 17]))
    case = inputs.decode_case(batch=batch, lens=lens, page_size=P, kv_dtype=kv_dtype,
                              layout=layout, seed=i, num_q_heads=group * hkv,
                              num_kv_heads=hkv, scales=scales, max_seq_len=max_len)
    what = (f"sweep {i}: B{batch} lens<={lmax} P{P} hkv{hkv} group{group} "
            f"{'e4m3' if kv_dtype == E4M3 else 'fp16'} {layout} splits{splits}")
    return case, splits, what


@pytest.mark.parametrize("i", range(32))
def test_random_configurations(pg, i):
    """Each configuration through decode and through sparse prefill (rows as
    sequences) against the oracle; empty and negative lengths give zeros."""
    case, splits, what = _sweep_case(i)
    print(what, flush=True)
    ref = oracle.paged_gqa(**case.oracle_kwargs())
    for prefill in (False, True):
        got = _run(pg, case, prefill=prefill, num_splits=splits)
        assert_parity(got, ref, what + (" prefill" if prefill else " decode"))
        assert np.all(got[case.lens <= 0] == 0)


@pytest.mark.parametrize("length,requested,S", [
    (16384, 32, 32), (16384, 45, 43), (16384, 64, 64), (16384, 100, 86), (16384, 128, 128),
    (12000, 190, 188), (16384, 256, 256), (16384, 0, None)])
def test_many_splits_merge(pg, length, requested, S):
    """Effective split counts (a request is rounded through a chunk length
    that is a multiple of 64 tokens) on each merge width: one wave up to 32
    splits, two waves up to 64, four beyond, with partial last chunks (43,
    86, 188) and two chunks per wave (188, 256).  A whole call and
    decode_partial + merge_partials against the oracle; the two agree bit for
    bit."""
    import torch

    case = inputs.decode_case(batch=2, lens=[length, length], page_size=128, kv_dtype=E4M3,
                              seed=79, scales="uniform")
    ref = oracle.paged_gqa(**case.oracle_kwargs())
    q, pool, table, lens = pg.device_case(case)
    n, hq, _ = q.shape
    got_S = pg.paged_gqa_num_splits(n, 1, case.max_seq_len, requested)
    print(f"many splits: L {length} requested {requested} -> {got_S}", flush=True)
    if S is not None:
        assert got_S == S
    whole = _run(pg, case, num_splits=requested)
    assert_parity(whole, ref, f"splits {got_S} whole call")
    po = torch.empty((n, hq, got_S, 256), dtype=torch.float32, device="cuda")
    pl = torch.empty((n, hq, got_S), dtype=torch.float32, device="cuda")
    pg.paged_gqa_decode_partial(q, pool, table, lens, case.max_seq_len, case.sm_scale, po, pl,
                                num_splits=requested)
    merged = torch.empty_like(q)
    pg.paged_gqa_merge_partials(po, pl, merged)
    torch.cuda.synchronize()
    assert np.array_equal(merged.cpu().numpy().view(np.uint16), whole.view(np.uint16))


def test_b1_long_context_auto_splits(pg):
    """One 16K sequence: the automatic plan takes its largest split count
    (more than 64, so the merge runs four waves per row)."""
    case = inputs.workload_case("decode_b1_16k_e4m3_p128")
    assert pg.paged_gqa_num_splits(1, 1, case.max_seq_len, 0) > 64
    _check(pg, case, "b1 16k auto splits")


def test_two_streams_at_once(pg):
    """The library keeps no per-call state: calls launched on two streams
    without synchronisation between them (decode, sparse prefill and masking
    interleaved) give the same bits as the same calls one after another."""
    import torch

    dec = inputs.decode_case(batch=4, lens=[5000, 17, 3000, 0], page_size=64, kv_dtype=E4M3,
                             seed=81, scales="uniform")
    pre = inputs.sparse_prefill_case(rows=64, selected_blocks=40, tail=2, pool_blocks=1024,
                                     seed=82)
    sam = inputs.sampler_case(rows=4, vocab=50_000, k=[20, 1, 256, 7], p=0.9, seed=83)
    d = pg.device_case(dec)
    r = pg.device_case(pre)
    z = torch.from_numpy(sam.logits).cuda()
    k = torch.from_numpy(np.array(sam.k, np.int32)).cuda()
    pp = torch.from_numpy(np.array(sam.p, np.float32)).cuda()

    def work(stream, outs):
        wsb = pg.paged_gqa_workspace_bytes(4, 6, 1, dec.max_seq_len, 0)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
        wsb2 = pg.paged_gqa_workspace_bytes(pre.n, 6, 1, pre.max_seq_len, 0)
        ws2 = torch.empty(max(wsb2, 16), dtype=torch.uint8, device="cuda")
        for _ in range(3):
            pg.paged_gqa_decode(d[0], d[1], d[2], d[3], dec.max_seq_len, dec.sm_scale, outs[0],
                                workspace=ws, stream=stream)
            pg.paged_gqa_prefill_sparse(r[0], r[1], r[2], r[3], pre.max_seq_len, pre.sm_scale,
                                        outs[1], workspace=ws2, stream=stream)
            pg.sampler_topk_topp_mask(z, k, pp, out=outs[2], stream=stream)

    def fresh():
        return [torch.empty_like(d[0]), torch.empty_like(r[0]), torch.empty_like(z)]

    ref = fresh()
    work(torch.cuda.current_stream(), ref)
    torch.cuda.synchronize()
    a, b = fresh(), fresh()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s1):
        work(s1, a)
    with torch.cuda.stream(s2):
        work(s2, b)
    torch.cuda.synchronize()
    for x, y, w in zip(a, b, ref):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.float16 else x.view(torch.int32),
                           w.view(torch.int16) if w.dtype == torch.float16 else w.view(torch.int32))
        assert torch.equal(y.view(torch.int16) if y.dtype == torch.float16 else y.view(torch.int32),
                           w.view(torch.int16) if w.dtype == torch.float16 else w.view(torch.int32))
    assert_parity(a[0].cpu().numpy(), oracle.paged_gqa(**dec.oracle_kwargs()), "two streams")
