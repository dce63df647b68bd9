"""GPU: paged_gqa_decode_noalloc, the decode entry point that allocates
nothing (its split partials live in the library's per-device scratch array),
against paged_gqa_decode with a caller workspace, through the C ABI: the
same bits on two calls in a row, the second smaller than the first."""
from __future__ import annotations

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


def _both(pg, case, num_splits=0):
    """(decode with its own workspace, decode_noalloc) outputs as fp16 bits."""
    import torch

    q, pool, table, lens = pg.device_case(case)
    n, hq, _ = q.shape
    wsb = pg.paged_gqa_workspace_bytes(n, hq, case.num_kv_heads, case.max_seq_len, num_splits)
    assert 0 < wsb <= pg.NOALLOC_SCRATCH_BYTES
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    ref = torch.full_like(q, float("nan"))
    pg.paged_gqa_decode(q, pool, table, lens, case.max_seq_len, case.sm_scale, ref,
                        num_kv_heads=case.num_kv_heads, workspace=ws, num_splits=num_splits)
    out = torch.full_like(q, float("nan"))
    pg.paged_gqa_decode_noalloc(q, pool, table, lens, case.max_seq_len, case.sm_scale, out,
                                num_kv_heads=case.num_kv_heads, num_splits=num_splits)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), out.cpu().numpy()


def test_noalloc_matches_decode_two_calls(pg):
    # First call: 16 sequences of 16K tokens, E4M3, 128-token pages, automatic
    # splits (16 per sequence here: 1.6 MB of partials).
    big = inputs.decode_case(batch=16, lens=[16384] * 16, page_size=128, kv_dtype=E4M3,
                             seed=71, scales="uniform")
    ref, got = _both(pg, big)
    assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))
    # Second call, smaller: ragged FP16 lengths with an empty and a one-token
    # sequence (the length-balanced split plan), 6 explicit splits.  What the
    # first call left in the scratch must not matter.
    small = inputs.decode_case(batch=3, lens=[5000, 0, 1], page_size=64, kv_dtype=FP16, seed=72)
    ref2, got2 = _both(pg, small, num_splits=6)
    assert np.array_equal(got2.view(np.uint16), ref2.view(np.uint16))
    assert_parity(got2, oracle.paged_gqa(**small.oracle_kwargs()), "noalloc ragged")
    assert np.all(got2[1] == 0)
