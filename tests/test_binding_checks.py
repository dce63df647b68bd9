"""The Python binding checks every tensor before its address reaches the
library (which sees only pointers): dtype, shape, layout and device, and
that a KV pool's tensors hold every element its strides address.  CPU
tensors suffice: each check raises before any device call."""
from __future__ import annotations

import numpy as np
import pytest

from fp8_kv_amd import inputs, pgqa

torch = pytest.importorskip("torch")


def host_case(name="decode_b8_1k_e4m3_p64"):
    case = inputs.workload_case(name)
    ks = torch.from_numpy(case.k_store)
    vs = ks if case.v_store is case.k_store else torch.from_numpy(case.v_store)
    kflat, vflat = ks.reshape(-1), vs.reshape(-1)
    pool = pgqa.KVPool(kflat[case.k_offset:], vflat[case.v_offset:], case.page_stride,
                       case.token_stride, case.head_stride, case.num_pages, case.page_size,
                       case.kv_dtype, case.k_scale, case.v_scale, storage=(ks, vs))
    return (case, torch.from_numpy(case.q), pool, torch.from_numpy(case.table),
            torch.from_numpy(case.lens))


@pytest.mark.parametrize("name", ["decode_b1_1k_fp16_p16", "decode_b16_16k_e4m3_p128",
                                  "prefill_sparse_4096x64_p16"])
def test_pool_extent_is_exact(name):
    """The extent the strides address fits the workloads' pools, and for the
    last tensor of each storage it ends exactly at the storage's end."""
    case, _, pool, _, _ = host_case(name)
    ext = pgqa._pool_extent(pool, case.num_kv_heads)
    assert ext <= pgqa._bytes_after(pool.k) and ext <= pgqa._bytes_after(pool.v)
    assert ext == pgqa._bytes_after(pool.v)


def test_short_pool_is_rejected():
    case, q, pool, table, lens = host_case()
    short = pgqa.KVPool(pool.k[:-1], pool.v, pool.page_stride, pool.token_stride,
                        pool.head_stride, pool.num_pages, pool.page_size, pool.kv_dtype)
    ext = pgqa._pool_extent(short, 1)
    assert pgqa._bytes_after(short.k) >= ext   # a view keeps its storage: still fits
    clone = short.k.clone()                      # a storage of its own, one byte short
    short.k = clone
    assert pgqa._bytes_after(clone) == ext - 1


def test_attention_argument_checks():
    case, q, pool, table, lens = host_case()
    out = torch.empty_like(q)

    def call(**kw):
        a = dict(q=q, kv=pool, page_table=table, seq_lens=lens, out=out)
        a.update(kw)
        pgqa.paged_gqa_decode(a["q"], a["kv"], a["page_table"], a["seq_lens"],
                              case.max_seq_len, case.sm_scale, a["out"])

    for kw, msg in ((dict(q=q.float()), "q: dtype"),
                    (dict(page_table=table[:-1]), "page table: shape"),
                    (dict(page_table=table.t()), "page table: shape"),
                    (dict(seq_lens=lens.long()), "lengths: dtype"),
                    (dict(seq_lens=lens[:-1]), "lengths: shape"),
                    (dict(out=out[:-1]), "out: shape"),
                    (dict(q=q.transpose(0, 1).contiguous().transpose(0, 1)), "q: must be contig"),
                    (dict(out=out.float()), "out: dtype"),
                    ({}, "q: must be a device tensor")):
        with pytest.raises(ValueError, match=msg):
            call(**kw)
    S = 4
    with pytest.raises(ValueError, match="q: must be a device tensor"):
        pgqa.paged_gqa_decode_partial(q, pool, table, lens, case.max_seq_len, case.sm_scale,
                                      torch.empty((q.shape[0], 6, S, 256)),
                                      torch.empty((q.shape[0], 6, S)), num_splits=S)
    with pytest.raises(ValueError, match="do not hold"):
        pgqa.paged_gqa_merge_partials(torch.empty((3, 4, 256)), torch.empty((3, 4)),
                                      torch.empty((2, 256), dtype=torch.float16))
    with pytest.raises(ValueError, match="out: shape"):
        pgqa.e4m3_decode_table(torch.empty(255))


def test_qsa_and_sampler_argument_checks():
    sc = torch.zeros((4, 100))
    with pytest.raises(ValueError, match="exceeds"):
        pgqa.qsa_topk_select(sc, 8, n_blocks=101)
    with pytest.raises(ValueError, match="scores: must be a device tensor"):
        pgqa.qsa_topk_select(sc, 8)
    tok = torch.zeros((4, 12), dtype=torch.int32)
    with pytest.raises(ValueError, match="tokens: must be a device tensor"):
        pgqa.qsa_build_page4_table(tok, torch.zeros(4, dtype=torch.int32),
                                   torch.zeros((1, 8), dtype=torch.int32), num_pages=8,
                                   page_size=16, vpages_per_page=4, out_stride=4)
    z = torch.zeros((4, 1000))
    with pytest.raises(ValueError, match="logits: must be a device tensor"):
        pgqa.sampler_topk_topp_mask(z, torch.zeros(4, dtype=torch.int32), torch.zeros(4))
    # Shape checks run before the device check on the first tensor that fails.
    e = pgqa._expect
    with pytest.raises(ValueError, match="k: dtype"):
        e(torch.zeros(4), "k", torch.int32, (4,))
    with pytest.raises(ValueError, match="out: shape"):
        e(torch.zeros((4, 999)), "out", torch.float32, (4, 1000), dense=False)
    e(torch.zeros((4, 1000)), "x", torch.float32, (4, None))        # passes
    with pytest.raises(ValueError, match="x: must be a device tensor"):
        pgqa._device(x=torch.zeros(3))
    assert np.all(np.isfinite(z.numpy()))
