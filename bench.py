#!/usr/bin/env python3
"""Benchmark: paged GQA decode, B=16 x 16K context, FP8-E4M3 KV, page 128.

One step = one paged_gqa_decode call over the whole batch (every stage of the
path: page-table gather, E4M3 dequant, QK^T, online softmax, PV, split
merge).  Inputs are resident in HBM before timing starts.  The KV pool is
replicated into R separate device copies and the steps rotate through them,
so consecutive calls cannot be served from the 256 MB last-level cache.

Prints ONE JSON line.  `value` is KV-read GB/s: algorithmic KV bytes per call
(every live token's K and V row read once) divided by the call time, the
median of five batches of exactly K calls, each batch's average measured with
HIP events on the stream the kernels run on, after SETTLE_MS of untimed calls
(the shader clock read after each batch is in `repeat`).  `roofline` uses the dominant
kernel alone (timed the same way) when the call has more than one.  Beside
them: `repeat` (the five batches), `warm` (one pool reused every call, so not
an HBM rate) and, for decode, `read_ceiling` (a plain streaming read of the
same number of bytes from the same rotated pools: the rate those bytes can
reach here).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("KV-read HBM GB/s (% of peak) and µs/call, paged GQA decode B16×16K E4M3")
HBM_PEAK_GBS = 8000.0
BALANCE_MAX_SEQS = 512  # sequences the library's balanced split plan covers
# Untimed work before the first timed batch: in the first tens of
# milliseconds of sustained HBM load the device's power management lowers
# the shader clock (1.9-2.1 GHz instead of 2.42 GHz, measured with
# clock_probe after each batch), which slows 20-call batches by up to 8%;
# after this much untimed work the clock has settled.
SETTLE_MS = 100.0
KERNEL_SOURCES = [os.path.join(ROOT, "fp8_kv_amd", "csrc", f)
                  for f in ("pgqa_kernels.hip", "pgqa_api.hip", "pgqa_internal.h")]


_C_TOKENS = re.compile(r'//[^\n]*|/\*.*?\*/|"(?:\\.|[^"\\])*"', re.S)


def code_of(text: str) -> str:
    """C/C++ source without comments, whitespace runs collapsed: what the
    compiler sees, so a comment edit does not count as a kernel change."""
    text = _C_TOKENS.sub(lambda m: " " if m.group(0).startswith("/") else m.group(0), text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, encoding="utf-8") as f:
            h.update(code_of(f.read()).encode())
    return h.hexdigest()[:16]


def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json")


def measured_traffic(src_hash: str, workload: str):
    """HBM bytes per launch of the attention kernel from committed rocprofv3
    counter runs on `workload`, if they were taken on the current kernel
    sources; else None."""
    try:
        with open(traffic_file(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != src_hash:
        return None
    return t.get("hbm_bytes_per_launch")



def cpu_baseline(case, budget_s: float) -> dict:
    """The fp64 oracle, as it is, on the host cores: repeat whole calls on
    the same workload until about `budget_s` seconds have passed."""
    import oracle

    n_calls, t0 = 0, time.perf_counter()
    while True:
        oracle.paged_gqa(**case.oracle_kwargs())
        n_calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n_calls >= 200:
            break
    per_call = el / n_calls
    return {"value": round(case.kv_bytes_read() / per_call / 1e9, 4), "unit": "GB/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{n_calls} whole calls of the same workload, {per_call * 1e3:.1f} ms each"}


def cpu_baseline_topk(case, budget_s: float) -> dict:
    """The oracle's top-k selection, as it is, on a bounded sample of rows
    (the first rows of the workload, doubling until about `budget_s`)."""
    import oracle

    rows, el = min(16, case.rows), 0.0
    while True:
        t0 = time.perf_counter()
        oracle.topk_select(case.scores[:rows], case.k, case.n_valid[:rows],
                           n_blocks=case.n_blocks)
        el = time.perf_counter() - t0
        if el >= budget_s / 3 or rows >= case.rows:
            break
        rows = min(case.rows, rows * 2)
    nv = case.n_valid[:rows].clip(0, case.n_blocks).astype("int64")
    gbs = float(nv.sum()) * 4 / el / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"first {rows} of {case.rows} rows, {el * 1e3:.1f} ms"}


def bench_topk(args) -> int:
    """QSA top-k selection: one step = one qsa_topk_select call over every
    row.  `value` is score-read GB/s: the eligible score bytes of all rows
    (read once) divided by the average call time; the call is one kernel."""
    import torch

    from fp8_kv_amd import inputs, pgqa

    pgqa.load()
    torch.cuda.set_device(0)
    case = inputs.topk_workload_case(args.workload)
    R = max(1, args.pools)
    scores = [torch.from_numpy(case.scores).to("cuda")]
    for _ in range(R - 1):
        scores.append(scores[0].clone())
    nv = torch.from_numpy(case.n_valid).to("cuda")
    idx = torch.empty((case.rows, case.k), dtype=torch.int32, device="cuda")
    cnt = torch.empty(case.rows, dtype=torch.int32, device="cuda")

    def call(i):
        pgqa.qsa_topk_select(scores[i % R], case.k, nv, n_blocks=case.n_blocks, out_idx=idx,
                             out_count=cnt)

    ms = time_steps(call, args.steps, args.warmup, R, not args.eager)
    score_bytes = case.score_bytes()
    alg_bytes = score_bytes + case.rows * case.k * 4 + case.rows * 4
    gbs = score_bytes / (ms * 1e-3) / 1e9
    kernel_gbs = alg_bytes / (ms * 1e-3) / 1e9
    result = {
        "metric": "score-read HBM GB/s and µs/call, QSA top-k block selection",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "u32 keys of f32 scores",
        "data": "synthetic",
        "config": {"workload": args.workload, "rows": case.rows, "n_blocks": case.n_blocks,
                   "k": case.k, "pools_rotated": R, "us_per_call": round(ms * 1e3, 3),
                   "score_bytes_per_call": score_bytes,
                   "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)},
        "roofline": {"bound": "hbm", "achieved": round(kernel_gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(kernel_gbs / HBM_PEAK_GBS, 4),
                     "traffic": None, "kernel": "topk_kernel",
                     "kernel_us": round(ms * 1e3, 3)},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_topk(case, args.cpu_budget)
    print(json.dumps(result), flush=True)
    return 0


def page4_alg_bytes(case) -> int:
    """Bytes one builder call must move: every row's selection entries and
    live length read, one block-table entry read per output page, the whole
    output row plus its length and status written."""
    rows = case.rows
    n_pages = case.meta["selected_blocks"] + (1 if case.meta["tail"] else 0)
    return rows * (case.n_tokens * 4 + 4 + n_pages * 4 + case.out_stride * 4 + 8)


def cpu_baseline_page4(case, budget_s: float) -> dict:
    """The oracle's table builder, as it is, on a bounded sample of rows (the
    first rows of the workload, doubling until about `budget_s`)."""
    import oracle

    rows, el = min(64, case.rows), 0.0
    while True:
        t0 = time.perf_counter()
        oracle.qsa_page4_table(case.tokens[:rows], case.live_len[:rows], case.block_table,
                               **case.builder_kwargs())
        el = time.perf_counter() - t0
        if el >= budget_s / 3 or rows >= case.rows:
            break
        rows = min(case.rows, rows * 2)
    gbs = page4_alg_bytes(case) * rows / case.rows / el / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"first {rows} of {case.rows} rows, {el * 1e3:.1f} ms"}


def bench_page4(args) -> int:
    """Virtual page-4 table building: one step = one qsa_build_page4_table
    call over every row.  `value` is the call's algorithmic bytes (selections
    read, block-table entries looked up, tables written) per average call
    time; the call is one kernel."""
    import torch

    from fp8_kv_amd import inputs, pgqa

    pgqa.load()
    torch.cuda.set_device(0)
    case = inputs.page4_workload_case(args.workload)
    R = max(1, args.pools)
    toks = [torch.from_numpy(case.tokens).to("cuda")]
    for _ in range(R - 1):
        toks.append(toks[0].clone())
    live = torch.from_numpy(case.live_len).to("cuda")
    bt = torch.from_numpy(case.block_table).to("cuda")
    out_t = torch.empty((case.rows, case.out_stride), dtype=torch.int32, device="cuda")
    out_l = torch.empty(case.rows, dtype=torch.int32, device="cuda")
    out_s = torch.empty(case.rows, dtype=torch.int32, device="cuda")
    kw = case.builder_kwargs()
    kw.pop("row_seq")

    def call(i):
        pgqa.qsa_build_page4_table(toks[i % R], live, bt, out_table=out_t, out_len=out_l,
                                   out_status=out_s, **kw)

    ms = time_steps(call, args.steps, args.warmup, R, not args.eager)
    alg = page4_alg_bytes(case)
    gbs = alg / (ms * 1e-3) / 1e9
    result = {
        "metric": "HBM GB/s and µs/call, virtual page-4 table build from QSA selections",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int32", "data": "synthetic",
        "config": {"workload": args.workload, "rows": case.rows, "tokens_per_row": case.n_tokens,
                   "page_size": case.page_size, "vpages_per_page": case.vpages_per_page,
                   "out_stride": case.out_stride, "selections_rotated": R,
                   "us_per_call": round(ms * 1e3, 3), "alg_bytes_per_call": alg,
                   "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "page4_kernel", "kernel_us": round(ms * 1e3, 3)},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_page4(case, args.cpu_budget)
    print(json.dumps(result), flush=True)
    return 0


def cpu_baseline_sampler(case, budget_s: float) -> dict:
    """The oracle's masking, as it is, on a bounded sample of rows (doubling
    from one row until about `budget_s`)."""
    import oracle

    rows, el = 1, 0.0
    while True:
        t0 = time.perf_counter()
        oracle.topk_topp_mask(case.logits[:rows], case.k[:rows], case.p[:rows],
                              k_max=case.k_max)
        el = time.perf_counter() - t0
        if el >= budget_s / 3 or rows >= case.rows:
            break
        rows = min(case.rows, rows * 2)
    gbs = rows * case.vocab * 8 / el / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle", "sample": f"first {rows} of {case.rows} rows, {el * 1e3:.1f} ms"}


def bench_sampler(args) -> int:
    """Combined top-k/top-p masking: one step = one sampler_topk_topp_mask
    call over every row (two kernels).  `value` is the call's algorithmic
    bytes (every logit read once and written once) per average call time."""
    import torch

    from fp8_kv_amd import inputs, pgqa

    pgqa.load()
    torch.cuda.set_device(0)
    case = inputs.sampler_workload_case(args.workload)
    R = max(1, args.pools)
    logits = [torch.from_numpy(case.logits).to("cuda")]
    for _ in range(R - 1):
        logits.append(logits[0].clone())
    k = torch.from_numpy(case.k).to("cuda")
    p = torch.from_numpy(case.p).to("cuda")
    out = torch.empty_like(logits[0])
    st = torch.empty(case.rows, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(8, pgqa.sampler_topk_topp_workspace_bytes(case.rows, case.vocab,
                                                                   case.k_max)),
                     dtype=torch.uint8, device="cuda")

    def call(i):
        pgqa.sampler_topk_topp_mask(logits[i % R], k, p, k_max=case.k_max, out=out, status=st,
                                    workspace=ws)

    ms = time_steps(call, args.steps, args.warmup, R, not args.eager)
    alg = case.rows * case.vocab * 8
    gbs = alg / (ms * 1e-3) / 1e9
    result = {
        "metric": "HBM GB/s and µs/call, combined top-k/top-p masking of sampler logits",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": args.workload, "rows": case.rows, "vocab": case.vocab,
                   "top_k": int(case.k[0]), "top_p": float(case.p[0]), "k_max": case.k_max,
                   "logit_copies_rotated": R, "us_per_call": round(ms * 1e3, 3),
                   "alg_bytes_per_call": alg,
                   "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "chunk_top_kernel + cut_kernel",
                     "kernel_us": round(ms * 1e3, 3)},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_sampler(case, args.cpu_budget)
    print(json.dumps(result), flush=True)
    return 0


def time_batches(step, steps: int, warmup: int, R: int, use_graph: bool,
                 batches: int = 1, settle_ms: float = 0.0, clocks: list | None = None
                 ) -> list[float]:
    """Average milliseconds per step over exactly `steps` steps, timed with HIP
    events on the stream the kernels run on; one average per batch.

    With use_graph the steps are captured into one HIP graph (up to
    kGraphSteps of them, cycling through the R pools, replayed as often as
    needed, the remainder eager), as a serving loop captures a whole decode
    step, so neither Python's per-call overhead nor graph-launch boundaries
    leave the GPU idle between steps.  Before each timed batch one untimed
    replay of the same graph is queued without waiting for it: the GPU runs
    it while the host submits the timed replays, so the first timed step
    starts as soon as that untimed replay ends, not when the host has finished
    submitting (with 20-step graphs the host's submission latency otherwise
    lands inside the events, spread over only 20 calls).

    settle_ms > 0: before the first batch, untimed replays keep the device
    busy for that long (see SETTLE_MS).  clocks: when given, the shader
    clock (MHz) probed right after each timed batch is appended to it."""
    import torch

    kGraphSteps = 512
    cur = torch.cuda.current_stream()
    G = min(steps, kGraphSteps)
    if use_graph and G > 0:
        side = torch.cuda.Stream()
        side.wait_stream(cur)
        with torch.cuda.stream(side):
            for i in range(R):
                step(i)
        cur.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(G):
                step(i)
        replay, per_replay = graph.replay, G
    else:
        def replay():
            for i in range(R):
                step(i)
        per_replay = R
    for i in range(warmup):
        step(i)
    if use_graph and G > 0:
        replay()  # the graph's first launch uploads it: keep that out of the timing
    torch.cuda.synchronize()
    if settle_ms > 0:
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record(cur)
        for _ in range(10000):  # bounded: ends by time long before this count
            for _ in range(8):
                replay()
            s1.record(cur)
            s1.synchronize()
            if s0.elapsed_time(s1) >= settle_ms:
                break
    probe_buf = torch.zeros(2, dtype=torch.int64, device="cuda") if clocks is not None else None
    out = []
    for _ in range(batches):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if use_graph and G > 0:
            replay()  # untimed: keeps the GPU busy while the timed steps are queued
        e0.record(cur)
        for _ in range(steps // per_replay):
            replay()
        for i in range(steps % per_replay):
            step(i)
        e1.record(cur)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / steps)
        if clocks is not None:
            from fp8_kv_amd import stream_read

            clocks.append(round(stream_read.clock_mhz(probe_buf, stream=cur)))
    return out


def time_steps(step, steps: int, warmup: int, R: int, use_graph: bool,
               batches: int = 3) -> float:
    """Median over `batches` batches of the average milliseconds per step,
    each batch exactly `steps` steps."""
    return float(np.median(time_batches(step, steps, warmup, R, use_graph, batches)))


def read_ceiling(pools, kv_bytes: int, steps: int, warmup: int, use_graph: bool) -> dict:
    """The plain streaming-read kernel over the same number of KV bytes, taken
    from the same rotated pools (K storage first, then V), timed like the
    attention kernel; the best of a few grid sizes.  The attainable rate for
    these bytes on this device, for context beside roofline.achieved."""
    import torch

    from fp8_kv_amd import stream_read as sr

    R = len(pools)
    spans = []
    for p in pools:
        ks, vs = (t.view(torch.uint8).reshape(-1) for t in p.storage)
        if vs.data_ptr() == ks.data_ptr():      # interleaved: one allocation
            spans.append((ks[:kv_bytes], None))
        else:
            half = kv_bytes // 2
            spans.append((ks[:half], vs[:kv_bytes - half]))
    sweep = {}
    for blocks in (1024, 2048, 4096):
        sink = torch.empty((blocks, 4), dtype=torch.int32, device="cuda")

        def step(i, sink=sink, blocks=blocks):
            a, b = spans[i % R]
            sr.stream_read(a, b, sink, blocks)

        sweep[blocks] = time_steps(step, steps, warmup, R, use_graph)
    blocks = min(sweep, key=sweep.get)
    ms = sweep[blocks]
    gbs = kv_bytes / (ms * 1e-3) / 1e9
    return {"kernel": "stream_read_kernel (16-byte non-temporal loads, no page indirection)",
            "us": round(ms * 1e3, 3), "GB/s": round(gbs, 2), "frac": round(gbs / HBM_PEAK_GBS, 4),
            "blocks": blocks, "sweep_us": {str(k): round(v * 1e3, 3) for k, v in sweep.items()}}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="decode_b16_16k_e4m3_p128")
    ap.add_argument("--pools", type=int, default=8,
                    help="device copies of the KV pool rotated between steps (1 = warm cache)")
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="launch every step from Python instead of replaying a captured graph")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        return 2

    from fp8_kv_amd import inputs

    if args.workload in inputs.TOPK_WORKLOADS:
        return bench_topk(args)
    if args.workload in inputs.PAGE4_WORKLOADS:
        return bench_page4(args)
    if args.workload in inputs.SAMPLER_WORKLOADS:
        return bench_sampler(args)

    import torch

    from fp8_kv_amd import pgqa

    pgqa.load()
    torch.cuda.set_device(0)
    case = inputs.workload_case(args.workload)
    prefill = args.workload.startswith("prefill")
    q, pool0, table, lens = pgqa.device_case(case)
    n, hq, _ = q.shape
    R = max(1, args.pools)
    pools = [pool0]
    for _ in range(R - 1):
        ks = pool0.storage[0].clone()
        vs = ks if pool0.storage[1] is pool0.storage[0] else pool0.storage[1].clone()
        kflat, vflat = ks.reshape(-1), vs.reshape(-1)
        pools.append(pgqa.KVPool(kflat[case.k_offset:], vflat[case.v_offset:], case.page_stride,
                                 case.token_stride, case.head_stride, case.num_pages,
                                 case.page_size, case.kv_dtype, case.k_scale, case.v_scale,
                                 storage=(ks, vs)))
    out = torch.empty_like(q)
    splits = pgqa.paged_gqa_num_splits(n, case.num_kv_heads, case.max_seq_len, args.num_splits)
    wsb = pgqa.paged_gqa_workspace_bytes(n, hq, case.num_kv_heads, case.max_seq_len,
                                         args.num_splits)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
    fn = pgqa.paged_gqa_prefill_sparse if prefill else pgqa.paged_gqa_decode
    part_o = torch.empty((n, hq, splits, 256), dtype=torch.float32, device="cuda")
    part_l = torch.empty((n, hq, splits), dtype=torch.float32, device="cuda")

    def call(i):  # one whole call: attention (+ merge when split)
        fn(q, pools[i % R], table, lens, case.max_seq_len, case.sm_scale, out,
           num_kv_heads=case.num_kv_heads, workspace=ws, num_splits=args.num_splits)

    def attention_only(i):  # the dominant kernel alone, same launch configuration
        pgqa.paged_gqa_decode_partial(q, pools[i % R], table, lens, case.max_seq_len,
                                      case.sm_scale, part_o, part_l,
                                      num_kv_heads=case.num_kv_heads,
                                      num_splits=args.num_splits)

    clocks: list = []
    batches = time_batches(call, args.steps, args.warmup, R, not args.eager, batches=5,
                           settle_ms=SETTLE_MS, clocks=clocks)
    ms = float(np.median(batches))  # five batches of exactly K steps each: their median
    # decode_partial runs the attention kernel of a whole call only when both
    # use the static split plan: decode (not prefill) with every length at
    # max_seq_len, or more sequences than the balanced plan covers.
    live = np.clip(case.lens, 0, case.max_seq_len)
    same_plan = not prefill and (bool(np.all(live == case.max_seq_len)) or n > BALANCE_MAX_SEQS)
    if splits == 1:
        kernel_ms, kernel_name = ms, "attention_kernel"
    elif same_plan:
        kernel_ms = time_steps(attention_only, args.steps, args.warmup, R, not args.eager)
        kernel_name = "attention_kernel"
    else:
        kernel_ms = ms
        kernel_name = "paged_gqa_decode whole call (attention + merge; its split plan has no " \
                      "stand-alone entry point)"
    kv_bytes = case.kv_bytes_read()
    gbs = kv_bytes / (ms * 1e-3) / 1e9
    kernel_gbs = kv_bytes / (kernel_ms * 1e-3) / 1e9

    src_hash = kernel_source_hash()
    traffic = measured_traffic(src_hash, args.workload)
    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 kv -> f16 mfma, f32 accumulate" if case.kv_dtype == inputs.KV_E4M3
                 else "f16 kv -> f16 mfma, f32 accumulate",
        "data": "synthetic",
        "config": {
            "workload": args.workload, "batch_or_rows": n, "q_heads": hq,
            "kv_heads": case.num_kv_heads, "head_dim": 256,
            "context": int(case.max_seq_len), "page_size": case.page_size,
            "kv_dtype": "fp8_e4m3" if case.kv_dtype == inputs.KV_E4M3 else "fp16",
            "layout": case.layout, "num_splits": splits, "pools_rotated": R,
            "us_per_call": round(ms * 1e3, 3), "kv_bytes_per_call": kv_bytes,
            "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "kernel_source_hash": src_hash,
        },
        "roofline": {"bound": "hbm", "achieved": round(kernel_gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(kernel_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic if kernel_name == "attention_kernel" else None,
                     "kernel": kernel_name, "kernel_us": round(kernel_ms * 1e3, 3)},
    }
    result["repeat"] = {"batches": len(batches), "steps_each": args.steps,
                        "us_per_call": [round(b * 1e3, 3) for b in batches],
                        "median_us": round(ms * 1e3, 3),
                        "first_us": round(batches[0] * 1e3, 3),
                        "spread_us": round((max(batches) - min(batches)) * 1e3, 3),
                        "settle_ms": SETTLE_MS, "sclk_mhz_after_each": clocks}
    if R > 1:
        warm_ms = time_steps(lambda i: call(0), args.steps, args.warmup, 1, not args.eager)
        result["warm"] = {
            "pools_rotated": 1, "us_per_call": round(warm_ms * 1e3, 3),
            "GB/s": round(kv_bytes / (warm_ms * 1e-3) / 1e9, 2),
            "note": "one pool reused every call: its bytes can stay in the 256 MB last-level "
                    "cache, so this is not an HBM rate"}
    if not prefill:
        result["read_ceiling"] = read_ceiling(pools, kv_bytes, args.steps, args.warmup,
                                              not args.eager)
    if prefill:
        # Rows select overlapping blocks of one pool, so most gathered bytes
        # are served by L2 and the last-level cache: the HBM-side rate comes
        # from the calibrated counters of this kernel source, when recorded.
        rf = result["roofline"]
        rf["gathered_GBs"] = round(kernel_gbs, 2)
        if traffic:
            hbm_gbs = traffic / (kernel_ms * 1e-3) / 1e9
            rf["achieved"] = round(hbm_gbs, 2)
            rf["frac"] = round(hbm_gbs / HBM_PEAK_GBS, 4)
            rf["note"] = ("achieved: calibrated HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, "
                          "profiles/traffic_<workload>.json) / kernel time; gathered_GBs: the "
                          "K/V bytes the rows gather / kernel time")
        else:
            rf["achieved"], rf["frac"] = None, None
            rf["note"] = ("no counter record for these kernel sources: the HBM-side rate is "
                          "unknown; gathered_GBs counts gathered K/V bytes, most served by L2")
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(case, args.cpu_budget)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
