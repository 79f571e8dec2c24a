#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

A step is one decode step of query-aware sparse block attention for the
whole batch: kvsp_score_topk (block scores from the resident summaries, Top-k
with the keep floor, spans, dense-fallback flags) followed by
kvsp_sparse_decode (split-KV attention over the kept blocks and the exact
window, log-sum-exp merge; flagged sequences attend densely). Summaries are
built once before timing, as they are resident between steps.

Prints ONE JSON line: steps/s for the step, selected-KV GB/s of the attention
call against the 8 TB/s HBM3E peak, and the CPU oracle timed on this host.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                  [--host-pool] [--no-dkv]

After the headline timing the line also carries the DKV variant (DKV
abstract) on its own workload, Qwen2.5-1.5B-like heads with 256-token jointly
low-rank blocks: the codec over every older block, and a DKV step (scores +
attention over the compressed kept blocks and the exact window) beside the
exact sparse step on the same selection (skip it with --no-dkv).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBPS = 8000.0
PCIE_PEAK_GBPS = 64.0  # PCIe 5.0 x16 host link, one direction
METRIC = "decode-attn steps/sec + selected-KV GB/s (% of HBM peak) on 1 MI355X"


def workloads():
    from query_aware_sparse_block_amd import workloads as wl
    return {
        "opt6.7b-mha-fp16-B4-L8192-keep1/2": lambda: wl.c2(L=8192, keep="1/2"),
        "opt6.7b-mha-fp16-B4-L8192-keep1/10": lambda: wl.c2(L=8192, keep="1/10"),
        "minicpm4.1-8b-gqa-bf16-L131072-keep1/32": lambda: wl.c3(keep="1/32"),
        "minicpm4.1-8b-gqa-bf16-L131072-keep1/8": lambda: wl.c3(keep="1/8"),
        "qwen2.5-1.5b-gqa-bf16-L65536-top16": lambda: wl.c4(L=65536),
        "serving-gqa-bf16-B64-L32768-keep1/32": lambda: wl.c5(keep="1/32"),
        "serving-gqa-bf16-B64-L32768-keep7/10-dense": lambda: wl.c5(keep="7/10"),
        "tiny-mha-fp32-L1024-top8": lambda: wl.c1("k8"),
    }


DEFAULT_WORKLOAD = "opt6.7b-mha-fp16-B4-L8192-keep1/2"


def attended_tokens_per_seq(case, num_selected, use_dense):
    """Tokens each sequence attends (byte accounting from the step's own
    outputs: k kept blocks plus the window, or the whole context)."""
    out = []
    for b in range(case.B):
        L = int(case.ctx_lens[b])
        if int(use_dense[b]):
            out.append(L)
            continue
        C = max(0, L - case.recent_window) // case.P
        out.append(int(num_selected[b]) * case.P + (L - C * case.P))
    return out


def attention_bytes(case, tokens):
    """Algorithmic bytes of one attention call: each attended token's key and
    value rows for every KV head (2*D*E per token per KV head), the queries,
    the outputs and lse, and the block-table / selection entries read."""
    E = {"fp32": 4, "fp16": 2, "bf16": 2}[case.dtype]
    kv = sum(tokens) * case.Hkv * 2 * case.D * E
    q = case.B * case.Hq * case.D * E
    out = case.B * case.Hq * (case.D + 1) * 4
    blocks = sum(-(-t // case.P) for t in tokens)
    table = blocks * 4 * 2
    return kv + q + out + table, kv


def summary_bytes(case):
    """Algorithmic bytes of one summary build: the keys of every full block
    (P*D*E per KV head) read, one float32 row per (block, KV head) written."""
    E = {"fp32": 4, "fp16": 2, "bf16": 2}[case.dtype]
    full = sum(int(L) // case.P for L in case.ctx_lens)
    return full * case.Hkv * (case.P * case.D * E + case.D * 4)


def scoring_bytes(case, plans_C):
    return sum(plans_C) * case.Hkv * case.D * 4 + case.B * case.Hq * case.D * 2


def cpu_model() -> str:
    """The host CPU's model name (Linux /proc/cpuinfo), or "unknown"."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def time_cpu_oracle(case, budget_s=10.0, threads=1):
    """The oracle, as it stands, timed on this host: one whole decode step
    (scores, Top-k, spans, attention for every (sequence, head); summaries
    precomputed like the GPU's). Repeated until `budget_s` of CPU work. With
    `threads` > 1 the (sequence, head) attentions run on that many threads."""
    import oracle
    summ = oracle.summaries(case.dtype, case.k_pool, case.block_table, case.ctx_lens, case.Hkv,
                            case.P, case.D)
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        oracle.decode_step(case.dtype, case.q, case.k_pool, case.v_pool, case.block_table,
                           case.ctx_lens, summ, Hkv=case.Hkv, P=case.P, threads=threads,
                           **case.select_params)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s or len(times) >= 50:
            break
    times.sort()
    med = times[len(times) // 2]
    how = "single-threaded" if threads == 1 else f"OpenMP over (sequence, head), {threads} threads"
    return dict(value=1.0 / med, unit="steps/s", cores=threads, kind="oracle",
                sample=f"{len(times)} whole steps of the same workload "
                       f"(median {med * 1e3:.1f} ms/step), {how}, C++ double")


def time_cpu_oracle_sampled(case, n_pairs=64, budget_s=20.0, threads=1):
    """For workloads too large for whole oracle steps: scores + Top-k for every
    sequence, attention for a sample of (sequence, head) pairs, scaled to the
    whole batch."""
    import numpy as np

    import oracle
    summ = oracle.summaries(case.dtype, case.k_pool, case.block_table, case.ctx_lens, case.Hkv,
                            case.P, case.D)
    rng = np.random.default_rng(0)
    pairs = set()
    while len(pairs) < min(n_pairs, case.B * case.Hq):
        pairs.add((int(rng.integers(case.B)), int(rng.integers(case.Hq))))
    mask = np.zeros((case.B, case.Hq), np.uint8)
    t0 = time.perf_counter()
    oracle.decode_step(case.dtype, case.q, case.k_pool, case.v_pool, case.block_table,
                       case.ctx_lens, summ, Hkv=case.Hkv, P=case.P, head_mask=mask,
                       threads=threads, **case.select_params)
    t_sel = time.perf_counter() - t0
    for b, h in pairs:
        mask[b, h] = 1
    t0 = time.perf_counter()
    oracle.decode_step(case.dtype, case.q, case.k_pool, case.v_pool, case.block_table,
                       case.ctx_lens, summ, Hkv=case.Hkv, P=case.P, head_mask=mask,
                       threads=threads, **case.select_params)
    t_with = time.perf_counter() - t0
    # with several threads the sampled pairs run in rounds of `threads`
    per_round = max(t_with - t_sel, 1e-9) / -(-len(pairs) // threads)
    total = t_sel + per_round * -(-(case.B * case.Hq) // threads)
    how = "single-threaded" if threads == 1 else f"OpenMP over (sequence, head), {threads} threads"
    return dict(value=1.0 / total, unit="steps/s", cores=threads, kind="oracle",
                sample=f"selection for all {case.B} sequences + attention for {len(pairs)} of "
                       f"{case.B * case.Hq} (sequence, head) pairs, scaled to the batch; "
                       f"{how}, C++ double")


DKV_WORKLOAD = "qwen2.5-1.5b-gqa-bf16-L65536-top16-dkv-R16"


def dkv_record_payload(case, n_resid):
    """Bytes of one compressed (block, KV head) record that carry data: anchor
    rows, rank-32 basis and coefficients (float32), residual rows and offsets."""
    E = {"fp32": 4, "fp16": 2, "bf16": 2}[case.dtype]
    return (2 * case.D * E + 32 * 2 * case.D * 4 + case.P * 32 * 4 + n_resid * 2 * case.D * E
            + 4 * n_resid)


def bench_dkv(args, capture, timed):
    """The DKV variant on its own workload (see the module docstring)."""
    import torch

    from query_aware_sparse_block_amd import device as dev
    from query_aware_sparse_block_amd import kvsp
    from query_aware_sparse_block_amd import profiling
    from query_aware_sparse_block_amd import workloads as wl

    n_resid = 16
    print(f"[bench] generating {DKV_WORKLOAD}", file=sys.stderr, flush=True)
    case = wl.c4_dkv(L=65536, n_resid=n_resid)
    dkv = kvsp.DkvParams(n_resid=n_resid)
    dc0 = dev.upload(case)
    buf0 = dev.alloc_buffers(dc0)
    dev.build_summaries(dc0, buf0)  # routing summaries are made before compression
    recs0 = dev.alloc_dkv_records(dc0, dkv)
    torch.cuda.synchronize()

    # the codec: one launch compresses every block older than the window
    dev.dkv_compress(dc0, dkv, recs0)  # warm
    torch.cuda.synchronize()
    n_comp = 5
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(n_comp):
        dev.dkv_compress(dc0, dkv, recs0)
    t1.record()
    torch.cuda.synchronize()
    comp_us = t0.elapsed_time(t1) / n_comp * 1e3

    # replicas of pool, summaries and records, rotated per step (cache hygiene
    # as for the headline workload)
    pool_bytes = dc0.k_pool.numel() * dc0.k_pool.element_size() * 2
    rec_total = recs0.numel()
    R = max(3, -(-(2 << 30) // (pool_bytes + rec_total)))
    reps, bufs, recs, wss = [dc0], [buf0], [recs0], [kvsp.alloc_dkv_workspace(dc0.layout, dkv)]
    for _ in range(R - 1):
        d = dev.DeviceCase(case, dc0.q.clone(), dc0.k_pool.clone(), dc0.v_pool.clone(),
                           dc0.block_table.clone(), dc0.ctx_lens.clone(), dc0.layout, dc0.params)
        b = dev.alloc_buffers(d)
        b.summaries.copy_(buf0.summaries)
        reps.append(d)
        bufs.append(b)
        recs.append(recs0.clone())
        wss.append(kvsp.alloc_dkv_workspace(d.layout, dkv))
    torch.cuda.synchronize()

    def dkv_step(i):
        j = i % R
        dev.score_topk(reps[j], bufs[j])
        dev.dkv_decode(reps[j], bufs[j], dkv, recs[j], wss[j])

    def exact_step(i):
        dev.decode_step(reps[i % R], bufs[i % R])

    for i in range(max(args.warmup, R)):
        dkv_step(i)
        exact_step(i)
    torch.cuda.synchronize()
    dkv_s = timed(capture(dkv_step))
    dec_s = timed(capture(lambda i: dev.dkv_decode(reps[i % R], bufs[i % R], dkv, recs[i % R],
                                                   wss[i % R])))
    exact_s = timed(capture(exact_step))
    exact_dec_s = timed(capture(lambda i: dev.sparse_decode(reps[i % R], bufs[i % R])))

    E = {"fp32": 4, "fp16": 2, "bf16": 2}[case.dtype]
    L = int(case.ctx_lens[0])
    C = max(0, L - case.recent_window) // case.P
    k = int(bufs[0].num_selected[0].item())
    window = L - C * case.P
    payload = dkv_record_payload(case, n_resid)
    exact_block = 2 * case.P * case.D * E
    dkv_bytes = (case.B * case.Hkv * (k * payload + window * 2 * case.D * E)
                 + case.B * case.Hq * case.D * E + case.B * case.Hq * (case.D + 1) * 4)
    exact_bytes = (case.B * case.Hkv * (k * case.P + window) * 2 * case.D * E
                   + case.B * case.Hq * case.D * E + case.B * case.Hq * (case.D + 1) * 4)
    steps = args.steps
    return {
        "workload": DKV_WORKLOAD,
        "n_resid": n_resid, "rank": 32, "kept_blocks": k, "candidate_blocks": C,
        "window_tokens": window, "pool_replicas": R,
        "record_payload_bytes": payload, "exact_block_bytes": exact_block,
        "block_size_ratio": exact_block / payload,
        "decode_traffic": profiling.recorded_traffic(DKV_WORKLOAD, profiling.DKV_TRAFFIC_FILE,
                                                     profiling.DKV_SOURCES),
        "decode_traffic_source": "profiles/dkv_attend_traffic.txt (rocprofv3 FETCH_SIZE and "
                                 "WRITE_SIZE per dkv_attend_kernel launch, scaled as the roofline "
                                 "traffic; null if the DKV decode sources changed)",
        "compress": {"us_per_launch": comp_us, "records": case.B * C * case.Hkv,
                     "us_per_record": comp_us / (case.B * C * case.Hkv)},
        "step_us": dkv_s / steps * 1e6,
        "decode_us": dec_s / steps * 1e6,
        "decode_bytes": dkv_bytes,
        "decode_gbps": dkv_bytes / (dec_s / steps) / 1e9,
        "exact_step_us": exact_s / steps * 1e6,
        "exact_decode_us": exact_dec_s / steps * 1e6,
        "exact_decode_bytes": exact_bytes,
        "note": "latency-bound (a few MiB per call): us/step is the figure of merit",
    }


def bench_budget(case, dc):
    """The budget controller (SparPR, "Dynamic budget control") on this machine:
    the pinned host-to-device copy bandwidth and the throughput of one block's
    K and V projection GEMM ([P x hidden] x [hidden x 2 Hkv D], hidden = Hq D),
    both measured here, priced by kvsp_budget_keep_ratio for the workload."""
    import torch

    from query_aware_sparse_block_amd import kvsp

    hidden = case.Hq * case.D
    n = 256 << 20
    host = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    devbuf = torch.empty(n, dtype=torch.uint8, device="cuda")
    devbuf.copy_(host, non_blocking=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record()
    for _ in range(reps):
        devbuf.copy_(host, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    h2d = reps * n / (e0.elapsed_time(e1) * 1e-3)
    del host, devbuf

    tdt = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}[case.dtype]
    x = torch.randn(case.P, hidden, device="cuda").to(tdt)
    w = torch.randn(hidden, 2 * case.Hkv * case.D, device="cuda").to(tdt).contiguous()
    for _ in range(10):
        torch.matmul(x, w)
    torch.cuda.synchronize()
    reps = 200
    e0.record()
    for _ in range(reps):
        torch.matmul(x, w)
    e1.record()
    torch.cuda.synchronize()
    gemm_s = e0.elapsed_time(e1) * 1e-3 / reps
    flops = 2.0 * case.P * hidden * 2 * case.Hkv * case.D / gemm_s
    del x, w

    den = 1024
    num, copy_s, rec_s = kvsp.kvsp_budget_keep_ratio(dc.layout, kvsp.BudgetModel(h2d, flops, hidden),
                                                     den)
    Cs = [max(0, int(L) - case.recent_window) // case.P for L in case.ctx_lens]
    ks = [min(C, max(case.keep_floor, -(-C * num // den))) for C in Cs]
    return {"h2d_gbps": h2d / 1e9, "proj_tflops": flops / 1e12, "hidden": hidden,
            "copy_us_per_block": copy_s * 1e6, "recompute_us_per_block": rec_s * 1e6,
            "keep": f"{num}/{den}", "keep_ratio": num / den, "kept_blocks_per_seq": sorted(set(ks)),
            "note": "kvsp_budget_keep_ratio with the measured copy bandwidth (256 MiB pinned "
                    "copies) and projection throughput (torch.matmul of one block's K|V "
                    "projection); reported only, the timed step keeps the workload's keep ratio"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--replicas", type=int, default=0,
                    help="device copies of the pool rotated per step (0: at least 3 and "
                         "enough for 2 GiB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--host-pool", action="store_true",
                    help="also time the decode over a host-resident (pinned, mapped) pool")
    ap.add_argument("--no-dkv", action="store_true",
                    help="skip the DKV codec and decode on the 256-token-block workload")
    ap.add_argument("--no-budget", action="store_true",
                    help="skip measuring the budget controller's copy and recompute prices")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has "
              "no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from query_aware_sparse_block_amd import device as dev
    from query_aware_sparse_block_amd import kvsp
    from query_aware_sparse_block_amd import profiling

    kvsp.library()
    wls = workloads()
    if args.workload not in wls:
        sys.exit(f"unknown workload {args.workload}; choose from {sorted(wls)}")
    print(f"[bench] generating {args.workload}", file=sys.stderr, flush=True)
    case = wls[args.workload]()
    dc0 = dev.upload(case)
    pool_bytes = dc0.k_pool.numel() * dc0.k_pool.element_size() * 2
    R = args.replicas or max(3, -(-(2 << 30) // pool_bytes))
    # Distinct device copies (different addresses), taken in turn, so a step
    # never finds in the 256 MB Infinity Cache what an earlier step read: at
    # least 3, so two other replicas' traffic separates two uses of one, and
    # enough for 2 GiB of pools.
    reps = [dc0]
    for _ in range(R - 1):
        reps.append(dev.DeviceCase(case, dc0.q.clone(), dc0.k_pool.clone(), dc0.v_pool.clone(),
                                   dc0.block_table.clone(), dc0.ctx_lens.clone(), dc0.layout,
                                   dc0.params))
    bufs = [dev.alloc_buffers(d) for d in reps]
    # Summaries of every replica (step 1, before timing: they are resident
    # between steps); each build is timed on its own.
    build_ev = []
    for d, bf in zip(reps, bufs):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dev.build_summaries(d, bf)
        e1.record()
        build_ev.append((e0, e1))
    torch.cuda.synchronize()
    build_us = sorted(a.elapsed_time(b) * 1e3 for a, b in build_ev)[len(build_ev) // 2]
    print(f"[bench] {R} replica(s) of {pool_bytes / 2**30:.2f} GiB resident", file=sys.stderr,
          flush=True)

    for i in range(args.warmup):
        dev.decode_step(reps[i % R], bufs[i % R])
    torch.cuda.synchronize()

    # Each timed region is one HIP graph holding all K calls (replicas taken
    # in turn), so host launch overhead does not enter the measurement. The
    # kernels reset their own completion counters, so the graphs hold kernel
    # nodes only.
    def capture(fn):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn(0)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(args.steps):
                fn(i)
        graph.replay()  # warm
        torch.cuda.synchronize()
        return graph

    def timed(graph):
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        graph.replay()
        stop.record()
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / 1e3  # seconds

    step_s = timed(capture(lambda i: dev.decode_step(reps[i % R], bufs[i % R])))
    attn_s = timed(capture(lambda i: dev.sparse_decode(reps[i % R], bufs[i % R])))
    sel_s = timed(capture(lambda i: dev.score_topk(reps[i % R], bufs[i % R])))

    # Decode-time append, timed on its own (it precedes scoring in a decode
    # loop): each sequence's newest token is written again with its own K/V
    # rows, so the pools and summaries keep their contents; when the contexts
    # end on a block boundary every call also re-derives that block's summary.
    ctx0 = dc0.ctx_lens.long()
    bt0 = dc0.block_table.long()
    last_phys = bt0[torch.arange(case.B, device=bt0.device), (ctx0 - 1) // case.P]
    last_t = (ctx0 - 1) % case.P
    k_last = dc0.k_pool[last_phys, :, last_t].contiguous()
    v_last = dc0.v_pool[last_phys, :, last_t].contiguous()
    pos_last = (ctx0 - 1).to(torch.int32)
    append_s = timed(capture(lambda i: dev.append_kv(reps[i % R], bufs[i % R], k_last, v_last,
                                                     pos_last)))
    completes = bool(((ctx0 % case.P) == 0).all().item())

    # With --host-pool: the pool in host RAM (mapped pinned memory, the SparPR
    # setting), where the decode reads its attended tiles across PCIe. A few
    # eager calls on replica 0's selection; pools above 4 GiB are skipped.
    host_pool = None
    if args.host_pool and pool_bytes <= (4 << 30):
        print("[bench] decode over a host-resident pool", file=sys.stderr, flush=True)
        hdc = dev.with_host_pool(dc0)
        dev.sparse_decode(hdc, bufs[0])  # warm
        torch.cuda.synchronize()
        n_host = 5
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(n_host):
            dev.sparse_decode(hdc, bufs[0])
        t1.record()
        torch.cuda.synchronize()
        host_pool = {"calls": n_host, "decode_us": t0.elapsed_time(t1) / n_host * 1e3}
        del hdc

    nsel = bufs[0].num_selected.cpu().numpy()
    dense = bufs[0].use_dense.cpu().numpy()
    tokens = attended_tokens_per_seq(case, nsel, dense)
    attn_bytes, kv_bytes = attention_bytes(case, tokens)
    Cs = [max(0, int(L) - case.recent_window) // case.P for L in case.ctx_lens]
    attn_avg = attn_s / args.steps
    achieved = attn_bytes / attn_avg / 1e9
    ms_per_step = step_s / args.steps * 1e3

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        big = sum(tokens) * case.Hq * case.D > 2e9
        cpu = time_cpu_oracle_sampled(case) if big else time_cpu_oracle(case)
        cpu["cores_available"] = os.cpu_count()
        cpu["cpu_model"] = cpu_model()
        # the same oracle with its (sequence, head) loop on the host's thread share
        threads = max(1, int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)))
        if threads > 1:
            mt = (time_cpu_oracle_sampled(case, threads=threads) if big
                  else time_cpu_oracle(case, budget_s=5.0, threads=threads))
            cpu["openmp"] = {k: mt[k] for k in ("value", "unit", "cores", "sample")}

    dkv = None if args.no_dkv else bench_dkv(args, capture, timed)
    budget = None if args.no_budget else bench_budget(case, reps[0])

    E = {"fp32": 4, "fp16": 2, "bf16": 2}[case.dtype]
    rec = {
        "metric": METRIC,
        "value": args.steps / step_s,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dtype,
        "data": "synthetic",
        "launch": "hipGraph of all K steps",
        "config": {
            "workload": args.workload,
            "batch": case.B, "q_heads": case.Hq, "kv_heads": case.Hkv, "head_dim": case.D,
            "block": case.P, "contexts": sorted(set(int(x) for x in case.ctx_lens)),
            "top_k": case.top_k, "keep": f"{case.keep_num}/{case.keep_den}",
            "keep_floor": case.keep_floor, "recent_window": case.recent_window,
            "gamma": f"{case.gamma_num}/{case.gamma_den}",
            "attended_tokens_per_seq": sorted(set(tokens)),
            "dense_sequences": int(dense.sum()), "pool_replicas": R,
        },
        "selected_kv_gbps": achieved,
        "selected_kv_hbm_frac": achieved / HBM_PEAK_GBPS,
        "step_gbps": (attn_bytes + scoring_bytes(case, Cs)) / (ms_per_step * 1e-3) / 1e9,
        "step_gbps_note": "attention bytes (selected K/V, q, table, out) + scoring bytes "
                          "(summaries, q) per step, over the step time",
        "kernels_us": {"score_topk": sel_s / args.steps * 1e6,
                       "sparse_decode": attn_avg * 1e6,
                       "step": ms_per_step * 1e3,
                       "append_kv": append_s / args.steps * 1e6},
        "append": {"completes_block": completes,
                   "bytes_written_per_launch": 2 * case.B * case.Hkv * case.D * E
                   + (case.B * case.Hkv * case.D * 4 if completes else 0),
                   "bytes_read_per_launch": case.B * case.Hkv * case.P * case.D * E
                   if completes else 0},
        "roofline": {
            "bound": "hbm",
            "kernel": "attend_kernel (the whole kvsp_sparse_decode call)",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "bytes_per_launch": attn_bytes,
            "kv_bytes_per_launch": kv_bytes,
            "per_unit": f"2*D*E = {2 * case.D * E} B per attended token per KV head",
            "traffic": profiling.recorded_traffic(args.workload),
            "traffic_source": "profiles/attend_traffic.txt (rocprofv3 FETCH_SIZE*2 + "
                              "WRITE_SIZE*1 per launch; null if the decode sources changed)",
        },
        "host_pool": None if host_pool is None else {
            **host_pool,
            "pcie_gbps": attn_bytes / (host_pool["decode_us"] * 1e-6) / 1e9,
            "pcie_peak_gbps": PCIE_PEAK_GBPS,
            "frac": attn_bytes / (host_pool["decode_us"] * 1e-6) / 1e9 / PCIE_PEAK_GBPS,
            "note": "kvsp_sparse_decode with K/V in mapped pinned host memory; bytes as roofline",
        },
        "scoring": {"bytes_per_launch": scoring_bytes(case, Cs),
                    "gbps": scoring_bytes(case, Cs) / (sel_s / args.steps) / 1e9},
        "summaries": {"us": build_us, "bytes_per_launch": summary_bytes(case),
                      "gbps": summary_bytes(case) / (build_us * 1e-6) / 1e9,
                      "note": "kvsp_build_summaries over every full block, median over replicas"},
        "dkv": dkv,
        "budget": budget,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
