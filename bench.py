#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

A step is one decode step of query-aware sparse block attention for the
whole batch: kvsp_score_topk (block scores from the resident summaries, Top-k
with the keep floor, spans, dense-fallback flags) followed by
kvsp_sparse_decode over the span list it wrote (split-KV attention over the
kept blocks and the exact window, log-sum-exp merge; flagged sequences attend
densely). Summaries are built once before timing, as they are resident
between steps.

Prints ONE JSON line. Its headline is the batched serving shape (64 sequences
of 32768 tokens, 32 query / 8 KV heads, bf16, keep 1/32, gamma 3/5): steps/s
for the step, selected-KV GB/s of the attention call against the 8 TB/s
HBM3E peak, and the CPU oracle timed on this host. The same line carries a
`configs` map with a record per other workload (the tiny fp32 case, the
OPT-like batch at keep 1/2 and 1/10, the MiniCPM-like context at keep 1/32,
1/16 and 1/8, the Qwen-like context at 65536 tokens, and the serving shape's
keep-7/10 dense fallback), each timed the same way; the decode over a
host-resident pool (PCIe) on the OPT-like batch; the DKV variant; and the
budget controller's measured inputs.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                  [--no-configs] [--config-steps N] [--no-host-pool] [--no-dkv]
                  [--no-budget]

The DKV variant (DKV abstract) runs on its own workload, Qwen2.5-1.5B-like
heads with 256-token jointly low-rank blocks: the codec over every older
block, and a DKV step (scores + attention over the compressed kept blocks and
the exact window) beside the exact sparse step on the same selection.
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
        "minicpm4.1-8b-gqa-bf16-L131072-keep1/16": lambda: wl.c3(keep="1/16"),
        "minicpm4.1-8b-gqa-bf16-L131072-keep1/8": lambda: wl.c3(keep="1/8"),
        "qwen2.5-1.5b-gqa-bf16-L65536-top16": lambda: wl.c4(L=65536),
        "serving-gqa-bf16-B64-L32768-keep1/32": lambda: wl.c5(keep="1/32"),
        "serving-gqa-bf16-B64-L32768-keep7/10-dense": lambda: wl.c5(keep="7/10"),
        "tiny-mha-fp32-L1024-top8": lambda: wl.c1("k8"),
    }


DEFAULT_WORKLOAD = "serving-gqa-bf16-B64-L32768-keep1/32"
# Timed beside the headline, each in a record of the `configs` map.
CONFIG_WORKLOADS = [
    "tiny-mha-fp32-L1024-top8",
    "opt6.7b-mha-fp16-B4-L8192-keep1/2",
    "opt6.7b-mha-fp16-B4-L8192-keep1/10",
    "minicpm4.1-8b-gqa-bf16-L131072-keep1/32",
    "minicpm4.1-8b-gqa-bf16-L131072-keep1/16",
    "minicpm4.1-8b-gqa-bf16-L131072-keep1/8",
    "qwen2.5-1.5b-gqa-bf16-L65536-top16",
    "serving-gqa-bf16-B64-L32768-keep7/10-dense",
]
HOST_POOL_WORKLOAD = "opt6.7b-mha-fp16-B4-L8192-keep1/2"
# Steps whose bytes at 8 TB/s take under this long are launch- and
# latency-bound: microseconds per step is their figure of merit.
LATENCY_BOUND_US = 5.0


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
    summ = oracle.stored_summaries(oracle.summaries(case.dtype, case.k_pool, case.block_table,
                                                    case.ctx_lens, case.Hkv, case.P, case.D))
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
    summ = oracle.stored_summaries(oracle.summaries(case.dtype, case.k_pool, case.block_table,
                                                    case.ctx_lens, case.Hkv, case.P, case.D))
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
    import numpy as np
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
    # subspace-iteration rounds the codec chose per record (older blocks only)
    lay = wl.dkv_record_layout(case.D, case.P, wl.ELEM_BYTES[case.dtype], n_resid)
    C0 = max(0, int(case.ctx_lens[0]) - case.recent_window) // case.P
    older = dc0.block_table[0, :C0].long()
    rounds = recs0[older][:, :, lay["rounds"]:lay["rounds"] + 4].contiguous().view(torch.int32)
    rounds = rounds.reshape(-1).cpu().numpy()

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
        "decode_traffic": profiling.recorded_traffic(DKV_WORKLOAD, kernel="dkv_attend"),
        "decode_traffic_source": "profiles/traffic_dkv_attend_<workload>.txt (rocprofv3 "
                                 "FETCH_SIZE and WRITE_SIZE per dkv_attend_kernel launch, scaled "
                                 "by a plain copy; null if the DKV decode sources changed)",
        "compress": {"us_per_launch": comp_us, "records": case.B * C * case.Hkv,
                     "us_per_record": comp_us / (case.B * C * case.Hkv),
                     "rounds_min": int(rounds.min()), "rounds_median": float(np.median(rounds)),
                     "rounds_max": int(rounds.max()),
                     "records_at_round_cap": int((rounds >= 64).sum()),
                     "rounds_note": "subspace-iteration rounds per record: 8, then as many as "
                                    "the measured Ritz-value ratio needs for a 1e-6 reduction, "
                                    "at most 64"},
        "step_us": dkv_s / steps * 1e6,
        "decode_us": dec_s / steps * 1e6,
        "decode_bytes": dkv_bytes,
        "decode_gbps": dkv_bytes / (dec_s / steps) / 1e9,
        "exact_step_us": exact_s / steps * 1e6,
        "exact_decode_us": exact_dec_s / steps * 1e6,
        "exact_decode_bytes": exact_bytes,
        "note": "latency-bound (a few MiB per call): us/step is the figure of merit",
    }


def bench_budget(case):
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
    layout = kvsp.kvsp_layout(case.B, case.Hq, case.Hkv, case.D, case.P, case.num_phys,
                              case.max_blocks, {"fp32": 0, "fp16": 1, "bf16": 2}[case.dtype])
    num, copy_s, rec_s = kvsp.kvsp_budget_keep_ratio(layout, kvsp.BudgetModel(h2d, flops, hidden),
                                                     den)
    Cs = [max(0, int(L) - case.recent_window) // case.P for L in case.ctx_lens]
    ks = [min(C, max(case.keep_floor, -(-C * num // den))) for C in Cs]
    return {"h2d_gbps": h2d / 1e9, "proj_tflops": flops / 1e12, "hidden": hidden,
            "copy_us_per_block": copy_s * 1e6, "recompute_us_per_block": rec_s * 1e6,
            "keep": f"{num}/{den}", "keep_ratio": num / den, "kept_blocks_per_seq": sorted(set(ks)),
            "note": "kvsp_budget_keep_ratio with the measured copy bandwidth (256 MiB pinned "
                    "copies) and projection throughput (torch.matmul of one block's K|V "
                    "projection); reported only, the timed step keeps the workload's keep ratio"}


def make_capture(steps):
    """capture(fn) -> a HIP graph holding fn(0..steps-1); timed(graph) -> the
    replay's seconds by HIP events on torch's current stream (the one every
    call below is enqueued on). The kernels reset their own completion
    counters, so the graphs hold kernel nodes only."""
    import torch

    def capture(fn):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn(0)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(steps):
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

    return capture, timed


class Measured:
    """One workload uploaded with its rotating replicas, timed as a step, as
    the attention call alone and as the selection call alone."""

    def __init__(self, name, case, steps, warmup, replicas=0):
        import torch

        from query_aware_sparse_block_amd import device as dev
        self.name, self.case, self.steps = name, case, steps
        dc0 = dev.upload(case)
        self.pool_bytes = dc0.k_pool.numel() * dc0.k_pool.element_size() * 2
        # Distinct device copies (different addresses), taken in turn, so a
        # step never finds in the 256 MB Infinity Cache what an earlier step
        # read: at least 3, so two other replicas' traffic separates two uses
        # of one, and enough for 2 GiB of pools.
        R = replicas or max(3, -(-(2 << 30) // self.pool_bytes))
        self.R = R
        self.reps = [dc0]
        for _ in range(R - 1):
            self.reps.append(dev.DeviceCase(case, dc0.q.clone(), dc0.k_pool.clone(),
                                            dc0.v_pool.clone(), dc0.block_table.clone(),
                                            dc0.ctx_lens.clone(), dc0.layout, dc0.params))
        self.bufs = [dev.alloc_buffers(d) for d in self.reps]
        # Summaries of every replica (step 1, before timing: they are resident
        # between steps); each build is timed on its own.
        build_ev = []
        for d, bf in zip(self.reps, self.bufs):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            dev.build_summaries(d, bf)
            e1.record()
            build_ev.append((e0, e1))
        torch.cuda.synchronize()
        self.build_us = sorted(a.elapsed_time(b) * 1e3 for a, b in build_ev)[len(build_ev) // 2]
        for i in range(warmup):
            dev.decode_step(self.reps[i % R], self.bufs[i % R])
        torch.cuda.synchronize()

    def time_calls(self):
        from query_aware_sparse_block_amd import device as dev
        capture, timed = make_capture(self.steps)
        R, reps, bufs = self.R, self.reps, self.bufs
        self.step_s = timed(capture(lambda i: dev.decode_step(reps[i % R], bufs[i % R])))
        self.attn_s = timed(capture(lambda i: dev.sparse_decode(reps[i % R], bufs[i % R])))
        self.sel_s = timed(capture(lambda i: dev.score_topk(reps[i % R], bufs[i % R])))
        case = self.case
        nsel = bufs[0].num_selected.cpu().numpy()
        self.dense = bufs[0].use_dense.cpu().numpy()
        self.tokens = attended_tokens_per_seq(case, nsel, self.dense)
        self.attn_bytes, self.kv_bytes = attention_bytes(case, self.tokens)
        self.Cs = [max(0, int(L) - case.recent_window) // case.P for L in case.ctx_lens]
        self.score_bytes = scoring_bytes(case, self.Cs)
        return self

    def record(self):
        """The per-workload figures shared by the headline and the configs map."""
        case, k = self.case, self.steps
        attn_us = self.attn_s / k * 1e6
        sel_us = self.sel_s / k * 1e6
        step_us = self.step_s / k * 1e6
        gbps = self.attn_bytes / (attn_us * 1e-6) / 1e9
        step_bytes = self.attn_bytes + self.score_bytes
        bound_us = step_bytes / (HBM_PEAK_GBPS * 1e9) * 1e6
        return {
            "workload": self.name,
            "batch": case.B, "q_heads": case.Hq, "kv_heads": case.Hkv, "head_dim": case.D,
            "dtype": case.dtype, "block": case.P,
            "contexts": sorted(set(int(x) for x in case.ctx_lens)),
            "top_k": case.top_k, "keep": f"{case.keep_num}/{case.keep_den}",
            "keep_floor": case.keep_floor, "recent_window": case.recent_window,
            "gamma": f"{case.gamma_num}/{case.gamma_den}",
            "attended_tokens_per_seq": sorted(set(self.tokens)),
            "dense_sequences": int(self.dense.sum()), "pool_replicas": self.R,
            "steps": k,
            "us_per_step": step_us,
            "steps_per_s": 1e6 / step_us,
            "score_topk_us": sel_us,
            "sparse_decode_us": attn_us,
            "attention_bytes": self.attn_bytes,
            "attention_gbps": gbps,
            "attention_hbm_frac": gbps / HBM_PEAK_GBPS,
            "scoring_bytes": self.score_bytes,
            "scoring_gbps": self.score_bytes / (sel_us * 1e-6) / 1e9,
            "scoring_hbm_frac": self.score_bytes / (sel_us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
            "step_gbps": step_bytes / (step_us * 1e-6) / 1e9,
            "step_us_at_hbm_peak": bound_us,
            "figure_of_merit": ("us_per_step (latency-bound: the step's bytes take "
                                f"{bound_us:.2f} us at 8 TB/s)") if bound_us < LATENCY_BOUND_US
                               else "attention_hbm_frac",
        }


def measure(name, steps, warmup, replicas=0):
    import torch
    print(f"[bench] {name}: generating", file=sys.stderr, flush=True)
    case = workloads()[name]()
    m = Measured(name, case, steps, warmup, replicas).time_calls()
    rec = m.record()
    print(f"[bench] {name}: {rec['us_per_step']:.2f} us/step, attention "
          f"{rec['attention_hbm_frac']:.3f} of HBM", file=sys.stderr, flush=True)
    return m, rec


def host_pool_record(steps, warmup):
    """kvsp_sparse_decode with K/V in mapped pinned host memory (the SparPR
    setting: the cache off the GPU, summaries on it): only the kept blocks
    and the window cross PCIe. A few eager calls on replica 0's selection."""
    import torch

    from query_aware_sparse_block_amd import device as dev
    name = HOST_POOL_WORKLOAD
    print(f"[bench] {name}: decode over a host-resident pool", file=sys.stderr, flush=True)
    case = workloads()[name]()
    m = Measured(name, case, steps, warmup, replicas=1)
    dc0, buf = m.reps[0], m.bufs[0]
    dev.score_topk(dc0, buf)
    hdc = dev.with_host_pool(dc0)
    dev.sparse_decode(hdc, buf)  # warm
    torch.cuda.synchronize()
    n_host = 5
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(n_host):
        dev.sparse_decode(hdc, buf)
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) / n_host * 1e3
    tokens = attended_tokens_per_seq(case, buf.num_selected.cpu().numpy(),
                                     buf.use_dense.cpu().numpy())
    nbytes, _ = attention_bytes(case, tokens)
    gbps = nbytes / (us * 1e-6) / 1e9
    del hdc
    return {"workload": name, "calls": n_host, "decode_us": us, "bytes_per_call": nbytes,
            "pcie_gbps": gbps, "pcie_peak_gbps": PCIE_PEAK_GBPS, "frac": gbps / PCIE_PEAK_GBPS,
            "note": "kvsp_sparse_decode with K/V in mapped pinned host memory (summaries, "
                    "queries and tables in HBM); bytes as the roofline's; PCIe-inclusive, "
                    "never the headline value"}


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
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload records of the configs map")
    ap.add_argument("--config-steps", type=int, default=200,
                    help="steps timed per record of the configs map")
    ap.add_argument("--no-host-pool", action="store_true",
                    help="skip the decode over a host-resident (pinned, mapped) pool")
    ap.add_argument("--no-dkv", action="store_true",
                    help="skip the DKV codec and decode on the 256-token-block workload")
    ap.add_argument("--no-budget", action="store_true",
                    help="skip measuring the budget controller's copy and recompute prices")
    ap.add_argument("--only-dkv", action="store_true",
                    help="run the DKV codec and decode alone and print their record (for "
                         "profiling the DKV kernels on their own)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has "
              "no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch

    from query_aware_sparse_block_amd import device as dev
    from query_aware_sparse_block_amd import kvsp
    from query_aware_sparse_block_amd import profiling

    kvsp.library()
    if args.only_dkv:
        capture, timed = make_capture(args.steps)
        print(json.dumps({"dkv": bench_dkv(args, capture, timed)}), flush=True)
        return
    if args.workload not in workloads():
        sys.exit(f"unknown workload {args.workload}; choose from {sorted(workloads())}")

    # ---- headline: exactly --steps timed steps after --warmup -----------------
    m, head = measure(args.workload, args.steps, args.warmup, args.replicas)
    case = m.case
    E = {"fp32": 4, "fp16": 2, "bf16": 2}[case.dtype]

    # Decode-time append, timed on its own (it precedes scoring in a decode
    # loop): each sequence's newest token is written again with its own K/V
    # rows, so the pools and summaries keep their contents; when the contexts
    # end on a block boundary every call also re-derives that block's summary.
    dc0 = m.reps[0]
    ctx0 = dc0.ctx_lens.long()
    bt0 = dc0.block_table.long()
    last_phys = bt0[torch.arange(case.B, device=bt0.device), (ctx0 - 1) // case.P]
    last_t = (ctx0 - 1) % case.P
    k_last = dc0.k_pool[last_phys, :, last_t].contiguous()
    v_last = dc0.v_pool[last_phys, :, last_t].contiguous()
    pos_last = (ctx0 - 1).to(torch.int32)
    capture, timed = make_capture(args.steps)
    R = m.R
    append_s = timed(capture(lambda i: dev.append_kv(m.reps[i % R], m.bufs[i % R], k_last, v_last,
                                                     pos_last)))
    completes = bool(((ctx0 % case.P) == 0).all().item())

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        big = sum(m.tokens) * case.Hq * case.D > 2e9 or case.B * case.Hq > 512
        cpu = time_cpu_oracle_sampled(case) if big else time_cpu_oracle(case)
        cpu["cores_available"] = os.cpu_count()
        cpu["cpu_model"] = cpu_model()
        # the same oracle with its (sequence, head) loop on the host's thread share
        threads = max(1, int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)))
        if threads > 1:
            mt = (time_cpu_oracle_sampled(case, threads=threads) if big
                  else time_cpu_oracle(case, budget_s=5.0, threads=threads))
            cpu["openmp"] = {k: mt[k] for k in ("value", "unit", "cores", "sample")}
    headline_bytes = (m.attn_bytes, m.kv_bytes, m.build_us)
    del m, dc0, k_last, v_last
    torch.cuda.empty_cache()

    configs = {}
    if not args.no_configs:
        for name in CONFIG_WORKLOADS:
            if name == args.workload:
                continue
            mc, rec = measure(name, args.config_steps, max(args.warmup, 5))
            rec["attention_traffic"] = profiling.recorded_traffic(name)
            rec["scoring_traffic"] = profiling.recorded_traffic(name, kernel="score")
            configs[name] = rec
            del mc
            torch.cuda.empty_cache()

    host_pool = None if args.no_host_pool else host_pool_record(args.config_steps, args.warmup)
    torch.cuda.empty_cache()
    capture, timed = make_capture(args.steps)
    dkv = None if args.no_dkv else bench_dkv(args, capture, timed)
    torch.cuda.empty_cache()
    budget = None if args.no_budget else bench_budget(case)

    attn_bytes, kv_bytes, build_us = headline_bytes
    attn_avg = head["sparse_decode_us"] * 1e-6
    achieved = attn_bytes / attn_avg / 1e9
    rec = {
        "metric": METRIC,
        "value": head["steps_per_s"],
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["us_per_step"] * 1e-3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dtype,
        "data": "synthetic",
        "launch": "hipGraph of all K steps",
        "decode_input": "span list (kvsp_score_topk's spans)",
        "config": {k: head[k] for k in ("workload", "batch", "q_heads", "kv_heads", "head_dim",
                                        "block", "contexts", "top_k", "keep", "keep_floor",
                                        "recent_window", "gamma", "attended_tokens_per_seq",
                                        "dense_sequences", "pool_replicas")},
        "selected_kv_gbps": achieved,
        "selected_kv_hbm_frac": achieved / HBM_PEAK_GBPS,
        "step_gbps": head["step_gbps"],
        "step_gbps_note": "attention bytes (selected K/V, q, table, out) + scoring bytes "
                          "(summaries, q) per step, over the step time",
        "kernels_us": {"score_topk": head["score_topk_us"],
                       "sparse_decode": head["sparse_decode_us"],
                       "step": head["us_per_step"],
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
            "traffic_source": "profiles/traffic_attend_<workload>.txt (rocprofv3 FETCH_SIZE and "
                              "WRITE_SIZE per launch, scaled by a plain copy; null if the decode "
                              "sources changed since)",
        },
        "scoring": {"bytes_per_launch": head["scoring_bytes"], "gbps": head["scoring_gbps"],
                    "hbm_frac": head["scoring_hbm_frac"],
                    "traffic": profiling.recorded_traffic(args.workload, kernel="score"),
                    "note": "kvsp_score_topk: fp32 summary rows of every candidate and the "
                            "queries read; traffic from profiles/traffic_score_<workload>.txt"},
        "summaries": {"us": build_us, "bytes_per_launch": summary_bytes(case),
                      "gbps": summary_bytes(case) / (build_us * 1e-6) / 1e9,
                      "note": "kvsp_build_summaries over every full block, median over replicas"},
        "configs": configs,
        "configs_note": f"each record: {args.config_steps} steps per timed graph over rotating "
                        "pool replicas, timed like the headline",
        "host_pool": host_pool,
        "dkv": dkv,
        "budget": budget,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
