"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
and the oracle on the same seeded inputs, and compare them.

Bars (written here once, used by every parity test):
  * summaries: within one float32 ulp of the oracle's double mean (the GPU
    rounds an exact sum once);
  * selection: bit-exact, except that where an oracle score lies within
    tau = 1e-6 * max(|s_(k)|, max_j |score_j|) of the k-th score s_(k) either
    choice is accepted; the GPU's set must hold every block above the band,
    none below it, and exactly k blocks. Where the sets differ, outputs are
    compared with the oracle recomputed on the GPU's set;
  * selection against the GPU's own float32 scores: exactly their k largest,
    equal scores (+0 and -0 alike) taken in ascending block order;
  * spans, counts and the dense flag: exact (spans of the GPU's own set);
  * outputs: max-abs error <= 2e-3 for fp16/bf16 caches and <= 1e-5 for fp32
    caches (float32 accumulation); lse within 1e-4.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from query_aware_sparse_block_amd import device as dev
from query_aware_sparse_block_amd import workloads as wl

OUT_TOL = {"fp32": 1e-5, "fp16": 2e-3, "bf16": 2e-3}
LSE_TOL = 1e-4
BAND_REL = 1e-6


def note(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def oracle_summaries(case: wl.Case):
    return oracle.summaries(case.dtype, case.k_pool, case.block_table, case.ctx_lens, case.Hkv,
                            case.P, case.D)


def run_gpu(case: wl.Case, *, dense_api=False, params=None):
    """Summaries, selection and attention on the GPU; returns host arrays."""
    dc = dev.upload(case)
    buf = dev.alloc_buffers(dc)
    dev.build_summaries(dc, buf)
    if dense_api:
        dev.dense_decode(dc, buf)
    else:
        dev.score_topk(dc, buf, params)
        dev.sparse_decode(dc, buf, params)
    torch.cuda.synchronize()
    res = {k: getattr(buf, k).cpu().numpy() for k in
           ("summaries", "scores", "selected", "num_selected", "spans", "num_spans", "use_dense",
            "out", "lse")}
    return res, dc, buf


def check_summaries(case: wl.Case, gpu_summ: np.ndarray, summ: np.ndarray):
    for b in range(case.B):
        full = int(case.ctx_lens[b]) // case.P
        phys = case.block_table[b, :full]
        ref = summ[b, :full]
        got = gpu_summ[phys].astype(np.float64)
        ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
        err = np.abs(got - ref)
        assert np.all(err <= ulp + 1e-30), f"summary off by {float((err / ulp).max())} ulp (b={b})"


def check_selection(case, r_or, gpu, b):
    """Band test for sequence b; returns the GPU's selected set."""
    plan = r_or["plan"][b]
    C, k = int(plan[1]), int(plan[3])
    assert int(gpu["num_selected"][b]) == k, (b, gpu["num_selected"][b], k)
    assert int(gpu["use_dense"][b]) == int(plan[4])
    sel_g = gpu["selected"][b, :k].astype(np.int64)
    sel_o = r_or["sel"][b, :k].astype(np.int64)
    assert np.all(np.diff(sel_g) > 0) and (k == 0 or (sel_g[0] >= 0 and sel_g[-1] < C))
    # the Top-k rule on the GPU's own scores: a stable descending sort keeps
    # equal scores in index order, so its first k are the lowest-index ties
    own = gpu["scores"][b, :C].astype(np.float64)
    expect = np.sort(np.argsort(-own, kind="stable")[:k])
    assert np.array_equal(sel_g, expect), f"b={b}: not the k best of its own scores"
    if not np.array_equal(sel_g, sel_o):
        score = r_or["scores"][b, :C]
        s_k = np.sort(score)[::-1][k - 1]
        tau = BAND_REL * max(abs(s_k), float(np.abs(score).max()))
        must = set(np.nonzero(score > s_k + tau)[0].tolist())
        never = set(np.nonzero(score < s_k - tau)[0].tolist())
        gs = set(sel_g.tolist())
        assert must <= gs, f"b={b}: GPU dropped blocks above the band"
        assert not (gs & never), f"b={b}: GPU kept blocks below the band"
    # spans of the GPU's own selection
    n = int(plan[0])
    sp_ref = oracle.spans(sel_g.astype(np.int32), C, n)
    nsp = int(gpu["num_spans"][b])
    assert nsp == len(sp_ref), (b, nsp, len(sp_ref))
    assert np.array_equal(gpu["spans"][b, :nsp], sp_ref)
    return sel_g


def check_scores(case, r_or, gpu):
    for b in range(case.B):
        C = int(r_or["plan"][b][1])
        if C == 0:
            continue
        ref = r_or["scores"][b, :C]
        got = gpu["scores"][b, :C].astype(np.float64)
        tol = BAND_REL * float(np.abs(ref).max()) + 1e-30
        assert np.max(np.abs(got - ref)) <= tol, (b, float(np.max(np.abs(got - ref))), tol)


def oracle_attention_on(case, b, sel, dense, heads=None, scale=0.0):
    """Oracle attention of sequence b over a given selection."""
    L = int(case.ctx_lens[b])
    plan = oracle.plan(L, case.P, case.recent_window, case.top_k, case.keep_num, case.keep_den,
                       case.keep_floor, case.gamma_num, case.gamma_den)
    toks = oracle.attended_tokens(L, case.P, plan["C"], np.asarray(sel, np.int32), dense)
    sc = scale if scale > 0 else 1.0 / np.sqrt(case.D)
    G = case.Hq // case.Hkv
    outs, lses = {}, {}
    for h in (range(case.Hq) if heads is None else heads):
        o, l = oracle.attend_tokens(case.dtype, case.q[b, h], case.k_pool, case.v_pool, case.Hkv,
                                    case.P, case.D, h // G, case.block_table[b], toks, sc)
        outs[h], lses[h] = o, l
    return outs, lses


def check_outputs(case, r_or, gpu, b, sel_g, heads=None):
    tol = OUT_TOL[case.dtype]
    dense = int(r_or["plan"][b][4])
    same = np.array_equal(sel_g, r_or["sel"][b, :len(sel_g)])
    hs = list(range(case.Hq)) if heads is None else list(heads)
    if same and not np.isnan(r_or["out"][b, hs[0]]).any():
        ref_out = {h: r_or["out"][b, h] for h in hs}
        ref_lse = {h: r_or["lse"][b, h] for h in hs}
    else:
        ref_out, ref_lse = oracle_attention_on(case, b, sel_g, dense, hs)
    for h in hs:
        err = float(np.max(np.abs(gpu["out"][b, h].astype(np.float64) - ref_out[h])))
        assert err <= tol, f"b={b} h={h}: max-abs {err:.3e} > {tol}"
        g_lse, r_lse = float(gpu["lse"][b, h]), float(ref_lse[h])
        if np.isneginf(r_lse):  # nothing attended (an empty sequence): out = 0, lse = -inf
            assert np.isneginf(g_lse), f"b={b} h={h}: lse {g_lse} for an empty sequence"
            continue
        lerr = abs(g_lse - r_lse)
        assert lerr <= LSE_TOL, f"b={b} h={h}: lse off by {lerr:.3e}"


def full_parity(case: wl.Case, head_mask=None, check_all_summaries=True):
    """Run both sides on `case` and apply every bar above."""
    note(f"[parity] {case.name} B={case.B} Hq={case.Hq} Hkv={case.Hkv} D={case.D} P={case.P} "
         f"{case.dtype} ctx={case.ctx_lens.tolist()[:8]}")
    gpu, _, _ = run_gpu(case)
    summ = oracle_summaries(case)
    if check_all_summaries:
        check_summaries(case, gpu["summaries"], summ)
    r_or = oracle.decode_step(case.dtype, case.q, case.k_pool, case.v_pool, case.block_table,
                              case.ctx_lens, summ, Hkv=case.Hkv, P=case.P, head_mask=head_mask,
                              **case.select_params)
    check_scores(case, r_or, gpu)
    for b in range(case.B):
        sel_g = check_selection(case, r_or, gpu, b)
        heads = None
        if head_mask is not None:
            heads = np.nonzero(head_mask[b])[0].tolist()
            if not heads:
                continue
        check_outputs(case, r_or, gpu, b, sel_g, heads)
    return gpu, r_or
