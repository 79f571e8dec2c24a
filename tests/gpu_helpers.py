"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
and the oracle on the same seeded inputs, and compare them.

Bars (written here once, used by every parity test):
  * summaries: bit-identical to the oracle's stored summaries (the double
    mean rounded to the nearest float32; the GPU sums in double and rounds
    once, and for these inputs the double sums are exact);
  * scores: the oracle scores from those stored summaries in double; a GPU
    score (double sums rounded once to float32) must lie within half a
    float32 ulp of it plus 4e-12 * T_j, where T_j = sum_h sum_d |q_h,d| *
    |s_j,g(h),d| bounds the rounding of the double sums on either side;
  * selection: bit-exact, except that where an oracle score lies within
    tau = 1e-6 * |s_(k)| + 4e-12 * max_j T_j of the k-th score s_(k) either
    choice is accepted; the GPU's set must hold every block above the band,
    none below it, and exactly k blocks. Where the sets differ, outputs are
    compared with the oracle recomputed on the GPU's set;
  * selection against the GPU's own float32 scores: exactly their k largest,
    equal scores (+0 and -0 alike) taken in ascending block order;
  * spans, counts and the dense flag: exact (spans of the GPU's own set);
  * the decode given the span list and given the selected list: the same
    outputs bit for bit (every sparse run does both);
  * outputs: max-abs error <= 2e-3 for fp16/bf16 caches and <= 1e-5 for fp32
    caches (float32 accumulation); lse within 1e-4.
"""

from __future__ import annotations

import os
import sys

import numpy as np
import torch

import oracle
from query_aware_sparse_block_amd import device as dev
from query_aware_sparse_block_amd import workloads as wl

OUT_TOL = {"fp32": 1e-5, "fp16": 2e-3, "bf16": 2e-3}
LSE_TOL = 1e-4
BAND_REL = 1e-6
SUM_REL = 4e-12   # rounding of double sums of up to 2^14 terms, relative to sum |terms|


def oracle_threads() -> int:
    """Host threads for the oracle's (sequence, head) attentions: the
    runner's thread share where it is set, else every core."""
    return max(1, int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1))


def note(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def oracle_summaries(case: wl.Case):
    """The oracle's stored summaries (float32-rounded means, held as double)
    by logical block; NaN where a block is not full."""
    return oracle.stored_summaries(
        oracle.summaries(case.dtype, case.k_pool, case.block_table, case.ctx_lens, case.Hkv,
                         case.P, case.D))


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
        # the same kept blocks handed over as the selected list: bit-identical
        out_sel = torch.full_like(buf.out, float("nan"))
        dev.sparse_decode(dc, buf, params, form="selected", out=out_sel)
    torch.cuda.synchronize()
    if not dense_api:
        assert torch.equal(out_sel, buf.out), "span and selected forms of the decode differ"
    res = {k: getattr(buf, k).cpu().numpy() for k in
           ("summaries", "scores", "selected", "num_selected", "spans", "num_spans", "use_dense",
            "out", "lse")}
    return res, dc, buf


def check_summaries(case: wl.Case, gpu_summ: np.ndarray, summ: np.ndarray):
    """GPU summaries of every full block against the oracle's stored ones, bit for bit."""
    for b in range(case.B):
        full = int(case.ctx_lens[b]) // case.P
        phys = case.block_table[b, :full]
        ref = summ[b, :full]
        got = gpu_summ[phys].astype(np.float64)
        if not np.array_equal(got, ref):
            bad = np.argwhere(got != ref)[0]
            raise AssertionError(f"summary differs at b={b} block/head/d={bad.tolist()}: "
                                 f"{got[tuple(bad)]!r} vs {ref[tuple(bad)]!r}")


def term_sums(case: wl.Case, summ: np.ndarray) -> np.ndarray:
    """T[b][j] = sum_h sum_d |q[b][h][d]| * |s[b][j][g(h)][d]| for every
    candidate (NaN-free where the summary exists): the size of the terms
    the scores sum, which bounds the rounding of those sums."""
    G = case.Hq // case.Hkv
    qa = np.abs(oracle.widen(case.dtype, case.q))                         # [B][Hq][D]
    qa = qa.reshape(case.B, case.Hkv, G, case.D).sum(axis=2)               # [B][Hkv][D]
    sa = np.abs(np.nan_to_num(summ, nan=0.0))                               # [B][mb][Hkv][D]
    return np.einsum("bjgd,bgd->bj", sa, qa)


def check_selection(case, r_or, gpu, b, T=None):
    """Band test for sequence b (T: term_sums of the case); returns the GPU's
    selected set."""
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
        floor = SUM_REL * float(T[b, :C].max()) if T is not None else 0.0
        tau = BAND_REL * abs(s_k) + floor
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


def check_scores(case, r_or, gpu, T):
    for b in range(case.B):
        C = int(r_or["plan"][b][1])
        if C == 0:
            continue
        ref = r_or["scores"][b, :C]
        got = gpu["scores"][b, :C].astype(np.float64)
        mag = np.maximum(np.abs(got), np.abs(ref)).astype(np.float32)
        tol = 0.5 * np.spacing(mag).astype(np.float64) + SUM_REL * T[b, :C]
        err = np.abs(got - ref)
        if not np.all(err <= tol):
            j = int(np.argmax(err - tol))
            raise AssertionError(f"b={b} j={j}: score {got[j]!r} vs oracle {ref[j]!r} "
                                 f"(tolerance {tol[j]:.3e})")


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


def full_parity(case: wl.Case, head_mask=None, check_all_summaries=True, summ=None,
                threads=None):
    """Run both sides on `case` and apply every bar above. `summ` may hold the
    oracle's stored summaries already; `threads` sets the oracle's host
    threads (default: oracle_threads())."""
    note(f"[parity] {case.name} B={case.B} Hq={case.Hq} Hkv={case.Hkv} D={case.D} P={case.P} "
         f"{case.dtype} ctx={case.ctx_lens.tolist()[:8]}")
    gpu, _, _ = run_gpu(case)
    if summ is None:
        summ = oracle_summaries(case)
    if check_all_summaries:
        check_summaries(case, gpu["summaries"], summ)
    r_or = oracle.decode_step(case.dtype, case.q, case.k_pool, case.v_pool, case.block_table,
                              case.ctx_lens, summ, Hkv=case.Hkv, P=case.P, head_mask=head_mask,
                              threads=threads or oracle_threads(), **case.select_params)
    T = term_sums(case, summ)
    check_scores(case, r_or, gpu, T)
    for b in range(case.B):
        sel_g = check_selection(case, r_or, gpu, b, T)
        heads = None
        if head_mask is not None:
            heads = np.nonzero(head_mask[b])[0].tolist()
            if not heads:
                continue
        check_outputs(case, r_or, gpu, b, sel_g, heads)
    return gpu, r_or
