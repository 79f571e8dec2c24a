"""Reference oracle for query-aware sparse block decode attention.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package; the library under
``query_aware_sparse_block_amd`` never does. The arithmetic lives in
``kvsp_oracle.cpp`` (plain C++, IEEE double); this module only builds it with
g++ and marshals numpy arrays through ctypes. Each wrapper names the page and
section its C function follows (see the C source for the full statement).
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvsp_oracle.cpp")
_LIB = os.path.join(_HERE, "libkvsp_oracle.so")

DTYPE_CODE = {"fp32": 0, "fp16": 1, "bf16": 2}

def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with g++ (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-fopenmp", "-Wall", "-Wextra", "-o", tmp, src]
        subprocess.check_call(cmd)
        os.replace(tmp, out)
    return out


def _bind(path: str):
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    L.kvsp_oracle_abi_version.restype = ctypes.c_int
    L.kvsp_oracle_widen.argtypes = [ctypes.c_int, P, i64, P]
    L.kvsp_oracle_plan.argtypes = [i32] * 9 + [P]
    L.kvsp_oracle_block_summary.argtypes = [ctypes.c_int, P, i32, i32, i32, i32, i32, P]
    L.kvsp_oracle_summaries.argtypes = [ctypes.c_int, P, i32, i32, i32, i32, P, i32, P, P]
    L.kvsp_oracle_scores.argtypes = [ctypes.c_int, P, P, i32, i32, i32, i32, P]
    L.kvsp_oracle_topk.argtypes = [P, i32, i32, P]
    L.kvsp_oracle_spans.argtypes = [P, i32, i32, i32, P]
    L.kvsp_oracle_spans.restype = i32
    L.kvsp_oracle_partial.argtypes = [ctypes.c_int, P, P, P, i32, i32, i32, i32, P, P, i32,
                                      f64, P, P, P]
    L.kvsp_oracle_merge.argtypes = [i32, P, P, P, i32, P, P]
    L.kvsp_oracle_attend_tokens.argtypes = [ctypes.c_int, P, P, P, i32, i32, i32, i32, P, P,
                                            i32, f64, P, P]
    L.kvsp_oracle_attended_tokens.argtypes = [i32, i32, i32, P, i32, i32, P]
    L.kvsp_oracle_attended_tokens.restype = i32
    L.kvsp_oracle_append.argtypes = [ctypes.c_int, P, P, i32, i32, i32, P, P, P, i32, P, i32, P,
                                     P]
    L.kvsp_oracle_decode_step.argtypes = ([ctypes.c_int] + [i32] * 6 + [P] * 6 + [i32] * 7
                                          + [f64] + [P] * 8 + [i32])
    return L


_lib = None


def lib():
    """The oracle build that every function below calls. Mutation tests swap
    it (``use_library``) to run the same pins against a modified build."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(_LIB)
    return _lib


def use_library(path):
    """Bind the functions below to another build of the oracle; returns the
    previous binding for ``restore_library``."""
    global _lib
    prev = _lib
    _lib = _bind(path)
    return prev


def restore_library(prev):
    global _lib
    _lib = prev


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def _code(dtype: str) -> int:
    return DTYPE_CODE[dtype]


def widen(dtype: str, raw: np.ndarray) -> np.ndarray:
    """Stored elements (float32 / uint16 bit patterns) -> float64."""
    raw = np.ascontiguousarray(raw)
    out = np.empty(raw.size, np.float64)
    lib().kvsp_oracle_widen(_code(dtype), _p(raw), raw.size, _p(out))
    return out.reshape(raw.shape)


def plan(L, P, W, top_k=0, keep_num=1, keep_den=1, keep_floor=1, gamma_num=1, gamma_den=1):
    """Integer selection plan [SparPR §Three decisions; DKV abstract]:
    returns dict n, C, k_req, k_eff, use_dense."""
    out = np.zeros(5, np.int32)
    lib().kvsp_oracle_plan(L, P, W, top_k, keep_num, keep_den, keep_floor, gamma_num, gamma_den,
                           _p(out))
    return dict(n=int(out[0]), C=int(out[1]), k_req=int(out[2]), k_eff=int(out[3]),
                use_dense=int(out[4]))


def block_summary(dtype, k_pool, Hkv, P, D, phys, g):
    """Mean key of one block for one KV head [SparPR ¶Query-Aware key-block selection]."""
    out = np.empty(D, np.float64)
    lib().kvsp_oracle_block_summary(_code(dtype), _p(k_pool), Hkv, P, D, phys, g, _p(out))
    return out


def summaries(dtype, k_pool, block_table, ctx_lens, Hkv, P, D):
    """Summaries by logical block, [B][max_blocks][Hkv][D] (NaN where not a full block)."""
    B, max_blocks = block_table.shape
    out = np.full((B, max_blocks, Hkv, D), np.nan, np.float64)
    lib().kvsp_oracle_summaries(_code(dtype), _p(k_pool), B, Hkv, P, D, _p(block_table),
                                max_blocks, _p(ctx_lens), _p(out))
    return out


def stored_summaries(summ: np.ndarray) -> np.ndarray:
    """The summaries as the GPU keeps them resident: each double mean rounded
    to the nearest float32, ties to even (the compact per-block summary is
    held in float32 [SparPR ¶Query-Aware key-block selection: summaries stay
    resident on the GPU and scoring reads only them]). Scores are computed
    from these stored values. NaN entries (no full block) stay NaN. The
    rounding is numpy's float64 -> float32 cast, which is IEEE
    round-to-nearest-even."""
    return np.asarray(summ, np.float64).astype(np.float32).astype(np.float64)


def append(dtype, k_pool, v_pool, k_new, v_new, block_table, positions, *, Hkv, P, D):
    """Decode-time append [SparPR opening paragraphs; ¶Query-Aware key-block
    selection]: writes each sequence's new K/V row at token positions[b]
    (skipped when negative) into k_pool / v_pool IN PLACE; returns
    (filled [B][Hkv][D] double, flags [B]) where flags[b] = 1 marks that the
    token completed its block and filled[b] is that block's mean key."""
    B = len(positions)
    assert k_pool.flags["C_CONTIGUOUS"] and v_pool.flags["C_CONTIGUOUS"]
    filled = np.full((B, Hkv, D), np.nan, np.float64)
    flags = np.zeros(B, np.int32)
    lib().kvsp_oracle_append(_code(dtype), _p(k_pool), _p(v_pool), Hkv, P, D,
                             _p(np.ascontiguousarray(k_new)), _p(np.ascontiguousarray(v_new)),
                             _p(np.ascontiguousarray(block_table, np.int32)),
                             block_table.shape[1], _p(np.ascontiguousarray(positions, np.int32)),
                             B, _p(filled), _p(flags))
    return filled, flags


def scores(dtype, q_b, summ_b, Hq, Hkv, D, C):
    """Block relevance scores of one sequence [SparPR ¶Query-Aware key-block selection]."""
    out = np.empty(max(C, 1), np.float64)
    lib().kvsp_oracle_scores(_code(dtype), _p(q_b), _p(np.ascontiguousarray(summ_b)), Hq, Hkv,
                             D, C, _p(out))
    return out[:C]


def topk(score: np.ndarray, k: int) -> np.ndarray:
    """Top-k by (score desc, index asc), ascending ids [SparPR ¶Query-Aware key-block selection]."""
    score = np.ascontiguousarray(score, np.float64)
    out = np.empty(max(k, 1), np.int32)
    lib().kvsp_oracle_topk(_p(score), score.size, k, _p(out))
    return out[:k]


def spans(sel: np.ndarray, C: int, n: int) -> np.ndarray:
    """Span merge of selected ∪ window blocks [SparPR ¶On-demand local recomputation]."""
    sel = np.ascontiguousarray(sel, np.int32)
    out = np.empty((len(sel) + n - C + 1, 2), np.int32)
    cnt = lib().kvsp_oracle_spans(_p(sel), len(sel), C, n, _p(out))
    return out[:cnt].copy()


def partial(dtype, q_h, k_pool, v_pool, Hkv, P, D, g, bt_row, tokens, scale):
    """Partial softmax (m, l, acc) over a token list [DKV abstract]."""
    tokens = np.ascontiguousarray(tokens, np.int32)
    acc = np.empty(D, np.float64)
    m = np.zeros(1, np.float64)
    l = np.zeros(1, np.float64)
    lib().kvsp_oracle_partial(_code(dtype), _p(q_h), _p(k_pool), _p(v_pool), Hkv, P, D, g,
                              _p(np.ascontiguousarray(bt_row, np.int32)), _p(tokens), tokens.size,
                              scale, _p(m), _p(l), _p(acc))
    return float(m[0]), float(l[0]), acc


def merge(ms, ls, accs):
    """Flash-style log-sum-exp merge of partials [DKV abstract]."""
    ms = np.ascontiguousarray(ms, np.float64)
    ls = np.ascontiguousarray(ls, np.float64)
    accs = np.ascontiguousarray(accs, np.float64)
    D = accs.shape[-1]
    out = np.empty(D, np.float64)
    lse = np.zeros(1, np.float64)
    lib().kvsp_oracle_merge(ms.size, _p(ms), _p(ls), _p(accs), D, _p(out), _p(lse))
    return out, float(lse[0])


def attended_tokens(L, P, C, sel, use_dense):
    sel = np.ascontiguousarray(sel, np.int32)
    out = np.empty(max(L, 1), np.int32)
    cnt = lib().kvsp_oracle_attended_tokens(L, P, C, _p(sel) if sel.size else None, sel.size,
                                            int(use_dense), _p(out))
    return out[:cnt].copy()


def attend_tokens(dtype, q_h, k_pool, v_pool, Hkv, P, D, g, bt_row, tokens, scale):
    """Softmax attention of one query head over an explicit token list."""
    tokens = np.ascontiguousarray(tokens, np.int32)
    out = np.empty(D, np.float64)
    lse = np.zeros(1, np.float64)
    lib().kvsp_oracle_attend_tokens(_code(dtype), _p(q_h), _p(k_pool), _p(v_pool), Hkv, P, D, g,
                                    _p(np.ascontiguousarray(bt_row, np.int32)), _p(tokens),
                                    tokens.size, scale, _p(out), _p(lse))
    return out, float(lse[0])


def decode_step(dtype, q, k_pool, v_pool, block_table, ctx_lens, summ, *, Hkv, P, top_k=0,
                keep_num=1, keep_den=1, keep_floor=1, recent_window=0, gamma_num=1,
                gamma_den=1, scale=0.0, head_mask=None, threads=1):
    """Steps 2-5 and the dense fallback for a batch (summaries given);
    ``threads`` > 1 runs the (sequence, head) attentions on that many host
    threads.

    Returns a dict with plan [B][5], scores, sel, spans, nspans, out, lse
    (out/lse NaN where head_mask is 0)."""
    B, Hq, D = q.shape
    max_blocks = block_table.shape[1]
    plan_a = np.zeros((B, 5), np.int32)
    scores_a = np.full((B, max_blocks), np.nan, np.float64)
    sel_a = np.full((B, max_blocks), -1, np.int32)
    spans_a = np.full((B, max_blocks + 1, 2), -1, np.int32)
    nspans_a = np.zeros(B, np.int32)
    out = np.full((B, Hq, D), np.nan, np.float64)
    lse = np.full((B, Hq), np.nan, np.float64)
    mask = None
    if head_mask is not None:
        mask = np.ascontiguousarray(head_mask, np.uint8)
    lib().kvsp_oracle_decode_step(
        _code(dtype), B, Hq, Hkv, D, P, max_blocks, _p(np.ascontiguousarray(q)), _p(k_pool),
        _p(v_pool), _p(np.ascontiguousarray(block_table, np.int32)),
        _p(np.ascontiguousarray(ctx_lens, np.int32)), _p(np.ascontiguousarray(summ)), top_k,
        keep_num, keep_den, keep_floor, recent_window, gamma_num, gamma_den, scale,
        _p(mask) if mask is not None else None, _p(plan_a), _p(scores_a), _p(sel_a), _p(spans_a),
        _p(nspans_a), _p(out), _p(lse), int(threads))
    return dict(plan=plan_a, scores=scores_a, sel=sel_a, spans=spans_a, nspans=nspans_a, out=out,
                lse=lse)
