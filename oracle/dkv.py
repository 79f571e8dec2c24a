"""Reference oracle for the DKV block codec and its decode, plain numpy float64.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module; the library under
``query_aware_sparse_block_amd`` never does.

Source: "DKV: Anchor + Low-Rank Differential KV-Cache Compression for Scalable
Long-Context Inference", abstract. In short:
- an older block keeps one token exactly (the anchor);
- the other tokens are stored as a rank-32 truncated SVD of their joint
  key|value difference from the anchor;
- a budget of whole tokens is also kept exactly: those whose rows the low-rank
  basis reconstructs worst;
- decoding routes the query to the top-K blocks, attends the compressed
  tokens through the low-rank factors and the residual and recent tokens
  exactly, and merges the two halves by log-sum-exp.

Readings taken where the abstract is silent:
- the anchor is the block's first token;
- the SVD is taken of X = [K - k_anchor | V - v_anchor] (P x 2D), without
  further centring or scaling;
- residual tokens are the n_resid rows of largest Euclidean reconstruction
  error ||X_t - X_hat_t||, ties to the lower token index; the basis is not
  refitted after they are removed;
- "routes to the top-K relevant blocks" uses the same block summaries, scores
  and Top-k as the main path, so this module only decodes a given selection;
- a log-sum-exp merge of partial softmaxes over disjoint token sets equals
  softmax attention over their union, so ``decode`` evaluates that union
  directly: every compressed token is decompressed explicitly (k_a + c_t W_K,
  v_a + c_t W_V), every residual and window token is taken exactly.

Where the exact SVD has repeated singular values at the cut, the truncated
subspace is not unique; the pins and parity tests use blocks with a gap there.
"""

from __future__ import annotations

import numpy as np


def block_delta(K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """X = [K - k_anchor | V - v_anchor] for one block (anchor = token 0)."""
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    return np.concatenate([K - K[0], V - V[0]], axis=1)


def compress_block(K: np.ndarray, V: np.ndarray, rank: int, n_resid: int) -> dict:
    """Codec of one (block, KV head): K, V are the block's exact [P][D] rows.

    Returns float64 fields:
      anchor_k, anchor_v  [D]      exact first-token rows
      basis               [r][2D]  top-r right singular vectors of X (rows)
      coef                [P][r]   X projected on the basis (= U_r * S_r)
      resid               [R]      ascending token offsets kept exactly
      resid_k, resid_v    [R][D]   their exact rows
      err                 [P]      ||X_t - coef_t basis|| (for the pins)
    """
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    P, D = K.shape
    X = block_delta(K, V)
    _, _, vt = np.linalg.svd(X, full_matrices=False)
    r_eff = min(rank, vt.shape[0])
    basis = np.zeros((rank, 2 * D))
    basis[:r_eff] = vt[:r_eff]
    coef = X @ basis.T
    err = np.linalg.norm(X - coef @ basis, axis=1)
    n_resid = min(n_resid, P)
    # largest error first, lower index first among equal errors
    order = sorted(range(P), key=lambda t: (-err[t], t))
    resid = np.array(sorted(order[:n_resid]), np.int64)
    return dict(anchor_k=K[0].copy(), anchor_v=V[0].copy(), basis=basis, coef=coef,
                resid=resid, resid_k=K[resid].copy(), resid_v=V[resid].copy(), err=err)


def reconstruct_block(rec: dict, P: int) -> tuple[np.ndarray, np.ndarray]:
    """The K and V rows the decode attends for a compressed block: each token
    decompressed from the anchor and the low-rank factors, residual tokens
    replaced by their exact rows."""
    D = rec["anchor_k"].shape[0]
    basis = np.asarray(rec["basis"], np.float64)
    coef = np.asarray(rec["coef"], np.float64)
    X_hat = coef[:P] @ basis
    K = rec["anchor_k"][None, :] + X_hat[:, :D]
    V = rec["anchor_v"][None, :] + X_hat[:, D:]
    resid = np.asarray(rec["resid"], np.int64)
    K[resid] = rec["resid_k"]
    V[resid] = rec["resid_v"]
    return K, V


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Softmax attention of one query over explicit rows; returns (out, lse)
    with lse the natural log of the normaliser of the scaled logits."""
    if K.shape[0] == 0:
        return np.zeros(V.shape[1]), -np.inf
    z = scale * (K @ q)
    m = z.max()
    e = np.exp(z - m)
    l = e.sum()
    return (e @ V) / l, m + np.log(l)


def window_start(L: int, P: int, W: int) -> int:
    """First window block: C = floor(max(0, L - W) / P)."""
    return max(0, L - W) // P


def decode(q, k_pool, v_pool, records, block_table, ctx_lens, selected, num_selected, *, Hkv,
           P, recent_window, scale):
    """DKV decode for a batch.

    q [B][Hq][D], pools [phys][Hkv][P][D] (float arrays of the stored values),
    records[(phys, g)] -> dict as from ``compress_block`` (values as stored),
    selected [B][*] ascending logical block ids (< C_b), num_selected [B].
    Attended set of sequence b: every token of each selected (compressed)
    block, then the exact window tokens [C_b * P, L_b).
    Returns out [B][Hq][D] and lse [B][Hq] (float64)."""
    q = np.asarray(q, np.float64)
    B, Hq, D = q.shape
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        L = int(ctx_lens[b])
        C = window_start(L, P, recent_window)
        n = -(-L // P)
        for g in range(Hkv):
            Ks, Vs = [], []
            for j in list(selected[b][: int(num_selected[b])]):
                Kb, Vb = reconstruct_block(records[(int(block_table[b][j]), g)], P)
                Ks.append(Kb)
                Vs.append(Vb)
            for j in range(C, n):
                phys = int(block_table[b][j])
                cnt = min(P, L - j * P)
                Ks.append(np.asarray(k_pool[phys, g, :cnt], np.float64))
                Vs.append(np.asarray(v_pool[phys, g, :cnt], np.float64))
            Kall = np.concatenate(Ks) if Ks else np.zeros((0, D))
            Vall = np.concatenate(Vs) if Vs else np.zeros((0, D))
            for h in range(g * G, (g + 1) * G):
                out[b, h], lse[b, h] = attend(q[b, h], Kall, Vall, scale)
    return out, lse


def compress_case(k_pool, v_pool, block_table, ctx_lens, *, Hkv, P, recent_window, rank,
                  n_resid) -> dict:
    """Codec of every block wholly older than the window (j < C_b), keyed by
    (physical block, KV head)."""
    recs = {}
    for b in range(len(ctx_lens)):
        C = window_start(int(ctx_lens[b]), P, recent_window)
        for j in range(C):
            phys = int(block_table[b][j])
            for g in range(Hkv):
                recs[(phys, g)] = compress_block(k_pool[phys, g], v_pool[phys, g], rank,
                                                 n_resid)
    return recs
