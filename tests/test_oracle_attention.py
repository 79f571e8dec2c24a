"""Pins for the oracle's attention (DKV abstract: exact recency window and
flash-style log-sum-exp merge; SparPR news page, On-demand local
recomputation with cost-aware fallback: the dense path; "KV cache
offloading", Why the cache leaves the GPU: dense decode reads every key and
value).

1. At 100 % keep the sparse result equals a textbook dense softmax written
   here in numpy over keys gathered in token order.
2. Merging the partials of any partition of the token set equals the single
   pass, in any merge order, with empty and singleton parts.
3. Exact special cases: one token gives V; equal logits give the mean of V;
   shuffling the physical pool changes nothing."""

import numpy as np
import pytest

import oracle
from query_aware_sparse_block_amd import workloads as wl


def _dense_numpy(case, b, h, scale):
    """Textbook softmax attention over all L tokens of sequence b, keys and
    values gathered in token order (no blocks, no table after the gather)."""
    L = int(case.ctx_lens[b])
    G = case.Hq // case.Hkv
    g = h // G
    t = np.arange(L)
    phys = case.block_table[b, t // case.P]
    K = wl.decode_f32(case.k_pool[phys, g, t % case.P], case.dtype).astype(np.float64)
    V = wl.decode_f32(case.v_pool[phys, g, t % case.P], case.dtype).astype(np.float64)
    q = wl.decode_f32(case.q[b, h], case.dtype).astype(np.float64)
    z = scale * (K @ q)
    w = np.exp(z - z.max())
    return (w @ V) / w.sum(), z.max() + np.log(w.sum())


def _summ(case):
    return oracle.summaries(case.dtype, case.k_pool, case.block_table, case.ctx_lens, case.Hkv,
                            case.P, case.D)


def _run(case, **over):
    params = dict(case.select_params)
    params.update(over)
    return oracle.decode_step(case.dtype, case.q, case.k_pool, case.v_pool, case.block_table,
                              case.ctx_lens, _summ(case), Hkv=case.Hkv, P=case.P, **params)


@pytest.mark.parametrize("dtype,Hq,Hkv,P,L,W", [
    ("fp32", 8, 8, 16, 1024, 32),
    ("fp16", 4, 2, 16, 333, 40),
    ("bf16", 6, 2, 64, 640, 0),
])
def test_full_keep_equals_textbook_dense(dtype, Hq, Hkv, P, L, W):
    case = wl.make_case("full", seed=7, B=2, Hq=Hq, Hkv=Hkv, D=64, P=P, dtype=dtype,
                        ctx_lens=[L, L - 17], shuffle=True, num_phys=2 * (-(-L // P)) + 5,
                        top_k=10 ** 6, keep_floor=1, recent_window=W)
    r = _run(case)
    scale = 1.0 / np.sqrt(case.D)
    for b in range(case.B):
        assert r["plan"][b, 3] == r["plan"][b, 1]          # k_eff == C
        for h in range(case.Hq):
            o, lse = _dense_numpy(case, b, h, scale)
            np.testing.assert_allclose(r["out"][b, h], o, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(r["lse"][b, h], lse, rtol=1e-12)


def test_dense_fallback_equals_textbook_dense():
    case = wl.c1("gamma")
    r = _run(case)
    assert r["plan"][0, 4] == 1
    for h in range(case.Hq):
        o, lse = _dense_numpy(case, 0, h, 1.0 / 8.0)
        np.testing.assert_allclose(r["out"][0, h], o, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_lse_merge_partition_invariance(seed):
    rng = np.random.default_rng(seed)
    case = wl.make_case("merge", seed=100 + seed, B=1, Hq=2, Hkv=1, D=32, P=8, dtype="bf16",
                        ctx_lens=[200], shuffle=True, num_phys=30)
    tokens = rng.permutation(200).astype(np.int32)[: int(rng.integers(1, 201))]
    scale = 0.3
    full_o, full_lse = oracle.attend_tokens("bf16", case.q[0, 1], case.k_pool, case.v_pool, 1,
                                            8, 32, 0, case.block_table[0], tokens, scale)
    for nparts in (1, 2, 7, 64):
        cuts = np.sort(rng.integers(0, len(tokens) + 1, nparts - 1))
        parts = np.split(tokens, cuts)          # includes empty parts when cuts repeat
        parts.append(np.array([], np.int32))    # always one explicit empty part
        ms, ls, accs = [], [], []
        for p in parts:
            m, l, acc = oracle.partial("bf16", case.q[0, 1], case.k_pool, case.v_pool, 1, 8, 32,
                                       0, case.block_table[0], p, scale)
            if len(p) == 0:
                assert m == -np.inf and l == 0.0 and not acc.any()
            ms.append(m), ls.append(l), accs.append(acc)
        for order in (np.arange(len(parts)), rng.permutation(len(parts))):
            o, lse = oracle.merge(np.array(ms)[order], np.array(ls)[order],
                                  np.array(accs)[order])
            np.testing.assert_allclose(o, full_o, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(lse, full_lse, rtol=1e-12)


def test_merge_all_empty():
    o, lse = oracle.merge(np.array([-np.inf, -np.inf]), np.zeros(2), np.zeros((2, 4)))
    assert lse == -np.inf and not o.any()


def test_single_token_gives_value_exactly():
    case = wl.make_case("one", seed=8, B=1, Hq=2, Hkv=2, D=16, P=4, dtype="fp16",
                        ctx_lens=[12])
    for t in range(12):
        o, lse = oracle.attend_tokens("fp16", case.q[0, 1], case.k_pool, case.v_pool, 2, 4, 16,
                                      1, case.block_table[0], np.array([t]), 0.25)
        v = oracle.widen("fp16", case.v_pool[case.block_table[0, t // 4], 1, t % 4])
        assert np.array_equal(o, v)
        k = oracle.widen("fp16", case.k_pool[case.block_table[0, t // 4], 1, t % 4])
        q = oracle.widen("fp16", case.q[0, 1])
        assert lse == pytest.approx(0.25 * float(np.dot(q, k)), rel=1e-15)


def test_equal_logits_give_mean_of_values():
    rng = np.random.default_rng(9)
    k_pool = np.ones((6, 1, 4, 8), np.float32)          # every key identical
    v_pool = (rng.integers(-16, 17, (6, 1, 4, 8)) / 8.0).astype(np.float32)
    q = rng.standard_normal(8).astype(np.float32)
    bt = np.array([3, 1, 5, 0, 2, 4], np.int32)
    tokens = np.array([0, 1, 5, 9, 10, 11, 22, 23], np.int32)
    o, lse = oracle.attend_tokens("fp32", q, k_pool, v_pool, 1, 4, 8, 0, bt, tokens, 0.5)
    V = np.stack([v_pool[bt[t // 4], 0, t % 4] for t in tokens]).astype(np.float64)
    np.testing.assert_allclose(o, V.mean(0), rtol=0, atol=1e-15)
    z = 0.5 * float(q.astype(np.float64).sum())
    assert lse == pytest.approx(z + np.log(len(tokens)), rel=1e-14)


def test_physical_shuffle_changes_nothing():
    a = wl.c1("k8")
    r0 = _run(a)
    # same logical data, scattered over a larger pool through a permutation
    rng = np.random.default_rng(10)
    num_phys = 100
    perm = rng.permutation(num_phys)[: a.max_blocks].astype(np.int32)
    k2 = np.zeros((num_phys,) + a.k_pool.shape[1:], a.k_pool.dtype)
    v2 = np.zeros_like(k2)
    k2[perm] = a.k_pool[a.block_table[0]]
    v2[perm] = a.v_pool[a.block_table[0]]
    b = wl.Case(**{**a.__dict__, "k_pool": k2, "v_pool": v2, "block_table": perm[None].copy()})
    r1 = _run(b)
    for key in ("sel", "spans", "nspans", "out", "lse", "plan"):
        assert np.array_equal(r0[key], r1[key], equal_nan=True), key


def test_head_mask_limits_work():
    case = wl.c1("k8")
    mask = np.zeros((1, 8), np.uint8)
    mask[0, 3] = 1
    r = oracle.decode_step(case.dtype, case.q, case.k_pool, case.v_pool, case.block_table,
                           case.ctx_lens, _summ(case), Hkv=8, P=16, head_mask=mask,
                           **case.select_params)
    full = _run(case)
    assert np.array_equal(r["out"][0, 3], full["out"][0, 3])
    assert np.isnan(r["out"][0, 2]).all()


def test_empty_sequence_step():
    # a sequence with no cached token: no candidate, nothing selected, no
    # span, and attention over the empty set gives out = 0, lse = -inf
    # (the empty-merge convention pinned above)
    case = wl.make_case("empty-oracle", seed=11, B=2, Hq=2, Hkv=1, D=64, P=16, dtype="fp32",
                        ctx_lens=[0, 40], max_blocks=3, top_k=1, keep_floor=1, recent_window=8)
    summ = oracle.summaries(case.dtype, case.k_pool, case.block_table, case.ctx_lens, 1, 16, 64)
    r = oracle.decode_step(case.dtype, case.q, case.k_pool, case.v_pool, case.block_table,
                           case.ctx_lens, summ, Hkv=1, P=16, **case.select_params)
    assert r["plan"][0].tolist() == [0, 0, 1, 0, 0]
    assert r["nspans"][0] == 0
    assert not r["out"][0].any() and np.isneginf(r["lse"][0]).all()
    assert np.isfinite(r["lse"][1]).all()


def test_threaded_decode_step_is_bit_identical():
    """Spreading the (sequence, head) attentions over host threads changes no
    result: every output of the step equals the single-threaded one."""
    case = wl.c2(L=1024, keep="1/10")
    summ = oracle.summaries(case.dtype, case.k_pool, case.block_table, case.ctx_lens, case.Hkv,
                            case.P, case.D)
    args = (case.dtype, case.q, case.k_pool, case.v_pool, case.block_table, case.ctx_lens, summ)
    one = oracle.decode_step(*args, Hkv=case.Hkv, P=case.P, threads=1, **case.select_params)
    many = oracle.decode_step(*args, Hkv=case.Hkv, P=case.P, threads=4, **case.select_params)
    for key in one:
        assert np.array_equal(one[key], many[key], equal_nan=True), key
