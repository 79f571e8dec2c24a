"""Pins of the oracle's decode-time append (SparPR page: the cache gains one
token per decoded token, opening paragraphs; a full block has a mean-key
summary, "Three decisions rather than one compression ratio", paragraph
"Query-Aware key-block selection").

Each pin is checked against something the append does not compute itself:
the input rows byte for byte, numpy's mean of independently decoded rows,
and the batch summary function on the final pool."""

import numpy as np

import oracle
from query_aware_sparse_block_amd import workloads as wl


def _rows(rng, B, Hkv, D, dtype):
    return wl.encode(rng.standard_normal((B, Hkv, D)).astype(np.float32), dtype)


def _empty_pool(num_phys, Hkv, P, D, dtype):
    return np.zeros((num_phys, Hkv, P, D), np.float32 if dtype == "fp32" else np.uint16)


def test_filling_a_block_token_by_token(dtype="bf16", Hkv=3, P=16, D=64):
    rng = np.random.default_rng(5)
    table = np.array([[4, 1, 3]], np.int32)  # logical block 1 lives in physical block 1
    kp, vp = _empty_pool(6, Hkv, P, D, dtype), _empty_pool(6, Hkv, P, D, dtype)
    ks, vs = [], []
    for t in range(P):
        k, v = _rows(rng, 1, Hkv, D, dtype), _rows(rng, 1, Hkv, D, dtype)
        ks.append(k[0]), vs.append(v[0])
        filled, flags = oracle.append(dtype, kp, vp, k, v, table, np.array([P + t], np.int32),
                                      Hkv=Hkv, P=P, D=D)
        assert flags[0] == (1 if t == P - 1 else 0)
    # token t of block 1 holds the t-th appended row, for every head
    assert np.array_equal(kp[1], np.stack(ks, axis=1))
    assert np.array_equal(vp[1], np.stack(vs, axis=1))
    # nothing else was touched
    others = [i for i in range(6) if i != 1]
    assert not kp[others].any() and not vp[others].any()
    # the completed block's summary is the mean of its decoded keys
    mean = wl.decode_f32(np.stack(ks, axis=1), dtype).astype(np.float64).mean(axis=1)
    np.testing.assert_allclose(filled[0], mean, rtol=1e-14, atol=1e-15)


def test_filling_a_block_fp16_and_fp32():
    test_filling_a_block_token_by_token("fp16", 2, 4, 64)
    test_filling_a_block_token_by_token("fp32", 1, 16, 128)


def test_negative_position_writes_nothing():
    rng = np.random.default_rng(6)
    kp = wl.encode(rng.standard_normal((4, 2, 16, 64)).astype(np.float32), "fp16")
    vp = kp.copy()
    k0, v0 = kp.copy(), vp.copy()
    filled, flags = oracle.append("fp16", kp, vp, _rows(rng, 2, 2, 64, "fp16"),
                                  _rows(rng, 2, 2, 64, "fp16"), np.array([[0], [1]], np.int32),
                                  np.array([-1, -5], np.int32), Hkv=2, P=16, D=64)
    assert np.array_equal(kp, k0) and np.array_equal(vp, v0)
    assert not flags.any() and np.isnan(filled).all()


def test_batch_append_lands_in_each_sequences_block_and_matches_summaries():
    # three sequences through a shuffled table: one completes a block, one
    # writes mid-block, one has no token this step
    rng = np.random.default_rng(7)
    dtype, Hkv, P, D, max_blocks = "bf16", 2, 16, 64, 4
    table = rng.permutation(12).astype(np.int32).reshape(3, max_blocks)
    kp = wl.encode(rng.standard_normal((12, Hkv, P, D)).astype(np.float32), dtype)
    vp = wl.encode(rng.standard_normal((12, Hkv, P, D)).astype(np.float32), dtype)
    k0, v0 = kp.copy(), vp.copy()
    k, v = _rows(rng, 3, Hkv, D, dtype), _rows(rng, 3, Hkv, D, dtype)
    pos = np.array([2 * P - 1, P + 5, -1], np.int32)
    filled, flags = oracle.append(dtype, kp, vp, k, v, table, pos, Hkv=Hkv, P=P, D=D)
    assert flags.tolist() == [1, 0, 0]
    expect_k, expect_v = k0.copy(), v0.copy()
    expect_k[table[0, 1], :, P - 1], expect_v[table[0, 1], :, P - 1] = k[0], v[0]
    expect_k[table[1, 1], :, 5], expect_v[table[1, 1], :, 5] = k[1], v[1]
    assert np.array_equal(kp, expect_k) and np.array_equal(vp, expect_v)
    # the filled summary is the batch summary of that block on the new pool
    summ = oracle.summaries(dtype, kp, table, np.array([2 * P, 0, 0], np.int32), Hkv, P, D)
    assert np.array_equal(filled[0], summ[0, 1])
