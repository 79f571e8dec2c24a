"""Synthetic inputs: determinism, shapes, value recipes, and the byte
accounting the benchmark uses, pinned to the worked example printed on the
"KV cache offloading" page (section "Why the cache leaves the GPU")."""

import json
import os

import numpy as np

import oracle
from query_aware_sparse_block_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kv_cache_worked_example.json")


def test_bytes_per_token_worked_example():
    g = json.load(open(GOLDEN))
    m = g["minicpm41_8b"]
    per_tok = wl.kv_bytes_per_token(m["layers"], m["kv_heads"], m["head_dim"], m["elem_bytes"])
    assert per_tok == g["bytes_per_token"]
    assert per_tok * g["tokens_one_sequence"] == g["bytes_one_sequence_gib"] * 2 ** 30
    assert per_tok * g["tokens_one_sequence"] * g["batch"] == g["bytes_batch_gib"] * 2 ** 30
    o = g["opt13b"]
    opt = wl.kv_bytes_per_token(o["layers"], o["kv_heads"], o["head_dim"], o["elem_bytes"])
    assert abs(opt / 1000 - o["approx_kb_per_token"]) / o["approx_kb_per_token"] < 0.05
    assert abs(opt / per_tok - o["ratio_vs_minicpm"]) < 0.1
    total = g["bytes_one_sequence_gib"] * 2 ** 30
    assert round(total / g["h100_hbm_bytes_per_s"] * 1e3, 1) == g["dense_read_ms_hbm_approx"]
    assert round(total / g["pcie_one_direction_bytes_per_s"] * 1e3) == g["dense_read_ms_pcie_approx"]


def test_generation_is_deterministic_and_chunk_parallel_safe():
    a = wl.c5(B=2, L=2048, workers=1)
    b = wl.c5(B=2, L=2048, workers=8)
    for key in ("q", "k_pool", "v_pool", "block_table", "ctx_lens"):
        assert np.array_equal(getattr(a, key), getattr(b, key))
    c = wl.c5(B=2, L=2048, seed=1)
    assert not np.array_equal(a.k_pool, c.k_pool)


def test_shapes_and_tables():
    c = wl.c5(B=4, L=4096)
    assert c.k_pool.shape == (4 * 64, 8, 64, 128) and c.k_pool.dtype == np.uint16
    assert sorted(c.block_table.reshape(-1).tolist()) == list(range(256))
    assert c.block_table.tolist() != np.arange(256).reshape(4, 64).tolist()
    t = wl.c1()
    assert t.k_pool.dtype == np.float32 and t.block_table.tolist() == [list(range(64))]


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1e-3], np.float32)
    bits = wl.f32_to_bf16_bits(x)
    assert bits.tolist()[:2] == [0x3F80, 0x3F80]           # tie -> even
    assert bits.tolist()[2] == 0x3F82                       # tie -> even (up)
    back = oracle.widen("bf16", bits)
    assert np.all(np.abs(back - x) <= np.abs(x) * 2 ** -8)


def test_needles_stand_out():
    c = wl.c2(L=1024, B=2, H=4)
    assert all(len(n) == 4 for n in c.meta["needles"])
    assert all(0 <= j < (1024 - 128) // 64 for n in c.meta["needles"] for j in n)


def test_buried_block_recipe_keeps_unit_variance():
    c = wl.c4(L=8192)
    j = c.meta["buried"][0]
    assert 0 <= j < (8192 - 1024) // 256
    k = wl.decode_f32(c.k_pool, "bf16")
    assert abs(float(k.std()) - 1.0) < 0.02
    q = wl.decode_f32(c.q, "bf16")
    assert abs(float(q.std()) - 1.0) < 0.15
