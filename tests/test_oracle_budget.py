"""Pins for the dynamic budget controller (SparPR, "Dynamic budget control":
copy price = data volume / host-to-device bandwidth x 2 for K and V;
recompute price proportional to block length x hidden squared; their ratio
sets the keep ratio, bounded below by the Minimum Keep Floor).

The oracle (oracle/budget.py) is checked against hand-computed worked
examples, numpy's byte count of real K and V arrays, the page's block length x
hidden squared scaling, and the selection oracle's floor. The library's
kvsp_budget_keep_ratio (host arithmetic, no GPU) must then agree with it
exactly on seeded random models and machines."""

import math

import numpy as np
import pytest

import oracle
from oracle import budget
from query_aware_sparse_block_amd import kvsp

E = {"fp32": 4, "fp16": 2, "bf16": 2}
CODE = {"fp32": 0, "fp16": 1, "bf16": 2}


def test_worked_example_opt_like_block():
    # OPT-6.7B-like block: 64 tokens, 32 KV heads x 128, fp16, hidden 4096.
    # K bytes = 64*32*128*2 = 524288; copy = 2*524288 / 25e9 = 4.194304e-5 s.
    # One projection = 2*64*4096*4096 = 2147483648 flop; K and V = 4294967296
    # flop; at 400e12 flop/s = 1.073741824e-5 s. Ratio = 0.256 exactly
    # (= 4096*2.5e10 / 4e14); in units of 1/4096: 1048.576 -> 1049.
    n, c, r = budget.controller(64, 32, 128, 2, 4096, 25e9, 400e12, 4096)
    assert c == pytest.approx(4.194304e-5, rel=1e-15)
    assert r == pytest.approx(1.073741824e-5, rel=1e-15)
    assert budget.keep_ratio(c, r) == pytest.approx(0.256, rel=1e-15)
    assert n == 1049


def test_worked_example_qwen_like_gqa_block():
    # Qwen2.5-1.5B-like: 256 tokens, 2 KV heads x 128, bf16, hidden 1536.
    # K bytes = 256*2*128*2 = 131072; copy = 262144 / 25e9 = 1.048576e-5 s.
    # K and V projections = 4*256*1536*256 = 402653184 flop; at 100e12 flop/s
    # = 4.02653184e-6 s. Ratio = 0.384 (= 1536*2.5e10 / 1e14); x 4096 =
    # 1572.864 -> 1573.
    n, c, r = budget.controller(256, 2, 128, 2, 1536, 25e9, 100e12, 4096)
    assert c == pytest.approx(1.048576e-5, rel=1e-15)
    assert r == pytest.approx(4.02653184e-6, rel=1e-15)
    assert n == 1573


def test_copy_price_is_the_bytes_of_k_and_v_over_bandwidth():
    # the volume of a real block's K and V arrays, counted by numpy
    for dtype, npt in (("fp16", np.float16), ("bf16", np.uint16), ("fp32", np.float32)):
        for P, Hkv, D in ((16, 1, 64), (64, 32, 128), (256, 8, 128)):
            k = np.zeros((Hkv, P, D), npt)
            v = np.zeros((Hkv, P, D), npt)
            bw = 31.5e9
            assert budget.copy_seconds(P, Hkv, D, E[dtype], bw) == pytest.approx(
                (k.nbytes + v.nbytes) / bw, rel=1e-15)


def test_recompute_price_scales_with_block_length_and_hidden_squared():
    # multi-head attention (num_kv_heads * head_dim = hidden): 4 * P * hidden^2 / F
    F = 123e12
    for P, H, D in ((64, 32, 128), (128, 16, 64), (16, 8, 128)):
        hidden = H * D
        r = budget.recompute_seconds(P, hidden, H, D, F)
        assert r == pytest.approx(4 * P * hidden ** 2 / F, rel=1e-15)
        assert budget.recompute_seconds(2 * P, hidden, H, D, F) == pytest.approx(2 * r, rel=1e-15)
        assert budget.recompute_seconds(P, 2 * hidden, 2 * H, D, F) == pytest.approx(4 * r, rel=1e-15)
    # grouped KV heads: the projections are narrower than hidden
    assert budget.recompute_seconds(64, 4096, 8, 128, F) == pytest.approx(
        budget.recompute_seconds(64, 4096, 32, 128, F) / 4, rel=1e-15)


def test_keep_ratio_falls_as_the_copy_grows_dearer_and_never_exceeds_one():
    args = dict(block_size=64, num_kv_heads=8, head_dim=128, elem_bytes=2, hidden=4096,
                proj_flops_per_s=200e12, keep_den=1 << 16)
    prev = None
    for bw in (1e13, 1e12, 1e11, 5e10, 2.5e10, 1e10, 1e9, 1e8):
        n, c, r = budget.controller(h2d_bytes_per_s=bw, **args)
        assert 1 <= n <= args["keep_den"]
        if r >= c:
            assert n == args["keep_den"]  # fetching is no dearer than rebuilding: keep all
        if prev is not None:
            assert n <= prev
        prev = n
    assert prev == math.ceil(budget.keep_ratio(c, r) * args["keep_den"])
    # a fast link: rebuilding (42.9 us at 100e12 flop/s) costs more than
    # fetching (1 MiB at 1e12 B/s = 1.05 us); the ratio itself is capped at 1
    n, c, r = budget.controller(64, 32, 128, 2, 4096, 1e12, 100e12, 1000)
    assert r > c and budget.keep_ratio(c, r) == 1.0 and n == 1000
    assert budget.keep_num(1e-12, 1000) == 1  # never rounded to zero
    assert budget.keep_num(0.0, 1000) == 1  # at least one unit, whatever the ratio


def test_keep_floor_bounds_the_controllers_keep_from_below():
    # the selection oracle with the controller's ratio: k = max(floor,
    # ceil(C * keep_num / keep_den)), capped at C
    n, _, _ = budget.controller(64, 32, 128, 2, 4096, 0.5e9, 100e12, 1024)  # a slow link: ratio ~ 0.02
    assert n < 1024 // 32
    for L, floor in ((8192, 0), (8192, 4), (8192, 64), (1000, 3)):
        p = oracle.plan(L, 64, 128, keep_num=n, keep_den=1024, keep_floor=floor)
        C = p["C"]
        assert p["k_eff"] == min(C, max(floor, -(-C * n // 1024)))


def _random_model(rng):
    Hkv = int(rng.choice([1, 2, 4, 8, 16, 32, 56]))
    D = int(rng.choice([64, 128]))
    P = int(rng.choice([16, 32, 64, 128, 256]))
    dtype = str(rng.choice(["fp32", "fp16", "bf16"]))
    G = int(rng.choice([1, 2, 4, 8]))
    hidden = int(rng.integers(1, 8)) * Hkv * D * G // int(rng.choice([1, 2]))
    bw = float(10 ** rng.uniform(8, 13))
    flops = float(10 ** rng.uniform(11, 16))
    den = int(rng.choice([1, 7, 100, 1024, 4096, 65536, 1 << 30]))
    return Hkv, D, P, dtype, G, max(hidden, 1), bw, flops, den


def test_library_matches_oracle_on_seeded_random_models():
    rng = np.random.default_rng(2024)
    for _ in range(400):
        Hkv, D, P, dtype, G, hidden, bw, flops, den = _random_model(rng)
        if Hkv * D > 7168:
            continue
        layout = kvsp.kvsp_layout(2, Hkv * G, Hkv, D, P, 8, 4, CODE[dtype])
        got = kvsp.kvsp_budget_keep_ratio(layout, kvsp.BudgetModel(bw, flops, hidden), den)
        want = budget.controller(P, Hkv, D, E[dtype], hidden, bw, flops, den)
        assert got == want, (Hkv, D, P, dtype, hidden, bw, flops, den)


# ---- planted mistakes: each must fail at least one pin above ----------------------

_PINS = [test_worked_example_opt_like_block, test_worked_example_qwen_like_gqa_block,
         test_copy_price_is_the_bytes_of_k_and_v_over_bandwidth,
         test_recompute_price_scales_with_block_length_and_hidden_squared,
         test_keep_ratio_falls_as_the_copy_grows_dearer_and_never_exceeds_one,
         test_keep_floor_bounds_the_controllers_keep_from_below]

_MUTANTS = {
    "K and V not doubled": ("return 2 * volume / h2d_bytes_per_s", "return volume / h2d_bytes_per_s"),
    "one projection only": ("return 2 * one_projection / proj_flops_per_s",
                            "return one_projection / proj_flops_per_s"),
    "KV heads dropped": ("hidden * (num_kv_heads * head_dim)", "hidden * head_dim"),
    "ratio inverted": ("min(1.0, recompute_s / copy_s)", "min(1.0, copy_s / recompute_s)"),
    "ratio not capped": ("min(1.0, recompute_s / copy_s)", "recompute_s / copy_s"),
    "rounded down": ("math.ceil(ratio * keep_den)", "math.floor(ratio * keep_den)"),
    "zero keep allowed": ("max(1, math.ceil(", "max(0, math.ceil("),
}


@pytest.mark.parametrize("name", sorted(_MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    import types
    old, new = _MUTANTS[name]
    src = open(budget.__file__).read()
    assert src.count(old) == 1
    mutant = types.ModuleType("budget_mutant")
    exec(compile(src.replace(old, new), "budget_mutant", "exec"), mutant.__dict__)
    monkeypatch.setitem(globals(), "budget", mutant)
    failed = 0
    for pin in _PINS:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1, f"no pin catches the mutant '{name}'"
