"""Pins for the oracle's element widening: every 16-bit pattern decoded by the
oracle must equal an independent decoder (numpy's binary16, and bfloat16 as
the top half of a binary32)."""

import numpy as np

import oracle


def test_fp16_all_patterns_match_numpy():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.widen("fp16", bits)
    ref = bits.view(np.float16).astype(np.float64)
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])
    # spot values fixed by the binary16 format
    assert oracle.widen("fp16", np.array([0x3C00, 0x0001, 0x7BFF, 0x8000], np.uint16)).tolist() == \
        [1.0, 2.0 ** -24, 65504.0, -0.0]


def test_bf16_all_patterns_match_binary32_top_half():
    bits = np.arange(1 << 16, dtype=np.uint32)
    got = oracle.widen("bf16", bits.astype(np.uint16))
    with np.errstate(invalid="ignore"):
        ref = (bits << 16).view(np.float32).astype(np.float64)
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert oracle.widen("bf16", np.array([0x3F80, 0xC000, 0x0001], np.uint16)).tolist() == \
        [1.0, -2.0, 2.0 ** -133]


def test_fp32_passthrough():
    x = np.random.default_rng(0).standard_normal(1000).astype(np.float32)
    assert np.array_equal(oracle.widen("fp32", x), x.astype(np.float64))
