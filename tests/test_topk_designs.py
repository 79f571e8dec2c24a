"""The designed Top-k inputs of the GPU test really reach the radix pass they
are named for: the first byte (from the top) at which the keys whose prefix
is at least the k-th key's prefix number exactly k. Checked on the CPU so the
GPU test cannot silently lose a case."""

import numpy as np
import pytest

from tests.test_gpu_topk_designed import KINDS, _design


def _order_keys(x):
    """Float32 -> unsigned keys in the order of the values, -0 equal to +0."""
    u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    key = np.where(u >> 31, (~u) & 0xFFFFFFFF, u | 0x80000000)
    key[x == 0] = 0x80000000
    return key


def _whole_at(x, k):
    key = _order_keys(x)
    kth = np.sort(key)[::-1][k - 1]
    for p in range(4):
        mask = (0xFFFFFFFF << (24 - 8 * p)) & 0xFFFFFFFF
        if int(np.sum((key & mask) >= (kth & mask))) == k:
            return p
    return None


EXPECTED = {"whole-at-byte-0": 0, "whole-at-byte-1": 1, "whole-at-byte-2": 2, "all-bytes": 3,
            "tie-whole": 0}


@pytest.mark.parametrize("C,k", [(200, 37), (500, 37), (500, 200), (1500, 20), (1500, 300), (5000, 37)])
def test_designs_reach_their_pass(C, k):
    rng = np.random.default_rng(C * 1000 + k)
    for kind in KINDS:
        x = _design(kind, C, k, rng)
        p = _whole_at(x, k)
        if kind in EXPECTED:
            assert p == EXPECTED[kind], (kind, p)
        elif kind in ("tie-cut", "all-equal"):
            assert p is None, (kind, p)  # the k-th key's equal run is cut
