"""GPU parity on seeded random configurations. Three hundred shapes drawn from a
fixed seed cover combinations that the hand-picked cases do not: every
dtype, head dims 64 and 128, block sizes 16 to 256, 1 to 8 KV heads with 1 to
20 query heads each, 1 to 6 sequences of ragged lengths (some empty, some
inside the window), top-k or keep ratios, floors, windows, dense fallbacks
and shuffled pools. Each runs the whole step (summaries, scores, Top-k,
spans, attention) on the GPU and is checked against the oracle with the
usual bars (tests/gpu_helpers.py). Sizes are bounded so that the oracle
finishes in seconds."""

import numpy as np
import pytest

from query_aware_sparse_block_amd import workloads as wl
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

N_CASES = 300


def random_case(i):
    rng = np.random.default_rng(90_000 + i)
    dtype = ["fp32", "fp16", "bf16"][rng.integers(3)]
    D = int(rng.choice([64, 128]))
    P = int(rng.choice([16, 32, 64, 128, 256]))
    Hkv = int(rng.integers(1, 9))
    G = int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16, 20]))
    B = int(rng.integers(1, 7))
    max_blocks = int(rng.integers(1, 41))
    # bound the oracle's work: attended tokens x query heads x head dim
    while B * max_blocks * P * Hkv * G * D > 4e7 and max_blocks > 1:
        max_blocks //= 2
    ctx = []
    for _ in range(B):
        kind = rng.integers(6)
        if kind == 0:
            ctx.append(0)
        elif kind == 1:
            ctx.append(max_blocks * P)
        else:
            ctx.append(int(rng.integers(1, max_blocks * P + 1)))
    W = int(rng.choice([0, int(rng.integers(1, 3 * P + 1))]))
    floor = int(rng.integers(0, 5))
    if floor == 0 and W == 0:
        floor = 1
    if rng.random() < 0.5:
        sel = dict(top_k=int(rng.integers(1, 12)))
    else:
        den = int(rng.integers(1, 11))
        sel = dict(top_k=0, keep_num=int(rng.integers(0, den + 1)), keep_den=den)
    if rng.random() < 0.3:
        gden = int(rng.integers(1, 6))
        sel.update(gamma_num=int(rng.integers(0, gden)), gamma_den=gden)
    extra = int(rng.integers(0, 8))
    return wl.make_case(f"rand{i}", seed=91_000 + i, B=B, Hq=Hkv * G, Hkv=Hkv, D=D, P=P,
                        dtype=dtype, ctx_lens=ctx, shuffle=bool(rng.integers(2)),
                        num_phys=B * max_blocks + extra, max_blocks=max_blocks,
                        recent_window=W, keep_floor=floor, **sel)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(i):
    H.full_parity(random_case(i))
