"""Fidelity invariants of the synthetic workloads under the oracle.

The SparPR news page measures fidelity with a needle planted at two depths
("Measured numbers on one laptop") and the DKV abstract with a buried
passcode. Without the texts or the models, the synthetic stand-ins plant a
needle block whose keys point at the query; query-aware selection must find
it. These check the oracle's scoring and Top-k end to end on such inputs."""

import numpy as np
import pytest

import oracle
from query_aware_sparse_block_amd import workloads as wl


def _step(case, **over):
    summ = oracle.summaries(case.dtype, case.k_pool, case.block_table, case.ctx_lens, case.Hkv,
                            case.P, case.D)
    params = dict(case.select_params)
    params.update(over)
    return oracle.decode_step(case.dtype, case.q, case.k_pool, case.v_pool, case.block_table,
                              case.ctx_lens, summ, Hkv=case.Hkv, P=case.P, **params)


@pytest.mark.parametrize("L", [1024, 2048, 4096])
@pytest.mark.parametrize("keep", ["1/2", "1/10"])
def test_needle_blocks_are_selected(L, keep):
    case = wl.c2(L=L, keep=keep, B=2, H=8)
    r = _step(case)
    for b in range(case.B):
        k = int(r["plan"][b, 3])
        sel = set(r["sel"][b, :k].tolist())
        needles = set(case.meta["needles"][b])
        if k >= len(needles):
            assert needles <= sel
        else:
            assert sel <= needles
    if all(int(r["plan"][b, 3]) >= 4 for b in range(case.B)):
        dense = _step(case, top_k=10 ** 6)
        # the unselected blocks hold a negligible share of the softmax mass
        np.testing.assert_allclose(r["out"], dense["out"], atol=1e-6)


@pytest.mark.parametrize("L", [4096, 8192, 16384])
def test_buried_block_is_selected(L):
    case = wl.c4(L=L)
    r = _step(case)
    k = int(r["plan"][0, 3])
    assert case.meta["buried"][0] in r["sel"][0, :k].tolist()
