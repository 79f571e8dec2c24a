"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (same entry points, same layouts).

Every family is checked completely: every summary, score, selection, span,
output and lse. That includes the batched serving shape (64 sequences of
32768 tokens in an 8 GiB pool, 2048 (sequence, head) outputs) at keep 1/32
and in its dense-fallback variant (keep 7/10 > gamma 3/5, every token of every
sequence attended); the oracle runs its (sequence, head) attentions on the
host's thread share."""

import dataclasses

import pytest

from query_aware_sparse_block_amd import workloads as wl
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("L", [1024, 2048, 4096, 8192])
@pytest.mark.parametrize("keep", ["1/2", "1/10"])
def test_opt_like_full(L, keep):
    case = wl.c2(L=L, keep=keep)
    gpu, r_or = H.full_parity(case)
    for b, needles in enumerate(case.meta["needles"]):
        k = int(gpu["num_selected"][b])
        sel = set(gpu["selected"][b, :k].tolist())
        assert set(needles) <= sel or sel <= set(needles)


@pytest.mark.parametrize("keep", ["1/32", "1/16", "1/8"])
def test_minicpm_like_full(keep):
    H.full_parity(wl.c3(keep=keep))


@pytest.mark.parametrize("L", [4096, 8192, 16384, 32768, 65536])
def test_qwen_like_full(L):
    case = wl.c4(L=L)
    gpu, _ = H.full_parity(case)
    k = int(gpu["num_selected"][0])
    assert case.meta["buried"][0] in gpu["selected"][0, :k].tolist()


@pytest.fixture(scope="module")
def serving_case():
    H.note("[fullsize] generating the batched serving workload (8 GiB pool)")
    case = wl.c5(keep="1/32")
    H.note("[fullsize] oracle summaries of the serving workload")
    return case, H.oracle_summaries(case)


def test_serving_full_sparse(serving_case):
    case, summ = serving_case
    gpu, r_or = H.full_parity(case, summ=summ)
    assert (gpu["num_selected"] == 16).all() and not gpu["use_dense"].any()


def test_serving_full_dense_fallback(serving_case):
    base, summ = serving_case
    case = dataclasses.replace(base, name="c5-keep7/10", keep_num=7, keep_den=10)
    gpu, r_or = H.full_parity(case, summ=summ)
    assert (gpu["num_selected"] == 359).all() and gpu["use_dense"].all()
