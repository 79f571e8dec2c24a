"""The streamed scoring path (summary sets above 64 MiB are read with
non-temporal loads, as a branch-free pipeline of passes) on a shape whose
summary row does not fill its lane group: 3 KV heads x 64 channels = 48
16-byte vectors per row, so lanes past the row's end read a clamped vector
that must be masked. Scores must match the oracle and the selection must be
exact, for every sequence."""

import numpy as np
import pytest

import oracle
from query_aware_sparse_block_amd import workloads as wl
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def test_streamed_scoring_with_partial_rows_matches_oracle():
    B, L, P = 64, 24576, 16
    ctx = np.full(B, L, np.int32)
    ctx[::7] = L - 37  # some sequences end inside a block
    case = wl.make_case("streamed-partial-rows", seed=9100, B=B, Hq=6, Hkv=3, D=64, P=P,
                        dtype="bf16", ctx_lens=ctx, top_k=5, keep_floor=1, recent_window=16)
    summary_bytes = B * case.max_blocks * case.Hkv * case.D * 4
    assert summary_bytes > (64 << 20)  # the streamed path
    H.note(f"[streamed scores] B={B} L={L} Hkv=3 D=64 summaries={summary_bytes >> 20} MiB")
    gpu, _, _ = H.run_gpu(case)
    summ = H.oracle_summaries(case)
    H.check_summaries(case, gpu["summaries"], summ)
    r_or = oracle.decode_step(case.dtype, case.q, case.k_pool, case.v_pool, case.block_table,
                              case.ctx_lens, summ, Hkv=case.Hkv, P=case.P, **case.select_params)
    T = H.term_sums(case, summ)
    H.check_scores(case, r_or, gpu, T)
    for b in range(B):
        H.check_selection(case, r_or, gpu, b, T)
