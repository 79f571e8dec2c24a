"""The allocation-free decode (kvsp_sparse_decode_noalloc) through the C ABI
against kvsp_sparse_decode on the same inputs: bit-identical outputs and lse,
on two calls in a row whose second is smaller (so it finds the first call's
partials and counters in the shared static scratch), in both forms of the kept
blocks, with a dense-fallback batch among them."""

import pytest
import torch

from query_aware_sparse_block_amd import device as dev
from query_aware_sparse_block_amd import kvsp
from query_aware_sparse_block_amd import workloads as wl
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _step(case):
    dc = dev.upload(case)
    buf = dev.alloc_buffers(dc)
    dev.build_summaries(dc, buf)
    dev.score_topk(dc, buf)
    return dc, buf


def _noalloc(dc, buf, form):
    out = torch.full_like(buf.out, float("nan"))
    lse = torch.full_like(buf.lse, float("nan"))
    kept = ((buf.spans, buf.num_spans, None, None) if form == "spans"
            else (None, None, buf.selected, buf.num_selected))
    kvsp.kvsp_sparse_decode_noalloc(dc.layout, dc.params, dc.q, dc.k_pool, dc.v_pool,
                                    dc.block_table, dc.ctx_lens, *kept, buf.use_dense, 0.0, out,
                                    lse)
    return out, lse


@pytest.mark.parametrize("form", ["spans", "selected"])
def test_noalloc_matches_the_workspace_decode_twice_in_a_row(form):
    # first: the serving shape scaled (8 x 8 KV heads, keep 1/32, several
    # chunks per group); second: a smaller OPT-like batch with a longer
    # selection; third: the first again at keep 7/10 (every sequence dense)
    cases = [wl.c5(keep="1/32", B=8, L=4096), wl.c2(L=1024, keep="1/2", B=2, H=8),
             wl.c5(keep="7/10", B=8, L=4096)]
    for case in cases:
        H.note(f"[noalloc] {form} {case.name} B={case.B} Hq={case.Hq} Hkv={case.Hkv}")
        dc, buf = _step(case)
        dev.sparse_decode(dc, buf, form=form)
        out, lse = _noalloc(dc, buf, form)
        torch.cuda.synchronize()
        assert torch.equal(out, buf.out), f"{case.name}: outputs differ"
        assert torch.equal(lse, buf.lse), f"{case.name}: lse differ"
