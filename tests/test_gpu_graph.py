"""The decode step captured in a HIP graph (through torch.cuda.CUDAGraph)
replays to the same bits as the eager step. The library records no memset
into a graph: its completion counters reset themselves inside the kernels.
Each replay follows eager work (output buffers cleared, another eager step)
and a synchronization, and is checked on its own."""

import numpy as np
import pytest
import torch

from query_aware_sparse_block_amd import device as dev
from query_aware_sparse_block_amd import workloads as wl
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

KEYS = ("selected", "num_selected", "spans", "num_spans", "use_dense", "scores", "out", "lse")


def _snapshot(buf):
    return {k: getattr(buf, k).cpu().numpy().copy() for k in KEYS}


@pytest.mark.parametrize("name,make", [
    ("serving-small", lambda: wl.c5(keep="1/32", B=8, L=4096)),
    ("serving-small-dense", lambda: wl.c5(keep="7/10", B=8, L=4096)),
    ("minicpm-small", lambda: wl.c3(keep="1/16", L=16384)),
    # scored by more than 64 workgroups / a table longer than 512 blocks: the
    # Top-k runs in a launch of its own
    ("serving-b16", lambda: wl.c5(keep="1/32", B=16, L=4096)),
    ("minicpm-long-table", lambda: wl.c3(keep="1/16", L=65536)),
])
def test_graph_replays_match_eager(name, make):
    H.note(f"[graph] {name}")
    case = make()
    dc = dev.upload(case)
    buf = dev.alloc_buffers(dc)
    other = dev.alloc_buffers(dc)
    dev.build_summaries(dc, buf)
    dev.build_summaries(dc, other)
    dev.decode_step(dc, buf)
    torch.cuda.synchronize()
    eager = _snapshot(buf)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dev.decode_step(dc, buf)  # warm-up on the capture stream's side
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dev.decode_step(dc, buf)
    torch.cuda.synchronize()

    for rep in range(3):
        # eager work between replays: reset the outputs to their initial fill
        # (entries past the counts are never written), run another step
        buf.selected.fill_(-1)
        buf.spans.fill_(-1)
        for k in ("out", "lse", "scores", "num_selected", "num_spans", "use_dense"):
            getattr(buf, k).zero_()
        dev.decode_step(dc, other)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _snapshot(buf)
        for k in KEYS:
            assert np.array_equal(got[k], eager[k]), f"replay {rep}: {k} differs"
    assert np.array_equal(_snapshot(other)["out"], eager["out"])


def test_graph_of_append_score_decode_replays():
    # a whole decode-loop step in one graph: append each sequence's token at
    # its last position (completing the block), then score, select and
    # attend. The appended rows are the rows already there, so every replay
    # must reproduce the eager step exactly, pools and summaries included.
    case = wl.c5(keep="1/32", B=8, L=4096)
    H.note("[graph] append + step, serving-small")
    dc = dev.upload(case)
    buf = dev.alloc_buffers(dc)
    dev.build_summaries(dc, buf)
    ctx = dc.ctx_lens.long()
    bt = dc.block_table.long()
    phys = bt[torch.arange(case.B, device=bt.device), (ctx - 1) // case.P]
    t = (ctx - 1) % case.P
    k_new = dc.k_pool[phys, :, t].contiguous()
    v_new = dc.v_pool[phys, :, t].contiguous()
    pos = (ctx - 1).to(torch.int32)

    def step():
        dev.append_kv(dc, buf, k_new, v_new, pos)
        dev.decode_step(dc, buf)

    step()
    torch.cuda.synchronize()
    eager = _snapshot(buf)
    summ0 = buf.summaries.clone()
    k0 = dc.k_pool.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        buf.selected.fill_(-1)
        buf.spans.fill_(-1)
        for k in ("out", "lse", "scores", "num_selected", "num_spans", "use_dense"):
            getattr(buf, k).zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _snapshot(buf)
        for k in KEYS:
            assert np.array_equal(got[k], eager[k]), f"replay {rep}: {k} differs"
        assert torch.equal(buf.summaries, summ0) and torch.equal(dc.k_pool, k0)


def test_graph_of_dkv_compress_score_decode_replays():
    # the DKV variant in one graph: compress every older block, then score,
    # select and decode over the compressed blocks and the exact window. The
    # codec is deterministic, so every replay must reproduce the eager step
    # and the eager records byte for byte.
    from query_aware_sparse_block_amd import kvsp
    case = wl.c4_dkv(L=8192, n_resid=8)
    H.note("[graph] dkv compress + score + decode, qwen-like 8192")
    dc = dev.upload(case)
    buf = dev.alloc_buffers(dc)
    dev.build_summaries(dc, buf)
    dkv = kvsp.DkvParams(n_resid=8)
    recs = dev.alloc_dkv_records(dc, dkv)
    ws = kvsp.alloc_dkv_workspace(dc.layout, dkv)

    def step():
        dev.dkv_compress(dc, dkv, recs)
        dev.score_topk(dc, buf)
        dev.dkv_decode(dc, buf, dkv, recs, ws)

    step()
    torch.cuda.synchronize()
    eager = _snapshot(buf)
    recs0 = recs.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        buf.selected.fill_(-1)
        buf.spans.fill_(-1)
        for k in ("out", "lse", "scores", "num_selected", "num_spans", "use_dense"):
            getattr(buf, k).zero_()
        recs.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _snapshot(buf)
        for k in KEYS:
            assert np.array_equal(got[k], eager[k]), f"replay {rep}: {k} differs"
        assert torch.equal(recs, recs0), f"replay {rep}: records differ"
