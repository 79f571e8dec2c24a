"""Concurrent calls on two streams. The library keeps no mutable global
state: calls on different streams, each with its own workspace, may overlap
and must give the same bits as the same calls made one at a time. Two
workloads of different shapes (a GQA serving batch and an MHA batch) step on
two default-priority streams, interleaved, several times; every result is
compared with its single-stream run."""

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


def test_two_streams_overlap_without_interference():
    H.note("[streams] serving-small + opt-like-small on two streams")
    cases = [wl.c5(keep="1/32", B=8, L=4096), wl.c2(L=2048, keep="1/2")]
    dcs = [dev.upload(c) for c in cases]
    bufs = [dev.alloc_buffers(d) for d in dcs]
    for d, b in zip(dcs, bufs):
        dev.build_summaries(d, b)
    torch.cuda.synchronize()
    alone = []
    for d, b in zip(dcs, bufs):
        dev.decode_step(d, b)
        torch.cuda.synchronize()
        alone.append(_snapshot(b))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for rep in range(4):
        for b in bufs:
            b.out.zero_()
            b.lse.zero_()
        torch.cuda.synchronize()
        for s in streams:
            s.wait_stream(torch.cuda.current_stream())
        for _ in range(3):  # several steps in flight on both streams
            for d, b, s in zip(dcs, bufs, streams):
                dev.decode_step(d, b, stream=s)
        torch.cuda.synchronize()
        for i, b in enumerate(bufs):
            got = _snapshot(b)
            for k in KEYS:
                assert np.array_equal(got[k], alone[i][k]), f"rep {rep}, case {i}: {k} differs"
