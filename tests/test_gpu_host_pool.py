"""The pool kept in host RAM: the same entry points, with K/V in mapped pinned
host memory, must give bit-identical results to a device-resident pool (the
kernels are the same; only the memory the tiles come from differs). This is
the SparPR page's setting, where the cache is off the GPU and only selected
blocks (plus the window) cross to it."""

import numpy as np
import pytest
import torch

from query_aware_sparse_block_amd import device as dev
from query_aware_sparse_block_amd import workloads as wl
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

KEYS = ("summaries", "scores", "selected", "num_selected", "spans", "num_spans", "use_dense",
        "out", "lse")


def _run(dc, dense_api=False):
    buf = dev.alloc_buffers(dc)
    dev.build_summaries(dc, buf)
    if dense_api:
        dev.dense_decode(dc, buf)
    else:
        dev.decode_step(dc, buf)
    torch.cuda.synchronize()
    return {k: getattr(buf, k).cpu().numpy() for k in KEYS}


@pytest.mark.parametrize("name,make", [
    ("serving-small", lambda: wl.c5(keep="1/32", B=8, L=4096)),
    ("serving-small-dense", lambda: wl.c5(keep="7/10", B=8, L=4096)),
    ("opt-like", lambda: wl.c2(L=2048, keep="1/10", B=2, H=8)),
    ("qwen-like", lambda: wl.c4(L=8192)),
])
def test_host_pool_matches_device_pool(name, make):
    H.note(f"[host pool] {name}")
    case = make()
    dc = dev.upload(case)
    on_device = _run(dc)
    on_host = _run(dev.with_host_pool(dc))
    for k in KEYS:
        assert np.array_equal(on_device[k], on_host[k]), k
    # and the device run itself against the oracle
    H.full_parity(case)


def test_dense_decode_from_host_pool():
    case = wl.c1("k8")
    H.note("[host pool] dense decode c1")
    dc = dev.upload(case)
    a = _run(dc, dense_api=True)
    b = _run(dev.with_host_pool(dc), dense_api=True)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["lse"], b["lse"])


def test_dkv_codec_and_decode_from_host_pool():
    # the DKV variant over a pool in host RAM: the codec reads the older blocks
    # and the decode the window rows across PCIe; records and outputs must be
    # bit-identical to those of the device-resident pool
    from query_aware_sparse_block_amd import kvsp
    case = wl.c4_dkv(L=8192, n_resid=8)
    H.note("[host pool] dkv compress + decode, qwen-like 8192")
    dkv = kvsp.DkvParams(n_resid=8)
    got = {}
    for where, dc in (("device", dev.upload(case)), ("host", None)):
        if dc is None:
            dc = dev.with_host_pool(dev.upload(case))
        buf = dev.alloc_buffers(dc)
        dev.build_summaries(dc, buf)
        recs = dev.alloc_dkv_records(dc, dkv)
        ws = kvsp.alloc_dkv_workspace(dc.layout, dkv)
        dev.dkv_compress(dc, dkv, recs)
        dev.score_topk(dc, buf)
        dev.dkv_decode(dc, buf, dkv, recs, ws)
        torch.cuda.synchronize()
        got[where] = (recs.cpu().numpy(), buf.selected.cpu().numpy(), buf.out.cpu().numpy(),
                      buf.lse.cpu().numpy())
    for a, b, name in zip(got["device"], got["host"], ("records", "selected", "out", "lse")):
        assert np.array_equal(a, b), name
