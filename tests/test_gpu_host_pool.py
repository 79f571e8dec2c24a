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


def _decode_forms(dc):
    """Summaries, selection and the decode in both forms of the kept blocks."""
    buf = dev.alloc_buffers(dc)
    dev.build_summaries(dc, buf)
    dev.score_topk(dc, buf)
    res = {}
    for form in ("spans", "selected"):
        out = torch.full_like(buf.out, float("nan"))
        dev.sparse_decode(dc, buf, form=form, out=out)
        torch.cuda.synchronize()
        res[form] = out.cpu().numpy()
    return res


# every row length the host-memory K path transposes (D * E = 128, 256 and
# 512 bytes) with one-head, four-head and sixteen-head items
_SHAPES = (("bf16", 64, 16), ("fp16", 64, 1), ("fp32", 128, 4), ("fp32", 64, 16),
           ("bf16", 128, 16), ("fp16", 128, 8))
_N_RANDOM = 24


def _shape_case(idx):
    """The first _N_RANDOM of the random-shape test's cases, then _SHAPES."""
    if idx < _N_RANDOM:
        from tests.test_gpu_random_shapes import random_case
        return random_case(idx)
    dtype, D, G = _SHAPES[idx - _N_RANDOM]
    return wl.make_case(f"host-{dtype}-D{D}-G{G}", seed=97_000 + D + G, B=3, Hq=2 * G, Hkv=2, D=D,
                        P=32, dtype=dtype, ctx_lens=[1000, 640, 31], top_k=5, keep_floor=2,
                        recent_window=40)


@pytest.mark.parametrize("idx", range(_N_RANDOM + len(_SHAPES)))
def test_host_pool_decode_shapes_match_device_pool(idx):
    # The decode reads K row-major from a host-memory pool and puts it in the
    # MFMA layout through LDS: the outputs must be bit-identical to the
    # device pool's for every dtype, head dim and head-group size, in both
    # forms of the kept blocks.
    case = _shape_case(idx)
    H.note(f"[host pool] shape {case.name}")
    dc = dev.upload(case)
    on_device = _decode_forms(dc)
    on_host = _decode_forms(dev.with_host_pool(dc))
    for form in ("spans", "selected"):
        assert np.array_equal(on_device[form], on_host[form], equal_nan=True), form


def test_host_pool_sixteen_head_fp32_items():
    # fp32, D = 128, 16 heads per KV head and enough (sequence, KV head)
    # pairs that items keep all 16 heads: the host-memory kernel with the
    # most LDS (row-major K staging plus the four waves' 16-head sums).
    case = wl.make_case("host-fp32-D128-G16-B4", seed=97_500, B=4, Hq=32, Hkv=2, D=128, P=32,
                        dtype="fp32", ctx_lens=[900, 1000, 33, 640], top_k=5, keep_floor=2,
                        recent_window=40)
    H.note(f"[host pool] shape {case.name}")
    dc = dev.upload(case)
    on_device = _decode_forms(dc)
    on_host = _decode_forms(dev.with_host_pool(dc))
    for form in ("spans", "selected"):
        assert np.array_equal(on_device[form], on_host[form], equal_nan=True), form
    H.full_parity(case)
