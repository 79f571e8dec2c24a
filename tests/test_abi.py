"""The C ABI without a GPU: libkvsp.so loads, exports every entry point the
public header declares, sizes workspaces, and rejects malformed calls on the
host before anything is enqueued. No kernel is launched here."""

import ctypes

import pytest
import torch

from query_aware_sparse_block_amd import kvsp

P = ctypes.c_void_p
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails its host checks


def _have_gpu():
    return torch.cuda.device_count() > 0


def _layout(**over):
    base = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=64,
                num_phys_blocks=64, max_blocks_per_seq=32, dtype=2)
    base.update(over)
    return kvsp.kvsp_layout(*[base[f] for f, _ in kvsp.kvsp_layout._fields_])


def _params(**over):
    base = dict(top_k=4, keep_num=1, keep_den=1, keep_floor=1, recent_window=64, gamma_num=1,
                gamma_den=1)
    base.update(over)
    return kvsp.kvsp_select_params(*[base[f] for f, _ in kvsp.kvsp_select_params._fields_])


def test_library_exports_every_declared_entry_point():
    lib = kvsp.library()
    names = kvsp.declared_entry_points()
    assert {"kvsp_build_summaries", "kvsp_score_topk", "kvsp_sparse_decode",
            "kvsp_dense_decode", "kvsp_append_kv", "kvsp_workspace_bytes", "kvsp_status_string",
            "kvsp_abi_version"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name
    assert lib.kvsp_abi_version() == 1


def test_status_strings():
    for code in (0, -1, -2, -3, -4):
        assert kvsp.status_string(code)
    assert kvsp.status_string(-99) == "unknown status"


def test_workspace_bytes():
    lib = kvsp.library()
    n = lib.kvsp_workspace_bytes(ctypes.byref(_layout()), ctypes.byref(_params()))
    assert n > 0 and n % 256 == 0
    big = lib.kvsp_workspace_bytes(ctypes.byref(_layout(batch=64)), ctypes.byref(_params()))
    assert big >= n
    assert lib.kvsp_workspace_bytes(ctypes.byref(_layout(head_dim=96)), ctypes.byref(_params())) == 0


@pytest.mark.parametrize("over,code", [
    (dict(head_dim=96), -2),
    (dict(block_size=48), -2),
    (dict(block_size=8), -2),
    (dict(block_size=512), -2),
    (dict(dtype=7), -2),
    (dict(num_q_heads=6, num_kv_heads=4), -1),
    (dict(batch=0), -1),
    (dict(max_blocks_per_seq=20000), -2),
    (dict(num_kv_heads=64, num_q_heads=64), -2),
])
def test_bad_layout_rejected(over, code):
    lib = kvsp.library()
    lay = _layout(**over)
    par = _params()
    nul = [None] * 10
    assert lib.kvsp_build_summaries(ctypes.byref(lay), None, None, None, None, None) == code
    assert lib.kvsp_append_kv(ctypes.byref(lay), *([None] * 7), None) == code
    assert lib.kvsp_score_topk(ctypes.byref(lay), ctypes.byref(par), *nul, None, 0, None) == code
    assert lib.kvsp_sparse_decode(ctypes.byref(lay), ctypes.byref(par), *([None] * 8),
                                  ctypes.c_float(0), None, None, None, 0, None) == code
    assert lib.kvsp_dense_decode(ctypes.byref(lay), *([None] * 5), ctypes.c_float(0), None,
                                 None, None, 0, None) == code


@pytest.mark.parametrize("over", [
    dict(keep_den=0), dict(gamma_den=0), dict(keep_floor=0, recent_window=0), dict(top_k=-1),
    dict(recent_window=-5), dict(keep_num=-1),
])
def test_bad_params_rejected(over):
    lib = kvsp.library()
    lay, par = _layout(), _params(**over)
    assert lib.kvsp_score_topk(ctypes.byref(lay), ctypes.byref(par), *([FAKE] * 10), FAKE,
                               1 << 30, None) == -1
    assert lib.kvsp_sparse_decode(ctypes.byref(lay), ctypes.byref(par), *([FAKE] * 8),
                                  ctypes.c_float(0), FAKE, FAKE, FAKE, 1 << 30, None) == -1


def test_null_pointers_rejected():
    lib = kvsp.library()
    lay, par = _layout(), _params()
    assert lib.kvsp_build_summaries(ctypes.byref(lay), None, FAKE, FAKE, FAKE, None) == -1
    for i in range(7):
        args = [FAKE] * 7
        args[i] = None
        assert lib.kvsp_append_kv(ctypes.byref(lay), *args, None) == -1
    args = [FAKE] * 10
    args[7] = None  # num_spans
    assert lib.kvsp_score_topk(ctypes.byref(lay), ctypes.byref(par), *args, FAKE, 1 << 30,
                               None) == -1
    assert lib.kvsp_sparse_decode(ctypes.byref(lay), ctypes.byref(par), FAKE, FAKE, None,
                                  *([FAKE] * 5), ctypes.c_float(0), FAKE, FAKE, FAKE, 1 << 30,
                                  None) == -1
    assert lib.kvsp_dense_decode(None, *([FAKE] * 5), ctypes.c_float(0), FAKE, FAKE, FAKE, 1 << 30,
                                 None) == -1


@pytest.mark.skipif(_have_gpu(), reason="fake pointers must never reach a real device")
def test_small_workspace_rejected():
    lib = kvsp.library()
    lay, par = _layout(), _params()
    need = lib.kvsp_workspace_bytes(ctypes.byref(lay), ctypes.byref(par))
    assert lib.kvsp_sparse_decode(ctypes.byref(lay), ctypes.byref(par), *([FAKE] * 8),
                                  ctypes.c_float(0), FAKE, FAKE, FAKE, need - 1, None) == -3
    assert lib.kvsp_dense_decode(ctypes.byref(lay), *([FAKE] * 5), ctypes.c_float(0), FAKE, FAKE,
                                 None, need, None) == -3
    # scores == NULL needs the workspace
    args = [FAKE] * 10
    args[4] = None
    assert lib.kvsp_score_topk(ctypes.byref(lay), ctypes.byref(par), *args, FAKE, need - 1,
                               None) == -3
