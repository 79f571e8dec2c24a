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
    assert lib.kvsp_abi_version() == 2


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
    (dict(batch=65537), -2),
    (dict(batch=2**31 - 1), -2),
    (dict(num_q_heads=2048, num_kv_heads=2), -2),
    (dict(num_q_heads=2**31 - 1, num_kv_heads=1), -2),
])
def test_bad_layout_rejected(over, code):
    lib = kvsp.library()
    lay = _layout(**over)
    par = _params()
    nul = [None] * 10
    assert lib.kvsp_build_summaries(ctypes.byref(lay), None, None, None, None, None) == code
    assert lib.kvsp_append_kv(ctypes.byref(lay), *([None] * 7), None) == code
    assert lib.kvsp_score_topk(ctypes.byref(lay), ctypes.byref(par), *nul, None, 0, None) == code
    assert lib.kvsp_sparse_decode(ctypes.byref(lay), ctypes.byref(par), *([None] * 10),
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
    assert lib.kvsp_sparse_decode(ctypes.byref(lay), ctypes.byref(par), *([FAKE] * 7),
                                  None, None, FAKE, ctypes.c_float(0), FAKE, FAKE, FAKE, 1 << 30,
                                  None) == -1


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
                                  *([FAKE] * 4), None, None, FAKE, ctypes.c_float(0), FAKE, FAKE,
                                  FAKE, 1 << 30, None) == -1


@pytest.mark.parametrize("kept", [
    (FAKE, FAKE, FAKE, FAKE),   # both forms
    (None, None, None, None),   # neither
    (FAKE, None, None, None),   # a span list without its counts
    (None, FAKE, None, None),
    (None, None, FAKE, None),   # a selected list without its counts
    (None, None, None, FAKE),
    (FAKE, None, FAKE, None),
])
def test_sparse_decode_takes_exactly_one_form_of_the_kept_blocks(kept):
    lib = kvsp.library()
    lay, par = _layout(), _params()
    assert lib.kvsp_sparse_decode(ctypes.byref(lay), ctypes.byref(par), *([FAKE] * 5), *kept,
                                  FAKE, ctypes.c_float(0), FAKE, FAKE, FAKE, 1 << 30, None) == -1
    assert lib.kvsp_dense_decode(None, *([FAKE] * 5), ctypes.c_float(0), FAKE, FAKE, FAKE, 1 << 30,
                                 None) == -1


@pytest.mark.skipif(_have_gpu(), reason="fake pointers must never reach a real device")
def test_small_workspace_rejected():
    lib = kvsp.library()
    lay, par = _layout(), _params()
    need = lib.kvsp_workspace_bytes(ctypes.byref(lay), ctypes.byref(par))
    assert lib.kvsp_sparse_decode(ctypes.byref(lay), ctypes.byref(par), *([FAKE] * 7),
                                  None, None, FAKE, ctypes.c_float(0), FAKE, FAKE, FAKE, need - 1,
                                  None) == -3
    assert lib.kvsp_dense_decode(ctypes.byref(lay), *([FAKE] * 5), ctypes.c_float(0), FAKE, FAKE,
                                 None, need, None) == -3
    # scores == NULL needs the workspace
    args = [FAKE] * 10
    args[4] = None
    assert lib.kvsp_score_topk(ctypes.byref(lay), ctypes.byref(par), *args, FAKE, need - 1,
                               None) == -3


# ---- DKV entry points (host checks only) ---------------------------------------

@pytest.mark.parametrize("D,P,dtype,R", [(128, 256, 2, 16), (64, 64, 0, 0), (128, 128, 1, 64),
                                         (64, 256, 2, 33)])
def test_dkv_record_bytes_match_the_packer(D, P, dtype, R):
    from query_aware_sparse_block_amd import workloads as wl
    lay = _layout(head_dim=D, block_size=P, dtype=dtype)
    n = kvsp.kvsp_dkv_record_bytes(lay, kvsp.DkvParams(n_resid=R))
    E = 4 if dtype == 0 else 2
    assert n == wl.dkv_record_layout(D, P, E, R)["bytes"] and n % 256 == 0
    ws = kvsp.kvsp_dkv_workspace_bytes(lay, kvsp.DkvParams(n_resid=R))
    assert ws >= kvsp.library().kvsp_workspace_bytes(ctypes.byref(lay), ctypes.byref(_params()))


@pytest.mark.parametrize("lay_over,dkv", [
    ({}, kvsp.DkvParams(rank=16)),
    ({}, kvsp.DkvParams(n_resid=65)),
    ({"block_size": 32}, kvsp.DkvParams()),
    ({"head_dim": 96}, kvsp.DkvParams()),
    ({"num_q_heads": 34, "num_kv_heads": 2}, kvsp.DkvParams()),
])
def test_dkv_unsupported_arguments(lay_over, dkv):
    lay = _layout(**lay_over)
    assert kvsp.kvsp_dkv_record_bytes(lay, dkv) == 0
    assert kvsp.kvsp_dkv_workspace_bytes(lay, dkv) == 0
    lib = kvsp.library()
    d = dkv.c()
    st = lib.kvsp_dkv_compress(ctypes.byref(lay), ctypes.byref(d), 64, *([FAKE] * 5), None)
    assert st in (-1, -2)


def test_dkv_compress_rejects_bad_calls():
    lib = kvsp.library()
    lay = _layout()
    d = kvsp.DkvParams().c()
    assert lib.kvsp_dkv_compress(ctypes.byref(lay), None, 64, *([FAKE] * 5), None) == -1
    assert lib.kvsp_dkv_compress(ctypes.byref(lay), ctypes.byref(d), -1, *([FAKE] * 5), None) == -1
    for i in range(5):
        args = [FAKE] * 5
        args[i] = None
        assert lib.kvsp_dkv_compress(ctypes.byref(lay), ctypes.byref(d), 64, *args, None) == -1
    bad = kvsp.DkvParams(power_iters=-1).c()
    assert lib.kvsp_dkv_compress(ctypes.byref(lay), ctypes.byref(bad), 64, *([FAKE] * 5),
                                 None) == -1


def test_dkv_decode_rejects_bad_calls():
    lib = kvsp.library()
    lay, par = _layout(), _params()
    d = kvsp.DkvParams().c()
    for i in range(8):  # q, pools, records, table, lengths, selection
        args = [FAKE] * 8
        args[i] = None
        assert lib.kvsp_dkv_decode(ctypes.byref(lay), ctypes.byref(par), ctypes.byref(d), *args,
                                   ctypes.c_float(0), FAKE, FAKE, FAKE, 1 << 30, None) == -1
    assert lib.kvsp_dkv_decode(ctypes.byref(lay), ctypes.byref(par), ctypes.byref(d), *([FAKE] * 8),
                               ctypes.c_float(0), None, FAKE, FAKE, 1 << 30, None) == -1  # out
    assert lib.kvsp_dkv_decode(ctypes.byref(lay), None, ctypes.byref(d), *([FAKE] * 8),
                               ctypes.c_float(0), FAKE, FAKE, FAKE, 1 << 30, None) == -1


@pytest.mark.skipif(_have_gpu(), reason="fake pointers must never reach a real device")
def test_dkv_decode_small_workspace_rejected():
    lib = kvsp.library()
    lay, par = _layout(), _params()
    dkv = kvsp.DkvParams()
    need = kvsp.kvsp_dkv_workspace_bytes(lay, dkv)
    d = dkv.c()
    assert lib.kvsp_dkv_decode(ctypes.byref(lay), ctypes.byref(par), ctypes.byref(d), *([FAKE] * 8),
                               ctypes.c_float(0), FAKE, FAKE, FAKE, need - 1, None) == -3


# ---- binding checks (no GPU: they raise before any pointer reaches the library) ----

class _FakeHostBuffer:
    def __init__(self, nbytes):
        self.nbytes = nbytes
        self.device_ptr = 0x1000


def test_binding_sizes_follow_the_header_layouts():
    lay = _layout(batch=3, num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                  num_phys_blocks=10, max_blocks_per_seq=5, dtype=1)
    z = kvsp._Sizes(lay)
    assert z.q == 3 * 8 * 64 * 2 and z.pool == 10 * 2 * 16 * 64 * 2
    assert z.table == z.row == 3 * 5 * 4 and z.per_seq == 3 * 4
    assert z.summaries == 10 * 2 * 64 * 4 and z.spans == 3 * 6 * 2 * 4
    assert z.out == 3 * 8 * 64 * 4 and z.lse == 3 * 8 * 4 and z.new_rows == 3 * 2 * 64 * 2
    assert z.cache_dtype == torch.float16


def test_binding_rejects_host_tensors_and_short_buffers():
    with pytest.raises(ValueError, match="contiguous device tensor"):
        kvsp._ptr(torch.zeros(4), "x", 16, torch.float32)
    with pytest.raises(ValueError, match="needs 64"):
        kvsp._ptr(_FakeHostBuffer(32), "k_pool", 64)
    assert kvsp._ptr(_FakeHostBuffer(64), "k_pool", 64).value == 0x1000
    assert kvsp._ptr(None, "lse") is None
    lay = _layout()
    with pytest.raises(ValueError):
        kvsp.kvsp_build_summaries(lay, torch.zeros(4), torch.zeros(4, dtype=torch.int32),
                                  torch.zeros(2, dtype=torch.int32), torch.zeros(4))


def test_budget_controller_rejects_bad_arguments_and_writes_nothing():
    lib = kvsp.library()
    num = ctypes.c_int32(-7)
    c, r = ctypes.c_double(-1.0), ctypes.c_double(-1.0)
    good = kvsp.kvsp_budget_model(25e9, 1e14, 4096)

    def call(layout, model, den, out=True):
        return lib.kvsp_budget_keep_ratio(
            ctypes.byref(layout) if layout is not None else None,
            ctypes.byref(model) if model is not None else None, den, ctypes.byref(c),
            ctypes.byref(r), ctypes.byref(num) if out else None)

    assert call(_layout(), good, 1024) == 0 and 1 <= num.value <= 1024
    num.value, c.value, r.value = -7, -1.0, -1.0
    bad_models = [kvsp.kvsp_budget_model(0.0, 1e14, 4096), kvsp.kvsp_budget_model(-1.0, 1e14, 4096),
                  kvsp.kvsp_budget_model(float("inf"), 1e14, 4096),
                  kvsp.kvsp_budget_model(float("nan"), 1e14, 4096),
                  kvsp.kvsp_budget_model(25e9, 0.0, 4096), kvsp.kvsp_budget_model(25e9, float("nan"), 4096),
                  kvsp.kvsp_budget_model(25e9, 1e14, 0), kvsp.kvsp_budget_model(25e9, 1e14, -5)]
    for m in bad_models:
        assert call(_layout(), m, 1024) == -1
    assert call(_layout(), None, 1024) == -1
    assert call(_layout(), good, 0) == -1
    assert call(_layout(), good, -3) == -1
    assert call(_layout(), good, 1024, out=False) == -1
    assert call(None, good, 1024) == -1
    assert call(_layout(head_dim=96), good, 1024) == -2
    assert call(_layout(batch=0), good, 1024) == -1
    assert (num.value, c.value, r.value) == (-7, -1.0, -1.0)
    # the outputs for the prices may be NULL
    assert lib.kvsp_budget_keep_ratio(ctypes.byref(_layout()), ctypes.byref(good), 1024, None,
                                      None, ctypes.byref(num)) == 0
    with pytest.raises(kvsp.KvspError):
        kvsp.kvsp_budget_keep_ratio(_layout(), kvsp.BudgetModel(0.0, 1e14, 4096), 1024)


def test_noalloc_decode_checks_arguments_before_any_device_call():
    # the allocation-free decode rejects what kvsp_sparse_decode rejects, and
    # layouts beyond its static scratch, before it looks the scratch up
    lib = kvsp.library()
    lay, par = _layout(), _params()
    kept = [FAKE, FAKE, None, None]
    assert lib.kvsp_sparse_decode_noalloc(ctypes.byref(lay), ctypes.byref(par), *([FAKE] * 5),
                                          FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(0), FAKE,
                                          FAKE, None) == -1  # both forms of the kept blocks
    assert lib.kvsp_sparse_decode_noalloc(ctypes.byref(lay), ctypes.byref(par), FAKE, None,
                                          *([FAKE] * 3), *kept, FAKE, ctypes.c_float(0), FAKE,
                                          FAKE, None) == -1  # no K pool
    assert lib.kvsp_sparse_decode_noalloc(ctypes.byref(_layout(head_dim=96)), ctypes.byref(par),
                                          *([FAKE] * 5), *kept, FAKE, ctypes.c_float(0), FAKE,
                                          FAKE, None) == -2
    assert lib.kvsp_sparse_decode_noalloc(ctypes.byref(lay), ctypes.byref(_params(keep_den=0)),
                                          *([FAKE] * 5), *kept, FAKE, ctypes.c_float(0), FAKE,
                                          FAKE, None) == -1
    # 8192 sequences x 8 KV heads: 65536 completion counters, beyond the 16384
    # the static scratch holds
    big = _layout(batch=8192, num_kv_heads=8, num_q_heads=32)
    assert lib.kvsp_sparse_decode_noalloc(ctypes.byref(big), ctypes.byref(par), *([FAKE] * 5),
                                          *kept, FAKE, ctypes.c_float(0), FAKE, FAKE, None) == -5
    assert "static scratch" in kvsp.status_string(-5)
