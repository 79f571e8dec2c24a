"""Python binding of libkvsp (see include/kvsp.h for the contract).

Argument marshalling only: shapes become a ``kvsp_layout``, tensors become
device pointers, the current torch stream becomes the ``hipStream_t``. Every
step of the computation runs in the HIP kernels of libkvsp.so; there is no
fallback. Importing this module does not load the library; the first call
does, and it raises if the library has not been built.
"""

from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# KVSP_LIBRARY selects another build of the same library (e.g. a tuning variant).
LIB_PATH = os.environ.get("KVSP_LIBRARY") or os.path.join(_PKG, "libkvsp.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "kvsp.h")

KVSP_OK = 0
STATUS_NAMES = {0: "KVSP_OK", -1: "KVSP_ERR_INVALID_ARG", -2: "KVSP_ERR_UNSUPPORTED",
                -3: "KVSP_ERR_WORKSPACE", -4: "KVSP_ERR_HIP", -5: "KVSP_ERR_TOO_LARGE"}
DTYPE_CODES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}


class kvsp_layout(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("num_phys_blocks", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class kvsp_select_params(ctypes.Structure):
    _fields_ = [("top_k", ctypes.c_int32), ("keep_num", ctypes.c_int32),
                ("keep_den", ctypes.c_int32), ("keep_floor", ctypes.c_int32),
                ("recent_window", ctypes.c_int32), ("gamma_num", ctypes.c_int32),
                ("gamma_den", ctypes.c_int32)]


class kvsp_dkv_params(ctypes.Structure):
    _fields_ = [("rank", ctypes.c_int32), ("n_resid", ctypes.c_int32),
                ("power_iters", ctypes.c_int32)]


class kvsp_budget_model(ctypes.Structure):
    _fields_ = [("h2d_bytes_per_s", ctypes.c_double), ("proj_flops_per_s", ctypes.c_double),
                ("hidden", ctypes.c_int32)]


class KvspError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {STATUS_NAMES.get(status, status)} "
                         f"({status_string(status)})")
        self.status = status


_lib = None


def library() -> ctypes.CDLL:
    """The loaded libkvsp.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m query_aware_sparse_block_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        LP, SP = ctypes.POINTER(kvsp_layout), ctypes.POINTER(kvsp_select_params)
        L.kvsp_abi_version.restype = i32
        L.kvsp_status_string.restype = ctypes.c_char_p
        L.kvsp_status_string.argtypes = [ctypes.c_int]
        L.kvsp_workspace_bytes.restype = sz
        L.kvsp_workspace_bytes.argtypes = [LP, SP]
        L.kvsp_append_kv.restype = ctypes.c_int
        L.kvsp_append_kv.argtypes = [LP, P, P, P, P, P, P, P, P]
        L.kvsp_build_summaries.restype = ctypes.c_int
        L.kvsp_build_summaries.argtypes = [LP, P, P, P, P, P]
        L.kvsp_score_topk.restype = ctypes.c_int
        L.kvsp_score_topk.argtypes = [LP, SP, P, P, P, P, P, P, P, P, P, P, P, sz, P]
        L.kvsp_sparse_decode.restype = ctypes.c_int
        L.kvsp_sparse_decode.argtypes = [LP, SP, P, P, P, P, P, P, P, P, P, P, ctypes.c_float, P,
                                         P, P, sz, P]
        L.kvsp_sparse_decode_noalloc.restype = ctypes.c_int
        L.kvsp_sparse_decode_noalloc.argtypes = [LP, SP, P, P, P, P, P, P, P, P, P, P,
                                                 ctypes.c_float, P, P, P]
        L.kvsp_dense_decode.restype = ctypes.c_int
        L.kvsp_dense_decode.argtypes = [LP, P, P, P, P, P, ctypes.c_float, P, P, P, sz, P]
        DP = ctypes.POINTER(kvsp_dkv_params)
        L.kvsp_dkv_record_bytes.restype = sz
        L.kvsp_dkv_record_bytes.argtypes = [LP, DP]
        L.kvsp_dkv_workspace_bytes.restype = sz
        L.kvsp_dkv_workspace_bytes.argtypes = [LP, DP]
        L.kvsp_dkv_compress.restype = ctypes.c_int
        L.kvsp_dkv_compress.argtypes = [LP, DP, i32, P, P, P, P, P, P]
        L.kvsp_dkv_decode.restype = ctypes.c_int
        L.kvsp_dkv_decode.argtypes = [LP, SP, DP, P, P, P, P, P, P, P, P, ctypes.c_float, P, P,
                                      P, sz, P]
        BP = ctypes.POINTER(kvsp_budget_model)
        L.kvsp_budget_keep_ratio.restype = ctypes.c_int
        L.kvsp_budget_keep_ratio.argtypes = [LP, BP, i32, ctypes.POINTER(ctypes.c_double),
                                             ctypes.POINTER(ctypes.c_double),
                                             ctypes.POINTER(ctypes.c_int32)]
        _lib = L
    return _lib


def declared_entry_points(header: str = HEADER_PATH) -> list[str]:
    """Function names declared in the public header."""
    text = open(header).read()
    return sorted(set(re.findall(r"\b(kvsp_[a-z_]+)\s*\(", text)))


def status_string(status: int) -> str:
    return library().kvsp_status_string(int(status)).decode()


kvsp_status_string = status_string


@dataclass
class SelectParams:
    top_k: int = 0
    keep_num: int = 1
    keep_den: int = 1
    keep_floor: int = 1
    recent_window: int = 0
    gamma_num: int = 1
    gamma_den: int = 1

    def c(self) -> kvsp_select_params:
        return kvsp_select_params(self.top_k, self.keep_num, self.keep_den, self.keep_floor,
                                  self.recent_window, self.gamma_num, self.gamma_den)


def make_layout(q: torch.Tensor, k_pool: torch.Tensor, block_table: torch.Tensor) -> kvsp_layout:
    """Layout from tensor shapes: q [B][Hq][D], pool [phys][Hkv][P][D],
    block_table [B][max_blocks]."""
    B, Hq, D = q.shape
    num_phys, Hkv, P, Dk = k_pool.shape
    assert Dk == D and block_table.shape[0] == B, "shape mismatch"
    return kvsp_layout(B, Hq, Hkv, D, P, num_phys, block_table.shape[1], DTYPE_CODES[q.dtype])


_ELEM_BYTES = {0: 4, 1: 2, 2: 2}
_CODE_DTYPES = {0: torch.float32, 1: torch.float16, 2: torch.bfloat16}


def _ptr(t, name="argument", nbytes=None, dtype=None):
    """Device address of a contiguous device tensor, or of a mapped pinned
    host buffer (an object with `device_ptr` and `nbytes`). With `nbytes`
    and `dtype` the buffer is checked against what the layout needs, so a
    short or mistyped buffer raises here instead of reaching a kernel. None
    passes through (the C entry points reject missing required pointers)."""
    if t is None:
        return None
    if hasattr(t, "device_ptr"):
        if nbytes is not None and t.nbytes < nbytes:
            raise ValueError(f"{name}: {t.nbytes} bytes, the layout needs {nbytes}")
        return ctypes.c_void_p(t.device_ptr)
    if not (t.is_cuda and t.is_contiguous()):
        raise ValueError(f"{name}: a contiguous device tensor is required")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if nbytes is not None and t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name}: {t.numel() * t.element_size()} bytes, the layout needs {nbytes}")
    return ctypes.c_void_p(t.data_ptr())


class _Sizes:
    """Bytes each buffer of the C ABI holds for a layout (kvsp.h layouts)."""

    def __init__(self, L: kvsp_layout):
        E = _ELEM_BYTES.get(L.dtype, 0)
        self.cache_dtype = _CODE_DTYPES.get(L.dtype)
        self.q = L.batch * L.num_q_heads * L.head_dim * E
        self.pool = L.num_phys_blocks * L.num_kv_heads * L.block_size * L.head_dim * E
        self.table = L.batch * L.max_blocks_per_seq * 4
        self.per_seq = L.batch * 4
        self.summaries = L.num_phys_blocks * L.num_kv_heads * L.head_dim * 4
        self.row = L.batch * L.max_blocks_per_seq * 4
        self.spans = L.batch * (L.max_blocks_per_seq + 1) * 2 * 4
        self.out = L.batch * L.num_q_heads * L.head_dim * 4
        self.lse = L.batch * L.num_q_heads * 4
        self.new_rows = L.batch * L.num_kv_heads * L.head_dim * E


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn: str, status: int):
    if status != KVSP_OK:
        raise KvspError(fn, status)


def kvsp_workspace_bytes(layout: kvsp_layout, params: SelectParams | None = None) -> int:
    p = (params or SelectParams()).c()
    return int(library().kvsp_workspace_bytes(ctypes.byref(layout), ctypes.byref(p)))


def alloc_workspace(layout: kvsp_layout, params: SelectParams | None = None,
                    device="cuda") -> torch.Tensor:
    n = kvsp_workspace_bytes(layout, params)
    return torch.zeros(max(n, 1), dtype=torch.uint8, device=device)  # counters start at zero


I32, F32 = torch.int32, torch.float32


def kvsp_append_kv(layout, k_new, v_new, block_table, positions, k_pool, v_pool, summaries,
                   stream=None):
    z = _Sizes(layout)
    _check("kvsp_append_kv", library().kvsp_append_kv(
        ctypes.byref(layout), _ptr(k_new, "k_new", z.new_rows, z.cache_dtype),
        _ptr(v_new, "v_new", z.new_rows, z.cache_dtype), _ptr(block_table, "block_table", z.table, I32),
        _ptr(positions, "positions", z.per_seq, I32), _ptr(k_pool, "k_pool", z.pool, z.cache_dtype),
        _ptr(v_pool, "v_pool", z.pool, z.cache_dtype), _ptr(summaries, "summaries", z.summaries, F32),
        _stream(stream)))


def kvsp_build_summaries(layout, k_pool, block_table, context_lens, summaries, stream=None):
    z = _Sizes(layout)
    _check("kvsp_build_summaries", library().kvsp_build_summaries(
        ctypes.byref(layout), _ptr(k_pool, "k_pool", z.pool, z.cache_dtype),
        _ptr(block_table, "block_table", z.table, I32),
        _ptr(context_lens, "context_lens", z.per_seq, I32),
        _ptr(summaries, "summaries", z.summaries, F32), _stream(stream)))


def kvsp_score_topk(layout, params: SelectParams, q, summaries, block_table, context_lens, scores,
                    selected, num_selected, spans, num_spans, use_dense, workspace=None,
                    stream=None):
    p = params.c()
    z = _Sizes(layout)
    ws_bytes = workspace.numel() if workspace is not None else 0
    _check("kvsp_score_topk", library().kvsp_score_topk(
        ctypes.byref(layout), ctypes.byref(p), _ptr(q, "q", z.q, z.cache_dtype),
        _ptr(summaries, "summaries", z.summaries, F32), _ptr(block_table, "block_table", z.table, I32),
        _ptr(context_lens, "context_lens", z.per_seq, I32), _ptr(scores, "scores", z.row, F32),
        _ptr(selected, "selected", z.row, I32), _ptr(num_selected, "num_selected", z.per_seq, I32),
        _ptr(spans, "spans", z.spans, I32), _ptr(num_spans, "num_spans", z.per_seq, I32),
        _ptr(use_dense, "use_dense", z.per_seq, I32), _ptr(workspace, "workspace"), ws_bytes,
        _stream(stream)))


def kvsp_sparse_decode(layout, params: SelectParams, q, k_pool, v_pool, block_table, context_lens,
                       spans, num_spans, selected, num_selected, use_dense, scale, out, lse,
                       workspace, stream=None):
    """The kept blocks come as (spans, num_spans) or as (selected,
    num_selected); pass None for the other pair."""
    p = params.c()
    z = _Sizes(layout)
    _check("kvsp_sparse_decode", library().kvsp_sparse_decode(
        ctypes.byref(layout), ctypes.byref(p), _ptr(q, "q", z.q, z.cache_dtype),
        _ptr(k_pool, "k_pool", z.pool, z.cache_dtype), _ptr(v_pool, "v_pool", z.pool, z.cache_dtype),
        _ptr(block_table, "block_table", z.table, I32),
        _ptr(context_lens, "context_lens", z.per_seq, I32), _ptr(spans, "spans", z.spans, I32),
        _ptr(num_spans, "num_spans", z.per_seq, I32), _ptr(selected, "selected", z.row, I32),
        _ptr(num_selected, "num_selected", z.per_seq, I32), _ptr(use_dense, "use_dense", z.per_seq, I32),
        ctypes.c_float(scale), _ptr(out, "out", z.out, F32), _ptr(lse, "lse", z.lse, F32),
        _ptr(workspace, "workspace"), workspace.numel(), _stream(stream)))


def kvsp_sparse_decode_noalloc(layout, params: SelectParams, q, k_pool, v_pool, block_table,
                               context_lens, spans, num_spans, selected, num_selected, use_dense,
                               scale, out, lse, stream=None):
    """kvsp_sparse_decode without a workspace: the library's static device
    scratch holds its counters and partials (see kvsp.h)."""
    p = params.c()
    z = _Sizes(layout)
    _check("kvsp_sparse_decode_noalloc", library().kvsp_sparse_decode_noalloc(
        ctypes.byref(layout), ctypes.byref(p), _ptr(q, "q", z.q, z.cache_dtype),
        _ptr(k_pool, "k_pool", z.pool, z.cache_dtype), _ptr(v_pool, "v_pool", z.pool, z.cache_dtype),
        _ptr(block_table, "block_table", z.table, I32),
        _ptr(context_lens, "context_lens", z.per_seq, I32), _ptr(spans, "spans", z.spans, I32),
        _ptr(num_spans, "num_spans", z.per_seq, I32), _ptr(selected, "selected", z.row, I32),
        _ptr(num_selected, "num_selected", z.per_seq, I32), _ptr(use_dense, "use_dense", z.per_seq, I32),
        ctypes.c_float(scale), _ptr(out, "out", z.out, F32), _ptr(lse, "lse", z.lse, F32),
        _stream(stream)))


def kvsp_dense_decode(layout, q, k_pool, v_pool, block_table, context_lens, scale, out, lse,
                      workspace, stream=None):
    z = _Sizes(layout)
    _check("kvsp_dense_decode", library().kvsp_dense_decode(
        ctypes.byref(layout), _ptr(q, "q", z.q, z.cache_dtype),
        _ptr(k_pool, "k_pool", z.pool, z.cache_dtype), _ptr(v_pool, "v_pool", z.pool, z.cache_dtype),
        _ptr(block_table, "block_table", z.table, I32),
        _ptr(context_lens, "context_lens", z.per_seq, I32), ctypes.c_float(scale),
        _ptr(out, "out", z.out, F32), _ptr(lse, "lse", z.lse, F32), _ptr(workspace, "workspace"),
        workspace.numel(), _stream(stream)))


@dataclass
class BudgetModel:
    h2d_bytes_per_s: float
    proj_flops_per_s: float
    hidden: int

    def c(self) -> kvsp_budget_model:
        return kvsp_budget_model(float(self.h2d_bytes_per_s), float(self.proj_flops_per_s),
                                 int(self.hidden))


def kvsp_budget_keep_ratio(layout: kvsp_layout, model: BudgetModel, keep_den: int):
    """(keep_num, copy_s, recompute_s) of the budget controller; keep_num / keep_den
    is the keep ratio for SelectParams."""
    m = model.c()
    num = ctypes.c_int32(-1)
    copy_s, rec_s = ctypes.c_double(0.0), ctypes.c_double(0.0)
    _check("kvsp_budget_keep_ratio", library().kvsp_budget_keep_ratio(
        ctypes.byref(layout), ctypes.byref(m), int(keep_den), ctypes.byref(copy_s),
        ctypes.byref(rec_s), ctypes.byref(num)))
    return int(num.value), float(copy_s.value), float(rec_s.value)


@dataclass
class DkvParams:
    rank: int = 32
    n_resid: int = 16
    power_iters: int = 0

    def c(self) -> kvsp_dkv_params:
        return kvsp_dkv_params(self.rank, self.n_resid, self.power_iters)


def kvsp_dkv_record_bytes(layout: kvsp_layout, dkv: DkvParams) -> int:
    p = dkv.c()
    return int(library().kvsp_dkv_record_bytes(ctypes.byref(layout), ctypes.byref(p)))


def kvsp_dkv_workspace_bytes(layout: kvsp_layout, dkv: DkvParams) -> int:
    p = dkv.c()
    return int(library().kvsp_dkv_workspace_bytes(ctypes.byref(layout), ctypes.byref(p)))


def alloc_dkv_workspace(layout: kvsp_layout, dkv: DkvParams, device="cuda") -> torch.Tensor:
    n = kvsp_dkv_workspace_bytes(layout, dkv)
    return torch.zeros(max(n, 1), dtype=torch.uint8, device=device)  # counters start at zero


def kvsp_dkv_compress(layout, dkv: DkvParams, recent_window, k_pool, v_pool, block_table,
                      context_lens, records, stream=None):
    p = dkv.c()
    z = _Sizes(layout)
    rec = kvsp_dkv_record_bytes(layout, dkv) * layout.num_phys_blocks * layout.num_kv_heads
    _check("kvsp_dkv_compress", library().kvsp_dkv_compress(
        ctypes.byref(layout), ctypes.byref(p), int(recent_window),
        _ptr(k_pool, "k_pool", z.pool, z.cache_dtype), _ptr(v_pool, "v_pool", z.pool, z.cache_dtype),
        _ptr(block_table, "block_table", z.table, I32),
        _ptr(context_lens, "context_lens", z.per_seq, I32), _ptr(records, "records", rec),
        _stream(stream)))


def kvsp_dkv_decode(layout, params: SelectParams, dkv: DkvParams, q, k_pool, v_pool, records,
                    block_table, context_lens, selected, num_selected, scale, out, lse, workspace,
                    stream=None):
    p = params.c()
    d = dkv.c()
    z = _Sizes(layout)
    rec = kvsp_dkv_record_bytes(layout, dkv) * layout.num_phys_blocks * layout.num_kv_heads
    _check("kvsp_dkv_decode", library().kvsp_dkv_decode(
        ctypes.byref(layout), ctypes.byref(p), ctypes.byref(d), _ptr(q, "q", z.q, z.cache_dtype),
        _ptr(k_pool, "k_pool", z.pool, z.cache_dtype), _ptr(v_pool, "v_pool", z.pool, z.cache_dtype),
        _ptr(records, "records", rec), _ptr(block_table, "block_table", z.table, I32),
        _ptr(context_lens, "context_lens", z.per_seq, I32), _ptr(selected, "selected", z.row, I32),
        _ptr(num_selected, "num_selected", z.per_seq, I32), ctypes.c_float(scale),
        _ptr(out, "out", z.out, F32), _ptr(lse, "lse", z.lse, F32), _ptr(workspace, "workspace"),
        workspace.numel(), _stream(stream)))
