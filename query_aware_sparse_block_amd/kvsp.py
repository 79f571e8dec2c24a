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
                -3: "KVSP_ERR_WORKSPACE", -4: "KVSP_ERR_HIP"}
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
        L.kvsp_sparse_decode.argtypes = [LP, SP, P, P, P, P, P, P, P, P, ctypes.c_float, P, P, P,
                                         sz, P]
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


def _ptr(t):
    """Device address of a contiguous device tensor, or of a mapped pinned
    host buffer (an object with `device_ptr`)."""
    if t is None:
        return None
    if hasattr(t, "device_ptr"):
        return ctypes.c_void_p(t.device_ptr)
    assert t.is_cuda and t.is_contiguous(), "device tensors must be contiguous"
    return ctypes.c_void_p(t.data_ptr())


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


def kvsp_append_kv(layout, k_new, v_new, block_table, positions, k_pool, v_pool, summaries,
                   stream=None):
    _check("kvsp_append_kv", library().kvsp_append_kv(
        ctypes.byref(layout), _ptr(k_new), _ptr(v_new), _ptr(block_table), _ptr(positions),
        _ptr(k_pool), _ptr(v_pool), _ptr(summaries), _stream(stream)))


def kvsp_build_summaries(layout, k_pool, block_table, context_lens, summaries, stream=None):
    _check("kvsp_build_summaries", library().kvsp_build_summaries(
        ctypes.byref(layout), _ptr(k_pool), _ptr(block_table), _ptr(context_lens),
        _ptr(summaries), _stream(stream)))


def kvsp_score_topk(layout, params: SelectParams, q, summaries, block_table, context_lens, scores,
                    selected, num_selected, spans, num_spans, use_dense, workspace=None,
                    stream=None):
    p = params.c()
    ws_bytes = workspace.numel() if workspace is not None else 0
    _check("kvsp_score_topk", library().kvsp_score_topk(
        ctypes.byref(layout), ctypes.byref(p), _ptr(q), _ptr(summaries), _ptr(block_table),
        _ptr(context_lens), _ptr(scores), _ptr(selected), _ptr(num_selected), _ptr(spans),
        _ptr(num_spans), _ptr(use_dense), _ptr(workspace), ws_bytes, _stream(stream)))


def kvsp_sparse_decode(layout, params: SelectParams, q, k_pool, v_pool, block_table, context_lens,
                       selected, num_selected, use_dense, scale, out, lse, workspace, stream=None):
    p = params.c()
    _check("kvsp_sparse_decode", library().kvsp_sparse_decode(
        ctypes.byref(layout), ctypes.byref(p), _ptr(q), _ptr(k_pool), _ptr(v_pool),
        _ptr(block_table), _ptr(context_lens), _ptr(selected), _ptr(num_selected),
        _ptr(use_dense), ctypes.c_float(scale), _ptr(out), _ptr(lse), _ptr(workspace),
        workspace.numel(), _stream(stream)))


def kvsp_dense_decode(layout, q, k_pool, v_pool, block_table, context_lens, scale, out, lse,
                      workspace, stream=None):
    _check("kvsp_dense_decode", library().kvsp_dense_decode(
        ctypes.byref(layout), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
        _ptr(context_lens), ctypes.c_float(scale), _ptr(out), _ptr(lse), _ptr(workspace),
        workspace.numel(), _stream(stream)))


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
    _check("kvsp_dkv_compress", library().kvsp_dkv_compress(
        ctypes.byref(layout), ctypes.byref(p), int(recent_window), _ptr(k_pool), _ptr(v_pool),
        _ptr(block_table), _ptr(context_lens), _ptr(records), _stream(stream)))


def kvsp_dkv_decode(layout, params: SelectParams, dkv: DkvParams, q, k_pool, v_pool, records,
                    block_table, context_lens, selected, num_selected, scale, out, lse, workspace,
                    stream=None):
    p = params.c()
    d = dkv.c()
    _check("kvsp_dkv_decode", library().kvsp_dkv_decode(
        ctypes.byref(layout), ctypes.byref(p), ctypes.byref(d), _ptr(q), _ptr(k_pool),
        _ptr(v_pool), _ptr(records), _ptr(block_table), _ptr(context_lens), _ptr(selected),
        _ptr(num_selected), ctypes.c_float(scale), _ptr(out), _ptr(lse), _ptr(workspace),
        workspace.numel(), _stream(stream)))
