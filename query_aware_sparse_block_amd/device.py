"""Device-side plumbing: upload a synthetic workload, own the output buffers,
and enqueue one decode step through the C ABI. PyTorch only provides device
memory and the stream; every computation is a libkvsp kernel."""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import kvsp
from .workloads import Case

_TORCH_DTYPE = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


def to_device(arr: np.ndarray, dtype: str | None, device) -> torch.Tensor:
    """Host array -> device tensor. 16-bit payloads travel as their bits."""
    if dtype in ("fp16", "bf16"):
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16))
        return t.to(device).view(_TORCH_DTYPE[dtype])
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


@dataclass
class DeviceCase:
    case: Case
    q: torch.Tensor
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    block_table: torch.Tensor
    ctx_lens: torch.Tensor
    layout: kvsp.kvsp_layout
    params: kvsp.SelectParams


def upload(case: Case, device="cuda") -> DeviceCase:
    q = to_device(case.q, case.dtype, device)
    k = to_device(case.k_pool, case.dtype, device)
    v = to_device(case.v_pool, case.dtype, device)
    bt = to_device(case.block_table.astype(np.int32), None, device)
    cl = to_device(case.ctx_lens.astype(np.int32), None, device)
    layout = kvsp.make_layout(q, k, bt)
    params = kvsp.SelectParams(**case.select_params)
    return DeviceCase(case, q, k, v, bt, cl, layout, params)


def with_host_pool(dc: DeviceCase) -> DeviceCase:
    """The same case with its K/V pool in mapped pinned host memory (queries,
    block table and lengths stay on the device). The kernels then read the
    pool across PCIe, and only the tiles they attend."""
    from . import hostmem
    return DeviceCase(dc.case, dc.q, hostmem.host_copy(dc.case.k_pool),
                      hostmem.host_copy(dc.case.v_pool), dc.block_table, dc.ctx_lens, dc.layout,
                      dc.params)


@dataclass
class StepBuffers:
    summaries: torch.Tensor
    scores: torch.Tensor
    selected: torch.Tensor
    num_selected: torch.Tensor
    spans: torch.Tensor
    num_spans: torch.Tensor
    use_dense: torch.Tensor
    out: torch.Tensor
    lse: torch.Tensor
    workspace: torch.Tensor


def alloc_buffers(dc: DeviceCase) -> StepBuffers:
    L = dc.layout
    dev = dc.q.device
    B, mb = L.batch, L.max_blocks_per_seq
    i32 = torch.int32
    return StepBuffers(
        summaries=torch.zeros((L.num_phys_blocks, L.num_kv_heads, L.head_dim), dtype=torch.float32,
                              device=dev),
        scores=torch.zeros((B, mb), dtype=torch.float32, device=dev),
        selected=torch.full((B, mb), -1, dtype=i32, device=dev),
        num_selected=torch.zeros(B, dtype=i32, device=dev),
        spans=torch.full((B, mb + 1, 2), -1, dtype=i32, device=dev),
        num_spans=torch.zeros(B, dtype=i32, device=dev),
        use_dense=torch.zeros(B, dtype=i32, device=dev),
        out=torch.zeros((B, L.num_q_heads, L.head_dim), dtype=torch.float32, device=dev),
        lse=torch.zeros((B, L.num_q_heads), dtype=torch.float32, device=dev),
        workspace=kvsp.alloc_workspace(L, dc.params, dev),
    )


def build_summaries(dc: DeviceCase, buf: StepBuffers, stream=None):
    kvsp.kvsp_build_summaries(dc.layout, dc.k_pool, dc.block_table, dc.ctx_lens, buf.summaries,
                              stream)


def append_kv(dc: DeviceCase, buf: StepBuffers, k_new, v_new, positions, stream=None):
    """Writes each sequence's new K/V row at positions[b] (device int32, -1 =
    none) and the summary of every block a new token completes."""
    kvsp.kvsp_append_kv(dc.layout, k_new, v_new, dc.block_table, positions, dc.k_pool, dc.v_pool,
                        buf.summaries, stream)


def score_topk(dc: DeviceCase, buf: StepBuffers, params=None, stream=None):
    kvsp.kvsp_score_topk(dc.layout, params or dc.params, dc.q, buf.summaries, dc.block_table,
                         dc.ctx_lens, buf.scores, buf.selected, buf.num_selected, buf.spans,
                         buf.num_spans, buf.use_dense, buf.workspace, stream)


def sparse_decode(dc: DeviceCase, buf: StepBuffers, params=None, scale=0.0, stream=None,
                  form="spans", out=None):
    """Attention over the kept blocks of kvsp_score_topk's outputs in `buf`,
    handed over as its span list (form="spans") or its selected list
    (form="selected"); into buf.out / buf.lse unless `out` is given."""
    if form == "spans":
        kept = (buf.spans, buf.num_spans, None, None)
    elif form == "selected":
        kept = (None, None, buf.selected, buf.num_selected)
    else:
        raise ValueError(f"unknown form {form!r}")
    kvsp.kvsp_sparse_decode(dc.layout, params or dc.params, dc.q, dc.k_pool, dc.v_pool,
                            dc.block_table, dc.ctx_lens, *kept, buf.use_dense, scale,
                            buf.out if out is None else out, buf.lse if out is None else None,
                            buf.workspace, stream)


def dense_decode(dc: DeviceCase, buf: StepBuffers, scale=0.0, stream=None):
    kvsp.kvsp_dense_decode(dc.layout, dc.q, dc.k_pool, dc.v_pool, dc.block_table, dc.ctx_lens,
                           scale, buf.out, buf.lse, buf.workspace, stream)


def decode_step(dc: DeviceCase, buf: StepBuffers, params=None, stream=None):
    """One decode step: score + Top-k + spans, then sparse attention (dense
    for flagged sequences). Summaries must already be resident."""
    score_topk(dc, buf, params, stream)
    sparse_decode(dc, buf, params, 0.0, stream)


# ---- DKV variant --------------------------------------------------------------------

def dkv_records_tensor(dc: DeviceCase, recs: dict, n_resid: int) -> torch.Tensor:
    """Host records keyed by (phys, g) (stored values, see workloads.dkv_pack)
    -> the device record array [num_phys][Hkv][record bytes]; absent records
    are zero bytes."""
    from . import workloads as wl
    c = dc.case
    lay = wl.dkv_record_layout(c.D, c.P, wl.ELEM_BYTES[c.dtype], n_resid)
    host = np.zeros((c.num_phys, c.Hkv, lay["bytes"]), np.uint8)
    for (phys, g), f in recs.items():
        host[phys, g] = wl.dkv_pack(f, c.dtype, c.P, n_resid)
    return torch.from_numpy(host).to(dc.q.device)


def alloc_dkv_records(dc: DeviceCase, dkv: kvsp.DkvParams) -> torch.Tensor:
    n = kvsp.kvsp_dkv_record_bytes(dc.layout, dkv)
    assert n > 0, "unsupported DKV arguments"
    L = dc.layout
    return torch.zeros((L.num_phys_blocks, L.num_kv_heads, n), dtype=torch.uint8,
                       device=dc.q.device)


def dkv_compress(dc: DeviceCase, dkv: kvsp.DkvParams, records: torch.Tensor, stream=None):
    kvsp.kvsp_dkv_compress(dc.layout, dkv, dc.params.recent_window, dc.k_pool, dc.v_pool,
                           dc.block_table, dc.ctx_lens, records, stream)


def dkv_decode(dc: DeviceCase, buf: StepBuffers, dkv: kvsp.DkvParams, records: torch.Tensor,
               workspace: torch.Tensor, scale=0.0, stream=None):
    """Attention over the compressed blocks buf.selected[:num_selected] and
    the exact window, into buf.out / buf.lse."""
    kvsp.kvsp_dkv_decode(dc.layout, dc.params, dkv, dc.q, dc.k_pool, dc.v_pool, records,
                         dc.block_table, dc.ctx_lens, buf.selected, buf.num_selected, scale,
                         buf.out, buf.lse, workspace, stream)
