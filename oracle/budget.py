"""Reference oracle for the dynamic budget controller, plain Python floats.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module; the library under
``query_aware_sparse_block_amd`` never does.

Source: SparPR news page ("SparPR: Runtime KV-Cache Recovery for
Resource-Constrained LLM Inference on Consumer Hardware"), section "Three
decisions rather than one compression ratio", paragraph "Dynamic budget
control". One block is priced two ways:
- copying it to the GPU: its data volume over the host-to-device bandwidth,
  counted twice because keys and values both travel;
- recomputing it: proportional to the block length and to the square of the
  hidden size, because the states are rebuilt from a checkpoint through the
  attention projection only.
The ratio of the two prices sets the keep ratio, which the Minimum Keep Floor
then bounds from below.

Readings where the page is silent:
- the volume is that of one KV tensor of the block over all KV heads
  (block_size x num_kv_heads x head_dim elements), so the copy price is
  2 x that volume / bandwidth;
- the recompute price is the flop count of the K and V projections of
  block_size hidden states (2 x block_size x hidden x (num_kv_heads x
  head_dim) each) over a measured projection throughput; with multi-head
  attention num_kv_heads x head_dim = hidden, which gives the page's
  block length x hidden squared;
- the map from the ratio to the keep ratio is min(1, recompute / copy);
- the keep ratio is handed to the selection as keep_num / keep_den with
  keep_num = min(keep_den, max(1, ceil(ratio x keep_den))) (rounded up, never
  zero); the selection's keep floor is the page's Minimum Keep Floor.
The arithmetic is IEEE double, as in the library (the rounding-up decision is
taken in the same precision).
"""

from __future__ import annotations

import math


def copy_seconds(block_size: int, num_kv_heads: int, head_dim: int, elem_bytes: int,
                 h2d_bytes_per_s: float) -> float:
    """Copy price of one block: data volume / host-to-device bandwidth, x2 for K and V."""
    volume = block_size * num_kv_heads * head_dim * elem_bytes  # bytes of K (or of V)
    return 2 * volume / h2d_bytes_per_s


def recompute_seconds(block_size: int, hidden: int, num_kv_heads: int, head_dim: int,
                      proj_flops_per_s: float) -> float:
    """Recompute price of one block: the K and V projections of its hidden states."""
    one_projection = 2 * block_size * hidden * (num_kv_heads * head_dim)  # multiply-adds x 2
    return 2 * one_projection / proj_flops_per_s


def keep_ratio(copy_s: float, recompute_s: float) -> float:
    """The ratio of the two prices, read as the keep ratio (at most 1)."""
    return min(1.0, recompute_s / copy_s)


def keep_num(ratio: float, keep_den: int) -> int:
    """The keep ratio in units of 1/keep_den, rounded up, at least 1."""
    return min(keep_den, max(1, math.ceil(ratio * keep_den)))


def controller(block_size, num_kv_heads, head_dim, elem_bytes, hidden, h2d_bytes_per_s,
               proj_flops_per_s, keep_den):
    """(keep_num, copy_s, recompute_s) for one model and machine."""
    c = copy_seconds(block_size, num_kv_heads, head_dim, elem_bytes, h2d_bytes_per_s)
    r = recompute_seconds(block_size, hidden, num_kv_heads, head_dim, proj_flops_per_s)
    return keep_num(keep_ratio(c, r), keep_den), c, r
