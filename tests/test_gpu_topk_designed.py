"""Top-k on designed scores. The radix select takes the k-th key's top byte
first and stops at the first pass whose digit is needed whole; these cases
place that pass at each of the four bytes, cut exact ties, take ties whole,
mix signs and zeros, and tie every candidate, on the fused selection (a short
table scored by few workgroups, one and two candidates a thread) and on the
separate Top-k launch (two and five candidates a thread).

Scores are made exact: the group-summed query is e_0 (head 0 of the group
holds 1.0 in channel 0, every other query element is 0) and every summary is
0 except channel 0 of KV head 0, which holds the designed float32 value, so
score j is that value bit for bit (+0 and -0 aside, which rank equal). The
expected selection, counts and spans come from the oracle's Top-k and span
merge on the same values (SparPR, "Query-Aware key-block selection": the k
best blocks by score; "On-demand local recomputation with cost-aware
fallback": kept blocks as contiguous spans)."""

import numpy as np
import pytest
import torch

import oracle
from query_aware_sparse_block_amd import device as dev
from query_aware_sparse_block_amd import workloads as wl
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _bits(u):
    return np.asarray(u, np.uint32).view(np.float32)


def _design(kind, C, k, rng):
    """Float32 scores of C candidates for which the k-th key is decided at a
    known radix pass (or by a tie), positions shuffled."""
    top = rng.permutation(C)[:k]
    x = np.empty(C, np.float32)
    rest = np.ones(C, bool)
    rest[top] = False
    if kind == "whole-at-byte-0":    # the k best alone in their exponent range
        x[top] = rng.uniform(2.0, 4.0, k)
        x[rest] = rng.uniform(0.5, 1.0, C - k)
    elif kind == "whole-at-byte-1":  # one exponent; the top 7 mantissa bits split them
        x[top] = rng.uniform(1.75, 2.0, k)
        x[rest] = rng.uniform(1.0, 1.5, C - k)
    elif kind == "whole-at-byte-2":  # the same top 16 bits; bits 8-15 split them
        x[top] = _bits(0x3F808000 + rng.integers(0, 0x8000, k))
        x[rest] = _bits(0x3F800000 + rng.integers(0, 0x4000, C - k))
    elif kind == "all-bytes":        # distinct keys differing in the low bytes only
        x[:] = _bits(0x3F800000 + rng.permutation(C))
    elif kind in ("tie-cut", "tie-whole"):
        hi = k // 2
        n_tie = k if kind == "tie-cut" else k - hi
        order = rng.permutation(C)
        x[:] = 1.0
        x[order[:hi]] = 5.0
        x[order[hi:hi + n_tie]] = 3.0
    elif kind == "signs-and-zeros":
        x[:] = rng.choice(np.array([-2.0, -1.0, -0.0, 0.0, 1.0, 2.0], np.float32), C)
        x *= np.where(rng.random(C) < 0.5, rng.uniform(0.5, 1.5, C), 1.0).astype(np.float32)
    elif kind == "all-equal":
        x[:] = 0.75
    else:
        raise ValueError(kind)
    return x


KINDS = ("whole-at-byte-0", "whole-at-byte-1", "whole-at-byte-2", "all-bytes", "tie-cut",
         "tie-whole", "signs-and-zeros", "all-equal")


@pytest.mark.parametrize("C,k", [(200, 1), (200, 37), (500, 37), (500, 200), (1500, 20), (1500, 300),
                                 (5000, 37)])
def test_designed_scores_select_exactly(C, k):
    case = wl.make_case(f"designed-C{C}-k{k}", seed=88_000 + C + k, B=1, Hq=2, Hkv=1, D=64, P=16,
                        dtype="fp32", ctx_lens=[16 * C], shuffle=True, top_k=k, keep_floor=1,
                        recent_window=0)
    q = np.zeros_like(case.q)
    q[0, 0, 0] = 1.0
    case = wl.Case(**{**case.__dict__, "q": q})
    plan = oracle.plan(16 * C, 16, 0, top_k=k, keep_floor=1)
    assert plan["C"] == C and plan["k_eff"] == k
    dc = dev.upload(case)
    buf = dev.alloc_buffers(dc)
    phys = torch.from_numpy(case.block_table[0, :C].astype(np.int64)).cuda()
    rng = np.random.default_rng(C * 1000 + k)
    for kind in KINDS:
        H.note(f"[designed top-k] C={C} k={k} {kind}")
        x = _design(kind, C, k, rng)
        buf.summaries.zero_()
        buf.summaries[phys, 0, 0] = torch.from_numpy(x).cuda()
        dev.score_topk(dc, buf)
        torch.cuda.synchronize()
        got = buf.scores[0, :C].cpu().numpy()
        assert np.array_equal(got, x), f"{kind}: scores are not the designed values"
        sel = buf.selected[0, :k].cpu().numpy()
        expect = oracle.topk(x.astype(np.float64), k)
        assert np.array_equal(sel, expect), f"{kind}: selection"
        assert int(buf.num_selected[0]) == k
        sp = oracle.spans(expect, C, plan["n"])
        nsp = int(buf.num_spans[0])
        assert nsp == len(sp), f"{kind}: span count"
        assert np.array_equal(buf.spans[0, :nsp].cpu().numpy(), sp), f"{kind}: spans"
        assert int(buf.use_dense[0]) == plan["use_dense"]
