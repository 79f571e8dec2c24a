"""GPU parity of the decode-time append (kvsp_append_kv) against the oracle.

A decode loop appends one token per sequence and step, with ragged starting
lengths, a shuffled pool and sequences that skip steps. After every step the
pools are compared byte for byte with the oracle's; every block a token
completes must carry the oracle's mean key (within one float32 ulp, the
summary bar) and be bit-identical to kvsp_build_summaries on the same pool.
Then a full decode step on the grown cache, scored from the summaries the
appends maintained, must meet every parity bar."""

import numpy as np
import pytest
import torch

import oracle
from query_aware_sparse_block_amd import device as dev
from query_aware_sparse_block_amd import workloads as wl
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _host(t, dtype):
    t = t.cpu()
    return t.numpy() if dtype == "fp32" else t.view(torch.int16).numpy().view(np.uint16)


def _ulp_close(got, ref):
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    return np.all(np.abs(got.astype(np.float64) - ref) <= ulp + 1e-30)


@pytest.mark.parametrize("dtype,Hq,Hkv,D,P", [("bf16", 8, 2, 128, 16), ("fp16", 4, 4, 64, 16),
                                              ("fp32", 6, 3, 64, 32), ("bf16", 16, 1, 128, 64),
                                              ("fp16", 12, 2, 128, 32), ("fp32", 8, 8, 128, 16)])
def test_decode_loop_appends_match_oracle(dtype, Hq, Hkv, D, P):
    B, steps = 3, 2 * P + 3
    start = np.array([P - 2, 3 * P, 5], np.int32)
    max_blocks = int(-(-(int(start.max()) + steps) // P))
    H.note(f"[append] {dtype} Hq={Hq} Hkv={Hkv} D={D} P={P} steps={steps}")
    case = wl.make_case(f"append-{dtype}", seed=80 + D + P, B=B, Hq=Hq, Hkv=Hkv, D=D, P=P,
                        dtype=dtype, ctx_lens=start, shuffle=True, max_blocks=max_blocks,
                        num_phys=B * max_blocks + 5, top_k=3, keep_floor=1, recent_window=P)
    dc = dev.upload(case)
    buf = dev.alloc_buffers(dc)
    dev.build_summaries(dc, buf)
    ref = dev.alloc_buffers(dc)
    k_host, v_host = case.k_pool.copy(), case.v_pool.copy()
    rng = np.random.default_rng(90 + D)
    ctx = start.copy()
    fills = 0
    for step in range(steps):
        k_new = wl.encode(rng.standard_normal((B, Hkv, D)).astype(np.float32), dtype)
        v_new = wl.encode(rng.standard_normal((B, Hkv, D)).astype(np.float32), dtype)
        pos = ctx.copy()
        pos[step % B] = -1 if step % 4 == 3 else pos[step % B]  # some steps skip a sequence
        dev.append_kv(dc, buf, dev.to_device(k_new, dtype, "cuda"),
                      dev.to_device(v_new, dtype, "cuda"), torch.from_numpy(pos).cuda())
        filled, flags = oracle.append(dtype, k_host, v_host, k_new, v_new, case.block_table, pos,
                                      Hkv=Hkv, P=P, D=D)
        torch.cuda.synchronize()
        assert np.array_equal(_host(dc.k_pool, dtype), k_host), f"K pool differs at step {step}"
        assert np.array_equal(_host(dc.v_pool, dtype), v_host), f"V pool differs at step {step}"
        gsum = buf.summaries.cpu().numpy()
        for b in np.nonzero(flags)[0]:
            phys = case.block_table[b, pos[b] // P]
            assert _ulp_close(gsum[phys], filled[b]), f"summary of b={b} off at step {step}"
            fills += 1
        ctx = np.where(pos >= 0, ctx + 1, ctx).astype(np.int32)
    assert fills >= B  # every sequence completed at least one block
    # the same summaries from the batch builder on the final pool, bit for bit
    grown = wl.Case(**{**case.__dict__, "k_pool": k_host, "v_pool": v_host, "ctx_lens": ctx})
    dc.ctx_lens.copy_(torch.from_numpy(ctx))
    dev.build_summaries(dc, ref)
    torch.cuda.synchronize()
    s_app, s_ref = buf.summaries.cpu().numpy(), ref.summaries.cpu().numpy()
    for b in range(B):
        phys = case.block_table[b, :ctx[b] // P]
        assert np.array_equal(s_app[phys], s_ref[phys])
    # a decode step on the grown cache, scored from the appended summaries
    dev.score_topk(dc, buf)
    dev.sparse_decode(dc, buf)
    torch.cuda.synchronize()
    gpu = {k: getattr(buf, k).cpu().numpy() for k in
           ("scores", "selected", "num_selected", "spans", "num_spans", "use_dense", "out", "lse")}
    summ = H.oracle_summaries(grown)
    r_or = oracle.decode_step(dtype, grown.q, k_host, v_host, grown.block_table, ctx, summ,
                              Hkv=Hkv, P=P, **grown.select_params)
    T = H.term_sums(grown, summ)
    H.check_scores(grown, r_or, gpu, T)
    for b in range(B):
        sel = H.check_selection(grown, r_or, gpu, b, T)
        H.check_outputs(grown, r_or, gpu, b, sel)


def test_append_at_the_bench_shape_rewrites_and_summarises_in_place():
    # OPT-like batch, L8192: appending each sequence's last token again (its
    # own row) leaves the pool unchanged and re-derives the last block's
    # summary bit-identically to the batch builder
    case = wl.c2(L=8192, keep="1/2")
    H.note("[append] c2 L8192 in-place")
    dc = dev.upload(case)
    buf = dev.alloc_buffers(dc)
    dev.build_summaries(dc, buf)
    torch.cuda.synchronize()
    before = buf.summaries.clone()
    L, P = 8192, case.P
    last = torch.from_numpy(case.block_table[:, (L - 1) // P].astype(np.int64)).cuda()
    k_new = dc.k_pool[last, :, P - 1].contiguous()
    v_new = dc.v_pool[last, :, P - 1].contiguous()
    k0 = dc.k_pool.clone()
    buf.summaries[last] = 0.0
    dev.append_kv(dc, buf, k_new, v_new, torch.full((case.B,), L - 1, dtype=torch.int32,
                                                     device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(dc.k_pool, k0)
    assert torch.equal(buf.summaries, before)
