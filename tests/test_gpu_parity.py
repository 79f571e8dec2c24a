"""GPU parity: the HIP path through the C ABI against the oracle on the same
seeded inputs, for every workload family (scaled so the oracle finishes in
seconds where the full size would not), every dtype and head-dim variant, and
the edge cases: ragged contexts, contexts inside the window, 100 % keep, the
dense fallback, mixed dense/sparse batches, partial head groups and shuffled
physical pools. Full-size runs live in test_gpu_fullsize.py."""

import numpy as np
import pytest
import torch

import oracle
from query_aware_sparse_block_amd import workloads as wl
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("variant", ["k8", "k2", "k64", "gamma", "shuffled"])
def test_tiny_fp32(variant):
    H.full_parity(wl.c1(variant))


@pytest.mark.parametrize("L", [1024, 2048])
@pytest.mark.parametrize("keep", ["1/2", "1/10"])
def test_opt_like_fp16_scaled(L, keep):
    gpu, r_or = H.full_parity(wl.c2(L=L, keep=keep, B=2, H=8))
    for b, needles in enumerate(wl.c2(L=L, keep=keep, B=2, H=8).meta["needles"]):
        k = int(gpu["num_selected"][b])
        sel = set(gpu["selected"][b, :k].tolist())
        assert set(needles) <= sel or sel <= set(needles)


@pytest.mark.parametrize("keep", ["1/32", "1/8"])
def test_minicpm_like_bf16_scaled(keep):
    H.full_parity(wl.c3(keep=keep, L=16384))


@pytest.mark.parametrize("L", [4096, 8192])
def test_qwen_like_bf16(L):
    case = wl.c4(L=L)
    gpu, _ = H.full_parity(case)
    k = int(gpu["num_selected"][0])
    assert case.meta["buried"][0] in gpu["selected"][0, :k].tolist()


@pytest.mark.parametrize("keep", ["1/32", "7/10"])
def test_serving_bf16_scaled(keep):
    case = wl.c5(keep=keep, B=8, L=4096)
    gpu, r_or = H.full_parity(case)
    assert (gpu["use_dense"] == (1 if keep == "7/10" else 0)).all()


@pytest.mark.parametrize("dtype,D", [("fp32", 128), ("fp16", 64), ("bf16", 64), ("fp32", 64)])
def test_dtype_and_head_dim_variants(dtype, D):
    case = wl.make_case(f"var-{dtype}-D{D}", seed=61, B=3, Hq=8, Hkv=2, D=D, P=32, dtype=dtype,
                        ctx_lens=[1000, 517, 64], shuffle=True, num_phys=100, top_k=5,
                        keep_floor=2, recent_window=100)
    H.full_parity(case)


def test_ragged_mixed_dense_and_partial_groups():
    # G = 3 (padded to 4), P = 16; short sequences fall back to dense (gamma 1/2)
    case = wl.make_case("ragged", seed=62, B=6, Hq=6, Hkv=2, D=128, P=16, dtype="fp16",
                        ctx_lens=[1, 15, 200, 1000, 777, 48], shuffle=True, num_phys=400,
                        top_k=3, keep_floor=1, recent_window=32, gamma_num=1, gamma_den=2)
    gpu, r_or = H.full_parity(case)
    assert set(r_or["plan"][:, 4].tolist()) == {0, 1}   # both paths in one batch


def test_large_group_over_sixteen_heads():
    # G = 24 -> two head groups of 16
    case = wl.make_case("g24", seed=63, B=2, Hq=48, Hkv=2, D=128, P=64, dtype="bf16",
                        ctx_lens=[2048, 1500], keep_num=1, keep_den=4, recent_window=64)
    H.full_parity(case)


def test_full_keep_equals_dense_api():
    case = wl.make_case("full-keep", seed=64, B=3, Hq=8, Hkv=4, D=128, P=64, dtype="bf16",
                        ctx_lens=[3000, 640, 129], shuffle=True, num_phys=150, top_k=10 ** 6,
                        keep_floor=1, recent_window=64)
    sparse, _ = H.full_parity(case)
    dense, _, _ = H.run_gpu(case, dense_api=True)
    np.testing.assert_allclose(sparse["out"], dense["out"], rtol=0, atol=2e-6)
    # and the dense entry point against the oracle's textbook dense attention
    summ = H.oracle_summaries(case)
    r = oracle.decode_step(case.dtype, case.q, case.k_pool, case.v_pool, case.block_table,
                           case.ctx_lens, summ, Hkv=case.Hkv, P=case.P, top_k=10 ** 6,
                           recent_window=64)
    assert np.max(np.abs(dense["out"] - r["out"])) <= 2e-3


def test_context_inside_window_and_single_token():
    case = wl.make_case("tiny-ctx", seed=65, B=4, Hq=4, Hkv=4, D=64, P=16, dtype="bf16",
                        ctx_lens=[1, 5, 16, 31], top_k=2, keep_floor=1, recent_window=32)
    gpu, r_or = H.full_parity(case)
    assert (r_or["plan"][:, 1] == 0).all()
    # one cached token: the output is that token's value
    v0 = wl.decode_f32(case.v_pool[case.block_table[0, 0], :, 0], "bf16")
    np.testing.assert_allclose(gpu["out"][0], v0, atol=1e-6)


def test_dense_decode_api_matches_oracle():
    case = wl.c5(keep="1/32", B=4, L=2048)
    H.note("[dense api] c5 B=4 L=2048")
    gpu, _, _ = H.run_gpu(case, dense_api=True)
    summ = H.oracle_summaries(case)
    r = oracle.decode_step(case.dtype, case.q, case.k_pool, case.v_pool, case.block_table,
                           case.ctx_lens, summ, Hkv=case.Hkv, P=case.P, top_k=10 ** 6,
                           recent_window=0)
    assert np.max(np.abs(gpu["out"] - r["out"])) <= 2e-3
    assert np.max(np.abs(gpu["lse"] - r["lse"])) <= 1e-4


def test_deterministic_and_layout_invariant():
    case = wl.c5(keep="1/32", B=4, L=2048)
    H.note("[determinism] c5 B=4 L=2048")
    a, _, _ = H.run_gpu(case)
    b, _, _ = H.run_gpu(case)
    for key in ("selected", "spans", "out", "lse", "scores"):
        assert np.array_equal(a[key], b[key]), key
    # same logical cache through an identity table
    ident = wl.Case(**{**case.__dict__,
                       "k_pool": np.ascontiguousarray(case.k_pool[case.block_table.reshape(-1)]),
                       "v_pool": np.ascontiguousarray(case.v_pool[case.block_table.reshape(-1)]),
                       "block_table": np.arange(case.block_table.size, dtype=np.int32)
                       .reshape(case.block_table.shape)})
    c, _, _ = H.run_gpu(ident)
    for key in ("selected", "spans", "out", "lse", "scores"):
        assert np.array_equal(a[key], c[key]), key


def test_scale_argument():
    case = wl.c1("k8")
    H.note("[scale] c1")
    from query_aware_sparse_block_amd import device as dev
    dc = dev.upload(case)
    buf = dev.alloc_buffers(dc)
    dev.build_summaries(dc, buf)
    dev.score_topk(dc, buf)
    dev.sparse_decode(dc, buf, scale=0.3)
    torch.cuda.synchronize()
    sel = buf.selected.cpu().numpy()[0, :8]
    ref, _ = H.oracle_attention_on(case, 0, sel, 0, heads=[0, 5], scale=0.3)
    out = buf.out.cpu().numpy()
    for h in (0, 5):
        assert np.max(np.abs(out[0, h] - ref[h])) <= 1e-5


def test_long_block_table_uses_two_kernel_selection():
    # 4400 blocks of 16 tokens: beyond what one workgroup selects in the fused
    # score+select launch, so scoring and Top-k run as separate kernels.
    case = wl.make_case("long-table", seed=66, B=1, Hq=2, Hkv=1, D=64, P=16, dtype="fp16",
                        ctx_lens=[70400], top_k=12, keep_floor=1, recent_window=40)
    H.full_parity(case)


def _repeat_blocks(case, period):
    """Every sequence's logical block j reads physical block table[j % period]:
    blocks with equal j % period have bit-identical summaries and scores."""
    bt = case.block_table.copy()
    for b in range(case.B):
        bt[b] = bt[b, np.arange(bt.shape[1]) % period]
    return wl.Case(**{**case.__dict__, "name": case.name + "-repeat", "block_table": bt})


@pytest.mark.parametrize("period,top_k", [(5, 7), (3, 1), (7, 30)])
def test_exact_ties_cut_by_top_k(period, top_k):
    # repeated summaries make groups of exactly equal scores; top_k cuts
    # through one of them, which the lowest block indices must fill
    base = wl.make_case("ties", seed=67, B=3, Hq=8, Hkv=2, D=64, P=16, dtype="bf16",
                        ctx_lens=[1600, 1111, 700], shuffle=True, num_phys=400, top_k=top_k,
                        keep_floor=1, recent_window=48)
    case = _repeat_blocks(base, period)
    gpu, r_or = H.full_parity(case)
    for b in range(case.B):
        C = int(r_or["plan"][b][1])
        k = int(r_or["plan"][b][3])
        assert np.array_equal(gpu["selected"][b, :k], r_or["sel"][b, :k])
        vals = gpu["scores"][b, :C]
        assert len(np.unique(vals)) <= period


def test_exact_ties_on_the_two_kernel_path():
    base = wl.make_case("ties-long", seed=68, B=1, Hq=2, Hkv=1, D=64, P=16, dtype="fp16",
                        ctx_lens=[70400], top_k=700, keep_floor=1, recent_window=40)
    case = _repeat_blocks(base, 11)
    gpu, r_or = H.full_parity(case)
    assert np.array_equal(gpu["selected"][0, :700], r_or["sel"][0, :700])


@pytest.mark.parametrize("max_blocks_pad", [0, 5000])
def test_zero_queries_tie_every_block(max_blocks_pad):
    # q = 0: every score is +0 or -0, all equal; the k lowest blocks are kept
    # and the output is the plain mean of the attended values
    base = wl.make_case("zero-q", seed=69, B=2, Hq=4, Hkv=2, D=64, P=16, dtype="fp16",
                        ctx_lens=[900, 333], keep_num=1, keep_den=3, keep_floor=1,
                        recent_window=20,
                        max_blocks=(max_blocks_pad or None), num_phys=(max_blocks_pad * 2 or None))
    case = wl.Case(**{**base.__dict__, "q": np.zeros_like(base.q)})
    gpu, r_or = H.full_parity(case)
    for b in range(case.B):
        k = int(r_or["plan"][b][3])
        assert np.array_equal(gpu["selected"][b, :k], np.arange(k))


@pytest.mark.parametrize("Hkv,D,G", [(6, 128, 2), (12, 64, 1), (24, 128, 1), (40, 128, 1)])
def test_summary_rows_of_any_head_count(Hkv, D, G):
    # summary rows of Hkv * D / 4 = 192, 192, 768 and 1280 16-byte vectors: none
    # is a whole number of lane groups, so the last vectors of a row are
    # partial; 40 heads also take the longest-row variant (32 vectors per lane)
    case = wl.make_case(f"hkv{Hkv}", seed=70 + Hkv, B=2, Hq=Hkv * G, Hkv=Hkv, D=D, P=16,
                        dtype="bf16", ctx_lens=[1024, 700], shuffle=True, num_phys=140, top_k=6,
                        keep_floor=1, recent_window=32)
    H.full_parity(case)


def test_long_table_with_three_kv_heads():
    # the two-kernel selection with a partial last lane group (48 vectors a row)
    case = wl.make_case("long-table-hkv3", seed=71, B=1, Hq=3, Hkv=3, D=64, P=16, dtype="bf16",
                        ctx_lens=[70000], top_k=9, keep_floor=1, recent_window=40)
    H.full_parity(case)


def test_more_items_than_workgroups_grid_stride():
    # 300 sequences x 8 KV heads = 2400 one-chunk items > 2048 launched
    # workgroups: later items are taken in grid-stride order
    ctx = [256 + 16 * (b % 13) for b in range(300)]
    case = wl.make_case("grid-stride", seed=72, B=300, Hq=16, Hkv=8, D=64, P=16, dtype="bf16",
                        ctx_lens=ctx, shuffle=True, num_phys=300 * 28 + 10, top_k=4,
                        keep_floor=1, recent_window=32)
    H.full_parity(case, head_mask=_sample_heads(case, 200, 3))


def _sample_heads(case, n, seed):
    rng = np.random.default_rng(seed)
    mask = np.zeros((case.B, case.Hq), np.uint8)
    while int(mask.sum()) < n:
        mask[rng.integers(case.B), rng.integers(case.Hq)] = 1
    mask[0, 0] = mask[case.B - 1, case.Hq - 1] = 1
    return mask


@pytest.mark.parametrize("dtype,Hq,Hkv,D,P,ctx", [
    ("fp32", 8, 2, 128, 256, [5000, 2300]),   # 128 KiB fp32 tiles
    ("bf16", 15, 5, 128, 64, [3000, 999]),    # G = 3 padded to 4, five KV heads
    ("fp16", 7, 7, 64, 32, [2048, 31]),       # odd MHA head count, a context inside the window
    ("bf16", 64, 4, 64, 16, [1500, 800]),     # G = 16 at D = 64
])
def test_uncommon_shapes(dtype, Hq, Hkv, D, P, ctx):
    case = wl.make_case(f"shape-{dtype}-{Hq}-{Hkv}-{D}-{P}", seed=73 + Hq + P, B=len(ctx), Hq=Hq,
                        Hkv=Hkv, D=D, P=P, dtype=dtype, ctx_lens=ctx, shuffle=True,
                        num_phys=len(ctx) * -(-max(ctx) // P) + 40, keep_num=1, keep_den=5,
                        keep_floor=2, recent_window=P + 7)
    H.full_parity(case)


def test_empty_sequences_in_a_batch():
    # sequences with no cached token attend nothing: out = 0 and lse = -inf
    # (the oracle's definition), no block is selected and no span emitted;
    # their neighbours in the batch are unaffected
    case = wl.make_case("empty", seed=74, B=4, Hq=8, Hkv=2, D=128, P=16, dtype="bf16",
                        ctx_lens=[0, 700, 0, 37], shuffle=True, num_phys=4 * 44 + 8, top_k=3,
                        keep_floor=1, recent_window=32)
    gpu, r_or = H.full_parity(case)
    for b in (0, 2):
        assert not gpu["out"][b].any() and np.isneginf(gpu["lse"][b]).all()
        assert gpu["num_selected"][b] == 0 and gpu["num_spans"][b] == 0


def test_largest_block_table():
    # 16384 blocks of 16 tokens (262144 tokens), the table-size limit: the
    # two-kernel selection at 16 candidates per thread of 16 wavefronts
    case = wl.make_case("max-table", seed=75, B=1, Hq=2, Hkv=1, D=64, P=16, dtype="fp16",
                        ctx_lens=[16384 * 16], top_k=40, keep_floor=1, recent_window=100)
    assert case.max_blocks == 16384
    H.full_parity(case)


def test_optional_outputs_may_be_null():
    # scores NULL (the selection keeps them in its workspace) and lse NULL on
    # every decode entry point: selection and outputs are bit-identical to
    # the run that returns them
    from query_aware_sparse_block_amd import device as dev
    from query_aware_sparse_block_amd import kvsp
    case = wl.c5(keep="1/32", B=4, L=2048)
    H.note("[optional] scores and lse NULL")
    gpu, dc, buf = H.run_gpu(case)
    sel2 = torch.full_like(buf.selected, -1)
    nsel2, nsp2, dense2 = (torch.zeros_like(buf.num_selected) for _ in range(3))
    spans2 = torch.full_like(buf.spans, -1)
    kvsp.kvsp_score_topk(dc.layout, dc.params, dc.q, buf.summaries, dc.block_table, dc.ctx_lens,
                         None, sel2, nsel2, spans2, nsp2, dense2, buf.workspace)
    out2 = torch.zeros_like(buf.out)
    kvsp.kvsp_sparse_decode(dc.layout, dc.params, dc.q, dc.k_pool, dc.v_pool, dc.block_table,
                            dc.ctx_lens, spans2, nsp2, None, None, dense2, 0.0, out2, None,
                            buf.workspace)
    torch.cuda.synchronize()
    assert torch.equal(sel2, buf.selected) and torch.equal(nsel2, buf.num_selected)
    assert torch.equal(spans2, buf.spans) and torch.equal(nsp2, buf.num_spans)
    assert torch.equal(out2, buf.out)
    dev.dense_decode(dc, buf)
    out3 = torch.zeros_like(buf.out)
    kvsp.kvsp_dense_decode(dc.layout, dc.q, dc.k_pool, dc.v_pool, dc.block_table, dc.ctx_lens, 0.0,
                           out3, None, buf.workspace)
    torch.cuda.synchronize()
    assert torch.equal(out3, buf.out)
    # DKV decode with lse NULL against the call that returns it
    case = wl.c4_dkv(L=4096, n_resid=8)
    dc = dev.upload(case)
    buf = dev.alloc_buffers(dc)
    dev.build_summaries(dc, buf)
    dkv = kvsp.DkvParams(n_resid=8)
    recs = dev.alloc_dkv_records(dc, dkv)
    ws = kvsp.alloc_dkv_workspace(dc.layout, dkv)
    dev.dkv_compress(dc, dkv, recs)
    dev.score_topk(dc, buf)
    dev.dkv_decode(dc, buf, dkv, recs, ws)
    out4 = torch.zeros_like(buf.out)
    kvsp.kvsp_dkv_decode(dc.layout, dc.params, dkv, dc.q, dc.k_pool, dc.v_pool, recs,
                         dc.block_table, dc.ctx_lens, buf.selected, buf.num_selected, 0.0, out4,
                         None, ws)
    torch.cuda.synchronize()
    assert torch.equal(out4, buf.out)


@pytest.mark.parametrize("bw,floor", [(2e9, 1), (0.5e9, 12), (1e12, 1)])
def test_budget_controller_drives_the_selection(bw, floor):
    # SparPR, "Dynamic budget control": the keep ratio the controller derives
    # for an OPT-like fp16 block (64 tokens, 16 heads x 128, hidden 2048) from
    # a slow, a very slow and a fast host link feeds kvsp_score_topk; the step
    # then meets every parity bar against the oracle run with the same ratio
    # and keep floor
    from query_aware_sparse_block_amd import kvsp
    B, NH, D, P, L = 3, 16, 128, 64, 4096
    layout = kvsp.kvsp_layout(B, NH, NH, D, P, B * L // P, L // P, 1)
    num, copy_s, rec_s = kvsp.kvsp_budget_keep_ratio(layout, kvsp.BudgetModel(bw, 100e12, NH * D), 1024)
    H.note(f"[budget] bw={bw:g} copy={copy_s:.3g}s recompute={rec_s:.3g}s keep={num}/1024 floor={floor}")
    case = wl.make_case(f"budget-bw{bw:g}", seed=7100 + floor, B=B, Hq=NH, Hkv=NH, D=D, P=P,
                        dtype="fp16", ctx_lens=[L, L - 100, 1000], values="needle",
                        keep_num=num, keep_den=1024, keep_floor=floor, recent_window=128)
    gpu, r_or = H.full_parity(case)
    for b in range(B):
        p = oracle.plan(int(case.ctx_lens[b]), P, 128, keep_num=num, keep_den=1024, keep_floor=floor)
        assert int(gpu["num_selected"][b]) == p["k_eff"]


@pytest.mark.parametrize("keep", ["1/2", "dense"])
def test_one_head_items_longer_than_the_id_window(keep):
    # one-head (MHA) items that attend more than 64 blocks: 64 sequences x 4
    # KV heads make 256 groups, so every group is a single chunk, and 16-token
    # blocks over 2048 tokens give 128 blocks per item; the per-wave window of
    # physical block ids is refreshed inside the streaming loop
    B, NH, P, L = 64, 4, 16, 2048
    params = dict(keep_num=1, keep_den=2) if keep == "1/2" else dict(keep_num=1, keep_den=1)
    case = wl.make_case(f"mha-long-items-{keep.replace('/', '_')}", seed=9300, B=B, Hq=NH, Hkv=NH,
                        D=128, P=P, dtype="fp16", ctx_lens=[L] * B, keep_floor=1,
                        recent_window=64, **params)
    H.note(f"[long items] keep={keep}")
    H.full_parity(case, check_all_summaries=False)
    if keep == "dense":
        gpu, dc, buf = H.run_gpu(case, dense_api=True)
        for b in (0, 17, 63):
            outs, _ = H.oracle_attention_on(case, b, [], True)
            for h, o in outs.items():
                assert np.max(np.abs(gpu["out"][b, h] - o)) <= 2e-3, (b, h)


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 4)])
def test_long_span_lists_and_long_items(Hq, Hkv):
    # keep 3/8 of 1535 candidates: about 360 spans per sequence, more than the
    # 256 the decode keeps in registers, and 64 sequences x 4 KV heads make
    # one chunk per group, so each item walks about 580 attended blocks and
    # refreshes its window of block ids from the span list many times; the
    # selected-list form must give the same bits (run_gpu checks it)
    case = wl.make_case(f"long-spans-{Hq}-{Hkv}", seed=9400 + Hq, B=64, Hq=Hq, Hkv=Hkv, D=64,
                        P=16, dtype="bf16", ctx_lens=[24576] * 64, shuffle=True,
                        keep_num=3, keep_den=8, keep_floor=1, recent_window=16)
    H.note(f"[long spans] Hq={Hq} Hkv={Hkv}")
    gpu, r_or = H.full_parity(case, check_all_summaries=False)
    assert int(gpu["num_spans"].min()) > 256
