"""GPU parity of the DKV block codec (DKV abstract) through the C ABI.

kvsp_dkv_compress computes the rank-32 basis by subspace iteration on 64
vectors with a Rayleigh-Ritz step (float32 products, double
orthonormalisation and eigensolver), not by an SVD, so a record is compared
with the oracle's codec through what the abstract fixes, not bit by bit:

* always: the anchor rows and the residual rows are byte copies of the pool;
  the residual offsets ascend; records of blocks inside the window are not
  touched; nonzero basis rows are orthonormal (1e-5) and other rows are zero;
  coef equals X basis^T (X = [K - k_a | V - v_a] from the stored values, in
  float64) within 1e-5 of the block's largest row norm; the residual tokens
  are the n_resid largest reconstruction errors of the record itself, up to a
  band of 1e-4 of the largest row norm (errors that close may order either
  way in float32); the captured energy never exceeds the Eckart-Young
  optimum (the oracle's SVD); the record's round count is the one asked
  for, or, by default, between the first 8 rounds and the cap of 64;
* with the default rounds, on every block: the captured energy is within
  1e-4 of the optimum; where the truncated subspace is numerically unique
  (s_32^2 - s_33^2 at least 1e-4 of s_32^2, as on iid, per-channel-scaled and
  planted low-rank blocks alike) the basis spans the oracle's subspace
  (projectors within 1e-3) and the residual tokens are the oracle's up to a
  band of 1e-3 of the largest row norm; and decoding the GPU records equals
  decoding the oracle's records (the codec bar: 2e-3 for every dtype);
* end to end: kvsp_dkv_decode over GPU-compressed records matches the oracle
  decode of the same records at the exact-path bars (2e-3 for 16-bit caches,
  1e-5 for fp32 caches; lse 1e-4).

Full size: the benchmark's DKV workload (65536 tokens, 504 records) in the
benchmark's launch configuration, on a seeded sample of records and every
output.

Special cases: a block of identical tokens (X = 0: zero basis and
coefficients, residual tokens the first n_resid offsets), an exactly rank-5
fp32 block (reconstruction exact to float32 rounding), n_resid 0 and 64, and
power_iters 1 (the properties hold after any number of rounds)."""

import numpy as np
import pytest
import torch

from oracle import dkv as DKV
from query_aware_sparse_block_amd import device as dev
from query_aware_sparse_block_amd import kvsp
from query_aware_sparse_block_amd import workloads as wl
from tests import gpu_helpers as H
from tests.test_gpu_dkv import oracle_fields

pytestmark = pytest.mark.gpu

ORTHO_TOL = 1e-5
COEF_REL = 1e-5
ERR_BAND_REL = 1e-4
ENERGY_REL = 1e-4
SUBSPACE_TOL = 1e-3
RESID_BAND_REL = 1e-3
UNIQUE_GAP = 1e-4
CODEC_OUT_TOL = 2e-3
FIRST_ROUNDS, ROUND_CAP = 8, 64
POISON = 0x5A


def codec_case(dtype, D, P, Hq, Hkv, ctx, W, seed, values="lowrank", n_spikes=8):
    max_blocks = -(-max(ctx) // P)
    extra = {"n_spikes": n_spikes} if values == "lowrank" else {}
    return wl.make_case(f"dkvc-{dtype}-D{D}-P{P}-{values}", seed=seed, B=len(ctx), Hq=Hq, Hkv=Hkv,
                        D=D, P=P, dtype=dtype, ctx_lens=ctx, shuffle=True, values=values,
                        num_phys=len(ctx) * max_blocks, max_blocks=max_blocks, recent_window=W,
                        top_k=4, **extra)


def compress_on_gpu(case, n_resid, iters=0):
    dc = dev.upload(case)
    dkv = kvsp.DkvParams(n_resid=n_resid, power_iters=iters)
    recs = dev.alloc_dkv_records(dc, dkv)
    recs.fill_(POISON)
    dev.dkv_compress(dc, dkv, recs)
    torch.cuda.synchronize()
    return dc, dkv, recs, recs.cpu().numpy()


def older_blocks(case):
    """(b, j, phys) of every block wholly older than the window."""
    out = []
    for b in range(case.B):
        C = DKV.window_start(int(case.ctx_lens[b]), case.P, case.recent_window)
        out += [(b, j, int(case.block_table[b, j])) for j in range(C)]
    return out


def pools_f64(case):
    return (wl.decode_f32(case.k_pool, case.dtype).astype(np.float64),
            wl.decode_f32(case.v_pool, case.dtype).astype(np.float64))


def check_record(case, raw, fields, K, V, n_resid, iters=0):
    """The property checks of the module docstring for one record; returns the
    oracle's codec of the block and whether it was compared subspace to
    subspace."""
    D, P = case.D, case.P
    X = DKV.block_delta(K, V)
    xmax = np.linalg.norm(X, axis=1).max()
    raw_k, raw_v = raw
    # byte copies
    assert np.array_equal(fields["anchor_k"], raw_k[0]) and np.array_equal(fields["anchor_v"], raw_v[0])
    resid = fields["resid"].astype(np.int64)
    assert np.all(np.diff(resid) > 0) and (n_resid == 0 or (resid[0] >= 0 and resid[-1] < P))
    assert np.array_equal(fields["resid_k"], raw_k[resid])
    assert np.array_equal(fields["resid_v"], raw_v[resid])
    # rounds
    if iters:
        assert fields["rounds"] == iters, fields["rounds"]
    else:
        assert FIRST_ROUNDS <= fields["rounds"] <= ROUND_CAP, fields["rounds"]
    # basis: orthonormal rows or zero rows
    Bm = fields["basis"].astype(np.float64)
    norms = np.linalg.norm(Bm, axis=1)
    nz = norms > 0.5
    assert np.all(nz | (norms == 0.0)), norms
    Bn = Bm[nz]
    assert np.abs(Bn @ Bn.T - np.eye(len(Bn))).max(initial=0.0) <= ORTHO_TOL
    # coefficients
    coef = fields["coef"].astype(np.float64)
    assert np.abs(coef - X @ Bm.T).max() <= COEF_REL * max(xmax, 1e-30)
    # residual tokens: the largest errors of this record, up to the band
    err = np.linalg.norm(X - coef @ Bm, axis=1)
    if n_resid:
        kth = np.sort(err)[::-1][n_resid - 1]
        tau = ERR_BAND_REL * max(xmax, 1e-30)
        chosen = np.zeros(P, bool)
        chosen[resid] = True
        assert np.all(chosen[err > kth + tau]), "a clearly larger error was not kept"
        assert not np.any(chosen[err < kth - tau]), "a clearly smaller error was kept"
    # energy against the Eckart-Young optimum
    ref = DKV.compress_block(K, V, 32, n_resid)
    opt = float(np.sum((X - ref["coef"] @ ref["basis"]) ** 2))
    got = float(np.sum((X - X @ Bm.T @ Bm) ** 2))
    scale = float(np.sum(X * X))
    assert got >= opt - 1e-6 * scale
    compared = False
    if iters == 0:
        assert got <= opt + ENERGY_REL * max(opt, 1e-30) + 1e-6 * scale, (got, opt)
        sv = np.linalg.svd(X, compute_uv=False)
        full = len(sv) > 32 and sv[31] > 1e-6 * sv[0]
        if full and sv[31] ** 2 - sv[32] ** 2 >= UNIQUE_GAP * sv[31] ** 2:
            Pg = Bm.T @ Bm
            Po = ref["basis"].T @ ref["basis"]
            assert np.abs(Pg - Po).max() <= SUBSPACE_TOL, np.abs(Pg - Po).max()
            if n_resid:
                eo = ref["err"]
                kth_o = np.sort(eo)[::-1][n_resid - 1]
                tau_o = RESID_BAND_REL * max(xmax, 1e-30)
                chosen = np.zeros(P, bool)
                chosen[resid] = True
                assert np.all(chosen[eo > kth_o + tau_o]), "the oracle keeps a clearly larger error"
                assert not np.any(chosen[eo < kth_o - tau_o]), "the oracle drops this token"
            compared = True
    return ref, compared


def raw_rows(case, phys, g):
    return case.k_pool[phys, g], case.v_pool[phys, g]


def run_codec_parity(case, n_resid, iters=0, decode=True, min_compared=0.9):
    """Compress every older block on the GPU, check each record (see
    check_record), require the subspace comparison on at least `min_compared`
    of them, and decode end to end."""
    H.note(f"dkv compress {case.name} R={n_resid} iters={iters}")
    dc, dkv, recs, host = compress_on_gpu(case, n_resid, iters)
    kp, vp = pools_f64(case)
    older = older_blocks(case)
    written = {(phys, g) for _, _, phys in older for g in range(case.Hkv)}
    for phys in range(case.num_phys):
        for g in range(case.Hkv):
            if (phys, g) not in written:
                assert np.all(host[phys, g] == POISON), f"record ({phys}, {g}) was touched"
    oracle_recs, gpu_recs = {}, {}
    n_cmp = 0
    for _, _, phys in older:
        for g in range(case.Hkv):
            f = wl.dkv_unpack(host[phys, g], case.dtype, case.D, case.P, n_resid)
            ref, compared = check_record(case, raw_rows(case, phys, g), f, kp[phys, g], vp[phys, g],
                                         n_resid, iters)
            n_cmp += compared
            oracle_recs[(phys, g)] = ref
            gpu_recs[(phys, g)] = f
    if iters == 0 and older:
        assert n_cmp >= min_compared * len(older) * case.Hkv, (n_cmp, len(older) * case.Hkv)
    if not decode:
        return
    # end to end: decode every older block of every sequence
    sel = np.full((case.B, case.max_blocks), -1, np.int32)
    nsel = np.zeros(case.B, np.int32)
    for b in range(case.B):
        C = DKV.window_start(int(case.ctx_lens[b]), case.P, case.recent_window)
        sel[b, :C] = np.arange(C)
        nsel[b] = C
    buf = dev.alloc_buffers(dc)
    buf.selected.copy_(torch.from_numpy(sel))
    buf.num_selected.copy_(torch.from_numpy(nsel))
    ws = kvsp.alloc_dkv_workspace(dc.layout, dkv)
    dev.dkv_decode(dc, buf, dkv, recs, ws)
    torch.cuda.synchronize()
    out = buf.out.cpu().numpy().astype(np.float64)
    lse = buf.lse.cpu().numpy().astype(np.float64)
    q = wl.decode_f32(case.q, case.dtype)
    scale = 1.0 / np.sqrt(case.D)
    args = dict(Hkv=case.Hkv, P=case.P, recent_window=case.recent_window, scale=scale)
    of = {key: oracle_fields(f, case.dtype) for key, f in gpu_recs.items()}
    ref, ref_lse = DKV.decode(q, kp, vp, of, case.block_table, case.ctx_lens, sel, nsel, **args)
    assert np.abs(out - ref).max() <= H.OUT_TOL[case.dtype]
    fin = np.isfinite(ref_lse)
    assert np.abs(lse[fin] - ref_lse[fin]).max(initial=0.0) <= H.LSE_TOL
    if iters == 0:
        ref2, _ = DKV.decode(q, kp, vp, oracle_recs, case.block_table, case.ctx_lens, sel, nsel,
                             **args)
        assert np.abs(ref - ref2).max() <= CODEC_OUT_TOL


@pytest.mark.parametrize("dtype,D,P,Hkv,R", [
    ("bf16", 128, 256, 2, 16),   # the DKV shape: 256-token blocks, Qwen2.5-1.5B-like heads
    ("fp16", 128, 128, 2, 8),
    ("fp32", 64, 256, 1, 8),
    ("bf16", 64, 256, 3, 8),
])
def test_compress_planted_low_rank_blocks_match_the_svd(dtype, D, P, Hkv, R):
    case = codec_case(dtype, D, P, 2 * Hkv, Hkv, [5 * P + 17, 3 * P], W=P, seed=800 + D + P,
                      n_spikes=R)
    run_codec_parity(case, R, min_compared=1.0)


@pytest.mark.parametrize("dtype,D,P,values,R", [
    ("bf16", 128, 64, "lowrank", 8),
    ("fp16", 64, 64, "iid", 16),
    ("bf16", 128, 256, "iid", 0),
    ("bf16", 128, 256, "iid", 16),     # the DKV shape without a planted gap
    ("bf16", 128, 256, "chscale", 16),
    ("fp32", 128, 128, "iid", 64),
    ("fp16", 64, 128, "chscale", 8),
    ("bf16", 128, 256, "lowrank", 40),  # more residual tokens than planted spikes
    ("bf16", 64, 64, "iid", 64),        # every token residual: the decode is exact attention
])
def test_compress_matches_the_svd_without_a_planted_gap(dtype, D, P, values, R):
    case = codec_case(dtype, D, P, 4, 2, [6 * P + 3, 2 * P + P // 2], W=P // 2,
                      seed=820 + D + P + R, values=values, n_spikes=8)
    run_codec_parity(case, R)


def test_compress_after_one_round_keeps_the_properties():
    case = codec_case("bf16", 128, 256, 2, 2, [4 * 256], W=0, seed=841, values="iid")
    # one round is far from converged: no bound on the captured energy
    run_codec_parity(case, 16, iters=1)


def test_compress_constant_and_rank_deficient_blocks():
    # fp32 pool: block 0 of each head holds one repeated token (X = 0), block 1
    # an exactly rank-5 difference; the rest stays iid
    case = codec_case("fp32", 64, 128, 4, 2, [4 * 128], W=0, seed=842, values="iid")
    rng = np.random.default_rng(842)
    phys0, phys1 = int(case.block_table[0, 0]), int(case.block_table[0, 1])
    for g in range(case.Hkv):
        row_k = rng.standard_normal(case.D).astype(np.float32)
        row_v = rng.standard_normal(case.D).astype(np.float32)
        case.k_pool[phys0, g] = row_k
        case.v_pool[phys0, g] = row_v
        A = rng.standard_normal((case.P, 5))
        Bm = rng.standard_normal((5, 2 * case.D))
        A[0] = 0.0
        X = A @ Bm
        case.k_pool[phys1, g] = (row_k + X[:, :case.D]).astype(np.float32)
        case.v_pool[phys1, g] = (row_v + X[:, case.D:]).astype(np.float32)
    R = 6
    dc, dkv, recs, host = compress_on_gpu(case, R)
    for g in range(case.Hkv):
        f0 = wl.dkv_unpack(host[phys0, g], case.dtype, case.D, case.P, R)
        assert np.all(f0["basis"] == 0.0) and np.all(f0["coef"] == 0.0)
        assert np.array_equal(f0["resid"], np.arange(R))
        f1 = wl.dkv_unpack(host[phys1, g], case.dtype, case.D, case.P, R)
        K, V = (case.k_pool[phys1, g].astype(np.float64), case.v_pool[phys1, g].astype(np.float64))
        X = DKV.block_delta(K, V)
        Bm = f1["basis"].astype(np.float64)
        rec_err = np.abs(X - f1["coef"].astype(np.float64) @ Bm).max()
        assert rec_err <= 1e-5 * np.abs(X).max(), rec_err
        norms = np.linalg.norm(Bm, axis=1)
        assert np.all((np.abs(norms - 1.0) < 1e-5) | (norms == 0.0))
    run_codec_parity(case, R, min_compared=0.0)


def test_compress_skips_window_blocks_and_empty_sequences():
    # sequence 1 is empty, sequence 2 lies wholly inside the window
    case = codec_case("bf16", 128, 64, 8, 2, [10 * 64 + 5, 0, 100], W=128, seed=843, values="iid")
    run_codec_parity(case, 4)


def test_dkv_workload_full_size():
    # the benchmark's DKV workload at its full size (65536 tokens, 252 older
    # 256-token blocks x 2 KV heads) in the benchmark's launch configuration:
    # codec over every older block, then scores, Top-k and the DKV decode.
    # A seeded sample of records is checked against the SVD (the planted
    # blocks have a clear gap); the decode is compared with the oracle on the
    # GPU's own selection and records, and with the oracle's records.
    case = wl.c4_dkv(L=65536, n_resid=16)
    H.note(f"dkv full size {case.name}")
    dc, dkv, recs, host = compress_on_gpu(case, 16)
    kp, vp = pools_f64(case)
    older = older_blocks(case)
    rng = np.random.default_rng(4242)
    sample = [older[i] for i in rng.choice(len(older), size=24, replace=False)]
    for _, _, phys in sample:
        for g in range(case.Hkv):
            f = wl.dkv_unpack(host[phys, g], case.dtype, case.D, case.P, 16)
            _, compared = check_record(case, raw_rows(case, phys, g), f, kp[phys, g], vp[phys, g],
                                       16)
            assert compared
    buf = dev.alloc_buffers(dc)
    dev.build_summaries(dc, buf)
    dev.score_topk(dc, buf)
    ws = kvsp.alloc_dkv_workspace(dc.layout, dkv)
    dev.dkv_decode(dc, buf, dkv, recs, ws)
    torch.cuda.synchronize()
    k = int(buf.num_selected[0].item())
    assert k == 16
    sel = buf.selected.cpu().numpy()
    nsel = buf.num_selected.cpu().numpy()
    out = buf.out.cpu().numpy().astype(np.float64)
    lse = buf.lse.cpu().numpy().astype(np.float64)
    used = {(int(case.block_table[0, j]), g) for j in sel[0, :k] for g in range(case.Hkv)}
    gpu_recs = {key: oracle_fields(wl.dkv_unpack(host[key[0], key[1]], case.dtype, case.D,
                                                 case.P, 16), case.dtype) for key in used}
    ref_recs = {key: DKV.compress_block(kp[key[0], key[1]], vp[key[0], key[1]], 32, 16)
                for key in used}
    q = wl.decode_f32(case.q, case.dtype)
    args = dict(Hkv=case.Hkv, P=case.P, recent_window=case.recent_window,
                scale=1.0 / np.sqrt(case.D))
    ref, ref_lse = DKV.decode(q, kp, vp, gpu_recs, case.block_table, case.ctx_lens, sel, nsel,
                              **args)
    assert np.abs(out - ref).max() <= H.OUT_TOL[case.dtype]
    assert np.abs(lse - ref_lse).max() <= H.LSE_TOL
    ref2, _ = DKV.decode(q, kp, vp, ref_recs, case.block_table, case.ctx_lens, sel, nsel, **args)
    assert np.abs(ref - ref2).max() <= CODEC_OUT_TOL


@pytest.mark.parametrize("i", range(12))
def test_compress_random_configurations(i):
    # seeded random shapes through the property checks and the decode:
    # dtype, head dim, block size, KV heads, residual budget, values, ragged
    # contexts and windows
    rng = np.random.default_rng(97_000 + i)
    dtype = ["fp32", "fp16", "bf16"][rng.integers(3)]
    D = int(rng.choice([64, 128]))
    P = int(rng.choice([64, 128, 256]))
    Hkv = int(rng.integers(1, 4))
    R = int(rng.integers(0, min(64, P) + 1))
    values = "lowrank" if rng.random() < 0.5 else "iid"
    ctx = [int(rng.integers(P, 5 * P + 1)) for _ in range(int(rng.integers(1, 4)))]
    W = int(rng.integers(0, 2 * P))
    case = codec_case(dtype, D, P, 2 * Hkv, Hkv, ctx, W, seed=98_000 + i, values=values,
                      n_spikes=max(R, 1))
    run_codec_parity(case, R)
