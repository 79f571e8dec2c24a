"""Seeded synthetic decode-step inputs shaped like the pages' workloads.

This module only draws random numbers and lays them out; it computes no
step of the method (no summaries, scores, selection or attention), so the
oracle and the GPU library can both consume its output without sharing any
of the method's arithmetic.

Shapes follow the models the pages evaluate: an OPT-6.7B-like multi-head
cache (SparPR news page, "Measured numbers on one laptop"), a
MiniCPM4.1-8B-like grouped-query cache ("KV cache offloading", "Why the cache
leaves the GPU"), a Qwen2.5-1.5B-like cache with 256-token blocks (DKV
abstract) and a batched paged pool. No weights or datasets are involved:
every value is drawn from a seeded PCG64 stream.

Storage: fp32 arrays are float32; fp16 and bf16 arrays hold the 16-bit
patterns as uint16, rounded to nearest-even from float32 draws.
"""

from __future__ import annotations

import os
import threading
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from fractions import Fraction

import numpy as np

ELEM_BYTES = {"fp32": 4, "fp16": 2, "bf16": 2}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); finite inputs."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, np.float32).astype(np.float16).view(np.uint16)


def encode(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "fp32":
        return np.ascontiguousarray(x, np.float32)
    if dtype == "fp16":
        return f32_to_f16_bits(x)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def decode_f32(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values -> float32 (exact for all three types)."""
    if dtype == "fp32":
        return np.asarray(raw, np.float32)
    if dtype == "fp16":
        return raw.view(np.float16).astype(np.float32)
    return (raw.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, *stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *stream])))


@dataclass
class Case:
    """One decode step's inputs for a whole batch."""
    name: str
    dtype: str
    B: int
    Hq: int
    Hkv: int
    D: int
    P: int
    q: np.ndarray            # [B][Hq][D]
    k_pool: np.ndarray       # [num_phys][Hkv][P][D]
    v_pool: np.ndarray       # [num_phys][Hkv][P][D]
    block_table: np.ndarray  # [B][max_blocks] int32, logical -> physical
    ctx_lens: np.ndarray     # [B] int32
    top_k: int = 0
    keep_num: int = 1
    keep_den: int = 1
    keep_floor: int = 1
    recent_window: int = 0
    gamma_num: int = 1
    gamma_den: int = 1
    meta: dict = field(default_factory=dict)

    @property
    def num_phys(self) -> int:
        return self.k_pool.shape[0]

    @property
    def max_blocks(self) -> int:
        return self.block_table.shape[1]

    @property
    def select_params(self) -> dict:
        return dict(top_k=self.top_k, keep_num=self.keep_num, keep_den=self.keep_den,
                    keep_floor=self.keep_floor, recent_window=self.recent_window,
                    gamma_num=self.gamma_num, gamma_den=self.gamma_den)


# ---- pool generation --------------------------------------------------------

_CHUNK_BLOCKS_TARGET = 1 << 22   # elements per generation chunk


def _encode_into(x: np.ndarray, dtype: str, dst: np.ndarray, tmp: np.ndarray | None):
    """Round float32 `x` into `dst` (same shape) without large temporaries."""
    if dtype == "fp32":
        dst[...] = x
    elif dtype == "fp16":
        dst.view(np.float16)[...] = x
    else:
        u = x.view(np.uint32)
        np.right_shift(u, np.uint32(16), out=tmp)
        np.bitwise_and(tmp, np.uint32(1), out=tmp)
        np.add(tmp, u, out=tmp)
        np.add(tmp, np.uint32(0x7FFF), out=tmp)
        np.right_shift(tmp, np.uint32(16), out=tmp)
        dst[...] = tmp


def _gen_pool(seed, stream, num_phys, Hkv, P, D, dtype, transform=None, workers=None):
    """Draw a [num_phys][Hkv][P][D] pool of N(0,1) values in independent
    chunks of whole physical blocks (chunk i uses its own PCG64 stream), apply
    `transform(first_block, f32_chunk)` in float32 and round to `dtype`.
    The result does not depend on `workers`."""
    per_block = Hkv * P * D
    blocks_per_chunk = max(1, _CHUNK_BLOCKS_TARGET // per_block)
    n_chunks = (num_phys + blocks_per_chunk - 1) // blocks_per_chunk
    out_dtype = np.float32 if dtype == "fp32" else np.uint16
    out = np.empty((num_phys, Hkv, P, D), out_dtype)
    local = threading.local()

    def work(ci):
        b0 = ci * blocks_per_chunk
        b1 = min(num_phys, b0 + blocks_per_chunk)
        nb = b1 - b0
        if getattr(local, "x", None) is None:
            local.x = np.empty((blocks_per_chunk, Hkv, P, D), np.float32)
            local.t = np.empty((blocks_per_chunk, Hkv, P, D), np.uint32)
        x, t = local.x[:nb], local.t[:nb]
        _rng(seed, stream, ci).standard_normal(out=x.reshape(-1), dtype=np.float32)
        if transform is not None:
            transform(b0, x)
        _encode_into(x, dtype, out[b0:b1], t)

    if workers is None:
        workers = min(16, os.cpu_count() or 1)
    if n_chunks == 1 or workers <= 1:
        for ci in range(n_chunks):
            work(ci)
    else:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(work, range(n_chunks)))
    return out


def _block_table(B, max_blocks, num_phys, shuffle, rng):
    if num_phys < B * max_blocks:
        raise ValueError(f"pool of {num_phys} blocks cannot hold {B} x {max_blocks} blocks")
    if shuffle:
        perm = rng.permutation(num_phys)[: B * max_blocks].astype(np.int32)
        return perm.reshape(B, max_blocks).copy()
    return np.arange(B * max_blocks, dtype=np.int32).reshape(B, max_blocks)


def make_case(name, *, seed, B, Hq, Hkv, D, P, dtype, ctx_lens, values="iid", shuffle=False,
              num_phys=None, max_blocks=None, workers=None, **params) -> Case:
    """General generator.

    values:
      "iid"      q, K, V iid N(0,1).
      "needle"   iid, then for 4 blocks per sequence drawn without replacement
                 from the blocks wholly older than the recent window, every
                 key of head g gets 3 * q[b][h] added (h = g; multi-head only).
      "chscale"  K and V scaled per (KV head, channel) by factors drawn from
                 LogNormal(0, 0.5), independently for K and V.
      "buried"   one block per sequence, drawn uniformly from the blocks wholly
                 older than the recent window, has keys 0.8*u_g + 0.6*z with a
                 per-head direction u_g ~ N(0, I); every query head h reads
                 0.8*u_g(h) + 0.6*z_h. All values stay N(0,1) marginally.
      "lowrank"  every (block, KV head) is jointly low-rank in K|V (see
                 ``_lowrank_transforms``), the premise of the DKV codec.
    """
    ctx_lens = np.asarray(ctx_lens, np.int32).reshape(B)
    if max_blocks is None:
        max_blocks = int(-(-int(ctx_lens.max()) // P))
    if num_phys is None:
        num_phys = B * max_blocks
    G = Hq // Hkv
    table_rng = _rng(seed, 1)
    bt = _block_table(B, max_blocks, num_phys, shuffle, table_rng)
    W = int(params.get("recent_window", 0))

    q32 = np.empty((B, Hq, D), np.float32)
    _rng(seed, 2).standard_normal(out=q32.reshape(-1), dtype=np.float32)
    meta = {}
    k_transform = v_transform = None

    def older_blocks(b):
        # blocks wholly older than the last W tokens
        return max(0, int(ctx_lens[b]) - W) // P

    if values == "needle":
        assert G == 1, "needle planting is defined for multi-head caches"
        nrng = _rng(seed, 5)
        needles = []
        for b in range(B):
            cands = older_blocks(b)
            take = min(4, cands)
            needles.append(sorted(nrng.choice(cands, size=take, replace=False).tolist())
                           if take else [])
        meta["needles"] = needles
        q_dec = decode_f32(encode(q32, dtype), dtype)
        phys_of = {}
        for b, js in enumerate(needles):
            for j in js:
                phys_of[int(bt[b, j])] = b

        def k_transform(b0, x):  # noqa: F811
            for phys, b in phys_of.items():
                if b0 <= phys < b0 + x.shape[0]:
                    x[phys - b0] += 3.0 * q_dec[b][:, None, :]
    elif values == "chscale":
        srng = _rng(seed, 6)
        ck = np.exp(0.5 * srng.standard_normal((Hkv, D))).astype(np.float32)
        cv = np.exp(0.5 * srng.standard_normal((Hkv, D))).astype(np.float32)
        meta["k_scale"], meta["v_scale"] = ck, cv

        def k_transform(b0, x):  # noqa: F811
            x *= ck[None, :, None, :]

        def v_transform(b0, x):  # noqa: F811
            x *= cv[None, :, None, :]
    elif values == "buried":
        brng = _rng(seed, 7)
        buried = [int(brng.integers(0, older_blocks(b))) if older_blocks(b) > 0 else -1
                  for b in range(B)]
        u = brng.standard_normal((B, Hkv, D)).astype(np.float32)
        meta["buried"] = buried
        rho, rest = np.float32(0.8), np.float32(0.6)
        for b in range(B):
            for h in range(Hq):
                q32[b, h] = rho * u[b, h // G] + rest * q32[b, h]
        phys_of = {int(bt[b, j]): b for b, j in enumerate(buried) if j >= 0}

        def k_transform(b0, x):  # noqa: F811
            for phys, b in phys_of.items():
                if b0 <= phys < b0 + x.shape[0]:
                    x[phys - b0] = rho * u[b][:, None, :] + rest * x[phys - b0]
    elif values == "lowrank":
        meta["n_spikes"] = int(params.get("n_spikes", 8))
        k_transform, v_transform = _lowrank_transforms(seed, Hkv, P, D, params)
    elif values != "iid":
        raise ValueError(values)

    k_pool = _gen_pool(seed, 3, num_phys, Hkv, P, D, dtype, k_transform, workers)
    v_pool = _gen_pool(seed, 4, num_phys, Hkv, P, D, dtype, v_transform, workers)
    return Case(name=name, dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, P=P, q=encode(q32, dtype),
                k_pool=k_pool, v_pool=v_pool, block_table=bt, ctx_lens=ctx_lens, meta=meta,
                **params)


LOWRANK_RANK = 32        # planted joint K|V rank per (block, KV head)
LOWRANK_NOISE = 0.05     # iid noise standard deviation
LOWRANK_SPIKE = 6.0      # norm of each planted distinctive token's K|V offset


def _lowrank_block(seed: int, phys: int, Hkv: int, P: int, D: int, n_spikes: int):
    """Per-physical-block draws shared by the K and V transforms:
    coefficients A [Hkv][P][32], bases B [Hkv][2D][32], means mu [Hkv][2D]
    and spike offsets [Hkv][P][2D] (zero except n_spikes rows per head,
    never token 0)."""
    rng = _rng(seed, 8, phys)
    r = LOWRANK_RANK
    A = rng.standard_normal((Hkv, P, r))
    Bm = rng.standard_normal((Hkv, 2 * D, r))
    mu = rng.standard_normal((Hkv, 2 * D))
    spikes = np.zeros((Hkv, P, 2 * D))
    for g in range(Hkv):
        rows = rng.choice(np.arange(1, P), size=min(n_spikes, P - 1), replace=False)
        for t in rows:
            u = rng.standard_normal(2 * D)
            spikes[g, t] = LOWRANK_SPIKE * u / np.linalg.norm(u)
    return A, Bm, mu, spikes


def _lowrank_transforms(seed, Hkv, P, D, params):
    """K|V rows of (block p, head g): mu + amp * A diag(s) B^T + noise + spikes,
    with s_j falling geometrically from 1 to 1/2 over the 32 planted
    directions and amp setting the signal's per-entry variance to 1. The
    iid N(0,1) pool draw, scaled by LOWRANK_NOISE, is the noise. The spikes
    are the distinctive tokens; their count is ``n_spikes`` (default 8)."""
    n_spikes = int(params.pop("n_spikes", 8))
    s = 0.5 ** (np.arange(LOWRANK_RANK) / (LOWRANK_RANK - 1))
    amp = 1.0 / np.sqrt(np.sum(s * s))

    def make(part):
        lo, hi = (0, D) if part == 0 else (D, 2 * D)

        def tf(b0, x):
            for i in range(x.shape[0]):
                A, Bm, mu, spikes = _lowrank_block(seed, b0 + i, Hkv, P, D, n_spikes)
                sig = amp * np.einsum("gtr,gdr->gtd", A * s, Bm[:, lo:hi])
                x[i] = (mu[:, None, lo:hi] + sig + spikes[:, :, lo:hi]
                        + LOWRANK_NOISE * x[i]).astype(np.float32)
        return tf

    return make(0), make(1)


def _ratio(keep) -> tuple[int, int]:
    f = Fraction(keep)
    return f.numerator, f.denominator


# ---- the five workload families ---------------------------------------------

def c1(variant="k8", seed=None) -> Case:
    """Tiny fp32 MHA step: batch 1, 8 heads, D 64, 1024 tokens in 16-token
    blocks, top-8 blocks + 32-token window, keep floor 4."""
    top_k, gamma, shuffle = 8, (1, 1), False
    num_phys = None
    if variant == "k2":
        top_k = 2
    elif variant == "k64":
        top_k = 64
    elif variant == "gamma":
        top_k, gamma = 64, (1, 10)
    elif variant == "shuffled":
        shuffle, num_phys = True, 96
    elif variant != "k8":
        raise ValueError(variant)
    vid = ["k8", "k2", "k64", "gamma", "shuffled"].index(variant)
    return make_case(f"c1-{variant}", seed=1000 + 10 * vid if seed is None else seed, B=1, Hq=8,
                     Hkv=8, D=64, P=16, dtype="fp32", ctx_lens=[1024], shuffle=shuffle,
                     num_phys=num_phys, top_k=top_k, keep_floor=4, recent_window=32,
                     gamma_num=gamma[0], gamma_den=gamma[1])


def c2(L=8192, keep="1/2", B=4, H=32, seed=None) -> Case:
    """OPT-6.7B-like MHA fp16: 32 heads, D 128, blocks of 64, keep 1/2 or
    1/10 of the candidate blocks, 128-token window, 4 planted needle blocks."""
    num, den = _ratio(keep)
    vid = [1024, 2048, 4096, 8192].index(L) if L in (1024, 2048, 4096, 8192) else 9
    return make_case(f"c2-L{L}-keep{num}/{den}", seed=2000 + 10 * vid if seed is None else seed,
                     B=B, Hq=H, Hkv=H, D=128, P=64, dtype="fp16", ctx_lens=[L] * B,
                     values="needle", keep_num=num, keep_den=den, recent_window=128)


def c3(keep="1/32", L=131072, seed=None) -> Case:
    """MiniCPM4.1-8B-like GQA bf16: 32 query / 2 KV heads, D 128, blocks of 64,
    keep 1/32, 1/16 or 1/8, 256-token window, per-channel LogNormal scales."""
    num, den = _ratio(keep)
    vid = {32: 0, 16: 1, 8: 2}.get(den, 9)
    return make_case(f"c3-L{L}-keep{num}/{den}", seed=3000 + 10 * vid if seed is None else seed,
                     B=1, Hq=32, Hkv=2, D=128, P=64, dtype="bf16", ctx_lens=[L],
                     values="chscale", keep_num=num, keep_den=den, recent_window=256)


def c4(L=65536, seed=None) -> Case:
    """Qwen2.5-1.5B-like GQA bf16: 12 query / 2 KV heads, D 128, blocks of 256,
    top-16 blocks + 1024-token window, query correlated with a buried block."""
    vid = {4096: 0, 8192: 1, 16384: 2, 32768: 3, 65536: 4}.get(L, 9)
    return make_case(f"c4-L{L}", seed=4000 + 10 * vid if seed is None else seed, B=1, Hq=12,
                     Hkv=2, D=128, P=256, dtype="bf16", ctx_lens=[L], values="buried", top_k=16,
                     recent_window=1024)


def c5(keep="1/32", B=64, L=32768, seed=None, workers=None) -> Case:
    """Batched serving shape bf16: batch 64, 32 query / 8 KV heads, D 128,
    32768 tokens each in blocks of 64 from a shuffled paged pool with a random
    block table, keep 1/32, no window, γ = 3/5 (keep 7/10 forces the dense
    fallback)."""
    num, den = _ratio(keep)
    vid = 0 if (num, den) == (1, 32) else 1
    max_blocks = L // 64
    return make_case(f"c5-B{B}-L{L}-keep{num}/{den}",
                     seed=5000 + 10 * vid if seed is None else seed, B=B, Hq=32, Hkv=8, D=128,
                     P=64, dtype="bf16", ctx_lens=[L] * B, shuffle=True,
                     num_phys=B * max_blocks, workers=workers, keep_num=num, keep_den=den,
                     recent_window=0, gamma_num=3, gamma_den=5)


def c4_dkv(L=65536, n_resid=16, seed=None) -> Case:
    """The c4 shape (Qwen2.5-1.5B-like, 256-token blocks, top-16 + 1024-token
    window) with jointly low-rank K|V blocks holding ``n_resid`` distinctive
    tokens each: the workload of the DKV codec (DKV abstract)."""
    vid = {4096: 0, 8192: 1, 16384: 2, 32768: 3, 65536: 4}.get(L, 9)
    case = make_case(f"c4dkv-L{L}-R{n_resid}", seed=4500 + 10 * vid if seed is None else seed,
                     B=1, Hq=12, Hkv=2, D=128, P=256, dtype="bf16", ctx_lens=[L],
                     values="lowrank", n_spikes=n_resid, top_k=16, recent_window=1024)
    case.meta["n_resid"] = n_resid
    return case


# ---- DKV compressed-block records (byte layout of the C ABI) ---------------

DKV_RANK = 32


def dkv_record_layout(D: int, P: int, elem_bytes: int, n_resid: int, rank: int = DKV_RANK):
    """Byte offsets of one (block, KV head) record and its padded size:
    anchor K and V rows (cache dtype), basis [rank][2D] fp32, coefficients
    [P][rank] fp32, residual K rows and V rows [n_resid][D] (cache dtype),
    residual token offsets [n_resid] int32, the codec's subspace-iteration
    rounds (int32); the record is padded to 256 B."""
    def up(x, a):
        return (x + a - 1) // a * a
    off = {"anchor": 0}
    off["basis"] = up(2 * D * elem_bytes, 16)
    off["coef"] = off["basis"] + rank * 2 * D * 4
    off["resid_k"] = off["coef"] + P * rank * 4
    off["resid_v"] = off["resid_k"] + n_resid * D * elem_bytes
    off["resid"] = off["resid_v"] + n_resid * D * elem_bytes
    off["rounds"] = off["resid"] + 4 * n_resid
    off["bytes"] = up(off["rounds"] + 4, 256)
    return off


def dkv_pack(fields: dict, dtype: str, P: int, n_resid: int) -> np.ndarray:
    """One record as uint8 bytes. ``fields`` hold stored values: anchor_k,
    anchor_v, resid_k, resid_v as the cache dtype's raw patterns (uint16 or
    float32), basis and coef as float32, resid as int; an optional
    ``rounds`` (int, default 0)."""
    D = fields["anchor_k"].shape[0]
    E = ELEM_BYTES[dtype]
    lay = dkv_record_layout(D, P, E, n_resid)
    buf = np.zeros(lay["bytes"], np.uint8)

    def put(off, arr):
        b = np.ascontiguousarray(arr).view(np.uint8).reshape(-1)
        buf[off:off + b.size] = b

    put(lay["anchor"], fields["anchor_k"])
    put(lay["anchor"] + D * E, fields["anchor_v"])
    put(lay["basis"], np.asarray(fields["basis"], np.float32))
    put(lay["coef"], np.asarray(fields["coef"], np.float32))
    put(lay["resid_k"], fields["resid_k"])
    put(lay["resid_v"], fields["resid_v"])
    put(lay["resid"], np.asarray(fields["resid"], np.int32))
    put(lay["rounds"], np.asarray([fields.get("rounds", 0)], np.int32))
    return buf


def dkv_unpack(buf: np.ndarray, dtype: str, D: int, P: int, n_resid: int) -> dict:
    """Inverse of ``dkv_pack`` (raw stored values, no arithmetic)."""
    E = ELEM_BYTES[dtype]
    lay = dkv_record_layout(D, P, E, n_resid)
    raw_t = np.float32 if dtype == "fp32" else np.uint16
    b = np.asarray(buf, np.uint8)

    def get(off, count, t):
        return b[off:off + count * np.dtype(t).itemsize].view(t).copy()

    return dict(
        anchor_k=get(lay["anchor"], D, raw_t),
        anchor_v=get(lay["anchor"] + D * E, D, raw_t),
        basis=get(lay["basis"], DKV_RANK * 2 * D, np.float32).reshape(DKV_RANK, 2 * D),
        coef=get(lay["coef"], P * DKV_RANK, np.float32).reshape(P, DKV_RANK),
        resid_k=get(lay["resid_k"], n_resid * D, raw_t).reshape(n_resid, D),
        resid_v=get(lay["resid_v"], n_resid * D, raw_t).reshape(n_resid, D),
        resid=get(lay["resid"], n_resid, np.int32),
        rounds=int(get(lay["rounds"], 1, np.int32)[0]),
    )


def dkv_random_records(case: Case, n_resid: int, seed: int, blocks=None) -> dict:
    """Synthetic records for decode tests, keyed by (phys, g): random
    anchors, bases, coefficients and residual rows (stored values), residual
    offsets a sorted random subset of the block. ``blocks`` limits the
    physical blocks (default: all)."""
    rng = _rng(seed, 9)
    D, P = case.D, case.P
    recs = {}
    phys_list = range(case.num_phys) if blocks is None else blocks
    for phys in phys_list:
        for g in range(case.Hkv):
            def draw(shape):
                return encode(rng.standard_normal(shape).astype(np.float32), case.dtype)
            recs[(int(phys), g)] = dict(
                anchor_k=draw(D), anchor_v=draw(D),
                basis=(rng.standard_normal((DKV_RANK, 2 * D)) / np.sqrt(2 * D)).astype(np.float32),
                coef=rng.standard_normal((P, DKV_RANK)).astype(np.float32),
                resid_k=draw((n_resid, D)), resid_v=draw((n_resid, D)),
                resid=np.sort(rng.choice(P, size=n_resid, replace=False)).astype(np.int32))
    return recs


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """Bytes one cached token occupies across a model: keys and values, for
    every layer and KV head ("KV cache offloading", "Why the cache leaves the
    GPU")."""
    return 2 * layers * kv_heads * head_dim * elem_bytes
