// Steps 4 and 5: split-KV attention over the kept blocks plus the exact
// recency window, and the flash-style log-sum-exp merge of the partials (DKV
// abstract). The same kernel is the dense fallback (SparPR news page, "On-
// demand local recomputation with cost-aware fallback") and the dense decode
// ("KV cache offloading", "Why the cache leaves the GPU": a dense step reads
// every stored key and value).
//
// Work decomposition. For sequence b the attended tokens form one ordered
// sequence: the tokens of selected[b][0..k) followed by the window [C*P, L)
// (or all of [0, L) when dense). Attended token i lives in attended block
// i / P at offset i % P, because every attended block but the last is full.
// That sequence is cut into at most max_chunks chunks of whole sub-tiles
// (SUB tokens); one wavefront handles one (sequence, KV head, head group,
// chunk) work item and loops over its sub-tiles with an online softmax.
// Waves walk the work items with a grid stride, so any mix of sparse and
// dense sequences fills the chip.
//
// Per sub-tile (SUB tokens, 8 KiB of keys):
//   K: 16-byte loads laid out as the A operand of v_mfma_f32_16x16x32_{bf16,
//      f16} (16x16x4 f32 for fp32 caches): row = token, contraction = head
//      dim. The B operand is the group's queries (up to 16 heads), so the
//      logits of all heads that share this KV head come from one read of K.
//   softmax: base-2 online softmax per head, probabilities staged in LDS.
//   V: 16-byte row-major loads (LPR lanes per row); each lane accumulates
//      acc[head][its EPV channels] += p * v in float32.
// HBM-bound: 2 * D * E bytes per attended token per KV head.

#include "kvsp_device.h"
#include "kvsp_internal.h"

namespace kvsp {

template <typename T, int D>
struct DecodeShape {
  static constexpr int E = T::kBytes;
  static constexpr int EPV = T::kPerVec;      // elements per 16-byte vector
  static constexpr int LPR = D * E / 16;      // lanes per K/V row
  static constexpr int RPL = kWave / LPR;     // rows per wave-wide load
  static constexpr int NRG = RPL;             // row groups in a wave
  static constexpr int SUB = 8192 / (D * E);  // tokens per sub-tile
  static constexpr int TILES = SUB / 16;      // 16-token MFMA tiles per sub-tile
  static constexpr int KLD = D * E / 64;      // K loads per lane per tile
  static constexpr int VLD = SUB / RPL;       // V loads per lane per sub-tile
  static constexpr int PROW = 16;             // floats per token row of p in LDS
};

struct SeqWork {
  int32_t L, Cw, k, dense, A, T, CT, nc;
};

__device__ __forceinline__ SeqWork seq_work(const DecodeArgs& a, int b, int sub) {
  SeqWork w;
  w.L = a.context_lens[b];
  const int n = (w.L + a.P - 1) / a.P;
  w.Cw = window_start_block(w.L, a.P, a.recent_window);
  w.dense = a.all_dense || (a.use_dense != nullptr && a.use_dense[b] != 0);
  w.k = w.dense ? 0 : a.num_selected[b];
  w.A = w.dense ? n : w.k + (n - w.Cw);
  w.T = w.dense ? w.L : w.k * a.P + (w.L - w.Cw * a.P);
  if (w.T > 0) {
    const int per = (w.T + sub * a.max_chunks - 1) / (sub * a.max_chunks);
    w.CT = per * sub;
    w.nc = (w.T + w.CT - 1) / w.CT;
  } else {
    w.CT = sub;
    w.nc = 1;
  }
  return w;
}

// Physical block of attended block `ab` (caller guarantees ab < A).
__device__ __forceinline__ int32_t attended_phys(const DecodeArgs& a, int b, const SeqWork& w,
                                                 int ab) {
  int32_t logical;
  if (w.dense) {
    logical = ab;
  } else if (ab < w.k) {
    logical = a.selected[static_cast<int64_t>(b) * a.max_blocks + ab];
  } else {
    logical = w.Cw + (ab - w.k);
  }
  return a.block_table[static_cast<int64_t>(b) * a.max_blocks + logical];
}

template <typename T>
struct QkMfma;

template <>
struct QkMfma<BF16> {
  __device__ static inline floatx4 step(const uint4& k, const uint4& q, floatx4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k),
                                                   __builtin_bit_cast(bf16x8, q), acc, 0, 0, 0);
  }
};

template <>
struct QkMfma<F16> {
  __device__ static inline floatx4 step(const uint4& k, const uint4& q, floatx4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, k),
                                                  __builtin_bit_cast(f16x8, q), acc, 0, 0, 0);
  }
};

template <>
struct QkMfma<F32> {
  // Four k=4 steps, one per float of the 16-byte vector.
  __device__ static inline floatx4 step(const uint4& k, const uint4& q, floatx4 acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(k.x), __uint_as_float(q.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(k.y), __uint_as_float(q.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(k.z), __uint_as_float(q.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(k.w), __uint_as_float(q.w), acc, 0, 0, 0);
    return acc;
  }
};

// Element offset, within a K row, of the 16-byte vector lane `lane` feeds to
// contraction step s of a 16x16 MFMA tile.
template <typename T>
__device__ __forceinline__ int k_elem_offset(int lane, int s) {
  if constexpr (T::kBytes == 2) {
    return (lane / 16) * 8 + 32 * s;
  } else {
    return (lane / 16) * 4 + 16 * s;
  }
}

template <typename T, int D, int GP>
__global__ __launch_bounds__(256) void attend_kernel(DecodeArgs a) {
  using S = DecodeShape<T, D>;
  constexpr int E = S::E;
  __shared__ float p_lds[4][S::SUB * S::PROW];
  __shared__ float alpha_lds[4][16];
  __shared__ float ml_lds[4][2][16];

  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int hl = lane % 16;  // head within the group (MFMA column)
  const int G = a.Hq / a.Hkv;
  const float NEG_INF = -__builtin_huge_valf();
  const int nwaves = gridDim.x * 4;

  for (int item = blockIdx.x * 4 + wave; item < a.total_items; item += nwaves) {
    int rest = item;
    const int c = rest % a.max_chunks;
    rest /= a.max_chunks;
    const int hg = rest % a.n_head_groups;
    rest /= a.n_head_groups;
    const int g = rest % a.Hkv;
    const int b = rest / a.Hkv;
    const SeqWork w = seq_work(a, b, S::SUB);
    if (c >= w.nc) continue;
    const int start = c * w.CT;
    const int end = min(w.T, start + w.CT);

    // Queries of this head group as the MFMA B operand.
    const int head_in_group = hg * GP + hl;
    const bool head_ok = hl < GP && head_in_group < G;
    const int hq_lane = g * G + head_in_group;
    uint4 qop[S::KLD];
#pragma unroll
    for (int s = 0; s < S::KLD; ++s) {
      if (head_ok) {
        const char* qp = static_cast<const char*>(a.q) +
                         (static_cast<int64_t>(b * a.Hq + hq_lane) * D + k_elem_offset<T>(lane, s)) * E;
        qop[s] = load16(qp);
      } else {
        qop[s] = make_uint4(0, 0, 0, 0);
      }
    }

    float m_run = NEG_INF, l_run = 0.f;
    float acc[GP][S::EPV];
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
      for (int e = 0; e < S::EPV; ++e) acc[h][e] = 0.f;

    // Physical ids of 64 consecutive attended blocks, one per lane.
    int gbase = start / a.P;
    int phys_v = 0;
    {
      const int ab = gbase + lane;
      if (ab < w.A) phys_v = attended_phys(a, b, w, ab);
    }

    const char* kbase = static_cast<const char*>(a.k_pool);
    const char* vbase = static_cast<const char*>(a.v_pool);
    for (int i0 = start; i0 < end; i0 += S::SUB) {
      const int a_last = (min(i0 + S::SUB, end) - 1) / a.P;
      if (a_last - gbase >= kWave) {
        gbase = i0 / a.P;
        const int ab = gbase + lane;
        phys_v = ab < w.A ? attended_phys(a, b, w, ab) : 0;
      }
      int64_t tile_row0[S::TILES];  // element index of the tile's first row
      bool tile_ok[S::TILES];
#pragma unroll
      for (int t = 0; t < S::TILES; ++t) {
        const int ti = i0 + 16 * t;
        tile_ok[t] = ti < end;
        const int ab = min(ti, end - 1) / a.P;
        const int64_t phys = __builtin_amdgcn_readlane(phys_v, ab - gbase);
        tile_row0[t] = ((phys * a.Hkv + g) * a.P + (ti % a.P)) * static_cast<int64_t>(D);
      }

      uint4 kv[S::TILES][S::KLD];
#pragma unroll
      for (int t = 0; t < S::TILES; ++t) {
        const int row = i0 + 16 * t + hl;
        const bool ok = tile_ok[t] && row < end;
#pragma unroll
        for (int s = 0; s < S::KLD; ++s) {
          kv[t][s] = ok ? load16(kbase + (tile_row0[t] + static_cast<int64_t>(hl) * D +
                                          k_elem_offset<T>(lane, s)) * E)
                        : make_uint4(0, 0, 0, 0);
        }
      }
      uint4 vv[S::VLD];
#pragma unroll
      for (int r = 0; r < S::VLD; ++r) {
        const int rr = r * S::RPL + lane / S::LPR;  // row within the sub-tile
        const int t = (r * S::RPL) / 16;
        const bool ok = i0 + rr < end;
        vv[r] = ok ? load16(vbase + (tile_row0[t] + static_cast<int64_t>(rr - 16 * t) * D +
                                     (lane % S::LPR) * S::EPV) * E)
                   : make_uint4(0, 0, 0, 0);
      }

      // Logits (base 2) of the sub-tile: lane holds head hl, tokens 4*(lane/16)+i.
      float s2[S::TILES][4];
      float mloc = NEG_INF;
#pragma unroll
      for (int t = 0; t < S::TILES; ++t) {
        floatx4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < S::KLD; ++s) st = QkMfma<T>::step(kv[t][s], qop[s], st);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = i0 + 16 * t + 4 * (lane / 16) + i;
          s2[t][i] = tok < end ? st[i] * a.scale_log2 : NEG_INF;
          mloc = fmaxf(mloc, s2[t][i]);
        }
      }
      mloc = fmaxf(mloc, lane_xor(mloc, 16));
      mloc = fmaxf(mloc, lane_xor(mloc, 32));
      const float m_new = fmaxf(m_run, mloc);
      const bool none = m_new == NEG_INF;
      const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      float psum = 0.f;
#pragma unroll
      for (int t = 0; t < S::TILES; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = none ? 0.f : __builtin_amdgcn_exp2f(s2[t][i] - m_new);
          psum += pv;
          p_lds[wave][(16 * t + 4 * (lane / 16) + i) * S::PROW + hl] = pv;
        }
      }
      psum += lane_xor(psum, 16);
      psum += lane_xor(psum, 32);
      l_run = l_run * alpha + psum;
      m_run = m_new;
      if (lane < 16) alpha_lds[wave][hl] = alpha;
      wave_lds_sync();

#pragma unroll
      for (int h = 0; h < GP; ++h) {
        const float al = alpha_lds[wave][h];
#pragma unroll
        for (int e = 0; e < S::EPV; ++e) acc[h][e] *= al;
      }
#pragma unroll
      for (int r = 0; r < S::VLD; ++r) {
        const int rr = r * S::RPL + lane / S::LPR;
        float vf[S::EPV];
        T::widen(vv[r], vf);
        const float* prow = &p_lds[wave][rr * S::PROW];
#pragma unroll
        for (int h = 0; h < GP; ++h) {
          const float ph = prow[h];
#pragma unroll
          for (int e = 0; e < S::EPV; ++e) acc[h][e] = fmaf(ph, vf[e], acc[h][e]);
        }
      }
      wave_lds_sync();
    }

    // Fold the row groups: every lane then holds the chunk's sums for its channels.
#pragma unroll
    for (int m = S::LPR; m < kWave; m <<= 1)
#pragma unroll
      for (int h = 0; h < GP; ++h)
#pragma unroll
        for (int e = 0; e < S::EPV; ++e) acc[h][e] += lane_xor(acc[h][e], m);

    if (lane < 16) {
      ml_lds[wave][0][hl] = m_run;
      ml_lds[wave][1][hl] = l_run;
    }
    wave_lds_sync();

    const int rg = lane / S::LPR;
    const int col = (lane % S::LPR) * S::EPV;
    if (w.nc == 1) {
#pragma unroll
      for (int h = 0; h < GP; ++h) {
        if (h % S::NRG != rg || hg * GP + h >= G) continue;
        const float lh = ml_lds[wave][1][h];
        const float inv = lh > 0.f ? 1.f / lh : 0.f;
        float* dst = a.out + (static_cast<int64_t>(b) * a.Hq + g * G + hg * GP + h) * D + col;
#pragma unroll
        for (int e = 0; e < S::EPV; ++e) dst[e] = acc[h][e] * inv;
      }
      if (a.lse != nullptr && head_ok && lane < 16) {
        a.lse[static_cast<int64_t>(b) * a.Hq + hq_lane] =
            l_run > 0.f ? (m_run + __builtin_log2f(l_run)) * 0.69314718055994531f : NEG_INF;
      }
    } else {
      const int64_t slot =
          ((static_cast<int64_t>(b) * a.Hkv + g) * a.n_head_groups + hg) * a.max_chunks + c;
#pragma unroll
      for (int h = 0; h < GP; ++h) {
        if (h % S::NRG != rg || hg * GP + h >= G) continue;
        float* dst = a.part_acc + (slot * GP + h) * D + col;
#pragma unroll
        for (int e = 0; e < S::EPV; ++e) dst[e] = acc[h][e];
      }
      if (lane < GP) {
        a.part_ml[(slot * GP + lane) * 2 + 0] = m_run;
        a.part_ml[(slot * GP + lane) * 2 + 1] = l_run;
      }
    }
    wave_lds_sync();
  }
}

// Log-sum-exp merge of a (sequence, KV head, head group)'s chunk partials:
//   M = max_c m_c, Lsum = sum_c l_c 2^(m_c - M), out = sum_c acc_c 2^(m_c - M) / Lsum.
template <int D, int GP>
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a, int sub) {
  const int lane = threadIdx.x % kWave;
  const int grp = blockIdx.x * 4 + threadIdx.x / kWave;
  const int n_groups = a.B * a.Hkv * a.n_head_groups;
  if (grp >= n_groups) return;
  const int hg = grp % a.n_head_groups;
  const int g = (grp / a.n_head_groups) % a.Hkv;
  const int b = grp / (a.n_head_groups * a.Hkv);
  const SeqWork w = seq_work(a, b, sub);
  if (w.nc <= 1) return;
  const int G = a.Hq / a.Hkv;
  const int64_t slot0 = static_cast<int64_t>(grp) * a.max_chunks;
  const float NEG_INF = -__builtin_huge_valf();
  for (int v = lane; v < GP * D / 4; v += kWave) {
    const int h = (4 * v) / D;
    const int d = (4 * v) % D;
    if (hg * GP + h >= G) continue;
    float M = NEG_INF;
    for (int c = 0; c < w.nc; ++c) {
      const float mc = a.part_ml[((slot0 + c) * GP + h) * 2];
      if (a.part_ml[((slot0 + c) * GP + h) * 2 + 1] > 0.f) M = fmaxf(M, mc);
    }
    float Ls = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    if (M != NEG_INF) {
      for (int c = 0; c < w.nc; ++c) {
        const float lc = a.part_ml[((slot0 + c) * GP + h) * 2 + 1];
        if (!(lc > 0.f)) continue;
        const float sc = __builtin_amdgcn_exp2f(a.part_ml[((slot0 + c) * GP + h) * 2] - M);
        Ls += lc * sc;
        const float4 pa = *reinterpret_cast<const float4*>(a.part_acc + ((slot0 + c) * GP + h) * D + d);
        o.x = fmaf(pa.x, sc, o.x);
        o.y = fmaf(pa.y, sc, o.y);
        o.z = fmaf(pa.z, sc, o.z);
        o.w = fmaf(pa.w, sc, o.w);
      }
    }
    const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
    const int hq = g * G + hg * GP + h;
    *reinterpret_cast<float4*>(a.out + (static_cast<int64_t>(b) * a.Hq + hq) * D + d) =
        make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
    if (d == 0 && a.lse != nullptr)
      a.lse[static_cast<int64_t>(b) * a.Hq + hq] =
          Ls > 0.f ? (M + __builtin_log2f(Ls)) * 0.69314718055994531f : NEG_INF;
  }
}

template <typename T, int D, int GP>
static hipError_t launch_decode_t(const DecodeArgs& a, int num_waves, hipStream_t stream) {
  const int wgs = (num_waves + 3) / 4;
  hipLaunchKernelGGL((attend_kernel<T, D, GP>), dim3(wgs), dim3(256), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.max_chunks == 1) return err;
  const int n_groups = a.B * a.Hkv * a.n_head_groups;
  hipLaunchKernelGGL((combine_kernel<D, GP>), dim3((n_groups + 3) / 4), dim3(256), 0, stream, a,
                     DecodeShape<T, D>::SUB);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_decode_d(const DecodeArgs& a, int gp, int num_waves, hipStream_t stream) {
  switch (gp) {
    case 1: return launch_decode_t<T, D, 1>(a, num_waves, stream);
    case 2: return launch_decode_t<T, D, 2>(a, num_waves, stream);
    case 4: return launch_decode_t<T, D, 4>(a, num_waves, stream);
    case 8: return launch_decode_t<T, D, 8>(a, num_waves, stream);
    default: return launch_decode_t<T, D, 16>(a, num_waves, stream);
  }
}

template <typename T>
static hipError_t launch_decode_dt(const DecodeArgs& a, int gp, int num_waves, hipStream_t stream) {
  return a.D == 64 ? launch_decode_d<T, 64>(a, gp, num_waves, stream)
                   : launch_decode_d<T, 128>(a, gp, num_waves, stream);
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, int group_pad, int num_waves,
                         hipStream_t stream) {
  if (dtype == KVSP_F32) return launch_decode_dt<F32>(a, group_pad, num_waves, stream);
  if (dtype == KVSP_F16) return launch_decode_dt<F16>(a, group_pad, num_waves, stream);
  return launch_decode_dt<BF16>(a, group_pad, num_waves, stream);
}

int decode_sub_tokens(int dtype, int D) {
  const int E = dtype == KVSP_F32 ? 4 : 2;
  return 8192 / (D * E);
}

}  // namespace kvsp
