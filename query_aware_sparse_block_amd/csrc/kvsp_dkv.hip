// DKV variant ("DKV: Anchor + Low-Rank Differential KV-Cache Compression for
// Scalable Long-Context Inference", abstract): attention over compressed
// blocks without decompressing their keys, and the block codec.
//
// A compressed (block, KV head) record holds the anchor rows k_a, v_a, a
// basis W = [W_K | W_V] (32 x 2D, fp32), coefficients C (P x 32, fp32) and R
// exact residual rows. Token t (not residual) stands for
//   k_t = k_a + C_t W_K,   v_t = v_a + C_t W_V.
// For a query q the logit is therefore <q, k_a> + C_t . (W_K q), and the
// softmax-weighted value sum over the block is
//   (sum_t p_t) v_a + (sum_t p_t C_t) W_V + sum_residual p_r v_r,
// so a block costs one pass over C, W and the residual rows.
//
// Decode work split. One launch covers both halves. A workgroup of 4 waves
// takes a (chunk, sequence, KV head) item, folded into one online softmax;
// each of the group's query heads (at most 16) is one MFMA column. A chunk is
// either a run of the sequence's selected compressed blocks or a run of
// 64-token groups of the exact window. A window group is treated as a block
// with no compressed token and up to 64 exact rows read from the pool (64
// divides every supported block size, so a group lies in one block); it takes
// the residual-row path below and skips the low-rank parts. Per block:
//   A. every wave stages its quarter of C in LDS, computes a partial
//      W_K q over a quarter of the channels (fp32 MFMA 16x16x4), the anchor
//      term, and the exact logits of one tile of 16 residual rows (the
//      QK^T MFMA of the exact path);
//   B. low-rank logits of the wave's tokens: C (16 tokens x 32) times
//      (W_K q) (32 x heads) on fp32 MFMA; residual tokens masked;
//   C. probabilities against the block maximum, and the wave's share of
//      p^T C (heads x 32), again fp32 MFMA, with p taken from the logit
//      registers as the A operand;
//   D. each wave owns D/4 output channels: (p^T C) W_V, the anchor term and
//      the residual PV on fp32 MFMA, then the online-softmax rescale.
// Chunks of one (sequence, KV head) merge through the workspace (device-scope
// stores, a completion counter, the last chunk merges).
#include <stddef.h>
#include <stdint.h>

#include "kvsp_device.h"
#include "kvsp_internal.h"

namespace kvsp {
namespace {

constexpr int kRank = 32;
constexpr int kMaxResid = 64;
constexpr int kCRow = 36;  // LDS row stride (floats) of staged coefficient rows
// LDS row stride of per-head rank vectors: 16-byte aligned, and rows 36
// floats apart put the 16 heads' 16-byte reads on distinct banks.
constexpr int kQRow = 36;
constexpr int kQaRow = 20;  // per-head anchor partials (16 used), same reasoning
constexpr float kLn2 = 0.69314718055994531f;

__device__ __forceinline__ floatx4 mfma4(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// out[s] = (p[0][hl][j] + p[1][hl][j]) + (p[2][hl][j] + p[3][hl][j]) for
// j = 8 gi + s: the four waves' partials of head hl, ranks 8 gi .. 8 gi + 7,
// read as 16-byte vectors.
__device__ __forceinline__ void sum_wave_partials(const float (&p)[4][16][kQRow], int hl, int gi,
                                                  float (&out)[8]) {
  float4 v[4][2];
#pragma unroll
  for (int w = 0; w < 4; ++w)
#pragma unroll
    for (int h = 0; h < 2; ++h) v[w][h] = *reinterpret_cast<const float4*>(&p[w][hl][8 * gi + 4 * h]);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    out[4 * h + 0] = (v[0][h].x + v[1][h].x) + (v[2][h].x + v[3][h].x);
    out[4 * h + 1] = (v[0][h].y + v[1][h].y) + (v[2][h].y + v[3][h].y);
    out[4 * h + 2] = (v[0][h].z + v[1][h].z) + (v[2][h].z + v[3][h].z);
    out[4 * h + 3] = (v[0][h].w + v[1][h].w) + (v[2][h].w + v[3][h].w);
  }
}

constexpr int kMergeBatch = 32;  // chunk partials requested together in the merge

template <typename T, int D, int TPW>
__global__ __launch_bounds__(256) void dkv_attend_kernel(DkvDecodeArgs a) {
  constexpr int E = T::kBytes;
  constexpr int DQ = D / 4;          // channels per wave for W_K q
  constexpr int QS = DQ / 4;         // per lane group: QS consecutive channels
  constexpr int NDT = D / 64;        // 16-channel output tiles per wave
  constexpr int TOKW = 16 * TPW;     // tokens per wave
  constexpr int KLD = D * E / 64;    // exact-row MFMA steps over D
  constexpr int RS = kMaxResid / 4;  // residual PV steps (4 rows each)

  __shared__ __align__(16) float c_lds[4][TOKW * kCRow];
  // Per-wave partials, read back as 16-byte vectors.
  __shared__ __align__(16) float qt_part[4][16][kQRow];
  __shared__ __align__(16) float qa_part[16][kQaRow];  // [head][4 * wave + lane group]
  __shared__ __align__(16) float cb_part[4][16][kQRow];
  __shared__ float p_res[kMaxResid][16];
  __shared__ __align__(16) float wmax[16][4];  // [head][wave]
  __shared__ __align__(16) float wsum[16][4];
  __shared__ __align__(16) float rsum[16][4];
  __shared__ uint32_t res_mask[8];
  __shared__ int last_flag;
  __shared__ float merge_w[16][kWave];  // split-KV merge: chunk weights per head
  __shared__ float merge_h[16][2];      // per head: normaliser, max

  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int hl = lane % 16;  // MFMA column: query head (or rank / channel)
  const int gi = lane / 16;  // lane group: MFMA k-slot, and row quad of outputs
  const int G = a.Hq / a.Hkv;
  const int n_pairs = a.B * a.Hkv;
  const int S = a.n_chunks + a.n_wchunks;  // chunk slots per (sequence, KV head)
  const int total = n_pairs * S;
  const float NEG_INF = -__builtin_huge_valf();
  const int dbase = wave * 16 * NDT;  // this wave's output channels

  if (wave == 0 && lane < 8) res_mask[lane] = 0;

  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const int c = item / n_pairs;
    const int pair = item - c * n_pairs;
    const int b = pair / a.Hkv;
    const int g = pair - b * a.Hkv;
    const int L = a.context_lens[b];
    const int C = window_start_block(L, a.P, a.recent_window);
    int k = a.num_selected[b];
    k = k < 0 ? 0 : (k > C ? C : k);
    const int per = k > 0 ? (k + a.n_chunks - 1) / a.n_chunks : 1;
    const int n_act_c = k > 0 ? (k + per - 1) / per : 0;
    const int wtok = L - C * a.P;            // exact window tokens
    const int wg = (wtok + 63) / 64;         // 64-token window groups
    const int wper = (wg + a.n_wchunks - 1) / a.n_wchunks;
    const int n_act_w = wg > 0 ? (wg + wper - 1) / wper : 0;
    // Active chunks: compressed ones first, then the window's. An empty
    // sequence keeps chunk 0 alone (no work: out 0, lse -inf).
    const int n_act = max(n_act_c + n_act_w, 1);
    const bool win = c >= a.n_chunks;        // uniform over the workgroup
    int idx, j0, j1;
    if (!win) {
      if (c >= max(n_act_c, n_act_c + n_act_w == 0 ? 1 : 0)) continue;
      idx = c;
      j0 = c * per;
      j1 = min(k, j0 + per);
    } else {
      const int w = c - a.n_chunks;
      if (w >= n_act_w) continue;
      idx = n_act_c + w;
      j0 = w * wper;
      j1 = min(wg, j0 + wper);
    }

    // Query operands (fixed for the item). Heads past G are zero columns: their
    // lanes read head 0 and zero it afterwards, so that no load sits behind a
    // per-lane branch (the compiler then waits for each such load alone).
    const bool head_ok = hl < G;
    const int64_t qrow = static_cast<int64_t>(b) * a.Hq + g * G + (head_ok ? hl : 0);
    float qreg[QS];
#pragma unroll
    for (int s = 0; s < QS; ++s) qreg[s] = T::load1(a.q, qrow * D + wave * DQ + gi * QS + s);
    uint4 qop[KLD];
#pragma unroll
    for (int s = 0; s < KLD; ++s)
      qop[s] = load16(static_cast<const char*>(a.q) + (qrow * D + k_elem_offset<T>(lane, s)) * E);
#pragma unroll
    for (int s = 0; s < QS; ++s) qreg[s] = head_ok ? qreg[s] : 0.f;
#pragma unroll
    for (int s = 0; s < KLD; ++s) qop[s] = head_ok ? qop[s] : make_uint4(0, 0, 0, 0);

    // Running softmax state of heads 4*gi + v, channels dbase + 16*dt + hl.
    float m_run[4], l_run[4];
    floatx4 acc[NDT];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      m_run[v] = NEG_INF;
      l_run[v] = 0.f;
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[dt] = floatx4{0.f, 0.f, 0.f, 0.f};

    for (int jj = j0; jj < j1; ++jj) {
      // Exact rows of this block: the record's residual rows, or a window
      // group's rows in the pool.
      const char* rec = nullptr;
      const char* rk_base;
      const char* rv_base;
      int R;
      if (!win) {
        const int jlog = a.selected[static_cast<int64_t>(b) * a.max_blocks + jj];
        const int64_t phys = a.block_table[static_cast<int64_t>(b) * a.max_blocks + jlog];
        rec = a.records + (phys * a.Hkv + g) * a.rec_bytes;
        rk_base = rec + a.off_rk;
        rv_base = rec + a.off_rv;
        R = a.n_resid;
      } else {
        const int t0 = C * a.P + 64 * jj;  // first token of the group
        const int lb = t0 / a.P;
        const int64_t phys = a.block_table[static_cast<int64_t>(b) * a.max_blocks + lb];
        const int64_t row0 = (phys * a.Hkv + g) * a.P + (t0 - lb * a.P);
        rk_base = static_cast<const char*>(a.k_pool) + row0 * D * E;
        rv_base = static_cast<const char*>(a.v_pool) + row0 * D * E;
        R = min(64, wtok - 64 * jj);
      }

      // ---- A: loads, W_K q partial, anchor term, exact-row logits ---------------
      // Every load of the block is issued before any of them is used, and
      // none sits behind a per-lane branch (rows past R are clamped to row
      // R - 1 and masked afterwards): the block's lines then arrive in one
      // round trip instead of one round trip per load.
      float wv[NDT][8];
      float va[NDT];
      float wk[2][QS];
      float ka[QS];
      uint4 cvec[2 * TPW];
      int rid = -1;
      if (!win) {
        const float* basis = reinterpret_cast<const float*>(rec + a.off_basis);
        if (R > 0) rid = reinterpret_cast<const int32_t*>(rec + a.off_ridx)[min(lane, R - 1)];
        const char* src = rec + a.off_coef + static_cast<int64_t>(wave) * TOKW * kRank * 4;
#pragma unroll
        for (int u = 0; u < 2 * TPW; ++u)  // 16-byte vectors of the wave's coefficient rows
          cvec[u] = load16(src + static_cast<int64_t>(lane + kWave * u) * 16);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int s = 0; s < QS; ++s)
            wk[nt][s] = basis[(16 * nt + hl) * 2 * D + wave * DQ + gi * QS + s];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int s = 0; s < 8; ++s) wv[dt][s] = basis[(gi * 8 + s) * 2 * D + D + dbase + 16 * dt + hl];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) va[dt] = T::load1(rec, D + dbase + 16 * dt + hl);
#pragma unroll
        for (int s = 0; s < QS; ++s) ka[s] = T::load1(rec, wave * DQ + gi * QS + s);
      }
      float vr[RS][NDT] = {};
      const int rlast = R > 0 ? R - 1 : 0;
#pragma unroll
      for (int s = 0; s < RS; ++s) {
        if (4 * s >= R) break;  // uniform
        const int row = min(4 * s + gi, rlast);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          vr[s][dt] = T::load1(rv_base, static_cast<int64_t>(row) * D + dbase + 16 * dt + hl);
      }
      const bool krows = 16 * wave < R;  // uniform over the wave
      uint4 kv[KLD];
      if (krows) {
        const char* kr = rk_base + static_cast<int64_t>(min(16 * wave + hl, R - 1)) * D * E;
#pragma unroll
        for (int s = 0; s < KLD; ++s) kv[s] = load16(kr + k_elem_offset<T>(lane, s) * E);
      }
      if (!win) {
        if (wave == 0 && lane < R && rid >= 0 && rid < a.P) atomicOr(&res_mask[rid >> 5], 1u << (rid & 31));
#pragma unroll
        for (int u = 0; u < 2 * TPW; ++u) {
          const int vi = lane + kWave * u;
          *reinterpret_cast<uint4*>(&c_lds[wave][(vi / 8) * kCRow + (vi % 8) * 4]) = cvec[u];
        }
        float qa = 0.f;
#pragma unroll
        for (int s = 0; s < QS; ++s) qa += qreg[s] * ka[s];
        floatx4 qt[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int s = 0; s < QS; ++s) qt[nt] = mfma4(qreg[s], wk[nt][s], qt[nt]);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int v = 0; v < 4; ++v) qt_part[wave][4 * gi + v][16 * nt + hl] = qt[nt][v];
        qa_part[hl][4 * wave + gi] = qa;
      } else {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          va[dt] = 0.f;
#pragma unroll
          for (int s = 0; s < 8; ++s) wv[dt][s] = 0.f;
        }
      }
      float rmax = NEG_INF;
      if (krows) {
        floatx4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KLD; ++s) sc = QkMfma<T>::step(kv[s], qop[s], sc);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = 16 * wave + 4 * gi + v;
          const float z = row < R ? sc[v] * a.scale_log2 : NEG_INF;
          p_res[row][hl] = z;
          rmax = fmaxf(rmax, z);
        }
      }
      __syncthreads();

      // ---- B: low-rank logits of this wave's tokens (none for a window group)
      float s2[TPW][4];
      float lmax = NEG_INF;
      if (!win) {
        float qtb[8];
        sum_wave_partials(qt_part, hl, gi, qtb);
        float qa_h = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float4 qa4 = *reinterpret_cast<const float4*>(&qa_part[hl][4 * w]);
          qa_h += qa4.x;
          qa_h += qa4.y;
          qa_h += qa4.z;
          qa_h += qa4.w;
        }
#pragma unroll
        for (int mt = 0; mt < TPW; ++mt) {
          const float* crow = &c_lds[wave][(16 * mt + hl) * kCRow + gi * 8];
          const float4 c0 = *reinterpret_cast<const float4*>(crow);
          const float4 c1 = *reinterpret_cast<const float4*>(crow + 4);
          const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
          floatx4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 8; ++s) sc = mfma4(cv[s], qtb[s], sc);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int tok = wave * TOKW + 16 * mt + 4 * gi + v;
            const bool resid = (res_mask[tok >> 5] >> (tok & 31)) & 1u;
            s2[mt][v] = resid ? NEG_INF : (sc[v] + qa_h) * a.scale_log2;
            lmax = fmaxf(lmax, s2[mt][v]);
          }
        }
      } else {
#pragma unroll
        for (int mt = 0; mt < TPW; ++mt)
#pragma unroll
          for (int v = 0; v < 4; ++v) s2[mt][v] = NEG_INF;
      }
      lmax = fold_max<16>(fmaxf(lmax, rmax));
      if (gi == 0) wmax[hl][wave] = lmax;
      __syncthreads();

      // ---- C: probabilities, p^T C, residual probabilities ------------------
      if (wave == 0 && lane < 8) res_mask[lane] = 0;  // every read of it is done
      const float4 wm = *reinterpret_cast<const float4*>(wmax[hl]);
      const float mb = fmaxf(fmaxf(wm.x, wm.y), fmaxf(wm.z, wm.w));
      float ls = 0.f;
#pragma unroll
      for (int mt = 0; mt < TPW; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float p = __builtin_amdgcn_exp2f(s2[mt][v] - mb);
          s2[mt][v] = p;
          ls += p;
        }
      if (!win) {  // a window group has no coefficients (its p here are all 0)
        floatx4 cb[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int mt = 0; mt < TPW; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v)
              cb[nt] = mfma4(s2[mt][v], c_lds[wave][(16 * mt + 4 * gi + v) * kCRow + 16 * nt + hl], cb[nt]);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int v = 0; v < 4; ++v) cb_part[wave][4 * gi + v][16 * nt + hl] = cb[nt][v];
      }
      ls = fold_sum<16>(ls);
      if (gi == 0) wsum[hl][wave] = ls;
      float rs = 0.f;
      if (16 * wave < R) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = 16 * wave + 4 * gi + v;
          const float p = row < R ? __builtin_amdgcn_exp2f(p_res[row][hl] - mb) : 0.f;
          p_res[row][hl] = p;
          rs += p;
        }
      }
      rs = fold_sum<16>(rs);
      if (gi == 0) rsum[hl][wave] = rs;
      __syncthreads();

      // ---- D: output channels of this wave -----------------------------------
      float alpha[4], beta[4], llr[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int h = 4 * gi + v;
        const float4 wm = *reinterpret_cast<const float4*>(wmax[h]);
        const float4 ws = *reinterpret_cast<const float4*>(wsum[h]);
        const float4 rs4 = *reinterpret_cast<const float4*>(rsum[h]);
        const float mbh = fmaxf(fmaxf(wm.x, wm.y), fmaxf(wm.z, wm.w));
        llr[v] = (ws.x + ws.y) + (ws.z + ws.w);
        const float lb = llr[v] + ((rs4.x + rs4.y) + (rs4.z + rs4.w));
        const float mn = fmaxf(m_run[v], mbh);
        alpha[v] = __builtin_amdgcn_exp2f(m_run[v] - mn);
        beta[v] = __builtin_amdgcn_exp2f(mbh - mn);
        l_run[v] = l_run[v] * alpha[v] + lb * beta[v];
        m_run[v] = mn;
      }
      float ca[8];
      if (win) {
#pragma unroll
        for (int s = 0; s < 8; ++s) ca[s] = 0.f;
      } else {
        sum_wave_partials(cb_part, hl, gi, ca);
      }
      // The residual probabilities, all read before the first product (rows
      // past R in the last step are 0; later steps are skipped).
      float pr[RS];
#pragma unroll
      for (int s = 0; s < RS; ++s) pr[s] = p_res[4 * s + gi][hl];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        // separate accumulators for the low-rank and the residual values, so
        // the two MFMA chains run side by side
        floatx4 t = {0.f, 0.f, 0.f, 0.f};
        floatx4 tr = {0.f, 0.f, 0.f, 0.f};
        if (!win) {
#pragma unroll
          for (int s = 0; s < 8; ++s) t = mfma4(ca[s], wv[dt][s], t);
        }
#pragma unroll
        for (int s = 0; s < RS; ++s)
          if (4 * s < R) tr = mfma4(pr[s], vr[s][dt], tr);
#pragma unroll
        for (int v = 0; v < 4; ++v)
          acc[dt][v] = acc[dt][v] * alpha[v] + beta[v] * ((t[v] + tr[v]) + llr[v] * va[dt]);
      }
      __syncthreads();  // LDS is reused by the next block
    }

    // ---- merge the chunks of (b, g) ------------------------------------------------
    // (chunk idx's partial lives at slot pair * S + idx)
    if (n_act == 1) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int h = 4 * gi + v;
        if (h >= G) continue;
        const int64_t hq = static_cast<int64_t>(b) * a.Hq + g * G + h;
        const float inv = l_run[v] > 0.f ? 1.f / l_run[v] : 0.f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) a.out[hq * D + dbase + 16 * dt + hl] = acc[dt][v] * inv;
        if (a.lse != nullptr && wave == 0 && hl == 0)
          a.lse[hq] = l_run[v] > 0.f ? (m_run[v] + __builtin_log2f(l_run[v])) * kLn2 : NEG_INF;
      }
      continue;
    }
    {
      // Rows of padding heads (h >= G) are never merged: their stores get an
      // offset past the buffer's range, which the hardware drops (no branch,
      // no memory traffic).
      const int64_t pbase = static_cast<int64_t>(pair) * S * 16;
      const __amdgpu_buffer_rsrc_t wacc =
          coherent_rsrc(a.part_acc + pbase * D, static_cast<uint32_t>(S * 16 * D * sizeof(float)));
      const __amdgpu_buffer_rsrc_t wml =
          coherent_rsrc(a.part_ml + pbase * 2, static_cast<uint32_t>(S * 16 * 2 * sizeof(float)));
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int h = 4 * gi + v;
        const bool real = h < G;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const uint32_t off = static_cast<uint32_t>(((idx * 16 + h) * D + dbase + 16 * dt + hl) * sizeof(float));
          store_coherent1(wacc, real ? off : kDroppedOffset, acc[dt][v]);
        }
        if (wave == 0 && hl == 0) {
          const uint32_t off = static_cast<uint32_t>((idx * 16 + h) * 2 * sizeof(float));
          store_coherent1(wml, real ? off : kDroppedOffset, m_run[v]);
          store_coherent1(wml, real ? off + 4 : kDroppedOffset, l_run[v]);
        }
      }
    }
    wait_stores_done();  // the partial is at the device coherence point before it is counted
    __syncthreads();
    if (threadIdx.x == 0) {
      const int old = __hip_atomic_fetch_add(a.counters + pair, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last_flag = old == n_act - 1;
    }
    __syncthreads();
    if (!last_flag) continue;
    // Every chunk's (m, l) at once: a wave per head (heads wave, wave + 4,
    // ... all requested together), a lane per chunk; lanes past n_act read
    // the last chunk and are masked. The chunk weights 2^(m_c - M) go to LDS.
    const int64_t slot0 = static_cast<int64_t>(pair) * S;
    constexpr int kHeadsPerWave = 16 / 4;  // at most 16 heads per KV head (the MFMA columns)
    float m_in[kHeadsPerWave], l_in[kHeadsPerWave];
    {
      const int cl = min(lane, n_act - 1);
#pragma unroll
      for (int i = 0; i < kHeadsPerWave; ++i) {
        const int h = min(wave + 4 * i, G - 1);
        m_in[i] = load_coherent(a.part_ml + ((slot0 + cl) * 16 + h) * 2);
        l_in[i] = load_coherent(a.part_ml + ((slot0 + cl) * 16 + h) * 2 + 1);
      }
    }
#pragma unroll
    for (int i = 0; i < kHeadsPerWave; ++i) {
      const int h = wave + 4 * i;
      if (h >= G) break;  // wave-uniform
      const bool has = lane < n_act;
      const float mc = has ? m_in[i] : NEG_INF;
      const float lc = has ? l_in[i] : 0.f;
      const bool valid = lc > 0.f;
      const float M = group_max<64>(valid ? mc : NEG_INF);
      const float wc = valid ? __builtin_amdgcn_exp2f(mc - M) : 0.f;
      const float Ls = group_sum<64>(wc * lc);
      merge_w[h][lane] = wc;
      if (lane == 0) {
        merge_h[h][0] = Ls;
        merge_h[h][1] = M;
      }
    }
    __syncthreads();
    // Weighted sums over the chunks: independent 16-byte device-coherent loads.
    const __amdgpu_buffer_rsrc_t prs = coherent_rsrc(
        a.part_acc + slot0 * 16 * D, static_cast<uint32_t>(n_act * 16 * D * sizeof(float)));
    for (int o = threadIdx.x; o < G * (D / 4); o += blockDim.x) {
      const int h = o / (D / 4);
      const int d = (o - h * (D / 4)) * 4;
      const int64_t hq = static_cast<int64_t>(b) * a.Hq + g * G + h;
      float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
      // All of a batch's loads are in flight together (one round trip per
      // batch). Chunk indices past n_act are clamped to the last chunk;
      // their weights merge_w[h][cc] are 0 (n_act <= S <= kWave).
      for (int c0 = 0; c0 < n_act; c0 += kMergeBatch) {
        float4 p[kMergeBatch];
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
          const int cc = min(c0 + u, n_act - 1);
          p[u] = load_coherent4(prs, static_cast<uint32_t>(((cc * 16 + h) * D + d) * sizeof(float)));
        }
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
          const float w = merge_w[h][min(c0 + u, kWave - 1)];
          num.x += w * p[u].x;
          num.y += w * p[u].y;
          num.z += w * p[u].z;
          num.w += w * p[u].w;
        }
      }
      const float Ls = merge_h[h][0];
      float4 o4 = make_float4(0.f, 0.f, 0.f, 0.f);
      if (Ls > 0.f) {
        o4.x = num.x / Ls;
        o4.y = num.y / Ls;
        o4.z = num.z / Ls;
        o4.w = num.w / Ls;
      }
      *reinterpret_cast<float4*>(a.out + hq * D + d) = o4;
      if (a.lse != nullptr && d == 0)
        a.lse[hq] = Ls > 0.f ? (merge_h[h][1] + __builtin_log2f(Ls)) * kLn2 : NEG_INF;
    }
    __syncthreads();
    if (threadIdx.x == 0) store_coherent_i(a.counters + pair, 0);  // ready for the next call
  }
}

template <typename T, int D>
hipError_t launch_dkv_decode_t(const DkvDecodeArgs& a, hipStream_t stream) {
  const int total = a.B * a.Hkv * (a.n_chunks + a.n_wchunks);
  const int grid = total < 2048 ? total : 2048;
  switch (a.P) {
    case 64: hipLaunchKernelGGL((dkv_attend_kernel<T, D, 1>), dim3(grid), dim3(256), 0, stream, a); break;
    case 128: hipLaunchKernelGGL((dkv_attend_kernel<T, D, 2>), dim3(grid), dim3(256), 0, stream, a); break;
    case 256: hipLaunchKernelGGL((dkv_attend_kernel<T, D, 4>), dim3(grid), dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dkv_decode_d(const DkvDecodeArgs& a, int D, hipStream_t stream) {
  if (D == 64) return launch_dkv_decode_t<T, 64>(a, stream);
  if (D == 128) return launch_dkv_decode_t<T, 128>(a, stream);
  return hipErrorInvalidValue;
}


// ---- codec ----------------------------------------------------------------------
// One workgroup (4 waves) per (sequence, block j < C, KV head). X = [K - k_a |
// V - v_a] (P x N, N = 2D, anchor a = token 0) streams through LDS as float32
// in 32-token chunks; the differences of two 16-bit values are exact there.
// The top-32 right singular subspace of X comes from subspace iteration on a
// block of 64 vectors followed by a Rayleigh-Ritz step: the 64-dimensional
// iterate converges to a subspace holding the top 32 at the rate
// (s_65 / s_32)^2 per round, whatever the gap between s_32 and s_33, and the
// Rayleigh-Ritz step picks the top 32 out of it.
//   Y = X Q    fp32 MFMA (N x 64 iterate Q, kept as Q^T in LDS);
//   Z = X^T Y  fp32 MFMA, accumulated in registers across the chunks;
//   Q = orth(Z)  Cholesky QR in double of the column-scaled Z: Q = Z S R^-1
//             with S the inverse column norms and R^T R the Gram of Z S. A
//             column whose squared pivot falls below kDropTol (its part
//             independent of the earlier columns is under 1e-5 of its norm)
//             is dropped, i.e. set to zero; so are zero columns.
//   Rayleigh-Ritz: H = Y^T Y = Q^T X^T X Q (64 x 64, fp32 MFMA, then
//             double), H = U diag(theta) U^T by cyclic Jacobi in double, and
//             the basis rows are (Q U)^T for the 32 largest Ritz values theta;
//             a row whose theta is at most kRitzDrop of the largest (a
//             direction X does not have) is set to zero.
// Rounds: with power_iters > 0 exactly that many. Otherwise kFirstRounds,
// then a Rayleigh-Ritz step whose Ritz values estimate the rate:
// rho = theta_64 / theta_32 (theta_64 <= s_64^2 and s_65 <= s_64, so rho
// bounds the rate of the remaining rounds by the measured spectrum), and the
// total becomes ceil(log(kConvTol) / log(rho)), between kFirstRounds and
// kRoundCap. The rounds run are written to the record.
// The start is a fixed pseudo-random matrix (murmur3's 32-bit finaliser of
// the element index), orthonormalised the same way. A last pass writes
// coef = X B^T and each token's squared float32 reconstruction error
// ||X_t - coef_t B||^2; the n_resid largest (ties to the lower offset) become
// the residual tokens.
constexpr int kIterVecs = 64;   // vectors of the subspace iterate (twice the rank)
constexpr int kXChunk = 32;     // tokens per X chunk in LDS
constexpr int kYRow = kIterVecs + 4;
constexpr double kDropTol = 1e-10;
constexpr double kRitzDrop = 1e-10;
constexpr int kFirstRounds = 8;
constexpr int kRoundCap = 64;
constexpr double kConvTol = 1e-6;
constexpr int kJacobiSweeps = 16;

template <int N>
struct CodecShared {
  float qt[kIterVecs][N + 4];  // Q^T (row i = iterate vector i); Z^T in place; the basis in rows 0..31
  union {
    float x[kXChunk][N + 4];                  // X chunk
    double u[kIterVecs][kIterVecs + 1];       // Rayleigh-Ritz eigenvectors (columns)
  } v;
  float y[kXChunk][kYRow];                    // Y = X Q of the chunk
  double g[kIterVecs][kIterVecs + 1];         // Gram of Z S (Cholesky QR) or H (Rayleigh-Ritz)
  double rdiag[kIterVecs];                     // 1 / the Cholesky diagonal (0 where dropped)
  double cs[kIterVecs];                       // column scales
  double jc[kIterVecs / 2], js[kIterVecs / 2];  // Jacobi rotations of one round
  double red[2][4];
  int32_t perm[kIterVecs];                    // Ritz vector index of the r-th largest value
  float anc[N];                               // anchor row [k_a | v_a]
  float err2[256];                            // per-token squared reconstruction error
  int32_t flag[256];
  int32_t ridx[kMaxResid];
  int32_t rounds;
};

__device__ __forceinline__ float codec_start_value(uint32_t i) {
  uint32_t x = i * 0x9E3779B9u + 0x7F4A7C15u;
  x ^= x >> 16;
  x *= 0x85EBCA6Bu;
  x ^= x >> 13;
  x *= 0xC2B2AE35u;
  x ^= x >> 16;
  return static_cast<float>(x >> 8) * (1.0f / 8388608.0f) - 1.0f;
}

typedef double doublex4 __attribute__((ext_vector_type(4)));

// W[i][j] = sum over the N channels of sh.qt[ra + i][c] * sh.qt[rb + j][c],
// i, j < 32, in double on v_mfma_f64_16x16x4f64, into sh.g: wave w (of 4)
// takes the 16 x 16 tile (w / 2, w % 2), four channels per step (lane l
// supplies row l % 16 of each operand at channel 4 s + l / 16, widened to
// double; result i of lane l is row 4 i + l / 16, column l % 16 of the tile,
// the layout of this instruction's output on gfx950, checked on the device).
template <int N>
__device__ __forceinline__ void codec_dot32(CodecShared<N>& sh, int tid, int ra, int rb) {
  const int wave = tid / kWave, lane = tid % kWave;
  const int ti = wave / 2, tj = wave % 2;
  const int m = lane % 16, kk = lane / 16;
  const float* arow = &sh.qt[ra + 16 * ti + m][kk];
  const float* brow = &sh.qt[rb + 16 * tj + m][kk];
  doublex4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 8
  for (int c = 0; c < N; c += 4)
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(static_cast<double>(arow[c]), static_cast<double>(brow[c]),
                                               acc, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) sh.g[16 * ti + 4 * i + kk][16 * tj + m] = acc[i];
}

// Cholesky QR, in place, of the 32 vectors in rows [r0, r0 + 32) of sh.qt:
// the Gram of the column-scaled vectors in double (codec_dot32, then scaled),
// a 32-step Cholesky with the
// drop rule above, and a forward substitution per channel in double. Starts
// after a barrier that published the rows and ends with one.
template <int N>
__device__ void codec_cholqr32(CodecShared<N>& sh, int tid, int r0) {
  codec_dot32<N>(sh, tid, r0, r0);
  __syncthreads();
  if (tid < kRank) {
    const double d = sh.g[tid][tid];
    sh.cs[tid] = d > 0.0 ? 1.0 / sqrt(d) : 0.0;
  }
  __syncthreads();
  for (int e = tid; e < kRank * kRank; e += 256) {
    const int i = e / kRank, j = e % kRank;
    sh.g[i][j] *= sh.cs[i] * sh.cs[j];
  }
  __syncthreads();
  for (int k = 0; k < kRank; ++k) {
    const double d = sh.g[k][k];
    const bool keep = d > kDropTol;
    const double rkk = keep ? sqrt(d) : 0.0;
    const double inv = keep ? 1.0 / rkk : 0.0;
    for (int e = tid; e < kRank * kRank; e += 256) {
      const int i = e / kRank, j = e % kRank;
      if (i > k && j >= i) sh.g[i][j] -= (sh.g[k][i] * inv) * (sh.g[k][j] * inv);
    }
    if (tid > k && tid < kRank) sh.g[tid][k] = sh.g[k][tid] * inv;
    if (tid == k) sh.rdiag[k] = inv;  // the substitution multiplies by 1 / r (0 if dropped)
    __syncthreads();
  }
  if (tid < N) {
    const int c = tid;
    double x[kRank];
#pragma unroll
    for (int j = 0; j < kRank; ++j) {
      double s = static_cast<double>(sh.qt[r0 + j][c]) * sh.cs[j];
#pragma unroll
      for (int i = 0; i < j; ++i) s -= x[i] * sh.g[j][i];
      x[j] = s * sh.rdiag[j];
    }
#pragma unroll
    for (int j = 0; j < kRank; ++j) sh.qt[r0 + j][c] = static_cast<float>(x[j]);
  }
  __syncthreads();
}

// Rows [32, 64) of sh.qt minus their projection on rows [0, 32), which are
// orthonormal: W = Q1^T Z2 in double (codec_dot32), then Z2 -= Q1 W in
// double, both on f64 MFMA.
template <int N>
__device__ void codec_project_out(CodecShared<N>& sh, int tid) {
  codec_dot32<N>(sh, tid, 0, kRank);
  __syncthreads();
  // Z2 -= Q1 W on v_mfma_f64_16x16x4f64, over the (channel, vector) plane of
  // Z2 in 16 x 16 tiles, tile t = (channels 16 (t / 2).., vectors 16 (t % 2)..)
  // taken by wave t % 4: the accumulator starts at Z2 and the A operand is
  // -Q1 (lane l supplies channel l % 16 of vector 4 s + l / 16), the B
  // operand W (row 4 s + l / 16, column l % 16); result i of lane l is
  // channel 4 i + l / 16, vector l % 16 of the tile.
  {
    const int wave = tid / kWave, lane = tid % kWave;
    const int m = lane % 16, kk = lane / 16;
    constexpr int NT = (N / 16) * (kRank / 16);
    for (int t = wave; t < NT; t += 4) {
      const int c0 = 16 * (t / 2), j0 = 16 * (t % 2);
      doublex4 acc;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = static_cast<double>(sh.qt[kRank + j0 + m][c0 + 4 * i + kk]);
#pragma unroll
      for (int s = 0; s < kRank / 4; ++s)
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(-static_cast<double>(sh.qt[4 * s + kk][c0 + m]),
                                                   sh.g[4 * s + kk][j0 + m], acc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) sh.qt[kRank + j0 + m][c0 + 4 * i + kk] = static_cast<float>(acc[i]);
    }
  }
  __syncthreads();
}

// Q^T <- orth(Z^T) in place on sh.qt, 64 vectors: the first 32 by Cholesky
// QR, the last 32 with the first 32 projected out (twice, so that what is
// left is orthogonal to working precision) and then by Cholesky QR. Starts
// after a barrier that published Z^T and ends with one.
template <int N>
__device__ void codec_orthonormalize(CodecShared<N>& sh, int tid) {
  codec_cholqr32<N>(sh, tid, 0);
  codec_project_out<N>(sh, tid);
  codec_project_out<N>(sh, tid);
  codec_cholqr32<N>(sh, tid, kRank);
}

// Members of pair m in round r of the circle tournament over 64 indices:
// every round pairs each index once, and 63 rounds pair every two indices.
__device__ __forceinline__ void jacobi_pair(int r, int m, int& p, int& q) {
  if (m == 0) {
    p = kIterVecs - 1;
    q = r;
  } else {
    p = (r + m) % (kIterVecs - 1);
    q = (r - m + kIterVecs - 1) % (kIterVecs - 1);
  }
}

// Cyclic Jacobi on the symmetric sh.g (64 x 64, double): sweeps of 63 rounds
// of 32 disjoint rotations until the off-diagonal part is negligible. The
// eigenvalues end on the diagonal; with VECTORS the eigenvectors end in the
// columns of sh.v.u. Starts after a barrier that published sh.g; ends with one.
template <int N, bool VECTORS>
__device__ void codec_jacobi(CodecShared<N>& sh, int tid) {
  constexpr int V = kIterVecs;
  if constexpr (VECTORS) {
    for (int e = tid; e < V * V; e += 256) sh.v.u[e / V][e % V] = (e / V == e % V) ? 1.0 : 0.0;
  }
  __syncthreads();
  for (int sweep = 0; sweep < kJacobiSweeps; ++sweep) {
    // stop once the off-diagonal square sum is below kOff of the total: 1e-16
    // for the Ritz vectors (an off-diagonal norm of 1e-8 of H's moves the
    // 32-vector subspace by 1e-8 over the relative gap at 32, far below the
    // float32 basis it feeds wherever that subspace is well defined), 1e-12
    // when only the Ritz values are wanted
    constexpr double kOff = VECTORS ? 1e-16 : 1e-12;
    double off = 0.0, all = 0.0;
    for (int e = tid; e < V * V; e += 256) {
      const double h = sh.g[e / V][e % V];
      all += h * h;
      if (e / V != e % V) off += h * h;
    }
    off = group_sum<kWave>(off);
    all = group_sum<kWave>(all);
    if (tid % kWave == 0) {
      sh.red[0][tid / kWave] = off;
      sh.red[1][tid / kWave] = all;
    }
    __syncthreads();
    const double off_t = sh.red[0][0] + sh.red[0][1] + sh.red[0][2] + sh.red[0][3];
    const double all_t = sh.red[1][0] + sh.red[1][1] + sh.red[1][2] + sh.red[1][3];
    __syncthreads();
    if (!(off_t > kOff * all_t)) break;  // uniform: every thread read the same sums
    for (int r = 0; r < V - 1; ++r) {
      if (tid < V / 2) {
        int p, q;
        jacobi_pair(r, tid, p, q);
        const double app = sh.g[p][p], aqq = sh.g[q][q], apq = sh.g[p][q];
        double c = 1.0, sn = 0.0;
        if (apq != 0.0) {
          // the rotation that zeroes (p, q): t = tan of its angle, the
          // smaller root of t^2 + 2 theta t - 1 = 0
          const double theta = (aqq - app) / (2.0 * apq);
          const double t = (theta >= 0.0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
          c = 1.0 / sqrt(t * t + 1.0);
          sn = t * c;
        }
        sh.jc[tid] = c;
        sh.js[tid] = sn;
      }
      __syncthreads();
      // H <- P^T H P, by 2 x 2 blocks of (pair m rows, pair n columns); P
      // maps (p, q) to (c p - s q, s p + c q)
      for (int e = tid; e < (V / 2) * (V / 2); e += 256) {
        const int m = e / (V / 2), n = e % (V / 2);
        int pm, qm, pn, qn;
        jacobi_pair(r, m, pm, qm);
        jacobi_pair(r, n, pn, qn);
        const double cm = sh.jc[m], sm = sh.js[m], cn = sh.jc[n], snn = sh.js[n];
        const double h00 = sh.g[pm][pn], h01 = sh.g[pm][qn], h10 = sh.g[qm][pn], h11 = sh.g[qm][qn];
        // rows: R_m^T B
        const double b00 = cm * h00 - sm * h10, b01 = cm * h01 - sm * h11;
        const double b10 = sm * h00 + cm * h10, b11 = sm * h01 + cm * h11;
        // columns: (R_m^T B) R_n
        sh.g[pm][pn] = cn * b00 - snn * b01;
        sh.g[pm][qn] = snn * b00 + cn * b01;
        sh.g[qm][pn] = cn * b10 - snn * b11;
        sh.g[qm][qn] = snn * b10 + cn * b11;
      }
      if constexpr (VECTORS) {
        for (int e = tid; e < V * (V / 2); e += 256) {
          const int i = e / (V / 2), n = e % (V / 2);
          int pn, qn;
          jacobi_pair(r, n, pn, qn);
          const double cn = sh.jc[n], snn = sh.js[n];
          const double up = sh.v.u[i][pn], uq = sh.v.u[i][qn];
          sh.v.u[i][pn] = cn * up - snn * uq;
          sh.v.u[i][qn] = snn * up + cn * uq;
        }
      }
      __syncthreads();
    }
  }
  // ranks of the eigenvalues, descending (ties to the lower index)
  if (tid < V) {
    const double t = sh.g[tid][tid];
    int rank = 0;
    for (int j = 0; j < V; ++j) {
      const double u = sh.g[j][j];
      rank += (u > t) || (u == t && j < tid);
    }
    sh.perm[rank] = tid;
  }
  __syncthreads();
}

// X rows [32 ch, 32 ch + 32) of the tile pair: codec_issue_chunk requests
// them into registers, codec_commit_chunk writes them to sh.v.x with the
// anchor subtracted.
template <typename T, int D>
struct CodecChunk {
  static constexpr int VPR = D * T::kBytes / 16;   // 16-byte vectors per K (or V) row
  static constexpr int VPC = kXChunk * VPR;         // per pool and chunk
  static constexpr int PER_THREAD = (2 * VPC + 255) / 256;  // K and V vectors per thread
  uint4 v[PER_THREAD];
};

template <typename T, int D>
__device__ __forceinline__ void codec_issue_chunk(CodecChunk<T, D>& cc, const char* ktile,
                                                  const char* vtile, int ch, int tid) {
  using CC = CodecChunk<T, D>;
#pragma unroll
  for (int u = 0; u < CC::PER_THREAD; ++u) {
    const int v = min(tid + 256 * u, 2 * CC::VPC - 1);
    const bool isv = v >= CC::VPC;
    const int w = isv ? v - CC::VPC : v;
    const int row = w / CC::VPR;
    const int col = (w % CC::VPR) * T::kPerVec;
    cc.v[u] = load16((isv ? vtile : ktile) + (static_cast<int64_t>(kXChunk * ch + row) * D + col) * T::kBytes);
  }
}

template <typename T, int D>
__device__ __forceinline__ void codec_commit_chunk(CodecShared<2 * D>& sh, const CodecChunk<T, D>& cc,
                                                   int tid) {
  using CC = CodecChunk<T, D>;
  constexpr int EPV = T::kPerVec;
#pragma unroll
  for (int u = 0; u < CC::PER_THREAD; ++u) {
    const int v = tid + 256 * u;
    if (v >= 2 * CC::VPC) continue;
    const bool isv = v >= CC::VPC;
    const int w = isv ? v - CC::VPC : v;
    const int row = w / CC::VPR;
    const int col = (w % CC::VPR) * EPV;
    float f[EPV];
    T::widen(cc.v[u], f);
    const int c0 = (isv ? D : 0) + col;
#pragma unroll
    for (int e = 0; e < EPV; e += 4) {
      float4 o;
      o.x = f[e + 0] - sh.anc[c0 + e + 0];
      o.y = f[e + 1] - sh.anc[c0 + e + 1];
      o.z = f[e + 2] - sh.anc[c0 + e + 2];
      o.w = f[e + 3] - sh.anc[c0 + e + 3];
      *reinterpret_cast<float4*>(&sh.v.x[row][c0 + e]) = o;
    }
  }
}

// Y = X Q for the chunk in sh.v.x: wave w computes token tile w % 2 against
// iterate vectors [32 (w / 2), 32 (w / 2) + 32) (two 16 x 16 tiles) and
// stores them in sh.y. BT basis tiles are used in total (4: the iterate; 2:
// the final 32-row basis, then only waves with w / 2 == 0 have work).
template <int N, int BT>
__device__ __forceinline__ void codec_y(CodecShared<N>& sh, int wave, int hl, int gi) {
  constexpr int NCG = N / 16;
  const int tt = wave % 2;
  const int bt0 = 2 * (wave / 2);
  if (bt0 >= BT) return;  // uniform per wave
  floatx4 yv[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll 4
  for (int cg = 0; cg < NCG; ++cg) {
    const float4 xa = *reinterpret_cast<const float4*>(&sh.v.x[16 * tt + hl][16 * cg + 4 * gi]);
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const float4 qb = *reinterpret_cast<const float4*>(&sh.qt[16 * (bt0 + rt) + hl][16 * cg + 4 * gi]);
      yv[rt] = mfma4(xa.x, qb.x, yv[rt]);
      yv[rt] = mfma4(xa.y, qb.y, yv[rt]);
      yv[rt] = mfma4(xa.z, qb.z, yv[rt]);
      yv[rt] = mfma4(xa.w, qb.w, yv[rt]);
    }
  }
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int v = 0; v < 4; ++v) sh.y[16 * tt + 4 * gi + v][16 * (bt0 + rt) + hl] = yv[rt][v];
}

template <typename T, int D>
__global__ __launch_bounds__(256) void dkv_compress_kernel(DkvCompressArgs a) {
  constexpr int E = T::kBytes;
  constexpr int N = 2 * D;
  constexpr int NCT = N / 64;      // 16-channel Z tiles per wave
  constexpr int VPR = D * E / 16;  // 16-byte vectors per K (or V) row
  constexpr int V = kIterVecs;
  __shared__ CodecShared<N> sh;

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int hl = lane % 16;
  const int gi = lane / 16;
  const int64_t total = static_cast<int64_t>(a.B) * a.max_blocks * a.Hkv;
  const int n_chunks = a.P / kXChunk;
  const int R = a.n_resid;

  for (int64_t item = blockIdx.x; item < total; item += gridDim.x) {
    const int g = static_cast<int>(item % a.Hkv);
    const int64_t bj = item / a.Hkv;
    const int j = static_cast<int>(bj % a.max_blocks);
    const int b = static_cast<int>(bj / a.max_blocks);
    if (j >= window_start_block(a.context_lens[b], a.P, a.recent_window)) continue;
    const int64_t phys = a.block_table[static_cast<int64_t>(b) * a.max_blocks + j];
    if (phys < 0 || phys >= a.num_phys) continue;
    const int64_t tile_off = (phys * a.Hkv + g) * a.P * static_cast<int64_t>(D) * E;
    const char* ktile = static_cast<const char*>(a.k_pool) + tile_off;
    const char* vtile = static_cast<const char*>(a.v_pool) + tile_off;
    char* rec = a.records + (phys * a.Hkv + g) * a.rec_bytes;

    // anchor: float32 copy for the differences, raw copy into the record
    for (int c = tid; c < N; c += 256) sh.anc[c] = c < D ? T::load1(ktile, c) : T::load1(vtile, c - D);
    if (tid < 2 * VPR) store16(rec + tid * 16, load16((tid < VPR ? ktile : vtile) + (tid % VPR) * 16));
    for (int e = tid; e < V * N; e += 256) sh.qt[e / N][e % N] = codec_start_value(e);
    __syncthreads();
    codec_orthonormalize<N>(sh, tid);

    // Passes over X: Z^T = (X^T X Q)^T into sh.qt (RITZ false), or H = Q^T
    // X^T X Q into sh.g (RITZ true).
    auto x_pass = [&](bool ritz) {
      floatx4 zacc[NCT][4];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int bt = 0; bt < 4; ++bt) zacc[ct][bt] = floatx4{0.f, 0.f, 0.f, 0.f};
      for (int ch = 0; ch < n_chunks; ++ch) {
        CodecChunk<T, D> now;
        codec_issue_chunk<T, D>(now, ktile, vtile, ch, tid);
        codec_commit_chunk<T, D>(sh, now, tid);
        __syncthreads();
        codec_y<N, 4>(sh, wave, hl, gi);
        __syncthreads();
        if (!ritz) {
          // Z^T += (X^T Y)^T: wave w takes channel tiles [NCT w, NCT (w + 1));
          // k-slot gi of step s is token 4 s + gi
#pragma unroll 2
          for (int s = 0; s < kXChunk / 4; ++s) {
            const int t = 4 * s + gi;
            float yb[4];
#pragma unroll
            for (int bt = 0; bt < 4; ++bt) yb[bt] = sh.y[t][16 * bt + hl];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
              const float xa = sh.v.x[t][16 * (wave * NCT + ct) + hl];
#pragma unroll
              for (int bt = 0; bt < 4; ++bt) zacc[ct][bt] = mfma4(xa, yb[bt], zacc[ct][bt]);
            }
          }
        } else {
          // H += Y^T Y: wave w takes row tile w, all four column tiles
#pragma unroll 2
          for (int s = 0; s < kXChunk / 4; ++s) {
            const int t = 4 * s + gi;
            const float ya = sh.y[t][16 * wave + hl];
#pragma unroll
            for (int bt = 0; bt < 4; ++bt) zacc[0][bt] = mfma4(ya, sh.y[t][16 * bt + hl], zacc[0][bt]);
          }
        }
        __syncthreads();  // x and y are overwritten next
      }
      if (!ritz) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int bt = 0; bt < 4; ++bt)
#pragma unroll
            for (int v = 0; v < 4; ++v)
              sh.qt[16 * bt + hl][16 * (wave * NCT + ct) + 4 * gi + v] = zacc[ct][bt][v];
      } else {
#pragma unroll
        for (int bt = 0; bt < 4; ++bt)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            sh.g[16 * wave + 4 * gi + v][16 * bt + hl] = static_cast<double>(zacc[0][bt][v]);
      }
      __syncthreads();
    };

    int rounds = a.power_iters > 0 ? a.power_iters : kRoundCap;
    bool ritz_done = false;  // uniform: the final Rayleigh-Ritz is already in sh
    for (int k = 0;; ++k) {
      if (a.power_iters == 0 && k == kFirstRounds) {
        // Rayleigh-Ritz of the current iterate: its values (the measured
        // rate) set the rounds, and when no more rounds are needed its
        // vectors are the final ones (the iterate does not change again)
        x_pass(true);
        codec_jacobi<N, true>(sh, tid);
        const double t32 = sh.g[sh.perm[kRank - 1]][sh.perm[kRank - 1]];
        const double t64 = sh.g[sh.perm[V - 1]][sh.perm[V - 1]];
        const double rho = t32 > 0.0 ? fmax(t64, 0.0) / t32 : 0.0;
        int want = kFirstRounds;
        if (rho >= 1.0) {
          want = kRoundCap;
        } else if (rho > 0.0) {
          const double need = ceil(log(kConvTol) / log(rho));
          want = need > kRoundCap ? kRoundCap : (need < kFirstRounds ? kFirstRounds : static_cast<int>(need));
        }
        rounds = want;  // the same on every thread (LDS values after a barrier)
        ritz_done = rounds <= k;
        __syncthreads();
      }
      if (k >= rounds) break;
      x_pass(false);
      codec_orthonormalize<N>(sh, tid);
    }

    // Rayleigh-Ritz: basis rows = (Q U)^T for the 32 largest Ritz values
    if (!ritz_done) {
      x_pass(true);
      codec_jacobi<N, true>(sh, tid);
    }
    {
      const double tmax = sh.g[sh.perm[0]][sh.perm[0]];
      if (tid < N) {
        const int c = tid;
        float qc[V];
#pragma unroll
        for (int i = 0; i < V; ++i) qc[i] = sh.qt[i][c];
#pragma unroll 1
        for (int r = 0; r < kRank; ++r) {
          const int pr = sh.perm[r];
          double acc = 0.0;
#pragma unroll
          for (int i = 0; i < V; ++i) acc += static_cast<double>(qc[i]) * sh.v.u[i][pr];
          const bool live = sh.g[pr][pr] > kRitzDrop * tmax && tmax > 0.0;
          sh.qt[r][c] = live ? static_cast<float>(acc) : 0.f;
        }
      }
    }
    __syncthreads();

    // last pass: coef = X B^T and the per-token squared errors
    for (int ch = 0; ch < n_chunks; ++ch) {
      CodecChunk<T, D> now;
      codec_issue_chunk<T, D>(now, ktile, vtile, ch, tid);
      codec_commit_chunk<T, D>(sh, now, tid);
      __syncthreads();
      codec_y<N, 2>(sh, wave, hl, gi);
      __syncthreads();
      for (int e = tid; e < kXChunk * kRank; e += 256) {
        const int t = e / kRank, r = e % kRank;
        reinterpret_cast<float*>(rec + a.off_coef)[(kXChunk * ch + t) * kRank + r] = sh.y[t][r];
      }
      // squared error of X - Y B for tokens [16 (w % 2), 16 (w % 2) + 16),
      // channel tiles of parity w / 2
      {
        const int tt = wave % 2;
        float sq[4] = {0.f, 0.f, 0.f, 0.f};
        for (int ct = wave / 2; ct < N / 16; ct += 2) {
          floatx4 xh = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int rg = 0; rg < 2; ++rg) {
            const float4 ya = *reinterpret_cast<const float4*>(&sh.y[16 * tt + hl][16 * rg + 4 * gi]);
            const int r0 = 16 * rg + 4 * gi;
            xh = mfma4(ya.x, sh.qt[r0 + 0][16 * ct + hl], xh);
            xh = mfma4(ya.y, sh.qt[r0 + 1][16 * ct + hl], xh);
            xh = mfma4(ya.z, sh.qt[r0 + 2][16 * ct + hl], xh);
            xh = mfma4(ya.w, sh.qt[r0 + 3][16 * ct + hl], xh);
          }
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float e = sh.v.x[16 * tt + 4 * gi + v][16 * ct + hl] - xh[v];
            sq[v] += e * e;
          }
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) sq[v] = group_sum<16>(sq[v]);
        // the two channel halves of a token tile are summed through LDS:
        // waves 0/1 write, waves 2/3 add after the barrier
        if (wave < 2) {
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (hl == 0) sh.err2[kXChunk * ch + 16 * tt + 4 * gi + v] = sq[v];
        }
        __syncthreads();
        if (wave >= 2) {
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (hl == 0) sh.err2[kXChunk * ch + 16 * tt + 4 * gi + v] += sq[v];
        }
      }
      __syncthreads();  // x and y are overwritten next
    }

    // basis rows
    for (int e = 4 * tid; e < kRank * N; e += 4 * 256) {
      const int r = e / N, c = e % N;
      *reinterpret_cast<float4*>(rec + a.off_basis + static_cast<int64_t>(e) * 4) =
          *reinterpret_cast<const float4*>(&sh.qt[r][c]);
    }
    // residual tokens: rank of each token's error, then ascending offsets
    if (tid < a.P) {
      const float e = sh.err2[tid];
      int rank = 0;
      for (int u = 0; u < a.P; ++u) {
        const float f = sh.err2[u];
        rank += (f > e) || (f == e && u < tid);
      }
      sh.flag[tid] = rank < R;
    }
    __syncthreads();
    if (tid < a.P && sh.flag[tid]) {
      int pos = 0;
      for (int u = 0; u < tid; ++u) pos += sh.flag[u];
      if (pos < R) sh.ridx[pos] = tid;
    }
    __syncthreads();
    if (tid < R) reinterpret_cast<int32_t*>(rec + a.off_ridx)[tid] = sh.ridx[tid];
    if (tid == 0) *reinterpret_cast<int32_t*>(rec + a.off_rounds) = rounds;
    for (int v = tid; v < R * 2 * VPR; v += 256) {
      const int row = v / (2 * VPR);
      const int w = v % (2 * VPR);
      const bool isv = w >= VPR;
      const int64_t src_off = static_cast<int64_t>(sh.ridx[row]) * D * E + (w % VPR) * 16;
      char* dst = rec + (isv ? a.off_rv : a.off_rk) + static_cast<int64_t>(row) * D * E + (w % VPR) * 16;
      store16(dst, load16((isv ? vtile : ktile) + src_off));
    }
    __syncthreads();  // LDS is reused by the next item
  }
}

template <typename T>
hipError_t launch_dkv_compress_d(const DkvCompressArgs& a, int D, hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(a.B) * a.max_blocks * a.Hkv;
  if (total <= 0) return hipSuccess;
  const int grid = total < 1024 ? static_cast<int>(total) : 1024;
  if (a.P % kXChunk != 0 || a.P > 256) return hipErrorInvalidValue;
  if (D == 64) {
    hipLaunchKernelGGL((dkv_compress_kernel<T, 64>), dim3(grid), dim3(256), 0, stream, a);
  } else if (D == 128) {
    hipLaunchKernelGGL((dkv_compress_kernel<T, 128>), dim3(grid), dim3(256), 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dkv_decode(const DkvDecodeArgs& a, int dtype, int D, hipStream_t stream) {
  switch (dtype) {
    case KVSP_F32: return launch_dkv_decode_d<F32>(a, D, stream);
    case KVSP_F16: return launch_dkv_decode_d<F16>(a, D, stream);
    case KVSP_BF16: return launch_dkv_decode_d<BF16>(a, D, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_dkv_compress(const DkvCompressArgs& a, int dtype, int D, hipStream_t stream) {
  switch (dtype) {
    case KVSP_F32: return launch_dkv_compress_d<F32>(a, D, stream);
    case KVSP_F16: return launch_dkv_compress_d<F16>(a, D, stream);
    case KVSP_BF16: return launch_dkv_compress_d<BF16>(a, D, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvsp
