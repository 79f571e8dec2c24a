// Steps 2 and 3: block relevance scores, Top-k with the keep floor, span
// merge and the dense-fallback flag (SparPR news page, "Three decisions rather
// than one compression ratio": paragraphs "Query-Aware key-block selection",
// "Dynamic budget control" and "On-demand local recomputation with cost-aware
// fallback").
//
// score_kernel: a block's score is sum_h <q_h, s_{j, g(h)}> over all query
// heads. By linearity it is computed as sum_g <qbar_g, s_{j,g}> with qbar_g the
// sum of the group's query heads (in ascending head order, in double). Each
// workgroup handles one sequence: it builds qbar in LDS once, then each wave
// streams whole summary rows (Hkv * D contiguous floats per physical block)
// with 16-byte loads and reduces the dot product in double. HBM-bound:
// Hkv * D * 4 bytes per candidate block.
//
// topk_kernel: one 1024-thread workgroup per sequence. The scores become
// order-preserving 32-bit keys (-0 folded onto +0); an MSB-first radix select
// (four 8-bit passes, LDS histograms) finds the k-th largest key T; blocks
// with key > T are kept, and of those equal to T the lowest indices fill the
// remaining places (ties go to the lower block index). Block-wide scans then
// emit the kept ids in ascending order and the span boundaries.

#include "kvsp_device.h"
#include "kvsp_internal.h"

namespace kvsp {

// ---- scores ---------------------------------------------------------------------

template <typename T>
__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a) {
  extern __shared__ double qbar[];  // [Hkv * D]
  const int b = blockIdx.y;
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const SelectArgs sel{a.top_k, a.keep_num, a.keep_den, a.keep_floor, a.recent_window,
                       a.gamma_num, a.gamma_den};
  const int L = a.context_lens[b];
  const int C = plan_sequence(L, a.P, sel).C;
  const int first = blockIdx.x * 4 * a.blocks_per_wave;
  if (first >= C) return;  // uniform over the workgroup

  const int G = a.Hq / a.Hkv;
  const int row = a.Hkv * a.D;
  const void* qb = static_cast<const char*>(a.q) + static_cast<int64_t>(b) * a.Hq * a.D * T::kBytes;
  for (int p = threadIdx.x; p < row; p += blockDim.x) {
    const int g = p / a.D;
    const int d = p % a.D;
    double s = 0.0;
    for (int h = 0; h < G; ++h) s += static_cast<double>(T::load1(qb, static_cast<int64_t>(g * G + h) * a.D + d));
    qbar[p] = s;
  }
  __syncthreads();

  const int j0 = first + wave * a.blocks_per_wave;
  const int j1 = min(C, j0 + a.blocks_per_wave);
  const int nvec = row / 4;
  for (int j = j0; j < j1; ++j) {
    const int64_t phys = a.block_table[static_cast<int64_t>(b) * a.max_blocks + j];
    const float4* srow = reinterpret_cast<const float4*>(a.summaries + phys * row);
    double acc = 0.0;
    for (int v = lane; v < nvec; v += kWave) {
      const float4 s = srow[v];
      const double* qv = qbar + 4 * v;
      acc += qv[0] * static_cast<double>(s.x);
      acc += qv[1] * static_cast<double>(s.y);
      acc += qv[2] * static_cast<double>(s.z);
      acc += qv[3] * static_cast<double>(s.w);
    }
    acc = wave_sum(acc);
    if (lane == 0) a.scores[static_cast<int64_t>(b) * a.max_blocks + j] = static_cast<float>(acc);
  }
}

template <typename T>
static hipError_t launch_score_t(const ScoreArgs& a, hipStream_t stream) {
  const int per_wg = 4 * a.blocks_per_wave;
  dim3 grid((a.max_blocks + per_wg - 1) / per_wg, a.B);
  const size_t lds = static_cast<size_t>(a.Hkv) * a.D * sizeof(double);
  hipLaunchKernelGGL((score_kernel<T>), grid, dim3(256), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_score(const ScoreArgs& a, int dtype, hipStream_t stream) {
  if (dtype == KVSP_F32) return launch_score_t<F32>(a, stream);
  if (dtype == KVSP_F16) return launch_score_t<F16>(a, stream);
  return launch_score_t<BF16>(a, stream);
}

// ---- Top-k, spans, dense flag -------------------------------------------------------

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kTopkMaxPerThread = 16;  // max_blocks <= 16384

// Larger float <=> larger key; -0.0 and +0.0 map to the same key.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  return x;
}

// Exclusive prefix sum of v over the workgroup in thread order; `total` gets
// the sum over all threads. Every thread must call it. tmp holds
// 2 * (kTopkWaves + 1) words: wave totals, then their exclusive scan.
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t* tmp, uint32_t& total) {
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const uint32_t incl = wave_incl_scan(v, lane);
  if (lane == kWave - 1) tmp[wave] = incl;
  __syncthreads();
  uint32_t* offs = tmp + kTopkWaves + 1;
  if (wave == 0) {
    const uint32_t w = lane < kTopkWaves ? tmp[lane] : 0u;
    const uint32_t wi = wave_incl_scan(w, lane);
    if (lane < kTopkWaves) offs[lane] = wi - w;
    if (lane == kTopkWaves - 1) offs[kTopkWaves] = wi;
  }
  __syncthreads();
  const uint32_t res = offs[wave] + incl - v;
  total = offs[kTopkWaves];
  __syncthreads();
  return res;
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t scan_tmp[2 * (kTopkWaves + 1)];
  __shared__ uint32_t bcast[2];
  extern __shared__ uint8_t kept[];  // [max_blocks] 0/1 per candidate
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t % kWave;
  const SelectArgs sel{a.top_k, a.keep_num, a.keep_den, a.keep_floor, a.recent_window,
                       a.gamma_num, a.gamma_den};
  const int L = a.context_lens[b];
  const SeqPlan p = plan_sequence(L, a.P, sel);
  const int C = p.C;
  const int k = p.k;
  const int R = (C + kTopkThreads - 1) / kTopkThreads;  // consecutive candidates per thread
  const int jbase = t * R;
  const int64_t row = static_cast<int64_t>(b) * a.max_blocks;

  uint32_t key[kTopkMaxPerThread];
#pragma unroll
  for (int r = 0; r < kTopkMaxPerThread; ++r) {
    const int j = jbase + r;
    key[r] = (r < R && j < C) ? order_key(a.scores[row + j]) : 0u;
  }

  // Radix select of the k-th largest key (only when 0 < k < C).
  uint32_t thresh = 0;
  int take_equal = 0;
  const bool partial = k > 0 && k < C;
  if (partial) {
    uint32_t prefix = 0, mask = 0;
    int krem = k;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      if (t < 256) hist[t] = 0;
      __syncthreads();
#pragma unroll
      for (int r = 0; r < kTopkMaxPerThread; ++r) {
        const int j = jbase + r;
        if (r < R && j < C && (key[r] & mask) == prefix) atomicAdd(&hist[(key[r] >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (t < kWave) {
        // lane owns digits 4*lane .. 4*lane+3; count keys in digits above
        uint32_t h[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = hist[4 * lane + i];
        const uint32_t local = h[0] + h[1] + h[2] + h[3];
        const uint32_t rev = __shfl(local, kWave - 1 - lane, kWave);
        const uint32_t rev_incl = wave_incl_scan(rev, lane);
        const uint32_t suffix_incl = __shfl(rev_incl, kWave - 1 - lane, kWave);
        uint32_t above = suffix_incl - local;  // keys in digits owned by higher lanes
        for (int i = 3; i >= 0; --i) {
          if (above < static_cast<uint32_t>(krem) && static_cast<uint32_t>(krem) <= above + h[i]) {
            bcast[0] = 4u * lane + i;
            bcast[1] = static_cast<uint32_t>(krem) - above;
          }
          above += h[i];
        }
      }
      __syncthreads();
      const uint32_t digit = bcast[0];
      krem = static_cast<int>(bcast[1]);
      prefix |= digit << shift;
      mask |= 0xFFu << shift;
      __syncthreads();
    }
    thresh = prefix;
    take_equal = krem;
  }

  // Kept flags in index order.
  uint32_t n_eq = 0;
#pragma unroll
  for (int r = 0; r < kTopkMaxPerThread; ++r) {
    const int j = jbase + r;
    if (partial && r < R && j < C && key[r] == thresh) ++n_eq;
  }
  uint32_t eq_total;
  uint32_t eq_before = block_excl_scan(n_eq, scan_tmp, eq_total);
  uint32_t keep_bits = 0, n_keep = 0;
#pragma unroll
  for (int r = 0; r < kTopkMaxPerThread; ++r) {
    const int j = jbase + r;
    if (!(r < R && j < C)) continue;
    bool keep;
    if (k >= C) {
      keep = true;
    } else if (k == 0) {
      keep = false;
    } else if (key[r] > thresh) {
      keep = true;
    } else if (key[r] == thresh) {
      keep = eq_before < static_cast<uint32_t>(take_equal);
      ++eq_before;
    } else {
      keep = false;
    }
    if (keep) {
      keep_bits |= 1u << r;
      ++n_keep;
    }
  }
  uint32_t keep_total;
  const uint32_t pos0 = block_excl_scan(n_keep, scan_tmp, keep_total);
  uint32_t pos = pos0;
#pragma unroll
  for (int r = 0; r < kTopkMaxPerThread; ++r) {
    const int j = jbase + r;
    if (r < R && j < C) {
      const bool keep = (keep_bits >> r) & 1u;
      kept[j] = keep ? 1 : 0;
      if (keep) a.selected[row + pos++] = j;
    }
  }
  __syncthreads();

  // Span boundaries: a run starts where a kept block follows a dropped one
  // and ends where a dropped one (or the candidate range end) follows.
  const bool window = p.n > C;
  uint32_t n_start = 0, n_end = 0;
#pragma unroll
  for (int r = 0; r < kTopkMaxPerThread; ++r) {
    const int j = jbase + r;
    if (r < R && j < C && ((keep_bits >> r) & 1u)) {
      if (j == 0 || !kept[j - 1]) ++n_start;
      if (j == C - 1 || !kept[j + 1]) ++n_end;
    }
  }
  uint32_t se_total;
  const uint32_t se_before = block_excl_scan((n_start << 16) | n_end, scan_tmp, se_total);
  uint32_t s_idx = se_before >> 16, e_idx = se_before & 0xFFFFu;
  int32_t* sp = a.spans + row * 2 + static_cast<int64_t>(b) * 2;  // [B][max_blocks+1][2]
#pragma unroll
  for (int r = 0; r < kTopkMaxPerThread; ++r) {
    const int j = jbase + r;
    if (r < R && j < C && ((keep_bits >> r) & 1u)) {
      if (j == 0 || !kept[j - 1]) sp[2 * s_idx++] = j;
      if (j == C - 1 || !kept[j + 1]) sp[2 * e_idx++ + 1] = (j == C - 1 && window) ? p.n : j + 1;
    }
  }
  if (t == 0) {
    const int sel_spans = static_cast<int>(se_total >> 16);
    const bool joined = C > 0 && k > 0 && kept[C - 1];
    int nsp = sel_spans;
    if (window && !joined) {
      sp[2 * nsp] = C;
      sp[2 * nsp + 1] = p.n;
      ++nsp;
    }
    a.num_selected[b] = k;
    a.num_spans[b] = nsp;
    a.use_dense[b] = p.dense;
  }
  (void)lane;
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t stream) {
  const size_t lds = static_cast<size_t>((a.max_blocks + 3) / 4 * 4);
  hipLaunchKernelGGL(topk_kernel, dim3(a.B), dim3(kTopkThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace kvsp
