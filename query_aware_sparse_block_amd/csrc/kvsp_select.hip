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

#include <algorithm>

#include "kvsp_device.h"
#include "kvsp_internal.h"

namespace kvsp {

// ---- scores ---------------------------------------------------------------------

// A group of LG lanes scores one block: the block's summary row (Hkv * D
// floats = LG * VPL 16-byte vectors) is split across the group, so a wave
// scores 64 / LG blocks per pass, and one DPP butterfly over LG lanes reduces
// all of them at once. The prologue issues its independent loads together
// (context length, the workgroup's block-table entries, the queries); the
// passes are double-buffered (up to 16 vectors per lane) so one pass's loads
// fly while the previous one is reduced. This scores the workgroup's block range of sequence b and
// returns C (the sequence's candidate count). COHERENT stores make the scores
// visible to other workgroups of the same launch.

// The group-summed queries in LDS. A lane of a group takes summary vectors
// gl, gl + LG, ... and multiplies each vector's 4 components by the matching
// query sums. Stored row-major (element x at qbar[x]), those reads have a
// 32-byte stride across the lanes and pile several lanes onto each bank
// (measured: a quarter of the serving call's time stalled on LDS bank
// conflicts). So when the group's LG * VPL vectors are at most 1024 (32 KiB
// of doubles), they are stored component-major with stride QS = LG * VPL:
// component c of vector i at qbar[c * QS + i], zero for i past the row's
// end, and a lane's reads are consecutive doubles across the group, at
// offsets known when compiling. Longer rows keep the row-major layout
// (QS = 0), which uses less LDS.
template <int LG, int VPL>
__host__ __device__ constexpr int qbar_stride() { return VPL <= 16 ? LG * VPL : 0; }
template <int LG, int VPL>
__host__ __device__ constexpr int qbar_doubles(int row) {
  return qbar_stride<LG, VPL>() ? 4 * qbar_stride<LG, VPL>() : row;
}

// STREAM (a.stream_rows as a template parameter) reads the summary rows with
// non-temporal loads and runs the passes as a branch-free pipeline.
template <typename T, int LG, int VPL, bool COHERENT, bool STREAM>
__device__ __forceinline__ int score_blocks(const ScoreArgs& a, double* qbar, int b) {
  constexpr int QS = qbar_stride<LG, VPL>();
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int per_wg = 4 * a.blocks_per_wave;
  const int first = blockIdx.x * per_wg;
  const int row = a.Hkv * a.D;
  const int nvec = row / 4;
  int32_t* phys_lds = reinterpret_cast<int32_t*>(qbar + qbar_doubles<LG, VPL>(row));
  const int64_t trow = static_cast<int64_t>(b) * a.max_blocks;
  // Block-table entries of this workgroup's range (in bounds of the row
  // whatever the context length; entries past C are never used).
  for (int i = threadIdx.x; i < per_wg; i += blockDim.x)
    phys_lds[i] = first + i < a.max_blocks ? a.block_table[trow + first + i] : 0;

  // qbar[g][d] = sum over the group's query heads, ascending, in double
  // (exact for 16-bit inputs). One 16-byte vector of q per head and thread;
  // the heads are loaded 16 at a time so a group costs one round trip.
  const int G = a.Hq / a.Hkv;
  constexpr int EPV = T::kPerVec;
  constexpr int QB = 16;
  const char* qb = static_cast<const char*>(a.q) + static_cast<int64_t>(b) * a.Hq * a.D * T::kBytes;
  for (int v = threadIdx.x; v < row / EPV; v += blockDim.x) {
    const int g = (v * EPV) / a.D;
    const int d0 = (v * EPV) % a.D;
    double s[EPV];
#pragma unroll
    for (int e = 0; e < EPV; ++e) s[e] = 0.0;
    for (int h0 = 0; h0 < G; h0 += QB) {
      uint4 qv[QB];
#pragma unroll
      for (int u = 0; u < QB; ++u)
        qv[u] = h0 + u < G ? load16(qb + (static_cast<int64_t>(g * G + h0 + u) * a.D + d0) * T::kBytes)
                           : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int u = 0; u < QB; ++u) {
        if (h0 + u < G) {
          float f[EPV];
          T::widen(qv[u], f);
#pragma unroll
          for (int e = 0; e < EPV; ++e) s[e] += static_cast<double>(f[e]);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      const int x = v * EPV + e;
      if constexpr (QS != 0) {
        qbar[(x % 4) * QS + x / 4] = s[e];
      } else {
        qbar[x] = s[e];
      }
    }
  }
  if constexpr (QS != 0) {
    for (int i = nvec + threadIdx.x; i < QS; i += blockDim.x)
#pragma unroll
      for (int c = 0; c < 4; ++c) qbar[c * QS + i] = 0.0;
  }
  const SelectArgs sel{a.top_k, a.keep_num, a.keep_den, a.keep_floor, a.recent_window,
                       a.gamma_num, a.gamma_den};
  const int C = plan_sequence(a.context_lens[b], a.P, sel).C;

  constexpr int BPP = kWave / LG;  // blocks per wave pass
  const int gl = lane % LG;
  const int slot = lane / LG;
  const int w0 = wave * a.blocks_per_wave;  // offset of this wave's blocks in the range
  const int j1 = min(C, first + w0 + a.blocks_per_wave);

  // The row's nvec vectors are spread as gl + LG * v; the group covers
  // LG * VPL >= nvec of them and the lanes past the row's end contribute 0.
  // The first pass reads its block-table entries itself (`direct`), so its
  // summary loads leave before the workgroup barrier that publishes qbar.
  // Large summary sets are read once per call with non-temporal loads
  // (a.stream_rows, uniform); small ones may stay cached between calls.
  auto issue = [&](int jb, float4 (&sv)[VPL], bool direct, bool repeat = false) {
    const int j = jb + slot;
    if (STREAM && !direct) {
      // Later streamed passes: no load behind a per-lane branch (such a load
      // is waited for alone, and the next pass's loads could not stay in
      // flight). A row past j1 reads the last live row of the range and a
      // vector past the row's end the row's last vector; consume masks both.
      // A repeat (the pipeline's pass past the end, whose data is never
      // used) keeps the instruction count, which the waits depend on, but
      // points every lane at the row's first vector: one line per load
      // instead of re-reading the rows.
      const int64_t phys = phys_lds[min(j, j1 - 1) - first];
      const float4* srow = reinterpret_cast<const float4*>(a.summaries + phys * row);
#pragma unroll
      for (int v = 0; v < VPL; ++v)
        sv[v] = __builtin_bit_cast(float4, load16_stream(srow + (repeat ? 0 : min(gl + LG * v, nvec - 1))));
      return;
    }
    int64_t phys = 0;
    if (j < j1) phys = direct ? a.block_table[trow + j] : phys_lds[j - first];
    const float4* srow = reinterpret_cast<const float4*>(a.summaries + phys * row);
    if constexpr (STREAM) {
#pragma unroll
      for (int v = 0; v < VPL; ++v)
        sv[v] = (j < j1 && gl + LG * v < nvec) ? __builtin_bit_cast(float4, load16_stream(srow + gl + LG * v))
                                              : make_float4(0.f, 0.f, 0.f, 0.f);
    } else {
#pragma unroll
      for (int v = 0; v < VPL; ++v)
        sv[v] = (j < j1 && gl + LG * v < nvec) ? srow[gl + LG * v] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto consume = [&](int jb, const float4 (&sv)[VPL]) {
    double acc = 0.0;
    if constexpr (STREAM) {
      // Straight-line: a per-lane conditional here becomes a branch around
      // the LDS reads, and every such branch waits for all loads in flight.
      // A vector past the row's end is weighted by 0.0 and adds a zero (the
      // sum starts at +0.0, so its bits are those of the sum over the row).
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        if constexpr (QS != 0) {
          // past the row's end the query sums are 0.0
          const double* qv = qbar + gl + LG * v;
          acc += qv[0] * static_cast<double>(sv[v].x);
          acc += qv[QS] * static_cast<double>(sv[v].y);
          acc += qv[2 * QS] * static_cast<double>(sv[v].z);
          acc += qv[3 * QS] * static_cast<double>(sv[v].w);
        } else {
          const double in = gl + LG * v < nvec ? 1.0 : 0.0;
          const double* qv = qbar + 4 * min(gl + LG * v, nvec - 1);
          acc += (qv[0] * in) * static_cast<double>(sv[v].x);
          acc += (qv[1] * in) * static_cast<double>(sv[v].y);
          acc += (qv[2] * in) * static_cast<double>(sv[v].z);
          acc += (qv[3] * in) * static_cast<double>(sv[v].w);
        }
      }
    } else {
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        if (gl + LG * v < nvec) {
          constexpr int CS = QS != 0 ? QS : 1;  // stride between a vector's components
          const double* qv = QS != 0 ? qbar + gl + LG * v : qbar + 4 * (gl + LG * v);
          acc += qv[0] * static_cast<double>(sv[v].x);
          acc += qv[CS] * static_cast<double>(sv[v].y);
          acc += qv[2 * CS] * static_cast<double>(sv[v].z);
          acc += qv[3 * CS] * static_cast<double>(sv[v].w);
        }
      }
    }
    acc = group_sum<LG>(acc);
    const int j = jb + slot;
    if (gl == 0 && j < j1) {
      if constexpr (COHERENT) {
        store_coherent(a.scores + trow + j, static_cast<float>(acc));
      } else {
        a.scores[trow + j] = static_cast<float>(acc);
      }
    }
  };

  int jb = first + w0;
  if constexpr (VPL <= 16) {
    float4 buf0[VPL], buf1[VPL];
    if (jb < j1) issue(jb, buf0, true);
    __syncthreads();  // qbar and the staged table entries
    if (first >= C) return C;  // uniform over the workgroup
    if constexpr (STREAM) {
      // Every pass issues one, so that a pass's use waits for that pass alone
      // (past the end the current pass is requested again; its data is not
      // used). The scheduling barriers keep the next pass's loads ahead of
      // this pass's arithmetic, which would otherwise be hoisted above them.
      while (jb < j1) {
        const int jn = jb + BPP;
        issue(jn < j1 ? jn : jb, buf1, false, jn >= j1);
        __builtin_amdgcn_sched_barrier(0);
        consume(jb, buf0);
        if (jn >= j1) break;
        const int jn2 = jn + BPP;
        issue(jn2 < j1 ? jn2 : jn, buf0, false, jn2 >= j1);
        __builtin_amdgcn_sched_barrier(0);
        consume(jn, buf1);
        jb = jn2;
      }
    } else {
      while (jb < j1) {
        const int jn = jb + BPP;
        if (jn < j1) issue(jn, buf1, false);
        consume(jb, buf0);
        if (jn >= j1) break;
        const int jn2 = jn + BPP;
        if (jn2 < j1) issue(jn2, buf0, false);
        consume(jn, buf1);
        jb = jn2;
      }
    }
  } else {
    // The longest rows: one buffer already holds 32 vectors per lane.
    float4 buf[VPL];
    if (jb < j1) issue(jb, buf, true);
    __syncthreads();
    if (first >= C) return C;
    for (; jb < j1; jb += BPP) {
      if (jb != first + w0) issue(jb, buf, false);
      consume(jb, buf);
    }
  }
  return C;
}

template <typename T, int LG, int VPL, bool STREAM>
__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a) {
  extern __shared__ double qbar[];  // group-summed queries (qbar_doubles), then [4 * bpw] ints
  score_blocks<T, LG, VPL, false, STREAM>(a, qbar, blockIdx.y);
}

template <typename T, int LG, int VPL>
static hipError_t launch_score_v(const ScoreArgs& a, hipStream_t stream) {
  const int per_wg = 4 * a.blocks_per_wave;
  dim3 grid((a.max_blocks + per_wg - 1) / per_wg, a.B);
  const size_t lds = static_cast<size_t>(qbar_doubles<LG, VPL>(a.Hkv * a.D)) * sizeof(double) +
                     per_wg * sizeof(int32_t);
  if (a.stream_rows)
    hipLaunchKernelGGL((score_kernel<T, LG, VPL, true>), grid, dim3(256), lds, stream, a);
  else
    hipLaunchKernelGGL((score_kernel<T, LG, VPL, false>), grid, dim3(256), lds, stream, a);
  return hipGetLastError();
}

// Group shape from the summary row length nvec = Hkv * D / 4 vectors (at
// least 16): LG, the largest power of two <= 64 with 8 * LG <= nvec lanes
// per block, and VPL, the fewest of 8, 16 or 32 vectors per lane that cover
// the row (16 at most below 64 lanes).
#ifndef KVSP_SCORE_MIN_VPL
#define KVSP_SCORE_MIN_VPL 8
#endif
ScoreShape score_shape(int Hkv, int D) {
  const int nvec = Hkv * D / 4;
  ScoreShape sh{2, KVSP_SCORE_MIN_VPL};
  while (sh.lg < kWave && 2 * sh.lg * KVSP_SCORE_MIN_VPL <= nvec) sh.lg *= 2;
  while (sh.lg * sh.vpl < nvec) sh.vpl *= 2;
  return sh;
}

// Calls F::template run<LG, VPL>() for the shape of (Hkv, D).
template <typename F>
static hipError_t with_score_shape(int Hkv, int D, F&& f) {
  const ScoreShape sh = score_shape(Hkv, D);
  const bool wide = sh.vpl >= 16;
  switch (sh.lg) {
    case 2: return wide ? f.template run<2, 16>() : f.template run<2, 8>();
    case 4: return wide ? f.template run<4, 16>() : f.template run<4, 8>();
    case 8: return wide ? f.template run<8, 16>() : f.template run<8, 8>();
    case 16: return wide ? f.template run<16, 16>() : f.template run<16, 8>();
    case 32: return wide ? f.template run<32, 16>() : f.template run<32, 8>();
    default:
      if (sh.vpl == 32) return f.template run<64, 32>();
      return wide ? f.template run<64, 16>() : f.template run<64, 8>();
  }
}

template <typename T>
struct ScoreLauncher {
  const ScoreArgs& a;
  hipStream_t stream;
  template <int LG, int VPL>
  hipError_t run() const { return launch_score_v<T, LG, VPL>(a, stream); }
};

template <typename T>
static hipError_t launch_score_t(const ScoreArgs& a, hipStream_t stream) {
  return with_score_shape(a.Hkv, a.D, ScoreLauncher<T>{a, stream});
}

hipError_t launch_score(const ScoreArgs& a, int dtype, hipStream_t stream) {
  if (dtype == KVSP_F32) return launch_score_t<F32>(a, stream);
  if (dtype == KVSP_F16) return launch_score_t<F16>(a, stream);
  return launch_score_t<BF16>(a, stream);
}

// ---- Top-k, spans, dense flag -------------------------------------------------------

constexpr int kTopkMaxPerThread = 16;  // candidates per thread: C <= 16 * threads

// Larger float <=> larger key; -0.0 and +0.0 map to the same key.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum of v over the workgroup in thread order; `total` gets
// the sum over all threads. Every thread must call it. tmp holds
// 2 * (WAVES + 1) words: wave totals, then their exclusive scan.
template <int WAVES>
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t* tmp, uint32_t& total) {
  const int lane = threadIdx.x % kWave;
  const uint32_t incl = wave_incl_scan(v);
  if constexpr (WAVES == 1) {
    total = __builtin_amdgcn_readlane(incl, kWave - 1);
    return incl - v;
  } else {
    const int wave = threadIdx.x / kWave;
    if (lane == kWave - 1) tmp[wave] = incl;
    __syncthreads();
    uint32_t* offs = tmp + WAVES + 1;
    if (wave == 0) {
      const uint32_t w = lane < WAVES ? tmp[lane] : 0u;
      const uint32_t wi = wave_incl_scan(w);
      if (lane < WAVES) offs[lane] = wi - w;
      if (lane == WAVES - 1) offs[WAVES] = wi;
    }
    __syncthreads();
    const uint32_t res = offs[wave] + incl - v;
    total = offs[WAVES];
    __syncthreads();
    return res;
  }
}

struct TopkShared {
  uint32_t hist[4][256];  // one histogram per radix pass, cleared together
  uint32_t scan_tmp[2 * (16 + 1)];
};

// Top-k, spans and the dense flag of sequence b, by a workgroup of WAVES
// wavefronts (every thread calls it). COHERENT reads scores written by other
// workgroups of the same launch.
//
// Thread t owns the R consecutive candidates t*R .. t*R+R-1 and also reads
// the scores of the candidate just before and just after them, so it can
// decide on its own whether its first and last candidates open or close a
// run. Each radix pass costs one barrier: the four histograms are cleared
// up front and every wavefront finds the pass's digit by itself. When every
// key equal to the threshold is kept (no tie is cut), one block-wide scan of
// (kept, run starts) places the selected ids and the spans; a cut tie adds
// one scan that ranks the equal keys by index.
template <int WAVES, bool COHERENT, int RMAX>
__device__ __forceinline__ void select_sequence_r(const TopkArgs& a, int b, TopkShared& sh) {
  constexpr int kTopkThreads = WAVES * kWave;
  const int t = threadIdx.x;
  const int lane = t % kWave;
  const SelectArgs sel{a.top_k, a.keep_num, a.keep_den, a.keep_floor, a.recent_window,
                       a.gamma_num, a.gamma_den};
  // Candidates are assigned from the row capacity, so the score loads do not
  // wait for the context length.
  const int R = (a.max_blocks + kTopkThreads - 1) / kTopkThreads;
  const int jbase = t * R;
  const int64_t row = static_cast<int64_t>(b) * a.max_blocks;
  auto score_at = [&](int j) -> float {
    if constexpr (COHERENT) {
      return load_coherent(a.scores + row + j);
    } else {
      return a.scores[row + j];
    }
  };
  float raw[RMAX];
  if constexpr (COHERENT && RMAX >= 4) {
    // RMAX consecutive scores as 16-byte loads (a range-checked buffer: past
    // the row's end they read 0; slots r >= R are never used).
    const __amdgpu_buffer_rsrc_t rs =
        coherent_rsrc(a.scores + row, static_cast<uint32_t>(a.max_blocks) * sizeof(float));
#pragma unroll
    for (int q = 0; q < RMAX / 4; ++q) {
      const float4 v = load_coherent4(rs, static_cast<uint32_t>(jbase + 4 * q) * sizeof(float));
      raw[4 * q + 0] = v.x;
      raw[4 * q + 1] = v.y;
      raw[4 * q + 2] = v.z;
      raw[4 * q + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
      const int j = jbase + r;
      raw[r] = (r < R && j < a.max_blocks) ? score_at(j) : 0.f;
    }
  }
  const float raw_prev = (jbase >= 1 && jbase - 1 < a.max_blocks) ? score_at(jbase - 1) : 0.f;
  const float raw_next = jbase + R < a.max_blocks ? score_at(jbase + R) : 0.f;
  const SeqPlan p = plan_sequence(a.context_lens[b], a.P, sel);
  const int C = p.C;
  const int k = p.k;

  uint32_t key[RMAX];
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    const int j = jbase + r;
    key[r] = (r < R && j < C) ? order_key(raw[r]) : 0u;
  }
  const bool has_prev = jbase >= 1 && jbase - 1 < C;
  const bool has_next = jbase + R < C;
  const uint32_t key_prev = has_prev ? order_key(raw_prev) : 0u;
  const uint32_t key_next = has_next ? order_key(raw_next) : 0u;

  // Radix select of the k-th largest key T (only when 0 < k < C), 8 bits a
  // pass from the top: after the last pass, `take_equal` of the `eq_total`
  // keys equal to T are kept.
  uint32_t thresh = 0;
  int take_equal = 0, eq_total = 0;
  const bool partial = k > 0 && k < C;
  if (partial) {
    for (int i = t; i < 4 * 256; i += kTopkThreads) (&sh.hist[0][0])[i] = 0;
    __syncthreads();
    uint32_t prefix = 0, mask = 0;
    int krem = k;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      uint32_t* hist = sh.hist[pass];
#pragma unroll
      for (int r = 0; r < RMAX; ++r) {
        const int j = jbase + r;
        if (r < R && j < C && (key[r] & mask) == prefix) atomicAdd(&hist[(key[r] >> shift) & 255u], 1u);
      }
      __syncthreads();
      // Every wavefront: lane owns digits 4*lane .. 4*lane+3; the digit is
      // the one where the count of keys in higher digits first reaches krem.
      uint32_t h[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] = hist[4 * lane + i];
      const uint32_t incl = wave_incl_scan(h[0] + h[1] + h[2] + h[3]);
      uint32_t above = __builtin_amdgcn_readlane(incl, kWave - 1) - incl;
      bool found = false;
      uint32_t d_sel = 0, k_sel = 0, n_sel = 0;
#pragma unroll
      for (int i = 3; i >= 0; --i) {
        if (above < static_cast<uint32_t>(krem) && static_cast<uint32_t>(krem) <= above + h[i]) {
          found = true;
          d_sel = 4u * lane + i;
          k_sel = static_cast<uint32_t>(krem) - above;
          n_sel = h[i];
        }
        above += h[i];
      }
      // exactly one lane holds the digit (krem lies in (0, keys with this prefix])
      const int src = __builtin_ctzll(__ballot(found) | (1ull << 63));
      const uint32_t digit = __builtin_amdgcn_readlane(d_sel, src);
      krem = static_cast<int>(__builtin_amdgcn_readlane(k_sel, src));
      eq_total = static_cast<int>(__builtin_amdgcn_readlane(n_sel, src));
      prefix |= digit << shift;
      mask |= 0xFFu << shift;
      // The digit's keys are all needed: the k best are exactly the keys
      // whose prefix is at least this one, so the threshold is the prefix
      // with zero low bits and no tie is cut (uniform: every wave reads the
      // same histogram).
      if (krem == eq_total) {
        krem = 0;
        eq_total = 0;
        break;
      }
    }
    thresh = prefix;
    take_equal = krem;
  }

  // Equal keys are kept in index order: rank them when a tie is cut.
  const bool cut_tie = partial && take_equal < eq_total;  // uniform
  uint32_t n_eq = 0;
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    const int j = jbase + r;
    if (r < R && j < C && key[r] == thresh) ++n_eq;
  }
  uint32_t eq_before = 0;
  if (cut_tie) {
    uint32_t eq_all;
    eq_before = block_excl_scan<WAVES>(n_eq, sh.scan_tmp, eq_all);
  }
  // Kept? for a candidate with key `kk` whose rank among the equal keys is eq_rank.
  auto kept = [&](uint32_t kk, uint32_t eq_rank) -> bool {
    if (!partial) return k >= C;
    if (kk != thresh) return kk > thresh;
    return !cut_tie || eq_rank < static_cast<uint32_t>(take_equal);
  };
  const bool keep_prev = has_prev && kept(key_prev, eq_before - 1u);
  const bool keep_next = has_next && kept(key_next, eq_before + n_eq);

  uint32_t keep_bits = 0, n_keep = 0, n_start = 0;
  {
    uint32_t eq_rank = eq_before;
    bool left = keep_prev;  // kept(j - 1)
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
      const int j = jbase + r;
      if (!(r < R && j < C)) continue;
      const bool kp = kept(key[r], eq_rank);
      if (key[r] == thresh) ++eq_rank;
      if (kp) {
        keep_bits |= 1u << r;
        ++n_keep;
        if (!left) ++n_start;
      }
      left = kp;
    }
  }
  // One scan places both: kept ids before this thread (high half) and runs
  // started before it (low half); C <= 16 * threads keeps each below 2^16.
  uint32_t totals;
  const uint32_t before = block_excl_scan<WAVES>((n_keep << 16) | n_start, sh.scan_tmp, totals);
  uint32_t pos = before >> 16;
  uint32_t s_idx = before & 0xFFFFu;
  // A run still open at this thread's first candidate has its end counted here.
  const bool first_kept = (keep_bits & 1u) != 0;
  uint32_t e_idx = s_idx - ((keep_prev && first_kept) ? 1u : 0u);
  const bool window = p.n > C;
  int32_t* sp = a.spans + row * 2 + static_cast<int64_t>(b) * 2;  // [B][max_blocks+1][2]
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    const int j = jbase + r;
    if (!(r < R && j < C) || !((keep_bits >> r) & 1u)) continue;
    const bool left = r == 0 ? keep_prev : ((keep_bits >> (r - 1)) & 1u) != 0;
    const bool right = r == R - 1 ? keep_next : ((keep_bits >> (r + 1)) & 1u) != 0;
    a.selected[row + pos++] = j;
    if (!left) sp[2 * s_idx++] = j;
    if (!right) sp[2 * e_idx++ + 1] = (j == C - 1 && window) ? p.n : j + 1;
  }
  // The thread holding candidate C - 1 knows whether the window joins the
  // last selected span; it writes the counts.
  const int writer = C > 0 ? (C - 1) / R : 0;
  if (t == writer) {
    const int sel_spans = static_cast<int>(totals & 0xFFFFu);
    const bool joined = C > 0 && ((keep_bits >> (C - 1 - jbase)) & 1u) != 0;
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

// Candidates per thread are bounded by RMAX at compile time, so the loops over
// a thread's candidates unroll to the bound the table actually needs.
template <int WAVES, bool COHERENT>
__device__ __forceinline__ void select_sequence(const TopkArgs& a, int b, TopkShared& sh) {
  const int R = (a.max_blocks + WAVES * kWave - 1) / (WAVES * kWave);
  if (R <= 1) {
    select_sequence_r<WAVES, COHERENT, 1>(a, b, sh);
  } else if (R <= 2) {
    select_sequence_r<WAVES, COHERENT, 2>(a, b, sh);
  } else if (R <= 4) {
    select_sequence_r<WAVES, COHERENT, 4>(a, b, sh);
  } else if (R <= 8) {
    select_sequence_r<WAVES, COHERENT, 8>(a, b, sh);
  } else {
    select_sequence_r<WAVES, COHERENT, kTopkMaxPerThread>(a, b, sh);
  }
}

template <int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void topk_kernel(TopkArgs a) {
  __shared__ TopkShared sh;
  select_sequence<WAVES, false>(a, blockIdx.x, sh);
}

template <int WAVES>
static hipError_t launch_topk_w(const TopkArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((topk_kernel<WAVES>), dim3(a.B), dim3(WAVES * kWave), 0, stream, a);
  return hipGetLastError();
}

// Scores and selection in one launch: each workgroup scores its block range;
// the last workgroup of a sequence to finish (counted with a self-resetting
// device-scope atomic) runs that sequence's Top-k on the scores the others
// published. Workgroup 0 of every sequence takes part even with no
// candidates, so every sequence gets its counts and spans.
template <typename T, int LG, int VPL, bool STREAM>
__global__ __launch_bounds__(256) void score_select_kernel(ScoreArgs sa, TopkArgs ta,
                                                           int32_t* counters) {
  extern __shared__ double lds[];
  const int b = blockIdx.y;
  const int C = score_blocks<T, LG, VPL, true, STREAM>(sa, lds, b);
  const int per_wg = 4 * sa.blocks_per_wave;
  const int first = blockIdx.x * per_wg;
  if (first >= C && blockIdx.x != 0) return;  // uniform: no blocks, not the anchor
  const int expected = C > 0 ? (C + per_wg - 1) / per_wg : 1;
  __shared__ int is_last;
  wait_stores_done();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int old = __hip_atomic_fetch_add(counters + b, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    is_last = old == expected - 1;
  }
  __syncthreads();
  if (!is_last) return;
  TopkShared& sh = *reinterpret_cast<TopkShared*>(lds);
  select_sequence<4, true>(ta, b, sh);
  if (threadIdx.x == 0) store_coherent_i(counters + b, 0);
}

// The Top-k runs in the scoring launch (by the last scoring workgroup of a
// sequence, four waves) only for tables of at most KVSP_FUSED_SELECT_MAX_BLOCKS
// blocks scored by at most KVSP_FUSED_SELECT_MAX_WORKGROUPS workgroups in all;
// otherwise the scores are written and a Top-k launch of its own follows,
// with KVSP_TOPK_PER_THREAD candidates a thread (up to sixteen waves). Measured:
// with many scoring workgroups per sequence their completion atomics and the
// four-wave Top-k of a long table cost more than a second launch.
#ifndef KVSP_FUSED_SELECT_MAX_BLOCKS
#define KVSP_FUSED_SELECT_MAX_BLOCKS 512
#endif
#ifndef KVSP_FUSED_SELECT_MAX_WORKGROUPS
#define KVSP_FUSED_SELECT_MAX_WORKGROUPS 64
#endif
#ifndef KVSP_TOPK_PER_THREAD
#define KVSP_TOPK_PER_THREAD 2
#endif
constexpr int kFusedSelectMaxBlocks = KVSP_FUSED_SELECT_MAX_BLOCKS;
static_assert(kFusedSelectMaxBlocks <= 4 * kWave * kTopkMaxPerThread,
              "the fused Top-k holds at most 16 candidates a thread");

template <typename T, int LG, int VPL>
static hipError_t launch_fused_v(const ScoreArgs& sa, const TopkArgs& ta, int32_t* counters,
                                 hipStream_t stream) {
  const int per_wg = 4 * sa.blocks_per_wave;
  dim3 grid((sa.max_blocks + per_wg - 1) / per_wg, sa.B);
  const size_t score_lds = static_cast<size_t>(qbar_doubles<LG, VPL>(sa.Hkv * sa.D)) * sizeof(double) +
                           per_wg * sizeof(int32_t);
  const size_t topk_lds = sizeof(TopkShared);
  const size_t lds = (std::max(score_lds, topk_lds) + 7) / 8 * 8;
  if (sa.stream_rows)
    hipLaunchKernelGGL((score_select_kernel<T, LG, VPL, true>), grid, dim3(256), lds, stream, sa, ta,
                       counters);
  else
    hipLaunchKernelGGL((score_select_kernel<T, LG, VPL, false>), grid, dim3(256), lds, stream, sa,
                       ta, counters);
  return hipGetLastError();
}

template <typename T>
struct FusedLauncher {
  const ScoreArgs& sa;
  const TopkArgs& ta;
  int32_t* counters;
  hipStream_t stream;
  template <int LG, int VPL>
  hipError_t run() const { return launch_fused_v<T, LG, VPL>(sa, ta, counters, stream); }
};

template <typename T>
static hipError_t launch_fused_t(const ScoreArgs& sa, const TopkArgs& ta, int32_t* counters,
                                 hipStream_t stream) {
  return with_score_shape(sa.Hkv, sa.D, FusedLauncher<T>{sa, ta, counters, stream});
}

bool fused_select_supported(int max_blocks, int64_t workgroups) {
  return max_blocks <= kFusedSelectMaxBlocks && workgroups <= KVSP_FUSED_SELECT_MAX_WORKGROUPS;
}

int64_t score_workgroups(const ScoreArgs& sa) {
  const int per_wg = 4 * sa.blocks_per_wave;
  return static_cast<int64_t>((sa.max_blocks + per_wg - 1) / per_wg) * sa.B;
}

hipError_t launch_score_select(const ScoreArgs& sa, const TopkArgs& ta, int32_t* counters,
                               int dtype, hipStream_t stream) {
  if (dtype == KVSP_F32) return launch_fused_t<F32>(sa, ta, counters, stream);
  if (dtype == KVSP_F16) return launch_fused_t<F16>(sa, ta, counters, stream);
  return launch_fused_t<BF16>(sa, ta, counters, stream);
}

// The fewest wavefronts that hold every candidate at KVSP_TOPK_PER_THREAD a
// thread (at most sixteen waves, which then hold up to 16 a thread).
hipError_t launch_topk(const TopkArgs& a, hipStream_t stream) {
  const int per_wave = kWave * KVSP_TOPK_PER_THREAD;
  const int waves = (a.max_blocks + per_wave - 1) / per_wave;
  if (waves <= 1) return launch_topk_w<1>(a, stream);
  if (waves <= 2) return launch_topk_w<2>(a, stream);
  if (waves <= 4) return launch_topk_w<4>(a, stream);
  if (waves <= 8) return launch_topk_w<8>(a, stream);
  return launch_topk_w<16>(a, stream);
}

}  // namespace kvsp
