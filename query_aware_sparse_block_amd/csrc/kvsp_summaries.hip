// Step 1: per-block mean-key summaries (SparPR news page, "Three decisions
// rather than one compression ratio", paragraph "Query-Aware key-block
// selection": each older block carries a small summary made ahead of time,
// its mean key, kept in GPU memory).
//
// One wavefront per (sequence, logical block, KV head) tile: workgroup
// (x, b) takes tiles 4x .. 4x+3 of sequence b in (block, KV head) order, so
// every wave has a tile whatever the number of KV heads, and the tiles of one
// workgroup are neighbours in the pool. A tile is P rows of D elements,
// contiguous in the pool; a wave streams it with 16-byte loads: LPR lanes
// cover one row and the wave covers 64 / LPR rows per load. Each lane
// accumulates its slice of the row in double, the row groups are folded with
// lane shuffles, and the mean is rounded once to float32. HBM-bound: P*D*E
// bytes read and D*4 bytes written per (block, KV head). A lane adds its rows
// in a fixed order (the append kernel repeats it, so both give the same bits).

#include "kvsp_device.h"
#include "kvsp_internal.h"

namespace kvsp {

// Row loads a lane keeps in flight.
#ifndef KVSP_SUMMARY_ROW_BATCH
#define KVSP_SUMMARY_ROW_BATCH 16
#endif
constexpr int kRowBatch = KVSP_SUMMARY_ROW_BATCH;

template <typename T, int D>
__global__ __launch_bounds__(256) void build_summaries_kernel(SummaryArgs a) {
  constexpr int E = T::kBytes;
  constexpr int EPV = T::kPerVec;
  constexpr int LPR = D * E / 16;  // lanes per row
  constexpr int RPL = kWave / LPR; // rows per wave-load
  const int b = blockIdx.y;
  const int tile_id = blockIdx.x * 4 + threadIdx.x / kWave;  // wave-uniform
  const int j = tile_id / a.Hkv;
  const int g = tile_id - j * a.Hkv;
  if (j >= a.max_blocks || j >= a.context_lens[b] / a.P) return;  // only full blocks have a summary
  const int64_t phys = a.block_table[static_cast<int64_t>(b) * a.max_blocks + j];
  const int lane = threadIdx.x % kWave;
  const int col = (lane % LPR) * EPV;
  const int row0 = lane / LPR;
  const char* tile = static_cast<const char*>(a.k_pool) +
                     ((phys * a.Hkv + g) * a.P) * static_cast<int64_t>(D) * E;
  double acc[EPV];
#pragma unroll
  for (int e = 0; e < EPV; ++e) acc[e] = 0.0;
  // Rows t = row0, row0 + RPL, ... in that order; kRowBatch rows' loads are
  // requested before any of them is added, so they are in flight together.
  for (int t0 = row0; t0 < a.P; t0 += kRowBatch * RPL) {
    uint4 raw[kRowBatch];
#pragma unroll
    for (int u = 0; u < kRowBatch; ++u) {
      const int t = t0 + u * RPL;
      raw[u] = t < a.P ? load16_stream(tile + (static_cast<int64_t>(t) * D + col) * E) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kRowBatch; ++u) {
      if (t0 + u * RPL < a.P) {
        float v[EPV];
        T::widen(raw[u], v);
#pragma unroll
        for (int e = 0; e < EPV; ++e) acc[e] += static_cast<double>(v[e]);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < EPV; ++e) acc[e] = fold_sum<LPR>(acc[e]);
  if (lane < LPR) {
    float* dst = a.summaries + (phys * a.Hkv + g) * D + col;
    const double inv_p = 1.0 / static_cast<double>(a.P);  // P is a power of two: exact
#pragma unroll
    for (int e = 0; e < EPV; ++e) dst[e] = static_cast<float>(acc[e] * inv_p);
  }
}

template <typename T, int D>
static hipError_t launch_summaries_t(const SummaryArgs& a, hipStream_t stream) {
  dim3 grid((a.max_blocks * a.Hkv + 3) / 4, a.B);
  hipLaunchKernelGGL((build_summaries_kernel<T, D>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_build_summaries(const SummaryArgs& a, int dtype, int D, hipStream_t stream) {
  if (dtype == KVSP_F32) return D == 64 ? launch_summaries_t<F32, 64>(a, stream) : launch_summaries_t<F32, 128>(a, stream);
  if (dtype == KVSP_F16) return D == 64 ? launch_summaries_t<F16, 64>(a, stream) : launch_summaries_t<F16, 128>(a, stream);
  return D == 64 ? launch_summaries_t<BF16, 64>(a, stream) : launch_summaries_t<BF16, 128>(a, stream);
}

}  // namespace kvsp
