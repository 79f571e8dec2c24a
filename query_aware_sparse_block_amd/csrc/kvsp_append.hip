// Decode-time append: the cache gains one token per sequence and decode step
// (SparPR news page, opening paragraphs), and a block that the new token
// completes gets its mean-key summary right away (same page, "Three decisions
// rather than one compression ratio", paragraph "Query-Aware key-block
// selection"), so the next scoring call can rank it.
//
// One wave per (sequence, KV head): workgroup (x, b) takes heads 4x .. 4x+3
// of sequence b. The new K
// and V rows (D*E bytes each) are written by the first LPR lanes with one
// 16-byte store each. When the token is the block's last, the wave sums the
// block exactly as the summary builder does (the same lanes take the same
// rows in the same order, accumulating in double, then the same fold), except
// that the new row comes from the input rather than from the pool it was just
// written to; the mean therefore matches that builder bit for bit.
// Latency-bound: 2*D*E bytes written per (sequence, KV head), plus P*D*E read
// and D*4 written when a block completes.

#include "kvsp_device.h"
#include "kvsp_internal.h"

namespace kvsp {

template <typename T, int D>
__global__ __launch_bounds__(256) void append_kv_kernel(AppendArgs a) {
  constexpr int E = T::kBytes;
  constexpr int EPV = T::kPerVec;
  constexpr int LPR = D * E / 16;   // lanes per row
  constexpr int RPL = kWave / LPR;  // rows per wave-load
  const int b = blockIdx.y;
  const int lane = threadIdx.x % kWave;
  const int g = blockIdx.x * 4 + threadIdx.x / kWave;
  if (g >= a.Hkv) return;  // wave-uniform
  const int col = (lane % LPR) * EPV;
  const int row0 = lane / LPR;
  const char* kn = static_cast<const char*>(a.k_new);
  const char* vn = static_cast<const char*>(a.v_new);
  const int64_t src = (static_cast<int64_t>(b) * a.Hkv + g) * D * E;
  // The new rows do not depend on the position: request them first.
  uint4 k_row = make_uint4(0, 0, 0, 0), v_row = make_uint4(0, 0, 0, 0);
  if (lane < LPR) {
    k_row = load16(kn + src + col * E);
    v_row = load16(vn + src + col * E);
  }
  const int p = a.positions[b];
  if (p < 0 || p >= a.max_blocks * a.P) return;  // no token for this sequence this step
  const int j = p / a.P;
  const int t_in = p % a.P;
  const int64_t phys = a.block_table[static_cast<int64_t>(b) * a.max_blocks + j];
  if (phys < 0 || phys >= a.num_phys) return;  // unmapped block: nothing to write
  char* kp = static_cast<char*>(a.k_pool);
  char* vp = static_cast<char*>(a.v_pool);
  {
    const int64_t tile = ((phys * a.Hkv + g) * a.P) * static_cast<int64_t>(D) * E;
    if (lane < LPR) {
      const int64_t off = static_cast<int64_t>(t_in) * D * E + col * E;
      store16(kp + tile + off, k_row);
      store16(vp + tile + off, v_row);
    }
    if (t_in == a.P - 1) {
      double acc[EPV];
#pragma unroll
      for (int e = 0; e < EPV; ++e) acc[e] = 0.0;
#pragma unroll 8
      for (int t = row0; t < a.P; t += RPL) {
        const char* rowp = t == a.P - 1 ? kn + src : kp + tile + static_cast<int64_t>(t) * D * E;
        float v[EPV];
        T::widen(load16(rowp + col * E), v);
#pragma unroll
        for (int e = 0; e < EPV; ++e) acc[e] += static_cast<double>(v[e]);
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
  }
}

template <typename T, int D>
static hipError_t launch_append_t(const AppendArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((append_kv_kernel<T, D>), dim3((a.Hkv + 3) / 4, a.B), dim3(256), 0, stream,
                     a);
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, int dtype, int D, hipStream_t stream) {
  if (dtype == KVSP_F32) return D == 64 ? launch_append_t<F32, 64>(a, stream) : launch_append_t<F32, 128>(a, stream);
  if (dtype == KVSP_F16) return D == 64 ? launch_append_t<F16, 64>(a, stream) : launch_append_t<F16, 128>(a, stream);
  return D == 64 ? launch_append_t<BF16, 64>(a, stream) : launch_append_t<BF16, 128>(a, stream);
}

}  // namespace kvsp
