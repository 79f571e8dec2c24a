// Device-side building blocks shared by the kvsp HIP kernels (gfx950).
// Internal header: not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvsp.h"

namespace kvsp {

constexpr int kWave = 64;

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((__vector_size__(16)));
typedef _Float16 f16x8 __attribute__((__vector_size__(16)));

// ---- element types ------------------------------------------------------------
// A 16-byte global load is the unit of every K/V/q access: 8 halves or 4 floats.

struct F32 {
  static constexpr int kBytes = 4;
  static constexpr int kPerVec = 4;
  __device__ static inline float load1(const void* base, int64_t i) {
    return static_cast<const float*>(base)[i];
  }
  __device__ static inline void widen(const uint4& v, float* o) {
    o[0] = __uint_as_float(v.x);
    o[1] = __uint_as_float(v.y);
    o[2] = __uint_as_float(v.z);
    o[3] = __uint_as_float(v.w);
  }
};

struct BF16 {
  static constexpr int kBytes = 2;
  static constexpr int kPerVec = 8;
  __device__ static inline float load1(const void* base, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(base)[i]) << 16);
  }
  // bfloat16 is the upper half of a binary32: widening is a shift / mask.
  __device__ static inline void widen(const uint4& v, float* o) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};

struct F16 {
  static constexpr int kBytes = 2;
  static constexpr int kPerVec = 8;
  __device__ static inline float load1(const void* base, int64_t i) {
    return static_cast<float>(static_cast<const _Float16*>(base)[i]);
  }
  __device__ static inline void widen(const uint4& v, float* o) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[i] & 0xFFFFu)));
      o[2 * i + 1] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[i] >> 16)));
    }
  }
};

__device__ __forceinline__ uint4 load16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// ---- cross-lane -----------------------------------------------------------------

__device__ __forceinline__ float lane_xor(float v, int mask) { return __shfl_xor(v, mask, kWave); }

__device__ __forceinline__ double lane_xor(double v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += lane_xor(v, m);
  return v;
}

// Orders LDS traffic between lanes of one wavefront (no workgroup barrier:
// the waves of a workgroup run independent work items).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// ---- device-coherent accesses ------------------------------------------------------
// Workgroups on different XCDs exchange split-KV partials through memory. The
// partials are stored and loaded with device-scope (sc1) accesses, which reach
// the device coherence point without write-back or invalidation of the whole
// L2; the completion counter is a device-scope atomic.

__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_coherent_i(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits until every memory access this wavefront issued has completed.
__device__ __forceinline__ void wait_stores_done() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---- per-sequence integer plan ----------------------------------------------------
// n blocks, C candidate blocks before the exact window [C*P, L), k kept blocks
// and the dense-fallback decision; see kvsp_select_params in kvsp.h.

struct SelectArgs {
  int32_t top_k, keep_num, keep_den, keep_floor, recent_window, gamma_num, gamma_den;
};

struct SeqPlan {
  int32_t n, C, k, dense;
};

__device__ __forceinline__ SeqPlan plan_sequence(int32_t L, int32_t P, const SelectArgs& s) {
  SeqPlan p;
  p.n = (L + P - 1) / P;
  const int32_t older = L > s.recent_window ? L - s.recent_window : 0;
  p.C = older / P;
  int64_t want;
  if (s.top_k > 0) {
    want = s.top_k;
  } else {
    const int64_t num = static_cast<int64_t>(p.C) * s.keep_num;
    want = (num + s.keep_den - 1) / s.keep_den;
  }
  if (want < s.keep_floor) want = s.keep_floor;
  if (want > p.C) want = p.C;
  p.k = static_cast<int32_t>(want);
  p.dense = (p.C > 0 && static_cast<int64_t>(p.k) * s.gamma_den >
                            static_cast<int64_t>(s.gamma_num) * p.C)
                ? 1
                : 0;
  return p;
}

// Window start block for the decode kernels (same definition as above).
__device__ __forceinline__ int32_t window_start_block(int32_t L, int32_t P, int32_t W) {
  return (L > W ? L - W : 0) / P;
}

}  // namespace kvsp
