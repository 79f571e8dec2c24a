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
typedef uint32_t u32x4 __attribute__((__vector_size__(16)));

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

__device__ __forceinline__ void store16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

// 16-byte non-temporal load, for data read once per call.
__device__ __forceinline__ uint4 load16_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// ---- cross-lane -----------------------------------------------------------------
// DPP row permutations and the gfx950 permlane16/32 swaps move data between
// lanes inside the VALU, without the LDS round trip of ds_bpermute.

template <int CTRL, int ROW_MASK = 0xf, int BANK_MASK = 0xf, bool BOUND_ZERO = true>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, ROW_MASK,
                                                           BANK_MASK, BOUND_ZERO));
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __uint_as_float(dpp_u32<CTRL, 0xf, 0xf, false>(__float_as_uint(x)));
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = dpp_u32<CTRL, 0xf, 0xf, false>(static_cast<uint32_t>(u));
  const uint32_t hi = dpp_u32<CTRL, 0xf, 0xf, false>(static_cast<uint32_t>(u >> 32));
  return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

template <int CTRL, typename F>
__device__ __forceinline__ F dpp_f(F x) {
  if constexpr (sizeof(F) == 8) {
    return dpp_f64<CTRL>(x);
  } else {
    return dpp_f32<CTRL>(x);
  }
}

// Partner values across 16-lane rows: lane l receives lane l ^ 16 (resp. l ^ 32).
__device__ __forceinline__ float xor16(float x) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  // s[0] = rows (0,0,2,2), s[1] = rows (1,1,3,3): the partner is whichever is not x.
  return __uint_as_float((threadIdx.x & 16) ? s[0] : s[1]);
}

__device__ __forceinline__ float xor32(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32) ? s[0] : s[1]);
}

__device__ __forceinline__ double xor16(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = static_cast<uint32_t>(u), hi = static_cast<uint32_t>(u >> 32);
  const auto sl = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  const auto sh = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  const bool up = threadIdx.x & 16;
  return __builtin_bit_cast(double, (static_cast<uint64_t>(up ? sh[0] : sh[1]) << 32) | (up ? sl[0] : sl[1]));
}

__device__ __forceinline__ double xor32(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = static_cast<uint32_t>(u), hi = static_cast<uint32_t>(u >> 32);
  const auto sl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  const auto sh = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  const bool up = threadIdx.x & 32;
  return __builtin_bit_cast(double, (static_cast<uint64_t>(up ? sh[0] : sh[1]) << 32) | (up ? sl[0] : sl[1]));
}

// Partner l ^ 8 (rotate each 16-lane row by 8).
template <typename F>
__device__ __forceinline__ F xor8(F x) { return dpp_f<0x128>(x); }

// Sum over the lanes that share lane % STRIDE (STRIDE = 8, 16 or 32): every
// lane receives the total of its residue class.
template <int STRIDE, typename F>
__device__ __forceinline__ F fold_sum(F v) {
  if constexpr (STRIDE <= 8) v += xor8(v);
  if constexpr (STRIDE <= 16) v += xor16(v);
  if constexpr (STRIDE <= 32) v += xor32(v);
  return v;
}

template <int STRIDE>
__device__ __forceinline__ float fold_max(float v) {
  if constexpr (STRIDE <= 8) v = fmaxf(v, xor8(v));
  if constexpr (STRIDE <= 16) v = fmaxf(v, xor16(v));
  if constexpr (STRIDE <= 32) v = fmaxf(v, xor32(v));
  return v;
}

// Sum over aligned groups of LANES consecutive lanes (1, 2, ..., 64); every
// lane of a group receives the group's total. Butterfly order: quad swaps,
// half-row mirror, row mirror, then the cross-row swaps.
template <int LANES, typename F>
__device__ __forceinline__ F group_sum(F v) {
  if constexpr (LANES >= 2) v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  if constexpr (LANES >= 4) v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  if constexpr (LANES >= 8) v += dpp_f<0x141>(v);  // row_half_mirror
  if constexpr (LANES >= 16) v += dpp_f<0x140>(v); // row_mirror
  if constexpr (LANES >= 32) v += xor16(v);
  if constexpr (LANES >= 64) v += xor32(v);
  return v;
}

// Maximum over aligned groups of LANES consecutive lanes (same butterfly).
template <int LANES>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (LANES >= 2) v = fmaxf(v, dpp_f<0xB1>(v));
  if constexpr (LANES >= 4) v = fmaxf(v, dpp_f<0x4E>(v));
  if constexpr (LANES >= 8) v = fmaxf(v, dpp_f<0x141>(v));
  if constexpr (LANES >= 16) v = fmaxf(v, dpp_f<0x140>(v));
  if constexpr (LANES >= 32) v = fmaxf(v, xor16(v));
  if constexpr (LANES >= 64) v = fmaxf(v, xor32(v));
  return v;
}


// Inclusive prefix sum over the wave (DPP row shifts and row broadcasts).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  const uint32_t t = x;
  x += dpp_u32<0x111>(t);             // row_shr:1
  x += dpp_u32<0x112>(t);             // row_shr:2
  x += dpp_u32<0x113>(t);             // row_shr:3
  x += dpp_u32<0x114, 0xf, 0xe>(x);   // row_shr:4, banks 1-3
  x += dpp_u32<0x118, 0xf, 0xc>(x);   // row_shr:8, banks 2-3
  x += dpp_u32<0x142, 0xa>(x);        // row_bcast:15 into rows 1 and 3
  x += dpp_u32<0x143, 0xc>(x);        // row_bcast:31 into rows 2 and 3
  return x;
}

// Orders LDS traffic between lanes of one wavefront (no workgroup barrier:
// the waves of a workgroup run independent work items). A wavefront's LDS
// operations execute in order, so wavefront-scope fences (which keep the
// compiler from moving memory operations across them and emit no wait) are
// enough. Workgroup scope would also wait for the wave's outstanding global
// loads, i.e. drain the next tile's prefetch at every call.
#ifndef KVSP_WAVE_SYNC_SCOPE
#define KVSP_WAVE_SYNC_SCOPE "wavefront"
#endif
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, KVSP_WAVE_SYNC_SCOPE);
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, KVSP_WAVE_SYNC_SCOPE);
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

// 16-byte device-coherent accesses through a buffer resource (range-checked:
// an offset past `bytes` reads zero and drops the write).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}

constexpr int kCachePolicySc1 = 16;  // device scope

__device__ __forceinline__ float4 load_coherent4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kCachePolicySc1));
}

__device__ __forceinline__ void store_coherent4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, float4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, byte_off, 0, kCachePolicySc1);
}

__device__ __forceinline__ void store_coherent1(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, byte_off, 0, kCachePolicySc1);
}

// A buffer offset past every range: a store there is dropped by the hardware.
constexpr uint32_t kDroppedOffset = 0xFFFFFFF0u;

// Waits until every memory access this wavefront issued has completed.
__device__ __forceinline__ void wait_stores_done() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---- QK^T on MFMA --------------------------------------------------------------
// One 16x16 tile of logits: rows are 16 key rows (A operand, one 16-byte vector
// per lane and contraction step), columns 16 query heads (B operand).

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
