// Device-side helpers shared by the gfx950 kernels of libpkv: 16-byte
// vector access, widening of stored values to fp32, rounding back, and
// reductions across the lanes of a wavefront (DPP within 16-lane rows).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

constexpr int kWave = 64;

template <int DT> struct Format;
template <> struct Format<PKV_F32>  { static constexpr int kBytes = 4; };
template <> struct Format<PKV_F16>  { static constexpr int kBytes = 2; };
template <> struct Format<PKV_BF16> { static constexpr int kBytes = 2; };
template <> struct Format<PKV_FP8_E4M3> { static constexpr int kBytes = 1; };

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Key and value loads.  NT: the nontemporal hint, for caches streamed once
// per step (measured on MI355X: ~11% more bandwidth on scattered 4 KiB
// tiles than plain loads).  Plain loads let blocks that several sequences
// of the batch share (a common prompt) be served again from L2 and the
// Infinity Cache: 1.4x faster on the shared-prefix sampling layer.
template <bool NT, typename T>
__device__ __forceinline__ T load_kv(const void* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
  return *reinterpret_cast<const T*>(p);
}

__device__ __forceinline__ void store16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// Widen one stored element held in the low (hi=false) or high half of a
// 32-bit word.  Exact for every format.
template <int DT>
__device__ __forceinline__ float widen_half(uint32_t w, bool hi);

template <>
__device__ __forceinline__ float widen_half<PKV_F16>(uint32_t w, bool hi) {
  uint16_t b = hi ? uint16_t(w >> 16) : uint16_t(w & 0xffffu);
  return float(__builtin_bit_cast(_Float16, b));
}

template <>
__device__ __forceinline__ float widen_half<PKV_BF16>(uint32_t w, bool hi) {
  return __builtin_bit_cast(float, hi ? (w & 0xffff0000u) : (w << 16));
}

// 16 stored bytes -> 16/kBytes floats.  E4M3 codes go through the
// hardware conversion (v_cvt_pk_f32_fp8 decodes OCP E4M3 on gfx950, NaN
// codes included; checked against the format definition on all 256 codes).
template <int DT>
__device__ __forceinline__ void widen16(const u32x4& raw, float* f) {
  if constexpr (DT == PKV_FP8_E4M3) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int w = (int)raw[i];
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
      f[4 * i] = lo[0];
      f[4 * i + 1] = lo[1];
      f[4 * i + 2] = hi[0];
      f[4 * i + 3] = hi[1];
    }
  } else if constexpr (DT == PKV_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // Copy the element out first: a bit_cast applied directly to an
      // ext_vector element reads element 0 with this compiler.
      const uint32_t w = raw[i];
      f[i] = __builtin_bit_cast(float, w);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = widen_half<DT>(raw[i], false);
      f[2 * i + 1] = widen_half<DT>(raw[i], true);
    }
  }
}

// fp32 -> stored format, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t narrow_bf16(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

__device__ __forceinline__ uint16_t narrow_f16(float x) {
  return __builtin_bit_cast(uint16_t, _Float16(x));   // v_cvt_f16_f32: RNE
}

template <int DT>
__device__ __forceinline__ void store_elem(void* base, size_t idx, float x) {
  if constexpr (DT == PKV_F32) {
    reinterpret_cast<float*>(base)[idx] = x;
  } else if constexpr (DT == PKV_F16) {
    reinterpret_cast<uint16_t*>(base)[idx] = narrow_f16(x);
  } else {
    reinterpret_cast<uint16_t*>(base)[idx] = narrow_bf16(x);
  }
}

template <int DT>
__device__ __forceinline__ float load_elem(const void* base, size_t idx) {
  if constexpr (DT == PKV_F32) {
    return reinterpret_cast<const float*>(base)[idx];
  } else {
    uint32_t w = reinterpret_cast<const uint16_t*>(base)[idx];
    return widen_half<DT>(w, false);
  }
}

// ---------------------------------------------------------------------------
// Lane reductions.  DPP controls (gfx9): quad_perm [1,0,3,2] = 0xB1,
// quad_perm [2,3,0,1] = 0x4E, row_half_mirror = 0x141, row_mirror = 0x140.
// After the k-th step every lane of an aligned group of 2^k lanes holds the
// same bit pattern (each step adds the same two operands in both partners).
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

__device__ __forceinline__ float shfl_xor_f(float x, int mask) {
  return __shfl_xor(x, mask, kWave);
}

// Sum over aligned groups of N lanes (N in 1..64, a power of two); every
// lane of a group receives the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp_f<0xB1>(x);
  if constexpr (N >= 4) x += dpp_f<0x4E>(x);
  if constexpr (N >= 8) x += dpp_f<0x141>(x);
  if constexpr (N >= 16) x += dpp_f<0x140>(x);
  if constexpr (N >= 32) x += shfl_xor_f(x, 16);
  if constexpr (N >= 64) x += shfl_xor_f(x, 32);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

}  // namespace pkv
