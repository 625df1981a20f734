// Device helpers shared by the gfx950 kernels: bf16 conversion, MFMA operand types,
// LDS-DMA helpers, wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace tcs {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int v8i_t __attribute__((ext_vector_type(8)));  // 32 fp8 codes: one fp8 MFMA operand

// Storage tags: the kernels move bf16 as raw 16-bit patterns.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16, round to nearest, ties to even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

template <typename T>
__device__ __forceinline__ float to_f32(T v);
template <>
__device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v.bits); }

template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return bf16_t{f32_to_bf16(v)}; }

// LDS pointer for the buffer-to-LDS load builtins.
#define TCS_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// s_waitcnt with one counter and the others left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// ---- wavefront reductions over groups of 16 consecutive lanes (DPP) ----
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// quad_perm [1,0,3,2] = 0xB1, quad_perm [2,3,0,1] = 0x4E, row_half_mirror = 0x141, row_mirror = 0x140
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  return v;
}
__device__ __forceinline__ float sum16(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// One lane's share of the dot product of a hidden row with head row `tok` of W
// (restricted heads: a few vocabulary rows, no log-sum-exp); summing over the 64
// lanes of the wave gives the product, before an fp8 row scale.  WK: 0 = fp32 h
// and W; 1 = bf16 h and W; 2 = bf16 h and E4M3 W.  bf16 rows: each lane takes 4
// consecutive elements per step, so d % 4 == 0 keeps every row 8-byte aligned.
template <int WK>
__device__ __forceinline__ float head_row_dot_lane(const void* __restrict__ h_row,
                                                   const void* __restrict__ W, int tok, int d,
                                                   int lane) {
  float acc = 0.f;
  if constexpr (WK == 0) {
    const float* hr = static_cast<const float*>(h_row);
    const float* wr = static_cast<const float*>(W) + size_t(tok) * d;
    for (int k = lane; k < d; k += 64) acc = fmaf(hr[k], wr[k], acc);
  } else {
    const uint2* hr = static_cast<const uint2*>(h_row);
    for (int k4 = lane; k4 < d / 4; k4 += 64) {
      const uint2 hv = hr[k4];
      float w[4];
      if constexpr (WK == 1) {
        const uint2 wv =
            reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(W) + size_t(tok) * d)[k4];
        w[0] = bf16_to_f32(uint16_t(wv.x));
        w[1] = bf16_to_f32(uint16_t(wv.x >> 16));
        w[2] = bf16_to_f32(uint16_t(wv.y));
        w[3] = bf16_to_f32(uint16_t(wv.y >> 16));
      } else {
        // four E4M3 codes -> bf16 (hardware conversion at scale 1, exact)
        const uint32_t wv =
            reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(W) + size_t(tok) * d)[k4];
        const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wv, 1.0f, false);
        const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wv, 1.0f, true);
        w[0] = float(lo[0]);
        w[1] = float(lo[1]);
        w[2] = float(hi[0]);
        w[3] = float(hi[1]);
      }
      acc = fmaf(bf16_to_f32(uint16_t(hv.x)), w[0], acc);
      acc = fmaf(bf16_to_f32(uint16_t(hv.x >> 16)), w[1], acc);
      acc = fmaf(bf16_to_f32(uint16_t(hv.y)), w[2], acc);
      acc = fmaf(bf16_to_f32(uint16_t(hv.y >> 16)), w[3], acc);
    }
  }
  return acc;
}

// (max, sum-of-exp) merge of two softmax partials.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  s = s * __expf(m - mn) + s2 * __expf(m2 - mn);
  m = mn;
}

}  // namespace tcs
