// Device helpers shared by the rnq kernels (gfx950 / CDNA4, wave64).
//
// Internal header of librnq.so: dtype codecs on packed 32-bit words, DPP
// cross-lane reductions, and the per-element quotient used by the FP8 step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rnq {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- dtype traits
// A 32-bit word holds two 16-bit values: element 2i in the low half, 2i+1 in
// the high half (little-endian row-major storage).

struct BF16 {
  static __device__ __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
  static __device__ __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
  // round both values to bf16, nearest even (v_cvt_pk_bf16_f32)
  static __device__ __forceinline__ uint32_t pack(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  }
};

struct F16 {
  static __device__ __forceinline__ float lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
  }
  static __device__ __forceinline__ float hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  }
  // round both values to fp16, nearest even
  static __device__ __forceinline__ uint32_t pack(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
};

// 8 consecutive 16-bit values (one 16-byte chunk) <-> 8 floats
template <class DT>
__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
  f[0] = DT::lo(v.x); f[1] = DT::hi(v.x);
  f[2] = DT::lo(v.y); f[3] = DT::hi(v.y);
  f[4] = DT::lo(v.z); f[5] = DT::hi(v.z);
  f[6] = DT::lo(v.w); f[7] = DT::hi(v.w);
}

template <class DT>
__device__ __forceinline__ uint4 pack8(const float* f) {
  uint4 v;
  v.x = DT::pack(f[0], f[1]);
  v.y = DT::pack(f[2], f[3]);
  v.z = DT::pack(f[4], f[5]);
  v.w = DT::pack(f[6], f[7]);
  return v;
}

// ------------------------------------------------------------ DPP reductions
// dpp_ctrl values (GFX9 DPP): quad_perm [1,0,3,2] = 0xB1 (xor 1),
// quad_perm [2,3,0,1] = 0x4E (xor 2), row_half_mirror = 0x141 (lane i <- 7-i
// within 8), row_mirror = 0x140 (lane i <- 15-i within 16).

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  uint64_t b = __builtin_bit_cast(uint64_t, v);
  int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, 0xF, 0xF, false);
  int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Sum over aligned groups of L lanes (L a power of two <= 64). Every lane of a
// group ends with the same value (each step adds a value to its partner's).
template <int L>
__device__ __forceinline__ double group_sum(double v) {
  if constexpr (L >= 2) v += dpp_f64<0xB1>(v);
  if constexpr (L >= 4) v += dpp_f64<0x4E>(v);
  if constexpr (L >= 8) v += dpp_f64<0x141>(v);
  if constexpr (L >= 16) v += dpp_f64<0x140>(v);
  if constexpr (L >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (L >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

template <int L>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (L >= 2) v += dpp_f32<0xB1>(v);
  if constexpr (L >= 4) v += dpp_f32<0x4E>(v);
  if constexpr (L >= 8) v += dpp_f32<0x141>(v);
  if constexpr (L >= 16) v += dpp_f32<0x140>(v);
  if constexpr (L >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (L >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

template <int L>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (L >= 2) v = fmaxf(v, dpp_f32<0xB1>(v));
  if constexpr (L >= 4) v = fmaxf(v, dpp_f32<0x4E>(v));
  if constexpr (L >= 8) v = fmaxf(v, dpp_f32<0x141>(v));
  if constexpr (L >= 16) v = fmaxf(v, dpp_f32<0x140>(v));
  if constexpr (L >= 32) v = fmaxf(v, __shfl_xor(v, 16, 64));
  if constexpr (L >= 64) v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}

// ------------------------------------------------------------- row scalars

// 1 / sqrt(v): correctly rounded square root, then correctly rounded division
// (hipcc lowers __builtin_sqrtf and '/' to IEEE-exact sequences).
__device__ __forceinline__ float rstd_of(float v) { return 1.0f / __builtin_sqrtf(v); }

// y / scale rounded to nearest, from r = RN(1/scale): q0 = RN(y r), the exact
// residual e = scale*q0 - y by one FMA, then q1 = RN(q0 - e r). For every
// bf16 or fp16 y and every fp32 scale this equals the IEEE quotient whenever
// |y/scale| >= 2^-100; below that both are far under the smallest e4m3
// subnormal and carry the same sign. Zeros keep their sign.
__device__ __forceinline__ float div_by_scale(float y, float scale, float r) {
  float q0 = y * r;
  float e = __builtin_fmaf(scale, q0, -y);
  return __builtin_fmaf(-e, r, q0);
}

// Four values -> four e4m3fn codes (OCP, nearest even) in one 32-bit word.
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

}  // namespace rnq
