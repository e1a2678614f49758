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
  // a rounded to bf16, as an fp32 value: one conversion with a zero low half
  static __device__ __forceinline__ float round(float a) { return __uint_as_float(pack(0.0f, a)); }
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
  // a rounded to fp16, as an fp32 value. The empty asm pins a as an fp32
  // value first: otherwise the compiler may fold the product that produced it
  // into one mixed-precision fma that rounds straight to fp16 (one rounding
  // where the operation rounds twice).
  static __device__ __forceinline__ float round(float a) {
    asm volatile("" : "+v"(a));
    return (float)(_Float16)a;
  }
};

// fp16 values kept as their bits (low 16 bits of a register) where the only
// consumers are further products and the store: rounding to fp16 is then one
// conversion, with no conversion back to fp32.
// a rounded to fp16 (nearest even), as bits; the empty asm keeps the product
// that made a from being folded into a mixed-precision fma that rounds once
__device__ __forceinline__ uint32_t f16_bits(float a) {
  asm volatile("" : "+v"(a));
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a);
}
// RN(h * b) in fp32 for an fp16 value h given as bits: one mixed-precision fma
// with a -0 addend (x + -0 = x for every x, -0 included, so the result is the
// fp32 product's rounding and sign; a +0 addend would turn a -0 product into
// +0). The compiler would rewrite an fma with a -0 addend into a plain
// multiply, which needs h converted first. The addend is the inline constant 0
// under the negate modifier: `neg(0)` (a bare `-0` assembles as integer 0).
__device__ __forceinline__ float mul_f16_f32(uint32_t h, float b) {
  float r;
  asm("v_fma_mix_f32 %0, %1, %2, neg(0) op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(b));
  return r;
}
// 8 fp16 values given as bits -> one 16-byte chunk
__device__ __forceinline__ uint4 pack8_bits(const uint32_t* h) {
  uint4 v;
  v.x = (h[0] & 0xffffu) | (h[1] << 16);
  v.y = (h[2] & 0xffffu) | (h[3] << 16);
  v.z = (h[4] & 0xffffu) | (h[5] << 16);
  v.w = (h[6] & 0xffffu) | (h[7] << 16);
  return v;
}

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

// ------------------------------------------------------- streaming accesses
// Data read once and codes written once: nontemporal hint (no reuse in cache).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void store_stream8(void* p, uint2 v) {
  const u32x2 w = {v.x, v.y};
  __builtin_nontemporal_store(w, (u32x2*)p);
}

// Raw buffer accesses: a wave-uniform base (the descriptor, in scalar
// registers) plus a 32-bit per-lane byte offset, so no per-lane 64-bit address
// arithmetic. Offsets at or past `bytes` read zero / are dropped by the
// hardware range check. Dword 3 of the descriptor: raw (untyped) 32-bit data.
// The base must be wave-uniform; it is read from the first active lane so
// that the descriptor is built in scalar registers whatever path the value
// took (a descriptor the compiler thinks divergent costs a loop per access).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // (readfirstlane returns int: convert through uint32_t so the low half is
  // zero-extended, never sign-extended into the high half)
  const uint64_t a = (uint64_t)base;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | (uint64_t)lo), 0, (int)bytes, 0x00020000);
}
constexpr int kNonTemporal = 2;  // cache-policy bit: streaming access, no reuse
__device__ __forceinline__ uint4 buf_load16_nt(rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNonTemporal);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 buf_load16(rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 buf_load16f(rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}
__device__ __forceinline__ uint2 buf_load8(rsrc_t r, uint32_t off) {
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t buf_load4(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ float buf_load4f(rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ void buf_store16(rsrc_t r, uint32_t off, uint4 v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(w, r, off, 0, 0);
}
__device__ __forceinline__ void buf_store16_nt(rsrc_t r, uint32_t off, uint4 v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(w, r, off, 0, kNonTemporal);
}
__device__ __forceinline__ void buf_store8_nt(rsrc_t r, uint32_t off, uint2 v) {
  const u32x2 w = {v.x, v.y};
  __builtin_amdgcn_raw_buffer_store_b64(w, r, off, 0, kNonTemporal);
}
// Stores with the sc1 cache-policy bit alone (device scope, no streaming
// hint). Which store policy suits an output was measured kernel by kernel
// (builds alternated in one process, with more rotated output buffers than the
// 256 MB Infinity Cache holds: ordinary and device-scope stores allocate there,
// and fewer buffers can stay resident): device-scope stores made the wide
// RMSNorm forward's y 12.95 -> 12.81 us at 4096 x 4096, while they made the row
// kernel's FP8 codes (320 -> 338 us at the 65,536-token prologue), path R's y,
// the grouped kernel's outputs and the narrow backward's grad_x slower than
// nontemporal stores, which those keep.
constexpr int kDeviceScope = 16;  // cache-policy bit sc1
__device__ __forceinline__ void buf_store16_dev(rsrc_t r, uint32_t off, uint4 v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(w, r, off, 0, kDeviceScope);
}
__device__ __forceinline__ void buf_store4(rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}

// Workgroup barrier that orders LDS only. __syncthreads() also fences global
// memory, which on this target waits for every outstanding global load and
// store of the wave (prefetches of the next rows included); the barriers here
// only ever protect LDS data, so they wait for the wave's LDS accesses alone.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ------------------------------------------------------------ DPP reductions
// dpp_ctrl values (GFX9 DPP): quad_perm [1,0,3,2] = 0xB1 (xor 1),
// quad_perm [2,3,0,1] = 0x4E (xor 2), row_half_mirror = 0x141 (lane i <- 7-i
// within 8), row_mirror = 0x140 (lane i <- 15-i within 16).

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  uint64_t b = __builtin_bit_cast(uint64_t, v);
  int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)b, CTRL, 0xF, 0xF, true);
  int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, true);
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

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}

// Max over aligned groups of L lanes of non-negative values (absolute values;
// +0 included, no NaN). For such floats the order of the bit patterns read as
// unsigned integers is the order of the values, so the lanes combine with an
// unsigned maximum, which takes the DPP operand directly (one instruction per
// step instead of a move and a float maximum).
template <int L>
__device__ __forceinline__ float group_max_nonneg(float f) {
  uint32_t v = __float_as_uint(f);
  if constexpr (L >= 2) v = max(v, dpp_u32<0xB1>(v));
  if constexpr (L >= 4) v = max(v, dpp_u32<0x4E>(v));
  if constexpr (L >= 8) v = max(v, dpp_u32<0x141>(v));
  if constexpr (L >= 16) v = max(v, dpp_u32<0x140>(v));
  if constexpr (L >= 32) v = max(v, (uint32_t)__shfl_xor((int)v, 16, 64));
  if constexpr (L >= 64) v = max(v, (uint32_t)__shfl_xor((int)v, 32, 64));
  return __uint_as_float(v);
}

// ------------------------------------------------------------- row scalars
// The row scalars are correctly rounded IEEE results. Each has a short
// sequence, checked bit for bit against the IEEE one over every input in its
// range (all normal positive floats for the reciprocal; v >= 2^-105 for the
// square root), and the IEEE sequence (which hipcc emits for '/' and
// __builtin_sqrtf) for anything outside that range.

// RN(1/s) for s in [2^-126, 2^126): hardware reciprocal (1 ulp) and one
// Newton step, r = r0 + r0 (1 - s r0) with fused multiply-adds.
__device__ __forceinline__ float rcp_rn_fast(float s) {
  const float r0 = __builtin_amdgcn_rcpf(s);
  const float e = __builtin_fmaf(-s, r0, 1.0f);
  return __builtin_fmaf(e, r0, r0);
}

// RN(sqrt(v)) for v in [2^-105, +inf]: hardware square root (1 ulp), then
// the neighbour whose square brackets v.
__device__ __forceinline__ float sqrt_rn_fast(float v) {
  float s = __builtin_amdgcn_sqrtf(v);
  const float sm = __uint_as_float(__float_as_uint(s) - 1u);
  const float sp = __uint_as_float(__float_as_uint(s) + 1u);
  const float rm = __builtin_fmaf(-sm, s, v);
  const float rp = __builtin_fmaf(-sp, s, v);
  s = (rm <= 0.0f) ? sm : s;
  s = (rp > 0.0f) ? sp : s;
  return s;
}

// rstd = RN(1 / RN(sqrt(v))), v = mean(x^2) + eps. All lanes of a wave take
// the same branch (the fast one unless some row is outside the checked range).
__device__ __forceinline__ float rstd_of(float v) {
  const bool fast = v >= 0x1p-100f && v <= 0x1p+120f;
  if (__builtin_amdgcn_ballot_w64(!fast) == 0) return rcp_rn_fast(sqrt_rn_fast(v));
  return 1.0f / __builtin_sqrtf(v);
}

// RN(1/s) for any positive normal s (fast path below 2^126).
__device__ __forceinline__ float rcp_rn(float s) {
  if (__builtin_amdgcn_ballot_w64(!(s < 0x1p+126f)) == 0) return rcp_rn_fast(s);
  return 1.0f / s;
}

// a / b rounded to nearest, given r = RN(1/b): q0 = RN(a r), the exact
// residual e = b*q0 - a by one FMA, then q1 = RN(q0 - e r). Checked bit for
// bit against IEEE division for every a with at most 11 significand bits
// (every bf16 or fp16 value) and every fp32 b, at normal exponents; the result
// differs only where |a/b| < 2^-100 (and then keeps the sign), which for the
// FP8 step is far below the smallest e4m3 subnormal. Zeros keep their sign.
__device__ __forceinline__ float div_by(float a, float b, float r) {
  const float q0 = a * r;
  const float e = __builtin_fmaf(b, q0, -a);
  return __builtin_fmaf(-e, r, q0);
}

// Four values -> four e4m3fn codes (OCP, nearest even) in one 32-bit word.
// The first conversion fills the low half; the previous contents of the word
// do not matter, so any register serves as its initial value.
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d, uint32_t any) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)any, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

}  // namespace rnq
