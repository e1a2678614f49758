// Measurement baselines for the fused prologue (not on the hot path).
//
// 1. The unfused plan of the chapter 13 ledger page ("norm+rope+quant, 3
//    kernels"): RMSNorm writes the normalised rows, a RoPE kernel reads them
//    and writes the rotated rows, a quantisation kernel reads those and writes
//    codes and one scale per row. Same arithmetic and rounding points as the
//    fused kernels, so the outputs are identical; only the traffic differs.
// 2. The chapter 28 page's designs A, B and C for QK-norm + RoPE + FP8: a
//    workgroup owns rows_per_block consecutive (token, head) rows (A: 1, B: 8,
//    C: every head of one token) and stages what its rows look up (both weight
//    vectors and the token's cos/sin row) once in LDS. The row arithmetic is the
//    row kernel's, so the outputs are identical to rnq_qk_norm_rope_fp8's.
#include "rnq_device.h"
#include "rnq_launch.h"

namespace rnq {

constexpr int BT = 256;
constexpr uint32_t kOut = 0x80000000u;

// ------------------------------------------------ unfused step 2: RoPE rows
// One workgroup per row: items are the 16-byte chunks before the tail (copied)
// and the R/16 pair chunks of the tail (chunk j of each half, rotated).
template <class DT>
__global__ __launch_bounds__(BT) void rope_rows_kernel(const uint16_t* __restrict__ in, const float* __restrict__ cos,
                                                       const float* __restrict__ sin, uint16_t* __restrict__ out,
                                                       uint32_t N, uint32_t R, uint32_t rows_per_token) {
  const uint32_t row = blockIdx.x;
  const uint32_t nc = (N - R) / 8, hc = R / 16, half = R / 2;
  const rsrc_t ri = make_rsrc(in + (size_t)row * N, 2u * N);
  const rsrc_t ro = make_rsrc(out + (size_t)row * N, 2u * N);
  const size_t trow = (size_t)(row / rows_per_token) * half;
  for (uint32_t i = threadIdx.x; i < nc + hc; i += BT) {
    if (i < nc) {
      buf_store16_nt(ro, 16u * i, buf_load16_nt(ri, 16u * i));
    } else {
      const uint32_t j = i - nc;
      const uint32_t lo_off = 2u * (N - R + 8 * j), hi_off = lo_off + 2u * half;
      float lo[8], hi[8];
      unpack8<DT>(buf_load16_nt(ri, lo_off), lo);
      unpack8<DT>(buf_load16_nt(ri, hi_off), hi);
      const float4 c0 = *(const float4*)(cos + trow + 8 * j), c1 = *(const float4*)(cos + trow + 8 * j + 4);
      const float4 s0 = *(const float4*)(sin + trow + 8 * j), s1 = *(const float4*)(sin + trow + 8 * j + 4);
      const float cc[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      const float ss[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
      float a[8], b[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        a[e] = DT::round((lo[e] * cc[e]) - (hi[e] * ss[e]));
        b[e] = DT::round((hi[e] * cc[e]) + (lo[e] * ss[e]));
      }
      buf_store16_nt(ro, lo_off, pack8<DT>(a));
      buf_store16_nt(ro, hi_off, pack8<DT>(b));
    }
  }
}

// ------------------------------------- unfused step 3: per-row FP8 quantise
// One workgroup per row; thread i owns chunks i, i + 256, ... (KC of them).
struct QuantRowsParams {
  const uint16_t* y;
  uint8_t* codes;
  float* scales;
  uint32_t N;
  float fp8_max, rcp_fp8_max, scale_floor;
  uint32_t scale_by_rcp, clamp;
};

template <class DT, int KC>
__global__ __launch_bounds__(BT) void quant_rows_kernel(QuantRowsParams p) {
  __shared__ float wmax[BT / 64];
  const uint32_t tid = threadIdx.x, row = blockIdx.x, nch = p.N / 8;
  const rsrc_t ry = make_rsrc(p.y + (size_t)row * p.N, 2u * p.N);
  float y[KC][8];
  uint32_t ch[KC];
  float m = 0.0f;
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    ch[k] = tid + BT * k;
    unpack8<DT>(buf_load16_nt(ry, ch[k] < nch ? 16u * ch[k] : kOut), y[k]);
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(y[k][i]));
  }
  m = group_max_nonneg<64>(m);
  if ((tid & 63) == 0) wmax[tid >> 6] = m;
  lds_barrier();
  float amax = wmax[0];
#pragma unroll
  for (int v = 1; v < BT / 64; ++v) amax = fmaxf(amax, wmax[v]);
  float scale;
  if (p.scale_by_rcp)
    scale = amax >= 1e-4f ? div_by(amax, p.fp8_max, p.rcp_fp8_max) : p.scale_floor;
  else
    scale = fmaxf(amax, 1e-4f) / p.fp8_max;
  const float rsc = rcp_rn(scale);
  const rsrc_t rq = make_rsrc(p.codes + (size_t)row * p.N, p.N);
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    float q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = div_by(y[k][i], scale, rsc);
    if (p.clamp) {
#pragma unroll
      for (int i = 0; i < 8; ++i) q[i] = __builtin_amdgcn_fmed3f(q[i], -p.fp8_max, p.fp8_max);
    }
    uint2 cw;
    cw.x = fp8x4(q[0], q[1], q[2], q[3], __float_as_uint(q[0]));
    cw.y = fp8x4(q[4], q[5], q[6], q[7], __float_as_uint(q[4]));
    buf_store8_nt(rq, ch[k] < nch ? 8u * ch[k] : kOut, cw);
  }
  if (tid == 0) p.scales[row] = scale;
}

template <class DT>
static hipError_t launch_quant_rows(const QuantRowsParams& p, uint32_t M, hipStream_t s) {
  const uint32_t nch = p.N / 8;
  const dim3 g(M), b(BT);
  if (nch <= BT) hipLaunchKernelGGL((quant_rows_kernel<DT, 1>), g, b, 0, s, p);
  else if (nch <= 2 * BT) hipLaunchKernelGGL((quant_rows_kernel<DT, 2>), g, b, 0, s, p);
  else if (nch <= 4 * BT) hipLaunchKernelGGL((quant_rows_kernel<DT, 4>), g, b, 0, s, p);
  else if (nch <= 8 * BT) hipLaunchKernelGGL((quant_rows_kernel<DT, 8>), g, b, 0, s, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

static void quant_constants(float fp8_max, float& rcp, float& floor_, uint32_t& by_rcp, uint32_t& clamp) {
  rcp = 1.0f / fp8_max;
  floor_ = 1e-4f / fp8_max;
  by_rcp = fp8_max >= 1.0f ? 1u : 0u;
  clamp = fp8_clamp_needed(fp8_max) ? 1u : 0u;
}

hipError_t launch_unfused_rope_quant(const uint16_t* normed, const float* cos, const float* sin, uint16_t* rotated,
                                     uint8_t* codes, float* scales, uint32_t M, uint32_t N, uint32_t R,
                                     uint32_t rows_per_token, float fp8_max, bool bf16, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL((rope_rows_kernel<BF16>), dim3(M), dim3(BT), 0, s, normed, cos, sin, rotated, N, R,
                       rows_per_token);
  else
    hipLaunchKernelGGL((rope_rows_kernel<F16>), dim3(M), dim3(BT), 0, s, normed, cos, sin, rotated, N, R,
                       rows_per_token);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  QuantRowsParams q = {};
  q.y = rotated;
  q.codes = codes;
  q.scales = scales;
  q.N = N;
  q.fp8_max = fp8_max;
  quant_constants(fp8_max, q.rcp_fp8_max, q.scale_floor, q.scale_by_rcp, q.clamp);
  return bf16 ? launch_quant_rows<BF16>(q, M, s) : launch_quant_rows<F16>(q, M, s);
}

// ------------------------------------------------ chapter 28 designs A / B / C
// L = D / 8 lanes per row (one 16-byte chunk each), rows_per_block rows per
// workgroup (RB lanes groups; threads rounded up to whole waves). The
// workgroup stages both weight vectors and the token's cos/sin row in LDS
// once (all its rows belong to one token: rows_per_block divides the heads),
// then every row is normalised, rotated (the partner chunk R/16 lanes away
// by a lane permute), reduced and quantised by its L lanes.
struct DesignParams {
  const uint16_t* x0;  // q [T, H0, D]
  const uint16_t* x1;  // k [T, H1, D]
  const uint16_t* w0;
  const uint16_t* w1;
  const float* cos;
  const float* sin;
  uint8_t* c0;
  uint8_t* c1;
  float* s0;
  float* s1;
  uint32_t total_rows, heads, heads0, rope, rows_per_block;
  float eps, fp8_max, rcp_fp8_max, scale_floor;
  uint32_t scale_by_rcp, clamp;
};

template <class DT, int D>
__global__ __launch_bounds__(1024) void design_kernel(DesignParams p) {
  constexpr int L = D / 8;
  __shared__ float w_s[2 * D];
  __shared__ float t_s[D];  // cos row then sin row (R/2 each, R <= D)
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const uint32_t ch = tid % L;
  const uint32_t r_in = tid / L;
  const uint32_t first = blockIdx.x * p.rows_per_block;
  const uint32_t tok = first / p.heads;
  const uint32_t half = p.rope / 2;

  // lookups, once per workgroup
  for (uint32_t i = tid; i < 2u * D; i += blockDim.x) {
    const uint16_t* w = i < (uint32_t)D ? p.w0 : (p.heads0 < p.heads ? p.w1 : p.w0);
    const uint16_t v = w[i % D];
    w_s[i] = DT::lo((uint32_t)v);
  }
  for (uint32_t i = tid; i < 2u * half; i += blockDim.x)
    t_s[i] = i < half ? p.cos[(size_t)tok * half + i] : p.sin[(size_t)tok * half + (i - half)];
  lds_barrier();

  const bool active = r_in < p.rows_per_block;
  const uint32_t row = first + (active ? r_in : 0);
  const uint32_t h = row - tok * p.heads;
  const bool second = h >= p.heads0;
  const uint32_t ri = second ? tok * (p.heads - p.heads0) + (h - p.heads0) : tok * p.heads0 + h;
  const uint16_t* src = (second ? p.x1 : p.x0) + (size_t)ri * D;
  float x[8];
  unpack8<DT>(*(const uint4*)(src + 8 * ch), x);
  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) acc = __builtin_fma((double)x[i], (double)x[i], acc);
  acc = group_sum<L>(acc);
  const float rstd = rstd_of((float)acc * (1.0f / (float)D) + p.eps);
  const float* w = w_s + (second ? D : 0) + 8 * ch;
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = DT::round((x[i] * rstd) * w[i]);

  // RoPE: tail chunk j of the lower half pairs with chunk j of the upper half
  const uint32_t t0 = (D - p.rope) / 8, hc = p.rope / 16;
  const bool tail = ch >= t0;
  const uint32_t j = ch - t0;
  const bool lo_half = tail && j < hc;
  const int src_lane = tail ? (int)lane + (lo_half ? (int)hc : -(int)hc) : (int)lane;
  float other[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) other[i] = __shfl(y[i], src_lane, 64);
  if (tail) {
    const uint32_t pj = lo_half ? j : j - hc;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float c = t_s[8 * pj + i], s = t_s[half + 8 * pj + i];
      y[i] = lo_half ? DT::round((y[i] * c) - (other[i] * s)) : DT::round((y[i] * c) + (other[i] * s));
    }
  }

  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(y[i]));
  const float amax = group_max_nonneg<L>(m);
  float scale;
  if (p.scale_by_rcp)
    scale = amax >= 1e-4f ? div_by(amax, p.fp8_max, p.rcp_fp8_max) : p.scale_floor;
  else
    scale = fmaxf(amax, 1e-4f) / p.fp8_max;
  const float rsc = rcp_rn(scale);
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = div_by(y[i], scale, rsc);
  if (p.clamp) {
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = __builtin_amdgcn_fmed3f(q[i], -p.fp8_max, p.fp8_max);
  }
  uint2 cw;
  cw.x = fp8x4(q[0], q[1], q[2], q[3], __float_as_uint(q[0]));
  cw.y = fp8x4(q[4], q[5], q[6], q[7], __float_as_uint(q[4]));
  if (active) {
    *(uint2*)((second ? p.c1 : p.c0) + (size_t)ri * D + 8 * ch) = cw;
    if (ch == 0) (second ? p.s1 : p.s0)[ri] = scale;
  }
}

hipError_t launch_design(const RowParams& rp, uint32_t rows_per_block, int D, bool bf16, hipStream_t s) {
  if (rp.total_rows == 0) return hipSuccess;
  DesignParams p = {};
  p.x0 = rp.x0;
  p.x1 = rp.x1;
  p.w0 = rp.w0;
  p.w1 = rp.w1;
  p.cos = rp.cos;
  p.sin = rp.sin;
  p.c0 = rp.c0;
  p.c1 = rp.c1;
  p.s0 = rp.s0;
  p.s1 = rp.s1;
  p.total_rows = rp.total_rows;
  p.heads = rp.heads;
  p.heads0 = rp.heads0;
  p.rope = rp.rope;
  p.rows_per_block = rows_per_block;
  p.eps = rp.eps;
  p.fp8_max = rp.fp8_max;
  quant_constants(rp.fp8_max, p.rcp_fp8_max, p.scale_floor, p.scale_by_rcp, p.clamp);
  const uint32_t threads = (rows_per_block * (uint32_t)(D / 8) + 63) / 64 * 64;
  if (threads > 1024) return hipErrorInvalidValue;
  const dim3 g(rp.total_rows / rows_per_block), b(threads);
  switch (D * (bf16 ? 1 : -1)) {
    case 64: hipLaunchKernelGGL((design_kernel<BF16, 64>), g, b, 0, s, p); break;
    case 128: hipLaunchKernelGGL((design_kernel<BF16, 128>), g, b, 0, s, p); break;
    case 256: hipLaunchKernelGGL((design_kernel<BF16, 256>), g, b, 0, s, p); break;
    case 512: hipLaunchKernelGGL((design_kernel<BF16, 512>), g, b, 0, s, p); break;
    case -64: hipLaunchKernelGGL((design_kernel<F16, 64>), g, b, 0, s, p); break;
    case -128: hipLaunchKernelGGL((design_kernel<F16, 128>), g, b, 0, s, p); break;
    case -256: hipLaunchKernelGGL((design_kernel<F16, 256>), g, b, 0, s, p); break;
    case -512: hipLaunchKernelGGL((design_kernel<F16, 512>), g, b, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------ HBM floor

// The memory floor of a byte pattern like the prologue's, for measurement: wave
// w reads the 2 KB block w of src (two 16-byte chunks per lane, 1 KB apart) and
// writes the 1 KB block w of dst (their XOR), with nontemporal loads, stores
// nontemporal or with device scope (DEV), and nothing else.
template <bool DEV>
__global__ __launch_bounds__(256) void stream_kernel(const uint8_t* src, uint8_t* dst, uint32_t blocks) {
  const uint32_t w = blockIdx.x * 4u + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63u;
  // waves past the last block read and write nothing (empty descriptors): an
  // early exit would be a branch ahead of the argument loads, which the
  // compiler then issues in a second dependent round
  const bool live = w < blocks;
  const size_t wb = live ? w : 0u;
  const rsrc_t rs = make_rsrc(src + wb * 2048u, live ? 2048u : 0u);
  const rsrc_t rd = make_rsrc(dst + wb * 1024u, live ? 1024u : 0u);
  const uint4 a = buf_load16_nt(rs, 16u * lane);
  const uint4 b = buf_load16_nt(rs, 1024u + 16u * lane);
  const uint4 v = make_uint4(a.x ^ b.x, a.y ^ b.y, a.z ^ b.z, a.w ^ b.w);
  if constexpr (DEV)
    buf_store16_dev(rd, 16u * lane, v);
  else
    buf_store16_nt(rd, 16u * lane, v);
}

// One workgroup that does nothing: the cost of a launch.
__global__ void empty_kernel() {}

hipError_t launch_stream(const void* src, void* dst, uint32_t blocks, bool device_scope, hipStream_t s) {
  if (blocks == 0) {
    hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, s);
  } else if (device_scope) {
    hipLaunchKernelGGL(stream_kernel<true>, dim3((blocks + 3) / 4), dim3(256), 0, s, (const uint8_t*)src,
                       (uint8_t*)dst, blocks);
  } else {
    hipLaunchKernelGGL(stream_kernel<false>, dim3((blocks + 3) / 4), dim3(256), 0, s, (const uint8_t*)src,
                       (uint8_t*)dst, blocks);
  }
  return hipGetLastError();
}

}  // namespace rnq
