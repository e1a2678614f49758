// RMSNorm -> partial NeoX RoPE -> FP8 e4m3fn with one scale per group of
// group_size consecutive elements, over rows of up to 16384 elements.
//
// Operation: tilelang-tutorial chapter 13 fusion page, rms_norm_rope_quant_fused
// (the normalised row cast to the input dtype, the tail rotated and cast, then
// every group of group_size elements quantised with its own scale =
// max(group absmax, 1e-4) / fp8_max, y / scale clamped to +-fp8_max and cast).
//
// Mapping: one 256-thread workgroup per row; thread i owns 16-byte chunks
// i, i+256, ... (KC of them). A group of group_size elements is GL =
// group_size / 8 consecutive chunks, i.e. GL consecutive lanes of one wave, so
// its absmax is a DPP reduction over those lanes. One group per row (GL = 0)
// takes the row's absmax instead: each wave's maximum, then the four through
// LDS (one more barrier). The rope tail's pairs live in different threads:
// the normalised tail goes through LDS (one barrier).
// Every global access is a buffer access with a row-uniform descriptor (lanes
// past the row's end use offsets outside its range).
//
// The same kernel without the quantiser (QUANT = false) is RMSNorm + RoPE
// (the fusion page's rms_norm_rope_fused) over rows wider than a head: it
// writes y only. Rows may sit in a token-strided view (x_token_stride
// elements between the first rows of consecutive tokens) and the cos/sin row
// of token t may be row positions[t] of a position-indexed table.
#include "rnq_device.h"
#include "rnq_launch.h"

namespace rnq {

constexpr int GT = 256;       // threads per workgroup
constexpr int GWV = GT / 64;  // waves
constexpr uint32_t kMaxRope = 1024;

// (Every kernel argument a workgroup needs before its first input load is
// read in one round: no branch precedes those loads, since the compiler issues
// no argument load past one. The token comes from a host-computed
// multiply-shift, the launcher gives every call a token stride and the table's
// row count, and a position-indexed table is a template case; with positions
// the table row is a second, dependent round, after the input loads.)
// The fields a workgroup needs before its first loads (its row of x, the
// weights, the tail's cos / sin values) come as leading scalar arguments, 14
// dwords that gfx950 preloads into scalar registers at wave launch: a
// workgroup then issues them without first loading its kernel arguments,
// which every workgroup (one per row) would otherwise wait for.
struct GroupHot {
  const uint16_t* x;
  uint64_t xs;  // token stride of x in elements
  const uint16_t* w;
  const float* cos;
  const float* sin;
  uint32_t n_shift_rope;  // N | div_shift << 15 | rope << 21
  uint32_t rows_per_token, div_magic, table_bytes;
  __device__ __forceinline__ uint32_t N() const { return n_shift_rope & 0x7fffu; }
  __device__ __forceinline__ uint32_t div_shift() const { return (n_shift_rope >> 15) & 0x3fu; }
  __device__ __forceinline__ uint32_t rope() const { return n_shift_rope >> 21; }
};

template <class DT, int KC, int GL, bool QUANT = true, bool POS = false>
__global__ __launch_bounds__(GT) void group_quant_kernel(const uint16_t* x, uint64_t xs, const uint16_t* w,
                                                         const float* cos, const float* sin, uint32_t n_shift_rope,
                                                         uint32_t rows_per_token, uint32_t div_magic,
                                                         uint32_t table_bytes, GroupQuantParams p) {
  const GroupHot hp{x, xs, w, cos, sin, n_shift_rope, rows_per_token, div_magic, table_bytes};
  const uint32_t N = hp.N();
  constexpr uint32_t kOutOfRange = 0x80000000u;
  __shared__ double part[GWV];
  __shared__ float tail_s[kMaxRope];
  __shared__ float wmax[GWV];
  const uint32_t tid = threadIdx.x;
  const uint32_t wave = tid >> 6;
  const uint32_t row = blockIdx.x;
  const uint32_t nch = N / 8;
  const uint32_t row_bytes = 2u * N;

  uint32_t ch[KC], off[KC];
  bool ok[KC];
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    ch[k] = tid + GT * k;
    ok[k] = ch[k] < nch;
    off[k] = ok[k] ? 16u * ch[k] : kOutOfRange;
  }
  // the row's token and its place in a (possibly strided) view
  const uint32_t tok = (uint32_t)(((uint64_t)row * hp.div_magic) >> hp.div_shift());
  const size_t xoff = (size_t)tok * hp.xs + (size_t)(row - tok * hp.rows_per_token) * N;
  const rsrc_t rx = make_rsrc(hp.x + xoff, row_bytes);
  const rsrc_t rw = make_rsrc(hp.w, row_bytes);
  uint4 xr[KC], wr[KC];
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    xr[k] = buf_load16_nt(rx, off[k]);
    wr[k] = buf_load16(rw, off[k]);
  }
  // the token's table row
  uint32_t trow = tok;
  if constexpr (POS) {
    // a workgroup-uniform index read through the constant address space (a
    // scalar load; the kernel never writes positions)
    typedef const __attribute__((address_space(4))) int32_t const_i32;
    trow = min((uint32_t)((const_i32*)p.positions)[tok], p.max_pos - 1);
  }
  // the rope tail's cos/sin values go out with the row: a thread's chunks are
  // 256 apart and the tail is at most 128 chunks, so a thread owns at most one
  // tail chunk and needs one set of 8 pair columns (other lanes read nothing)
  const uint32_t R = hp.rope(), half = R / 2;
  const uint32_t t0 = nch - R / 8, hc = R / 16;  // first tail chunk, chunks per half
  uint32_t toff = kOutOfRange;
#pragma unroll
  for (int k = 0; k < KC; ++k)
    if (ok[k] && R > 0 && ch[k] >= t0) {
      const uint32_t j = ch[k] - t0;
      toff = 4u * (trow * half + 8u * (j < hc ? j : j - hc));
    }
  const rsrc_t rcos = make_rsrc(hp.cos, hp.table_bytes), rsin = make_rsrc(hp.sin, hp.table_bytes);
  const float4 tc0 = buf_load16f(rcos, toff), tc1 = buf_load16f(rcos, toff + 16u);
  const float4 ts0 = buf_load16f(rsin, toff), ts1 = buf_load16f(rsin, toff + 16u);

  // ---- sum of squares: fp64 (exact for 16-bit inputs); waves added in ascending order
  double acc = 0.0;
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    float xf[8];
    unpack8<DT>(xr[k], xf);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = __builtin_fma((double)xf[i], (double)xf[i], acc);
  }
  acc = group_sum<64>(acc);
  if ((tid & 63) == 0) part[wave] = acc;
  lds_barrier();
  double tot = part[0];
#pragma unroll
  for (int v = 1; v < GWV; ++v) tot += part[v];
  const float ssq = (float)tot;            // one rounding of the exact sum
  const float rstd = rstd_of(ssq / (float)N + p.eps);

  // ---- normalise: (x * rstd) * w, rounded to the input dtype
  float y[KC][8];
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    float xf[8], wf[8];
    unpack8<DT>(xr[k], xf);
    unpack8<DT>(wr[k], wf);
#pragma unroll
    for (int i = 0; i < 8; ++i) y[k][i] = DT::round((xf[i] * rstd) * wf[i]);
  }

  // ---- RoPE on the last R columns: pair p <-> p + R/2, the other half through LDS
  if (R > 0) {
#pragma unroll
    for (int k = 0; k < KC; ++k)
      if (ok[k] && ch[k] >= t0) {
        float* d = tail_s + 8 * (ch[k] - t0);
        *(float4*)d = make_float4(y[k][0], y[k][1], y[k][2], y[k][3]);
        *(float4*)(d + 4) = make_float4(y[k][4], y[k][5], y[k][6], y[k][7]);
      }
    lds_barrier();
#pragma unroll
    for (int k = 0; k < KC; ++k)
      if (ok[k] && ch[k] >= t0) {
        const uint32_t j = ch[k] - t0;
        const bool lo_half = j < hc;
        const float cc[8] = {tc0.x, tc0.y, tc0.z, tc0.w, tc1.x, tc1.y, tc1.z, tc1.w};
        const float ss[8] = {ts0.x, ts0.y, ts0.z, ts0.w, ts1.x, ts1.y, ts1.z, ts1.w};
        const float* other = tail_s + 8 * (lo_half ? j + hc : j - hc);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if (lo_half) {
            const float lo = y[k][i], hi = other[i];
            y[k][i] = DT::round((lo * cc[i]) - (hi * ss[i]));
          } else {
            const float hi = y[k][i], lo = other[i];
            y[k][i] = DT::round((hi * cc[i]) + (lo * ss[i]));
          }
        }
      }
  }

  if (!QUANT || p.y != nullptr) {
    const rsrc_t ry = make_rsrc(p.y + (size_t)row * N, row_bytes);
#pragma unroll
    for (int k = 0; k < KC; ++k) buf_store16_nt(ry, off[k], pack8<DT>(y[k]));
  }
  if constexpr (!QUANT) return;

  // ---- per-group absmax, scale and codes
  const uint32_t n_groups = N / p.group_size;
  const rsrc_t rq = make_rsrc(p.codes + (size_t)row * N, N);
  const rsrc_t rs = make_rsrc(p.scales + (size_t)row * n_groups, 4u * n_groups);
  float row_amax = 0.0f;
  if constexpr (GL == 0) {
    // one group per row: the row's absmax (lanes past the row's end hold zeros)
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < KC; ++k)
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(y[k][i]));
    m = group_max_nonneg<64>(m);
    if ((tid & 63) == 0) wmax[wave] = m;
    lds_barrier();
    row_amax = wmax[0];
#pragma unroll
    for (int v = 1; v < GWV; ++v) row_amax = fmaxf(row_amax, wmax[v]);
  }
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    float amax = row_amax;
    if constexpr (GL > 0) {
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(y[k][i]));
      amax = group_max_nonneg<GL>(m);
    }
    // scale = RN(max(amax, 1e-4) / fp8_max); amax is a 16-bit float value
    float scale;
    if (p.scale_by_rcp)
      scale = amax >= 1e-4f ? div_by(amax, p.fp8_max, p.rcp_fp8_max) : p.scale_floor;
    else
      scale = fmaxf(amax, 1e-4f) / p.fp8_max;
    const float rsc = rcp_rn(scale);
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
    buf_store8_nt(rq, ok[k] ? 8u * ch[k] : kOutOfRange, cw);
    // the group's first lane stores its scale (chunk 0 for a whole-row group)
    uint32_t soff = kOutOfRange;
    if constexpr (GL > 0) {
      if (ok[k] && ch[k] % GL == 0) soff = 4u * (ch[k] / GL);
    } else {
      if (ch[k] == 0) soff = 0;
    }
    buf_store4(rs, soff, scale);
  }
}

// --------------------------------------------------------------- launcher

// (the leading, preloaded arguments: see GroupHot)
#define RNQ_GROUP_HOT(p)                                                                                  \
  (p).x, (p).xs, (p).w, (p).cos, (p).sin, (p).N | (p).div_shift << 15 | (p).rope << 21, (p).rows_per_token, \
      (p).div_magic, (p).rope > 0 ? (p).max_pos * ((p).rope / 2) * 4u : 0u, (p)

template <class DT, int KC>
static hipError_t launch_kc(const GroupQuantParams& p, dim3 g, hipStream_t s) {
  if (p.group_size == p.N && (p.N > 512 || (p.N & (p.N - 1)) != 0)) {  // one group per row (not one wave's lanes)
    hipLaunchKernelGGL((group_quant_kernel<DT, KC, 0>), g, dim3(GT), 0, s, RNQ_GROUP_HOT(p));
    return hipGetLastError();
  }
  switch (p.group_size / 8) {
    case 1: hipLaunchKernelGGL((group_quant_kernel<DT, KC, 1>), g, dim3(GT), 0, s, RNQ_GROUP_HOT(p)); break;
    case 2: hipLaunchKernelGGL((group_quant_kernel<DT, KC, 2>), g, dim3(GT), 0, s, RNQ_GROUP_HOT(p)); break;
    case 4: hipLaunchKernelGGL((group_quant_kernel<DT, KC, 4>), g, dim3(GT), 0, s, RNQ_GROUP_HOT(p)); break;
    case 8: hipLaunchKernelGGL((group_quant_kernel<DT, KC, 8>), g, dim3(GT), 0, s, RNQ_GROUP_HOT(p)); break;
    case 16: hipLaunchKernelGGL((group_quant_kernel<DT, KC, 16>), g, dim3(GT), 0, s, RNQ_GROUP_HOT(p)); break;
    case 32: hipLaunchKernelGGL((group_quant_kernel<DT, KC, 32>), g, dim3(GT), 0, s, RNQ_GROUP_HOT(p)); break;
    case 64: hipLaunchKernelGGL((group_quant_kernel<DT, KC, 64>), g, dim3(GT), 0, s, RNQ_GROUP_HOT(p)); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class DT>
static hipError_t launch_dt(const GroupQuantParams& p, dim3 g, hipStream_t s) {
  const uint32_t nch = p.N / 8;
  if (nch <= GT) return launch_kc<DT, 1>(p, g, s);
  if (nch <= 2 * GT) return launch_kc<DT, 2>(p, g, s);
  if (nch <= 4 * GT) return launch_kc<DT, 4>(p, g, s);
  if (nch <= 8 * GT) return launch_kc<DT, 8>(p, g, s);
  return hipErrorInvalidValue;
}

template <class DT, bool POS>
static hipError_t launch_norm_rope_dt(const GroupQuantParams& p, dim3 g, hipStream_t s) {
  const uint32_t nch = p.N / 8;
  if (nch <= GT)
    hipLaunchKernelGGL((group_quant_kernel<DT, 1, 0, false, POS>), g, dim3(GT), 0, s, RNQ_GROUP_HOT(p));
  else if (nch <= 2 * GT)
    hipLaunchKernelGGL((group_quant_kernel<DT, 2, 0, false, POS>), g, dim3(GT), 0, s, RNQ_GROUP_HOT(p));
  else if (nch <= 4 * GT)
    hipLaunchKernelGGL((group_quant_kernel<DT, 4, 0, false, POS>), g, dim3(GT), 0, s, RNQ_GROUP_HOT(p));
  else if (nch <= 8 * GT)
    hipLaunchKernelGGL((group_quant_kernel<DT, 8, 0, false, POS>), g, dim3(GT), 0, s, RNQ_GROUP_HOT(p));
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// the row -> token division, a token stride for every call, and the table's
// row count (position-indexed: the caller's; otherwise one row per token)
static void set_rows(GroupQuantParams& p) {
  div_magic_for(p.rows_per_token, p.div_magic, p.div_shift);
  if (p.xs == 0) p.xs = (uint64_t)p.rows_per_token * p.N;
  if (p.positions == nullptr) p.max_pos = (p.M - 1) / p.rows_per_token + 1;
}

hipError_t launch_wide_norm_rope(GroupQuantParams p, bool bf16, hipStream_t stream) {
  if (p.M == 0 || p.N == 0) return hipSuccess;
  if (p.rope > kMaxRope || p.y == nullptr || p.rows_per_token == 0) return hipErrorInvalidValue;
  p.group_size = 0;
  set_rows(p);
  const dim3 grid(p.M);
  if (p.positions != nullptr)
    return bf16 ? launch_norm_rope_dt<BF16, true>(p, grid, stream) : launch_norm_rope_dt<F16, true>(p, grid, stream);
  return bf16 ? launch_norm_rope_dt<BF16, false>(p, grid, stream) : launch_norm_rope_dt<F16, false>(p, grid, stream);
}

hipError_t launch_group_quant(GroupQuantParams p, bool bf16, hipStream_t stream) {
  if (p.M == 0 || p.N == 0) return hipSuccess;
  if (p.rope > kMaxRope || p.rows_per_token == 0 || p.positions != nullptr) return hipErrorInvalidValue;
  set_rows(p);
  p.rcp_fp8_max = 1.0f / p.fp8_max;
  p.scale_floor = 1e-4f / p.fp8_max;
  p.scale_by_rcp = p.fp8_max >= 1.0f ? 1u : 0u;
  p.clamp = fp8_clamp_needed(p.fp8_max) ? 1u : 0u;
  const dim3 grid(p.M);
  return bf16 ? launch_dt<BF16>(p, grid, stream) : launch_dt<F16>(p, grid, stream);
}

}  // namespace rnq
