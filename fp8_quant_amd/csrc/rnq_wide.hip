// Wide-row RMSNorm forward and backward (rows of up to 16384 elements).
//
// Operation: tilelang-tutorial chapter 17 page "rmsnorm_tl.py" - the RMSNorm
// forward kernel (fp32 accumulation, y = x * rsqrt(mean(x^2) + eps) * w) and
// RMSNormTileLang.backward:
//   xn = x * rstd, g = grad_y * w,
//   grad_x = rstd * (g - xn * mean(g * xn)),  grad_w = sum over rows of grad_y * xn.
//
// Mapping: one 256-thread workgroup (4 waves) per row at a time; thread i owns
// 16-byte chunks i, i+256, ... of the row (KC chunks). Row sums: per-lane
// partials, a DPP/shuffle butterfly over the wave, then the four wave totals
// are added in ascending wave order through LDS (double-buffered by row
// parity so one barrier per reduction suffices). The next row's loads are
// issued before the current row is reduced.
//
// Backward grad_w is deterministic: workgroup b owns a fixed contiguous range
// of rows and accumulates grad_y * xn for its columns in registers, in row
// order; the per-workgroup partials go to the caller's workspace [blocks, N];
// a second kernel adds them per column in ascending workgroup order.
#include "rnq_device.h"
#include "rnq_launch.h"

namespace rnq {

constexpr int WT = 256;  // threads per workgroup
constexpr int WW = WT / 64;

template <class DT, int KC>
__global__ __launch_bounds__(WT) void wide_fwd_kernel(WideFwdParams p) {
  __shared__ double part[2][WW];
  const uint32_t tid = threadIdx.x;
  const uint32_t wave = tid >> 6;
  const uint32_t nch = p.N / 8;
  uint32_t row = blockIdx.x;
  if (row >= p.M) return;

  float w[KC][8];
  bool ok[KC];
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    const uint32_t c = tid + WT * k;
    ok[k] = c < nch;
    if (ok[k]) unpack8<DT>(*(const uint4*)(p.w + 8 * (size_t)c), w[k]);
    else for (int i = 0; i < 8; ++i) w[k][i] = 0.f;
  }

  uint4 x[KC];
#pragma unroll
  for (int k = 0; k < KC; ++k)
    x[k] = ok[k] ? *(const uint4*)(p.x + (size_t)row * p.N + 8 * (size_t)(tid + WT * k)) : make_uint4(0, 0, 0, 0);

  uint32_t parity = 0;
  for (; row < p.M; row += gridDim.x) {
    const uint32_t nrow = row + gridDim.x;
    const bool has_next = nrow < p.M;
    uint4 nx[KC];
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      nx[k] = x[k];
      if (has_next && ok[k]) nx[k] = *(const uint4*)(p.x + (size_t)nrow * p.N + 8 * (size_t)(tid + WT * k));
    }

    float xf[KC][8];
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      unpack8<DT>(x[k], xf[k]);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc = __builtin_fma((double)xf[k][i], (double)xf[k][i], acc);
    }
    acc = group_sum<64>(acc);
    if ((tid & 63) == 0) part[parity][wave] = acc;
    __syncthreads();
    double tot = part[parity][0];
#pragma unroll
    for (int v = 1; v < WW; ++v) tot += part[parity][v];
    parity ^= 1u;

    const float ssq = (float)tot;
    const float ms = ssq / (float)p.N;
    const float rstd = rstd_of(ms + p.eps);
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      if (!ok[k]) continue;
      float o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = (xf[k][i] * rstd) * w[k][i];
      *(uint4*)(p.y + (size_t)row * p.N + 8 * (size_t)(tid + WT * k)) = pack8<DT>(o);
    }
    if (p.rstd != nullptr && tid == 0) p.rstd[row] = rstd;
#pragma unroll
    for (int k = 0; k < KC; ++k) x[k] = nx[k];
  }
}

template <class DT, int KC>
__global__ __launch_bounds__(WT) void wide_bwd_kernel(WideBwdParams p) {
  __shared__ double part_d[2][WW];
  __shared__ float part_f[2][WW];
  const uint32_t tid = threadIdx.x;
  const uint32_t wave = tid >> 6;
  const uint32_t nch = p.N / 8;
  const uint32_t r0 = blockIdx.x * p.rows_per_block;
  const uint32_t r1 = min(r0 + p.rows_per_block, p.M);

  float w[KC][8], dw[KC][8];
  bool ok[KC];
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    const uint32_t c = tid + WT * k;
    ok[k] = c < nch;
    if (ok[k]) unpack8<DT>(*(const uint4*)(p.w + 8 * (size_t)c), w[k]);
    else for (int i = 0; i < 8; ++i) w[k][i] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) dw[k][i] = 0.f;
  }

  uint4 x[KC], gy[KC];
  if (r0 < r1) {
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      const size_t off = (size_t)r0 * p.N + 8 * (size_t)(tid + WT * k);
      x[k] = ok[k] ? *(const uint4*)(p.x + off) : make_uint4(0, 0, 0, 0);
      gy[k] = ok[k] ? *(const uint4*)(p.gy + off) : make_uint4(0, 0, 0, 0);
    }
  }

  uint32_t parity = 0;
  for (uint32_t row = r0; row < r1; ++row) {
    const bool has_next = row + 1 < r1;
    uint4 nx[KC], ng[KC];
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      nx[k] = x[k];
      ng[k] = gy[k];
      if (has_next && ok[k]) {
        const size_t off = (size_t)(row + 1) * p.N + 8 * (size_t)(tid + WT * k);
        nx[k] = *(const uint4*)(p.x + off);
        ng[k] = *(const uint4*)(p.gy + off);
      }
    }

    float xf[KC][8], gf[KC][8];
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      unpack8<DT>(x[k], xf[k]);
      unpack8<DT>(gy[k], gf[k]);
    }

    float rstd;
    if (p.rstd != nullptr) {
      rstd = p.rstd[row];
    } else {
      double acc = 0.0;
#pragma unroll
      for (int k = 0; k < KC; ++k)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc = __builtin_fma((double)xf[k][i], (double)xf[k][i], acc);
      acc = group_sum<64>(acc);
      if ((tid & 63) == 0) part_d[parity][wave] = acc;
      __syncthreads();
      double tot = part_d[parity][0];
#pragma unroll
      for (int v = 1; v < WW; ++v) tot += part_d[parity][v];
      rstd = rstd_of((float)tot / (float)p.N + p.eps);
    }

    // C = mean(g * xn): lane-sequential fp32 sum, wave butterfly, waves in ascending order
    float xn[KC][8], g[KC][8];
    float dot = 0.f;
#pragma unroll
    for (int k = 0; k < KC; ++k)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        xn[k][i] = xf[k][i] * rstd;
        g[k][i] = gf[k][i] * w[k][i];
        dot += g[k][i] * xn[k][i];
      }
    dot = group_sum<64>(dot);
    if ((tid & 63) == 0) part_f[parity][wave] = dot;
    __syncthreads();
    float tot = part_f[parity][0];
#pragma unroll
    for (int v = 1; v < WW; ++v) tot += part_f[parity][v];
    parity ^= 1u;
    const float C = tot / (float)p.N;

#pragma unroll
    for (int k = 0; k < KC; ++k) {
      if (!ok[k]) continue;
      float o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        o[i] = rstd * (g[k][i] - xn[k][i] * C);
        dw[k][i] += gf[k][i] * xn[k][i];
      }
      *(uint4*)(p.gx + (size_t)row * p.N + 8 * (size_t)(tid + WT * k)) = pack8<DT>(o);
    }
#pragma unroll
    for (int k = 0; k < KC; ++k) { x[k] = nx[k]; gy[k] = ng[k]; }
  }

#pragma unroll
  for (int k = 0; k < KC; ++k) {
    if (!ok[k]) continue;
    float* dst = p.partial + (size_t)blockIdx.x * p.N + 8 * (size_t)(tid + WT * k);
    *(float4*)dst = make_float4(dw[k][0], dw[k][1], dw[k][2], dw[k][3]);
    *(float4*)(dst + 4) = make_float4(dw[k][4], dw[k][5], dw[k][6], dw[k][7]);
  }
}

// grad_w[j] = sum over b ascending of partial[b, j]; one thread per 4 columns.
__global__ __launch_bounds__(WT) void dw_reduce_kernel(const float* __restrict__ partial, float* __restrict__ gw,
                                                       uint32_t blocks, uint32_t N) {
  const uint32_t c4 = blockIdx.x * WT + threadIdx.x;
  if (4 * c4 >= N) return;
  float4 acc = *(const float4*)(partial + 4 * (size_t)c4);
  uint32_t b = 1;
  for (; b + 8 <= blocks; b += 8) {
    float4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = *(const float4*)(partial + (size_t)(b + i) * N + 4 * (size_t)c4);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      acc.x += v[i].x; acc.y += v[i].y; acc.z += v[i].z; acc.w += v[i].w;
    }
  }
  for (; b < blocks; ++b) {
    const float4 v = *(const float4*)(partial + (size_t)b * N + 4 * (size_t)c4);
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  *(float4*)(gw + 4 * (size_t)c4) = acc;
}

// ----------------------------------------------------------------- launchers

template <class DT>
static hipError_t fwd_kc(const WideFwdParams& p, int kc, dim3 g, dim3 b, hipStream_t s) {
  switch (kc) {
    case 1: hipLaunchKernelGGL((wide_fwd_kernel<DT, 1>), g, b, 0, s, p); break;
    case 2: hipLaunchKernelGGL((wide_fwd_kernel<DT, 2>), g, b, 0, s, p); break;
    case 4: hipLaunchKernelGGL((wide_fwd_kernel<DT, 4>), g, b, 0, s, p); break;
    case 8: hipLaunchKernelGGL((wide_fwd_kernel<DT, 8>), g, b, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class DT>
static hipError_t bwd_kc(const WideBwdParams& p, int kc, dim3 g, dim3 b, hipStream_t s) {
  switch (kc) {
    case 1: hipLaunchKernelGGL((wide_bwd_kernel<DT, 1>), g, b, 0, s, p); break;
    case 2: hipLaunchKernelGGL((wide_bwd_kernel<DT, 2>), g, b, 0, s, p); break;
    case 4: hipLaunchKernelGGL((wide_bwd_kernel<DT, 4>), g, b, 0, s, p); break;
    case 8: hipLaunchKernelGGL((wide_bwd_kernel<DT, 8>), g, b, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

static int chunks_per_lane(uint32_t N) {
  const uint32_t nch = N / 8;
  int kc = 1;
  while ((uint32_t)(kc * WT) < nch) kc *= 2;
  return kc;  // 1, 2, 4 or 8 for N <= 16384
}

hipError_t launch_wide_fwd(const WideFwdParams& p, bool bf16, hipStream_t stream) {
  const int kc = chunks_per_lane(p.N);
  uint32_t blocks = 2048;  // 8 workgroups per CU; each walks rows with a grid stride
  if (blocks > p.M) blocks = p.M;
  dim3 grid(blocks), block(WT);
  return bf16 ? fwd_kc<BF16>(p, kc, grid, block, stream) : fwd_kc<F16>(p, kc, grid, block, stream);
}

uint32_t bwd_blocks(int64_t M, int64_t N) {
  (void)N;
  const int64_t target = 256;
  return (uint32_t)(M < target ? (M > 0 ? M : 1) : target);
}

hipError_t launch_wide_bwd(const WideBwdParams& p, bool bf16, hipStream_t stream) {
  const int kc = chunks_per_lane(p.N);
  dim3 grid(p.blocks), block(WT);
  hipError_t e = bf16 ? bwd_kc<BF16>(p, kc, grid, block, stream) : bwd_kc<F16>(p, kc, grid, block, stream);
  if (e != hipSuccess) return e;
  const uint32_t threads = (p.N / 4 + WT - 1) / WT;
  hipLaunchKernelGGL(dw_reduce_kernel, dim3(threads), dim3(WT), 0, stream, (const float*)p.partial, p.gw, p.blocks, p.N);
  return hipGetLastError();
}

}  // namespace rnq
