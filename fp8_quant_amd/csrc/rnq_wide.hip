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
// a second kernel adds them per column in a fixed order (see dw_reduce_kernel).
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

// Backward. BT threads; thread i owns chunks i, i+BT, ... (KC of them). Loads
// of the next RING-1 rows are kept in flight ahead of the row being computed.
template <class DT, int KC, int BT>
__global__ __launch_bounds__(BT) void wide_bwd_kernel(WideBwdParams p) {
  constexpr int BW = BT / 64;
  __shared__ double part_d[2][BW];
  __shared__ float part_f[2][BW];
  const uint32_t tid = threadIdx.x;
  const uint32_t wave = tid >> 6;
  const uint32_t nch = p.N / 8;
  const uint32_t r0 = blockIdx.x * p.rows_per_block;
  const uint32_t r1 = min(r0 + p.rows_per_block, p.M);

  float w[KC][8], dw[KC][8];
  bool ok[KC];
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    const uint32_t c = tid + BT * k;
    ok[k] = c < nch;
    if (ok[k]) unpack8<DT>(*(const uint4*)(p.w + 8 * (size_t)c), w[k]);
    else for (int i = 0; i < 8; ++i) w[k][i] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) dw[k][i] = 0.f;
  }

  auto load_row = [&](uint32_t row, uint4* xs, uint4* gs) {
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      xs[k] = make_uint4(0, 0, 0, 0);
      gs[k] = make_uint4(0, 0, 0, 0);
      if (row < r1 && ok[k]) {
        const size_t off = (size_t)row * p.N + 8 * (size_t)(tid + BT * k);
        xs[k] = load_stream16(p.x + off);
        gs[k] = load_stream16(p.gy + off);
      }
    }
  };

  constexpr int RING = KC >= 4 ? 2 : (KC == 2 ? 3 : 4);  // bounded by registers
  uint4 xr[RING][KC], gr[RING][KC];
#pragma unroll
  for (int j = 0; j < RING - 1; ++j) load_row(r0 + j, xr[j], gr[j]);

  uint32_t parity = 0;
  for (uint32_t row = r0; row < r1; ++row) {
    load_row(row + RING - 1, xr[RING - 1], gr[RING - 1]);
    uint4 (&x0)[KC] = xr[0];
    uint4 (&g0)[KC] = gr[0];

    float xf[KC][8], gf[KC][8];
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      unpack8<DT>(x0[k], xf[k]);
      unpack8<DT>(g0[k], gf[k]);
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
      for (int v = 1; v < BW; ++v) tot += part_d[parity][v];
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
    for (int v = 1; v < BW; ++v) tot += part_f[parity][v];
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
      const uint4 v = pack8<DT>(o);
      __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, (u32x4*)(p.gx + (size_t)row * p.N + 8 * (size_t)(tid + BT * k)));
    }
#pragma unroll
    for (int j = 0; j < RING - 1; ++j)
#pragma unroll
      for (int k = 0; k < KC; ++k) { xr[j][k] = xr[j + 1][k]; gr[j][k] = gr[j + 1][k]; }
  }

#pragma unroll
  for (int k = 0; k < KC; ++k) {
    if (!ok[k]) continue;
    float* dst = p.partial + (size_t)blockIdx.x * p.N + 8 * (size_t)(tid + BT * k);
    *(float4*)dst = make_float4(dw[k][0], dw[k][1], dw[k][2], dw[k][3]);
    *(float4*)(dst + 4) = make_float4(dw[k][4], dw[k][5], dw[k][6], dw[k][7]);
  }
}

// grad_w[j] = sum over b of partial[b, j] in a fixed order. A workgroup owns 64
// columns (16 float4 column groups); its 16 row phases each add partial rows
// phase, phase+16, ... in ascending order, then phase sums are added in
// ascending phase order.
constexpr int RQ = 16;  // column float4 groups per workgroup
constexpr int RP = 16;  // row phases
__global__ __launch_bounds__(RQ * RP) void dw_reduce_kernel(const float* __restrict__ partial, float* __restrict__ gw,
                                                           uint32_t blocks, uint32_t N) {
  __shared__ float4 acc_s[RP][RQ];
  const uint32_t cq = threadIdx.x % RQ, ph = threadIdx.x / RQ;
  const uint32_t c4 = blockIdx.x * RQ + cq;  // float4 column group
  const bool ok = 4 * c4 < N;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (ok) {
    for (uint32_t b = ph; b < blocks; b += RP) {
      const float4 v = *(const float4*)(partial + (size_t)b * N + 4 * (size_t)c4);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
  }
  acc_s[ph][cq] = acc;
  __syncthreads();
  if (ph == 0 && ok) {
    float4 t = acc_s[0][cq];
#pragma unroll
    for (int i = 1; i < RP; ++i) {
      const float4 v = acc_s[i][cq];
      t.x += v.x; t.y += v.y; t.z += v.z; t.w += v.w;
    }
    *(float4*)(gw + 4 * (size_t)c4) = t;
  }
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

// 512 threads for rows wider than 2048 (1, 2 or 4 chunks per lane), 256 below (1 chunk).
template <class DT>
static hipError_t bwd_kc(const WideBwdParams& p, int kc, dim3 g, hipStream_t s) {
  if (p.N <= 2048) {
    hipLaunchKernelGGL((wide_bwd_kernel<DT, 1, 256>), g, dim3(256), 0, s, p);
    return hipGetLastError();
  }
  switch (kc) {
    case 1: hipLaunchKernelGGL((wide_bwd_kernel<DT, 1, 512>), g, dim3(512), 0, s, p); break;
    case 2: hipLaunchKernelGGL((wide_bwd_kernel<DT, 2, 512>), g, dim3(512), 0, s, p); break;
    case 4: hipLaunchKernelGGL((wide_bwd_kernel<DT, 4, 512>), g, dim3(512), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

static int chunks_per_lane(uint32_t N, uint32_t threads) {
  const uint32_t nch = N / 8;
  int kc = 1;
  while ((uint32_t)kc * threads < nch) kc *= 2;
  return kc;  // 1, 2, 4 or 8 for N <= 16384 (8 only with 256 threads)
}

hipError_t launch_wide_fwd(const WideFwdParams& p, bool bf16, hipStream_t stream) {
  const int kc = chunks_per_lane(p.N, WT);
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
  dim3 grid(p.blocks);
  const int kc = chunks_per_lane(p.N, p.N > 2048 ? 512 : 256);
  hipError_t e = bf16 ? bwd_kc<BF16>(p, kc, grid, stream) : bwd_kc<F16>(p, kc, grid, stream);
  if (e != hipSuccess) return e;
  const uint32_t cols4 = p.N / 4;
  hipLaunchKernelGGL(dw_reduce_kernel, dim3((cols4 + RQ - 1) / RQ), dim3(RQ * RP), 0, stream,
                     (const float*)p.partial, p.gw, p.blocks, p.N);
  return hipGetLastError();
}

}  // namespace rnq
