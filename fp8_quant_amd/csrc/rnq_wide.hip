// Wide-row RMSNorm forward and backward (rows of up to 16384 elements).
//
// Operation: tilelang-tutorial chapter 17 page "rmsnorm_tl.py" - the RMSNorm
// forward kernel (fp32 accumulation, y = x * rsqrt(mean(x^2) + eps) * w) and
// RMSNormTileLang.backward:
//   xn = x * rstd, g = grad_y * w,
//   grad_x = rstd * (g - xn * mean(g * xn)),  grad_w = sum over rows of grad_y * xn.
//
// Mapping: a workgroup (256 threads, or 512 for the backward of wide rows)
// holds whole rows; thread i owns 16-byte chunks i, i+256, ... of a row (KC
// chunks). Row sums: per-lane partials, a DPP/shuffle butterfly over the
// wave, then the wave totals are added in ascending wave order through LDS.
//
// Backward grad_w is deterministic: workgroup b owns a fixed contiguous range
// of rows and accumulates grad_y * xn for its columns in registers, in row
// order; the per-workgroup partials go to the caller's workspace [blocks, N];
// a second kernel adds them per column in a fixed order (dw_reduce_kernel).
//
// The backward of RMSNorm followed by the partial NeoX RoPE (chapter 13 fusion
// page's rotation of the last R columns) first takes grad_y back through the
// rotation: the transposed rotation (g_lo c + g_hi s, g_hi c - g_lo s) of each
// pair p <-> p + R/2 of the tail, in fp32 (the casts to the input dtype count
// as identities, as in the chapter 17 backward). A pair's two chunks belong to
// different threads here, so each row's grad_y tail and its cos/sin row pass
// through LDS, under the barrier the row sums take anyway.
#include "rnq_device.h"
#include "rnq_launch.h"

namespace rnq {

constexpr int WT = 256;  // threads per workgroup
constexpr int WW = WT / 64;

// Forward. Workgroup b normalises rows b*RB .. b*RB + RB - 1 (a last partial
// group repeats row M - 1, writing identical bytes). All its loads are issued
// at once (buffer accesses, lanes past the row's end out of the descriptor's
// range); one barrier for the RB rows' sums of squares.
// (its parameters, 11 dwords, are scalar arguments: gfx950 preloads them, so
// a workgroup issues its loads without first loading its kernel arguments)
template <class DT, int KC, int RB>
__global__ __launch_bounds__(WT) void wide_fwd_kernel(const uint16_t* x_in, const uint16_t* w_in, uint16_t* y_out,
                                                      float* rstd_out, uint32_t M, uint32_t N, float eps) {
  const WideFwdParams p{x_in, w_in, y_out, rstd_out, M, N, eps};
  constexpr uint32_t kOutOfRange = 0x80000000u;
  __shared__ double part[RB][WW];
  const uint32_t tid = threadIdx.x;
  const uint32_t wave = tid >> 6;
  const uint32_t nch = p.N / 8;
  const uint32_t row_bytes = 2u * p.N;
  const uint32_t first = blockIdx.x * RB;

  uint32_t off[KC];
  bool ok[KC];
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    const uint32_t c = tid + WT * k;
    ok[k] = c < nch;
    off[k] = ok[k] ? 16u * c : kOutOfRange;
  }
  uint4 x[RB][KC];
#pragma unroll
  for (int j = 0; j < RB; ++j) {
    const rsrc_t rx = make_rsrc(p.x + (size_t)min(first + (uint32_t)j, p.M - 1) * p.N, row_bytes);
#pragma unroll
    for (int k = 0; k < KC; ++k) x[j][k] = buf_load16_nt(rx, off[k]);
  }
  uint4 wr[KC];
  const rsrc_t rw = make_rsrc(p.w, row_bytes);
#pragma unroll
  for (int k = 0; k < KC; ++k) wr[k] = buf_load16(rw, off[k]);

#pragma unroll
  for (int j = 0; j < RB; ++j) {
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      float xf[8];
      unpack8<DT>(x[j][k], xf);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc = __builtin_fma((double)xf[i], (double)xf[i], acc);
    }
    acc = group_sum<64>(acc);
    if ((tid & 63) == 0) part[j][wave] = acc;
  }
  lds_barrier();

#pragma unroll
  for (int j = 0; j < RB; ++j) {
    double tot = part[j][0];
#pragma unroll
    for (int v = 1; v < WW; ++v) tot += part[j][v];
    const float ssq = (float)tot;
    const float ms = ssq / (float)p.N;
    const float rstd = rstd_of(ms + p.eps);
    const uint32_t row = min(first + (uint32_t)j, p.M - 1);
    const rsrc_t ry = make_rsrc(p.y + (size_t)row * p.N, row_bytes);
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      float xf[8], w[8], o[8];
      unpack8<DT>(x[j][k], xf);
      unpack8<DT>(wr[k], w);
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = (xf[i] * rstd) * w[i];
      // (device-scope stores: 12.95 -> 12.81 us against nontemporal ones at
      // 4096 x 4096, builds alternated in one process, outputs rotated past
      // the Infinity Cache)
      buf_store16_dev(ry, off[k], pack8<DT>(o));
    }
    if (p.rstd != nullptr && tid == 0) p.rstd[row] = rstd;
  }
}

// Backward. BT threads; thread i owns chunks i, i+BT, ... (KC of them). The
// workgroup walks its rows in batches of RB: one barrier per batch for each of
// the two row reductions (sum of squares when rstd is recomputed, then
// mean(g * xn)), and the next batch's loads are in flight while a batch is
// computed. Every global access is a buffer access with a row-uniform
// descriptor; lanes past the row's end use offsets outside the descriptor's
// range (dropped by the hardware), and a batch that runs past the workgroup's
// last row re-reads that row and writes its identical grad_x again, so no
// access in the loop is conditional and the in-order memory counter is waited
// on precisely. grad_w partials accumulate in ascending row order.
constexpr uint32_t kMaxBwdRope = 1024;

template <class DT, int KC, int BT, int RB, bool SAVED, bool ROPE = false>
__global__ __launch_bounds__(BT) void wide_bwd_kernel(WideBwdParams p) {
  constexpr int BW = BT / 64;
  constexpr uint32_t kOutOfRange = 0x80000000u;
  // table values a thread loads per row (cos then sin of the row's table row,
  // R <= 1024 values in all)
  constexpr int TPT = ROPE ? (int)((kMaxBwdRope + BT - 1) / BT) : 1;
  __shared__ double part_d[2][RB][BW];
  __shared__ float part_f[2][RB][BW];
  // RoPE: each row's cos/sin values and its grad_y tail (16-bit values), by ring parity
  __shared__ float tab_s[ROPE ? 2 : 1][RB][ROPE ? kMaxBwdRope : 1];
  __shared__ uint4 gt_s[ROPE ? 2 : 1][RB][ROPE ? kMaxBwdRope / 8 : 1];
  const uint32_t tid = threadIdx.x;
  const uint32_t wave = tid >> 6;
  const uint32_t nch = p.N / 8;
  const uint32_t r0 = blockIdx.x * p.rows_per_block;
  // the partition gives every block rows (r0 < r1); a block without rows would
  // run no batch and write a zero partial row. (No early exit: a branch here
  // would come before the kernel-argument loads the first batch needs, and
  // the compiler issues none past a branch.)
  const uint32_t r1 = min(r0 + p.rows_per_block, p.M);
  const uint32_t nrows = r1 > r0 ? r1 - r0 : 0u;
  const uint32_t row_bytes = 2u * p.N;

  // the weight row (16-bit values, N * 2 bytes, and one spare 16-byte slot),
  // read where it is used
  extern __shared__ uint4 w_s[];
  float dw[KC][8];
  bool ok[KC];
  uint32_t off[KC];  // byte offset of the lane's chunk k in a row (out of range past the end)
  uint4 wcs[KC];
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    const uint32_t c = tid + BT * k;
    ok[k] = c < nch;
    off[k] = ok[k] ? 16u * c : kOutOfRange;
    wcs[k] = buf_load16(make_rsrc(p.w, row_bytes), off[k]);
#pragma unroll
    for (int i = 0; i < 8; ++i) dw[k][i] = 0.f;
  }
  auto wk = [&](int k, float* wf) {  // this lane's 8 weights of chunk k (zeros past the row's end)
    const uint4 wc = w_s[ok[k] ? tid + BT * k : 0u];
    unpack8<DT>(ok[k] ? wc : make_uint4(0, 0, 0, 0), wf);
  };

  // RoPE geometry: R = p.rope columns at the end of the row, chunks t0 .. nch - 1,
  // hc chunks per half; thread-owned table values e = tid + BT m (cos for e < R/2,
  // then sin), out of the table's range past R
  const uint32_t R = ROPE ? p.rope : 0u, half = R / 2;
  const uint32_t t0 = nch - R / 8, hc = R / 16;
  const rsrc_t rcos = make_rsrc(p.cos, ROPE ? p.table_bytes : 0u);
  const rsrc_t rsin = make_rsrc(p.sin, ROPE ? p.table_bytes : 0u);
  auto table_off = [&](uint32_t row, int m, bool& is_sin) {
    const uint32_t e = tid + BT * m;
    is_sin = e >= half;
    if (e >= R) return kOutOfRange;
    const uint32_t t = (uint32_t)(((uint64_t)row * p.div_magic) >> p.div_shift);
    return 4u * (t * half + (is_sin ? e - half : e));
  };

  auto load_batch = [&](uint32_t first, uint4 (&xs)[RB][KC], uint4 (&gs)[RB][KC], float (&ts)[RB][TPT]) {
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      const size_t row = min(first + (uint32_t)j, r1 - 1);
      const rsrc_t rx = make_rsrc(p.x + row * p.N, row_bytes);
      const rsrc_t rg = make_rsrc(p.gy + row * p.N, row_bytes);
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        xs[j][k] = buf_load16_nt(rx, off[k]);
        gs[j][k] = buf_load16_nt(rg, off[k]);
      }
      if constexpr (ROPE) {
#pragma unroll
        for (int m = 0; m < TPT; ++m) {
          bool is_sin;
          const uint32_t o = table_off((uint32_t)row, m, is_sin);
          // (both loads go out; the unused one is out of range and reads nothing)
          const float c = buf_load4f(rcos, is_sin ? kOutOfRange : o);
          const float sv = buf_load4f(rsin, is_sin ? o : kOutOfRange);
          ts[j][m] = is_sin ? sv : c;
        }
      }
    }
  };

  uint4 xr[2][RB][KC], gr[2][RB][KC];
  float tr[2][RB][TPT];
  load_batch(r0, xr[0], gr[0], tr[0]);
  // the weights go to LDS once the first batch is in flight too (they were
  // loaded first, so waiting for them waits for no row); lanes past the row
  // store their zeros in the spare slot: a store under a branch would let the
  // compiler sink the weight load under it, behind the barrier
#pragma unroll
  for (int k = 0; k < KC; ++k) w_s[ok[k] ? tid + BT * k : nch] = wcs[k];
  lds_barrier();
  uint32_t parity = 0;

  // one batch; cur / nxt are compile-time ring slots
  auto batch = [&](uint32_t first, uint4 (&xc)[RB][KC], uint4 (&gc)[RB][KC], float (&tc)[RB][TPT],
                   uint4 (&xn_)[RB][KC], uint4 (&gn)[RB][KC], float (&tn)[RB][TPT]) {
    load_batch(first + RB, xn_, gn, tn);
    if constexpr (ROPE) {
      // this batch's table rows and grad_y tails into LDS (read after the next barrier)
#pragma unroll
      for (int j = 0; j < RB; ++j) {
#pragma unroll
        for (int m = 0; m < TPT; ++m)
          if (tid + BT * m < R) tab_s[parity][j][tid + BT * m] = tc[j][m];
#pragma unroll
        for (int k = 0; k < KC; ++k)
          if (ok[k] && tid + BT * k >= t0) gt_s[parity][j][tid + BT * k - t0] = gc[j][k];
      }
    }
    float rstd[RB];
    if constexpr (SAVED) {
#pragma unroll
      for (int j = 0; j < RB; ++j) rstd[j] = p.rstd[min(first + (uint32_t)j, r1 - 1)];
      if constexpr (ROPE) lds_barrier();
    } else {
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        double acc = 0.0;
#pragma unroll
        for (int k = 0; k < KC; ++k) {
          float xf[8];
          unpack8<DT>(xc[j][k], xf);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc = __builtin_fma((double)xf[i], (double)xf[i], acc);
        }
        acc = group_sum<64>(acc);
        if ((tid & 63) == 0) part_d[parity][j][wave] = acc;
      }
      lds_barrier();
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        double tot = part_d[parity][j][0];
#pragma unroll
        for (int v = 1; v < BW; ++v) tot += part_d[parity][j][v];
        rstd[j] = rstd_of((float)tot / (float)p.N + p.eps);
      }
    }

    // RoPE: grad_y through the transposed rotation on the tail (fp32), kept in registers
    float gnr[ROPE ? RB : 1][ROPE ? KC : 1][8];
    if constexpr (ROPE) {
#pragma unroll
      for (int j = 0; j < RB; ++j)
#pragma unroll
        for (int k = 0; k < KC; ++k) {
          unpack8<DT>(gc[j][k], gnr[j][k]);
          const uint32_t c = tid + BT * k;
          if (ok[k] && c >= t0) {
            const uint32_t tj = c - t0;
            const bool lo_half = tj < hc;
            const uint32_t pj = lo_half ? tj : tj - hc;  // pair columns 8 pj .. 8 pj + 7 of the half
            float pf[8];
            unpack8<DT>(gt_s[parity][j][lo_half ? tj + hc : tj - hc], pf);
            const float* cs = tab_s[parity][j] + 8 * pj;
            const float* sn = tab_s[parity][j] + half + 8 * pj;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const float own = gnr[j][k][i] * cs[i];
              const float other = pf[i] * sn[i];
              gnr[j][k][i] = lo_half ? own + other : own - other;
            }
          }
        }
    }
    auto grad = [&](int j, int k, float* gf) {  // this lane's 8 output-gradient values of chunk k, row j
      if constexpr (ROPE) {
#pragma unroll
        for (int i = 0; i < 8; ++i) gf[i] = gnr[j][k][i];
      } else {
        unpack8<DT>(gc[j][k], gf);
      }
    };

    // C = mean(g * xn): lane-sequential fp32 sum, wave butterfly, waves in ascending order
    float C[RB];
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        float xf[8], gf[8], w[8];
        unpack8<DT>(xc[j][k], xf);
        grad(j, k, gf);
        wk(k, w);
#pragma unroll
        for (int i = 0; i < 8; ++i) dot += (gf[i] * w[i]) * (xf[i] * rstd[j]);
      }
      dot = group_sum<64>(dot);
      if ((tid & 63) == 0) part_f[parity][j][wave] = dot;
    }
    lds_barrier();
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      float tot = part_f[parity][j][0];
#pragma unroll
      for (int v = 1; v < BW; ++v) tot += part_f[parity][j][v];
      C[j] = tot / (float)p.N;
    }
    parity ^= 1u;

#pragma unroll
    for (int j = 0; j < RB; ++j) {
      const uint32_t row = min(first + (uint32_t)j, r1 - 1);
      const bool real = first + (uint32_t)j < r1;  // a repeated row adds nothing to grad_w
      const rsrc_t rdx = make_rsrc(p.gx + (size_t)row * p.N, row_bytes);
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        float xf[8], gf[8], o[8], w[8];
        unpack8<DT>(xc[j][k], xf);
        grad(j, k, gf);
        wk(k, w);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float xn = xf[i] * rstd[j];
          o[i] = rstd[j] * ((gf[i] * w[i]) - xn * C[j]);
          if (real) dw[k][i] += gf[i] * xn;
        }
        buf_store16_nt(rdx, off[k], pack8<DT>(o));
      }
    }
  };

  // batches alternate between the two ring slots
  const uint32_t nb = (nrows + RB - 1) / RB;
  uint32_t b = 0;
  for (; b + 2 <= nb; b += 2) {
    batch(r0 + b * RB, xr[0], gr[0], tr[0], xr[1], gr[1], tr[1]);
    batch(r0 + (b + 1) * RB, xr[1], gr[1], tr[1], xr[0], gr[0], tr[0]);
  }
  if (b < nb) batch(r0 + b * RB, xr[0], gr[0], tr[0], xr[1], gr[1], tr[1]);

#pragma unroll
  for (int k = 0; k < KC; ++k) {
    const rsrc_t rp = make_rsrc(p.partial + (size_t)blockIdx.x * p.N, 4u * p.N);
    const uint32_t po = ok[k] ? 2u * off[k] : kOutOfRange;  // 8 floats per chunk
    buf_store16(rp, po, make_uint4(__float_as_uint(dw[k][0]), __float_as_uint(dw[k][1]),
                                   __float_as_uint(dw[k][2]), __float_as_uint(dw[k][3])));
    buf_store16(rp, po + 16u, make_uint4(__float_as_uint(dw[k][4]), __float_as_uint(dw[k][5]),
                                         __float_as_uint(dw[k][6]), __float_as_uint(dw[k][7])));
  }
}

// grad_w[j] = sum over b of partial[b, j] in a fixed order. A workgroup of 8
// waves owns a strip of 32 columns (8 float4 groups) and every partial row:
// lane (r, c) of wave w (r = lane / 8, c = lane % 8) adds the rows
// 64 u + 8 w + r (u = 0, 1, ...) of column group c in ascending u, with 8
// rows' loads in flight; each load instruction reads 8 whole 128-byte row
// segments. Rows past the last are outside the buffer descriptor (zero). The
// 8 row lanes of a column are then added by an xor butterfly, the 8 waves by
// a pairwise tree in LDS.
constexpr int RDW = 8;   // waves per workgroup
constexpr int RU = 8;    // loads in flight per lane
constexpr int RCQ = 8;   // float4 column groups per strip
__global__ __launch_bounds__(64 * RDW) void dw_reduce_kernel(const float* __restrict__ partial, float* __restrict__ gw,
                                                            uint32_t blocks, uint32_t N) {
  __shared__ float4 red[RDW][RCQ];
  const uint32_t tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const uint32_t c = lane % RCQ, r = lane / RCQ;
  const uint32_t c4 = blockIdx.x * RCQ + c;  // float4 column group
  const bool ok = 4 * c4 < N;
  const rsrc_t rp = make_rsrc(partial, 4u * blocks * N);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  // (blocks >= 1, so the first strip of rows is read without a loop test: no
  // branch before the kernel-argument loads it needs)
  uint32_t b0 = 0;
  do {
    float4 v[RU];
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      const uint32_t row = b0 + 64u * u + RCQ * wave + r;
      v[u] = buf_load16f(rp, ok ? 4u * (row * N + 4u * c4) : 0x80000000u);
    }
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      acc.x += v[u].x; acc.y += v[u].y; acc.z += v[u].z; acc.w += v[u].w;
    }
    b0 += 64 * RU;
  } while (b0 < blocks);
#pragma unroll
  for (int m = RCQ; m < 64; m *= 2) {
    acc.x += __shfl_xor(acc.x, m, 64);
    acc.y += __shfl_xor(acc.y, m, 64);
    acc.z += __shfl_xor(acc.z, m, 64);
    acc.w += __shfl_xor(acc.w, m, 64);
  }
  if (r == 0) red[wave][c] = acc;
  lds_barrier();
#pragma unroll
  for (int h = RDW / 2; h >= 1; h /= 2) {
    if (wave < (uint32_t)h && r == 0) {
      const float4 o = red[wave + h][c];
      float4& t = red[wave][c];
      t.x += o.x; t.y += o.y; t.z += o.z; t.w += o.w;
    }
    lds_barrier();
  }
  if (tid < (uint32_t)RCQ && ok) *(float4*)(gw + 4 * (size_t)c4) = red[0][c];
}

// ----------------------------------------------------------------- launchers

#ifndef RNQ_FWD_ROWS
#define RNQ_FWD_ROWS 1
#endif
template <class DT>
static hipError_t fwd_kc(const WideFwdParams& p, int kc, hipStream_t s) {
  constexpr int B = RNQ_FWD_ROWS;
  const dim3 b(WT);
  switch (kc) {
    case 1: hipLaunchKernelGGL((wide_fwd_kernel<DT, 1, B>), dim3((p.M + B - 1) / B), b, 0, s, p.x, p.w, p.y, p.rstd, p.M, p.N, p.eps); break;
    case 2: hipLaunchKernelGGL((wide_fwd_kernel<DT, 2, B>), dim3((p.M + B - 1) / B), b, 0, s, p.x, p.w, p.y, p.rstd, p.M, p.N, p.eps); break;
    case 4: hipLaunchKernelGGL((wide_fwd_kernel<DT, 4, 1>), dim3(p.M), b, 0, s, p.x, p.w, p.y, p.rstd, p.M, p.N, p.eps); break;
    case 8: hipLaunchKernelGGL((wide_fwd_kernel<DT, 8, 1>), dim3(p.M), b, 0, s, p.x, p.w, p.y, p.rstd, p.M, p.N, p.eps); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// 512 threads for rows wider than 2048 (1, 2 or 4 chunks per lane), 256 below
// (1 chunk); rows per batch: 4 chunks' worth of rows per lane.
#ifndef RNQ_BWD_BATCH
#define RNQ_BWD_BATCH 2
#endif
template <class DT, bool SAVED, bool ROPE>
static hipError_t bwd_kc(const WideBwdParams& p, int kc, dim3 g, hipStream_t s) {
  constexpr int B = RNQ_BWD_BATCH;
  const size_t lds = 2 * (size_t)p.N + 16;  // the weight row and a spare 16-byte slot
  if (p.N <= 2048) {
    hipLaunchKernelGGL((wide_bwd_kernel<DT, 1, 256, B, SAVED, ROPE>), g, dim3(256), lds, s, p);
    return hipGetLastError();
  }
  switch (kc) {
    case 1: hipLaunchKernelGGL((wide_bwd_kernel<DT, 1, 512, B, SAVED, ROPE>), g, dim3(512), lds, s, p); break;
    case 2:
      hipLaunchKernelGGL((wide_bwd_kernel<DT, 2, 512, (B > 2 ? B / 2 : 1), SAVED, ROPE>), g, dim3(512), lds, s, p);
      break;
    case 4:
      hipLaunchKernelGGL((wide_bwd_kernel<DT, 4, 512, (B > 4 ? B / 4 : 1), SAVED, ROPE>), g, dim3(512), lds, s, p);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class DT>
static hipError_t bwd_dt(const WideBwdParams& p, int kc, dim3 g, hipStream_t s) {
  const bool saved = p.rstd != nullptr, rope = p.rope > 0;
  if (rope) return saved ? bwd_kc<DT, true, true>(p, kc, g, s) : bwd_kc<DT, false, true>(p, kc, g, s);
  return saved ? bwd_kc<DT, true, false>(p, kc, g, s) : bwd_kc<DT, false, false>(p, kc, g, s);
}

static int chunks_per_lane(uint32_t N, uint32_t threads) {
  const uint32_t nch = N / 8;
  int kc = 1;
  while ((uint32_t)kc * threads < nch) kc *= 2;
  return kc;  // 1, 2, 4 or 8 for N <= 16384 (8 only with 256 threads)
}

hipError_t launch_wide_fwd(const WideFwdParams& p, bool bf16, hipStream_t stream) {
  const int kc = chunks_per_lane(p.N, WT);
  return bf16 ? fwd_kc<BF16>(p, kc, stream) : fwd_kc<F16>(p, kc, stream);
}

// Blocks of contiguous rows, every block owning at least one row: about 256
// (one workgroup per CU), or 512 (two) for the RoPE backward of the
// workgroup-per-row kernel up to 8192 rows. At 4096 x 4096 that kernel's plain
// backward took 24.8 us with 256 blocks against 26.0 with 512 (half the
// partial rows of grad_w to write and read back), its RoPE backward 27.9 us
// with 512 against 30.5 with 256 (its per-batch LDS exchange of the tail needs
// the second workgroup's waves to hide behind). The wave-per-row kernel holds
// one workgroup per CU (its LDS) and takes 256 either way.
uint32_t bwd_blocks(int64_t M, int64_t N, int64_t rope_dim) {
  if (M <= 0) return 1;
  const bool two_per_cu = rope_dim > 0 && M <= 8192 && !row_bwd_fits(N, rope_dim);
  const int64_t target = two_per_cu ? 512 : 256;
  const int64_t rpb = (M + target - 1) / target;
  return (uint32_t)((M + rpb - 1) / rpb);
}

hipError_t launch_wide_bwd(WideBwdParams p, bool bf16, hipStream_t stream) {
  if (row_bwd_fits(p.N, p.rope)) return launch_row_bwd(p, bf16, stream);
  dim3 grid(p.blocks);
  const int kc = chunks_per_lane(p.N, p.N > 2048 ? 512 : 256);
  if (p.rope > kMaxBwdRope || p.rope % 16 != 0 || p.rope > p.N) return hipErrorInvalidValue;
  if (p.rows_per_token == 0) p.rows_per_token = 1;
  // row / rows_per_token by multiply-shift (exact for every row < 2^31)
  div_magic_for(p.rows_per_token, p.div_magic, p.div_shift);
  hipError_t e = bf16 ? bwd_dt<BF16>(p, kc, grid, stream) : bwd_dt<F16>(p, kc, grid, stream);
  if (e != hipSuccess) return e;
  return launch_dw_reduce(p.partial, p.gw, p.blocks, p.N, stream);
}

hipError_t launch_dw_reduce(const float* partial, float* gw, uint32_t blocks, uint32_t N, hipStream_t stream) {
  const uint32_t cols4 = N / 4;
  hipLaunchKernelGGL(dw_reduce_kernel, dim3((cols4 + RCQ - 1) / RCQ), dim3(64 * RDW), 0, stream, partial, gw, blocks, N);
  return hipGetLastError();
}

}  // namespace rnq
