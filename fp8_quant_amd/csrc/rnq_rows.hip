// Row kernel: RMSNorm -> partial NeoX RoPE -> (optional) per-row FP8 e4m3fn.
//
// Operation: tilelang-tutorial chapter 13 fusion page, torch_reference_fused
// and the two fused kernels; chapter 28 case study, the QK-norm prologue
// (rows are (token, head) pairs; every head of a token uses the token's
// cos/sin row; one fp32 scale per row).
//
// Mapping (gfx950, wave64).
//  * A row of D elements is split into D/16 "units" of two 16-byte chunks:
//    a rope unit holds chunk j of the lower half of the rope tail and chunk j
//    of the upper half (so each lane owns both members of its RoPE pairs and
//    no exchange is needed); a plain unit holds two adjacent chunks.
//  * L lanes own a row, UPL units each (lane u owns units u, u+L, ...), so a
//    wave covers G = 64/L rows per "pass". Per-row work (reductions, rstd,
//    scale) runs once per lane for its 16*UPL elements, so a wider share per
//    lane means less of that work per element.
//  * A workgroup (RW waves) owns RW*PPW consecutive passes of the flattened
//    (token, head) rows; every wave issues the global loads of all its passes
//    first, then the workgroup stages the two weight vectors (as fp32) and,
//    when a token spans at least one pass, the cos/sin rows of the tokens it
//    covers into LDS; rows then read their weights and table values from LDS.
//  * Row sums: sum of squares in fp64 (exact for 16-bit inputs) and the
//    absmax, each reduced over the L lanes with DPP.
//  * Workgroups are renumbered so that neighbouring row ranges (which share
//    boundary tokens) run on the same XCD and its L2.
#include <math.h>

#include "rnq_device.h"
#include "rnq_launch.h"

namespace rnq {

#ifndef RNQ_ROWS_WAVES
#define RNQ_ROWS_WAVES 4
#endif
constexpr int RW = RNQ_ROWS_WAVES;  // waves per workgroup
constexpr int RT = 64 * RW;

struct Lane {
  uint32_t row;   // flattened (token, head) index (clamped into range)
  uint32_t tok;
  uint32_t ri;    // row index inside its tensor
  bool second;    // row of tensor 1 (k)
  bool valid;
};

template <int G>
__device__ __forceinline__ Lane locate(const RowParams& p, uint32_t first_row, uint32_t pass, uint32_t slot) {
  Lane r;
  uint32_t row = first_row + pass * (uint32_t)G + slot;
  r.valid = row < p.total_rows;
  row = r.valid ? row : p.total_rows - 1;
  r.row = row;
  const uint32_t t = (uint32_t)(((uint64_t)row * p.div_magic) >> p.div_shift);  // row / heads
  const uint32_t h = row - t * p.heads;
  r.tok = t;
  r.second = h >= p.heads0;
  r.ri = r.second ? t * (p.heads - p.heads0) + (h - p.heads0) : t * p.heads0 + h;
  return r;
}

template <class DT, int L, int UPL, int PPW, bool QUANT, bool CLAMP, bool TBL_LDS>
__global__ __launch_bounds__(RT) void rows_kernel(RowParams p) {
  constexpr int D = 16 * L * UPL;
  constexpr int G = 64 / L;
  constexpr int PPB = RW * PPW;  // passes per workgroup
  extern __shared__ float lds[];  // [2][D] weights, then cos [ntok][half], sin [ntok][half]

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u;
  const uint32_t wave = tid >> 6;
  const uint32_t u = lane % L;
  const uint32_t slot = lane / L;

  // XCD-aware renumbering: hardware places workgroup b on XCD b % 8; give the
  // workgroups of one XCD a contiguous stretch of the row space.
  uint32_t blk = blockIdx.x;
  {
    const uint32_t nb = gridDim.x, full = nb & ~7u;
    if (blk < full) blk = (blk & 7u) * (full >> 3) + (blk >> 3);
  }
  const uint32_t first_row = blk * (uint32_t)(PPB * G);
  const uint32_t R = p.rope, half = R / 2;
  const uint32_t n_plain = (D - R) / 16;

  // ---- this lane's columns
  uint32_t off_a[UPL], off_b[UPL], cs_off[UPL];
  bool rope_u[UPL];
#pragma unroll
  for (int k = 0; k < UPL; ++k) {
    const uint32_t v = u + L * k;
    rope_u[k] = v >= n_plain;
    if (!rope_u[k]) {
      off_a[k] = 16 * v;
      off_b[k] = off_a[k] + 8;
      cs_off[k] = 0;
    } else {
      const uint32_t j = v - n_plain;
      off_a[k] = (D - R) + 8 * j;
      off_b[k] = off_a[k] + half;
      cs_off[k] = 8 * j;
    }
  }

  // ---- issue every global load of this wave's passes
  Lane ln[PPW];
  uint4 xa[PPW][UPL], xb[PPW][UPL];
#pragma unroll
  for (int i = 0; i < PPW; ++i) {
    ln[i] = locate<G>(p, first_row, wave * PPW + i, slot);
    const uint16_t* src = (ln[i].second ? p.x1 : p.x0) + (size_t)ln[i].ri * D;
#pragma unroll
    for (int k = 0; k < UPL; ++k) {
      xa[i][k] = load_stream16(src + off_a[k]);
      xb[i][k] = load_stream16(src + off_b[k]);
    }
  }

  // ---- stage weights (fp32) and the covered tokens' table rows in LDS
  float* w_lds = lds;
  float* cos_lds = lds + 2 * D;
  const uint32_t last_row = min(first_row + (uint32_t)(PPB * G), p.total_rows) - 1;
  const uint32_t t0 = (uint32_t)(((uint64_t)first_row * p.div_magic) >> p.div_shift);
  const uint32_t t1 = (uint32_t)(((uint64_t)last_row * p.div_magic) >> p.div_shift);
  const uint32_t ntok = t1 - t0 + 1;
  float* sin_lds = cos_lds + ntok * half;
  if (tid < D / 8) {
    float f[8];
    unpack8<DT>(*(const uint4*)(p.w0 + 8 * tid), f);
#pragma unroll
    for (int i = 0; i < 8; ++i) w_lds[8 * tid + i] = f[i];
    if (p.heads0 < p.heads) unpack8<DT>(*(const uint4*)(p.w1 + 8 * tid), f);
#pragma unroll
    for (int i = 0; i < 8; ++i) w_lds[D + 8 * tid + i] = f[i];
  }
  if constexpr (TBL_LDS) {
    const uint32_t q4 = half / 4;  // float4s per table row
    for (uint32_t c = tid; c < ntok * q4; c += RT) {
      const uint32_t t = c / q4, o = c - t * q4;
      const size_t g = (size_t)(t0 + t) * half + 4 * o;
      *(float4*)(cos_lds + t * half + 4 * o) = *(const float4*)(p.cos + g);
      *(float4*)(sin_lds + t * half + 4 * o) = *(const float4*)(p.sin + g);
    }
  }
  __syncthreads();

#pragma unroll
  for (int i = 0; i < PPW; ++i) {
    const Lane& r = ln[i];
    const float* w = w_lds + (r.second ? D : 0);

    // ---- sum of squares: fp64 (exact for 16-bit inputs), reduced over the row's lanes
    float xv[UPL][16];
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < UPL; ++k) {
      unpack8<DT>(xa[i][k], xv[k]);
      unpack8<DT>(xb[i][k], xv[k] + 8);
#pragma unroll
      for (int e = 0; e < 16; ++e) acc = __builtin_fma((double)xv[k][e], (double)xv[k][e], acc);
    }
    acc = group_sum<L>(acc);
    const float ssq = (float)acc;               // one rounding of the exact sum
    const float ms = ssq * (1.0f / (float)D);   // D is a power of two: equals ssq / D
    const float rstd = rstd_of(ms + p.eps);

    uint4 ya[UPL], yb[UPL];
#pragma unroll
    for (int k = 0; k < UPL; ++k) {
      // ---- normalise: (x * rstd) * w, rounded to the input dtype
      const float4 wa0 = *(const float4*)(w + off_a[k]), wa1 = *(const float4*)(w + off_a[k] + 4);
      const float4 wb0 = *(const float4*)(w + off_b[k]), wb1 = *(const float4*)(w + off_b[k] + 4);
      const float wv[16] = {wa0.x, wa0.y, wa0.z, wa0.w, wa1.x, wa1.y, wa1.z, wa1.w,
                            wb0.x, wb0.y, wb0.z, wb0.w, wb1.x, wb1.y, wb1.z, wb1.w};
      float n[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) n[e] = (xv[k][e] * rstd) * wv[e];
      ya[k] = pack8<DT>(n);
      yb[k] = pack8<DT>(n + 8);

      // ---- RoPE on the tail: lo' = lo c - hi s, hi' = hi c + lo s, each rounded to dtype
      if (rope_u[k]) {
        float4 c0, c1, s0, s1;
        if constexpr (TBL_LDS) {
          const uint32_t o = (r.tok - t0) * half + cs_off[k];
          c0 = *(const float4*)(cos_lds + o); c1 = *(const float4*)(cos_lds + o + 4);
          s0 = *(const float4*)(sin_lds + o); s1 = *(const float4*)(sin_lds + o + 4);
        } else {
          const size_t o = (size_t)r.tok * half + cs_off[k];
          c0 = *(const float4*)(p.cos + o); c1 = *(const float4*)(p.cos + o + 4);
          s0 = *(const float4*)(p.sin + o); s1 = *(const float4*)(p.sin + o + 4);
        }
        const float cc[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        const float ss[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        float lo[8], hi[8], ra[8], rb[8];
        unpack8<DT>(ya[k], lo);
        unpack8<DT>(yb[k], hi);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          ra[e] = (lo[e] * cc[e]) - (hi[e] * ss[e]);
          rb[e] = (hi[e] * cc[e]) + (lo[e] * ss[e]);
        }
        ya[k] = pack8<DT>(ra);
        yb[k] = pack8<DT>(rb);
      }
    }

    const size_t ebase = (size_t)r.ri * D;
    if (r.valid) {
      uint16_t* dst = r.second ? p.y1 : p.y0;
      if (dst != nullptr) {
#pragma unroll
        for (int k = 0; k < UPL; ++k) {
          *(uint4*)(dst + ebase + off_a[k]) = ya[k];
          *(uint4*)(dst + ebase + off_b[k]) = yb[k];
        }
      }
      if (p.rstd != nullptr && u == 0) p.rstd[r.row] = rstd;
    }

    if constexpr (QUANT) {
      float yv[UPL][16];
      float m = 0.0f;
#pragma unroll
      for (int k = 0; k < UPL; ++k) {
        unpack8<DT>(ya[k], yv[k]);
        unpack8<DT>(yb[k], yv[k] + 8);
#pragma unroll
        for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(yv[k][e]));
      }
      const float amax = group_max<L>(m);
      // scale = RN(max(amax, 1e-4) / fp8_max); amax is a 16-bit float value
      float scale;
      if (p.scale_by_rcp)
        scale = amax >= 1e-4f ? div_by(amax, p.fp8_max, p.rcp_fp8_max) : p.scale_floor;
      else
        scale = fmaxf(amax, 1e-4f) / p.fp8_max;
      const float rs = rcp_rn(scale);
      uint8_t* cdst = (r.second ? p.c1 : p.c0) + ebase;
#pragma unroll
      for (int k = 0; k < UPL; ++k) {
        float q[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          q[e] = div_by(yv[k][e], scale, rs);
          if constexpr (CLAMP) q[e] = __builtin_amdgcn_fmed3f(q[e], -p.fp8_max, p.fp8_max);
        }
        uint2 ca, cb;
        ca.x = fp8x4(q[0], q[1], q[2], q[3], ya[k].x);
        ca.y = fp8x4(q[4], q[5], q[6], q[7], ya[k].y);
        cb.x = fp8x4(q[8], q[9], q[10], q[11], yb[k].x);
        cb.y = fp8x4(q[12], q[13], q[14], q[15], yb[k].y);
        if (r.valid) {
          store_stream8(cdst + off_a[k], ca);
          store_stream8(cdst + off_b[k], cb);
        }
      }
      if (r.valid && u == 0) (r.second ? p.s1 : p.s0)[r.ri] = scale;
    }
  }
}

// --------------------------------------------------------------- launcher

// Passes per wave: one pass keeps the smallest unit of work (best balance for
// launches of a few tens of thousands of passes); two passes amortise the
// per-wave setup once there are many workgroups per CU.
constexpr uint32_t kTwoPassesFrom = 1u << 18;  // passes in the launch

template <class DT, int L, int UPL, bool QUANT, bool CLAMP>
static hipError_t launch_shape(const RowParams& p, int ppw, bool tbl_lds, dim3 grid, size_t lds, hipStream_t s) {
  if (ppw == 2) {
    if (tbl_lds)
      hipLaunchKernelGGL((rows_kernel<DT, L, UPL, 2, QUANT, CLAMP, true>), grid, dim3(RT), lds, s, p);
    else
      hipLaunchKernelGGL((rows_kernel<DT, L, UPL, 2, QUANT, CLAMP, false>), grid, dim3(RT), lds, s, p);
  } else {
    if (tbl_lds)
      hipLaunchKernelGGL((rows_kernel<DT, L, UPL, 1, QUANT, CLAMP, true>), grid, dim3(RT), lds, s, p);
    else
      hipLaunchKernelGGL((rows_kernel<DT, L, UPL, 1, QUANT, CLAMP, false>), grid, dim3(RT), lds, s, p);
  }
  return hipGetLastError();
}

// One 16-byte chunk of each half of a unit per lane: 8 lanes own a 128-wide
// row, so each wave-wide access covers whole 128-byte (input) / 64-byte
// (codes) spans of 8 rows.
template <class DT, bool QUANT, bool CLAMP>
static hipError_t launch_dt(const RowParams& p, int D, int ppw, bool tbl_lds, dim3 grid, size_t lds, hipStream_t s) {
  switch (D) {
    case 64: return launch_shape<DT, 4, 1, QUANT, CLAMP>(p, ppw, tbl_lds, grid, lds, s);
    case 128: return launch_shape<DT, 8, 1, QUANT, CLAMP>(p, ppw, tbl_lds, grid, lds, s);
    case 256: return launch_shape<DT, 16, 1, QUANT, CLAMP>(p, ppw, tbl_lds, grid, lds, s);
    case 512: return launch_shape<DT, 32, 1, QUANT, CLAMP>(p, ppw, tbl_lds, grid, lds, s);
    default: return hipErrorInvalidValue;
  }
}

// e4m3fn code magnitude of a positive value below 480 (nearest even), host side.
static int e4m3_magnitude(double v) {
  if (v < 0x1p-6) return (int)nearbyint(v * 512.0);
  int e = 0;
  const double m = frexp(v, &e) * 2.0;  // v = m * 2^(e-1), m in [1, 2)
  int mant = (int)nearbyint((m - 1.0) * 8.0);
  int ex = e - 1;
  if (mant == 8) { mant = 0; ++ex; }
  return ((ex + 7) << 3) | mant;
}

// The clamp to +-fp8_max can only change a code when some quotient lands
// above fp8_max; every |y / scale| is at most fp8_max * (1 + 2^-22), so the
// clamp is needed only if that margin reaches a different code.
static bool clamp_needed(float fp8_max) {
  return e4m3_magnitude((double)fp8_max * (1.0 + 0x1p-20)) != e4m3_magnitude((double)fp8_max);
}

static int lanes_per_row(int D) { return D / 16; }

hipError_t launch_rows(RowParams p, int head_dim, bool bf16, bool quant, hipStream_t stream) {
  const uint32_t G = 64u / (uint32_t)lanes_per_row(head_dim);
  p.passes = (uint32_t)((p.total_rows + G - 1) / G);
  const int ppw = p.passes >= kTwoPassesFrom ? 2 : 1;
  const uint32_t rows_per_block = RW * (uint32_t)ppw * G;  // waves x passes x rows per pass
  // t = row / heads by multiply-shift: shift = 31 + ceil(log2 heads), magic = ceil(2^shift / heads);
  // exact for every row < 2^31.
  uint32_t lg = 0;
  while ((1u << lg) < p.heads) ++lg;
  p.div_shift = 31 + lg;
  p.div_magic = (uint32_t)((((uint64_t)1 << p.div_shift) + p.heads - 1) / p.heads);

  // table rows through LDS when a token spans at least one pass (rows of a token share them)
  const bool tbl_lds = p.rope > 0 && p.heads >= G;
  const uint32_t max_tok = tbl_lds ? (rows_per_block - 1) / p.heads + 2 : 0;
  const size_t lds = sizeof(float) * (2 * (size_t)head_dim + 2 * (size_t)max_tok * (p.rope / 2));
  dim3 grid((p.total_rows + rows_per_block - 1) / rows_per_block);
  // scale = RN(max(amax, 1e-4) / fp8_max) through the reciprocal of fp8_max
  // when fp8_max >= 1 (no overflow for any 16-bit amax)
  p.rcp_fp8_max = 1.0f / p.fp8_max;
  p.scale_floor = 1e-4f / p.fp8_max;
  p.scale_by_rcp = p.fp8_max >= 1.0f ? 1u : 0u;
  const bool clamp = quant && clamp_needed(p.fp8_max);
  if (bf16) {
    if (!quant) return launch_dt<BF16, false, false>(p, head_dim, ppw, tbl_lds, grid, lds, stream);
    return clamp ? launch_dt<BF16, true, true>(p, head_dim, ppw, tbl_lds, grid, lds, stream)
                 : launch_dt<BF16, true, false>(p, head_dim, ppw, tbl_lds, grid, lds, stream);
  }
  if (!quant) return launch_dt<F16, false, false>(p, head_dim, ppw, tbl_lds, grid, lds, stream);
  return clamp ? launch_dt<F16, true, true>(p, head_dim, ppw, tbl_lds, grid, lds, stream)
               : launch_dt<F16, true, false>(p, head_dim, ppw, tbl_lds, grid, lds, stream);
}

}  // namespace rnq
