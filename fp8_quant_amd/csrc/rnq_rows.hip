// Row kernel: RMSNorm -> partial NeoX RoPE -> (optional) per-row FP8 e4m3fn.
//
// Operation: tilelang-tutorial chapter 13 fusion page, torch_reference_fused
// and the two fused kernels; chapter 28 case study, the QK-norm prologue
// (rows are (token, head) pairs; every head of a token uses the token's
// cos/sin row; one fp32 scale per row).
//
// Mapping (gfx950, wave64). A row of D = 16*L elements is owned by L lanes;
// a wave handles G = 64/L rows at a time (a "pass"). Each lane holds two
// 16-byte chunks of its row:
//   * rope lanes hold chunk j of the lower half of the rope tail and chunk j
//     of the upper half, so both members of each of its 8 RoPE pairs are in
//     its own registers (no LDS exchange);
//   * lanes outside the tail hold two adjacent chunks.
// Row reductions (sum of squares in fp64, absmax) are DPP butterflies across
// the L lanes. Each wave walks a contiguous range of passes; with whole
// tokens per wave its lanes keep the token's cos/sin values in registers and
// reload them only when the token changes. Loads of the next pass are issued
// before the current pass is computed.
#include "rnq_device.h"
#include "rnq_launch.h"

namespace rnq {

struct RowRef {
  uint32_t row;  // flattened (token, head) index, clamped into range
  uint32_t tok;
  uint32_t ri;   // row index inside its tensor
  bool second;   // true: row of the second tensor (k)
  bool valid;
};

template <int G>
__device__ __forceinline__ RowRef locate(const RowParams& p, uint32_t pass, uint32_t slot) {
  RowRef r;
  uint32_t row = pass * (uint32_t)G + slot;
  r.valid = row < p.total_rows;
  row = r.valid ? row : p.total_rows - 1;
  r.row = row;
  // t = row / H by multiply-shift (exact for row < 2^31, see the launcher)
  uint32_t t = (uint32_t)(((uint64_t)row * p.div_magic) >> p.div_shift);
  uint32_t h = row - t * p.heads;
  r.tok = t;
  r.second = h >= p.heads0;
  r.ri = r.second ? t * (p.heads - p.heads0) + (h - p.heads0) : t * p.heads0 + h;
  return r;
}

template <class DT, int L, bool QUANT>
__global__ __launch_bounds__(256) void rows_kernel(RowParams p) {
  constexpr int D = 16 * L;
  constexpr int G = 64 / L;
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t u = lane % L;       // unit within the row
  const uint32_t slot = lane / L;    // row slot within the pass
  const uint32_t wave = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const uint32_t p_begin = wave * p.passes_per_wave;
  if (p_begin >= p.passes) return;
  const uint32_t p_end = min(p_begin + p.passes_per_wave, p.passes);

  // ---- this lane's columns
  const uint32_t R = p.rope;
  const uint32_t n_plain = (D - R) / 16;  // units outside the rope tail
  const bool rope_lane = u >= n_plain;
  uint32_t off_a, off_b, cs_off = 0;
  if (!rope_lane) {
    off_a = 16 * u;
    off_b = off_a + 8;
  } else {
    const uint32_t j = u - n_plain;
    off_a = (D - R) + 8 * j;
    off_b = off_a + R / 2;
    cs_off = 8 * j;
  }
  const uint32_t half = R / 2;

  // ---- weights of both tensors, as fp32, for this lane's 16 columns
  float w0a[8], w0b[8], w1a[8], w1b[8];
  unpack8<DT>(*(const uint4*)(p.w0 + off_a), w0a);
  unpack8<DT>(*(const uint4*)(p.w0 + off_b), w0b);
  if (p.heads0 < p.heads) {
    unpack8<DT>(*(const uint4*)(p.w1 + off_a), w1a);
    unpack8<DT>(*(const uint4*)(p.w1 + off_b), w1b);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) { w1a[i] = w0a[i]; w1b[i] = w0b[i]; }
  }

  // ---- first pass: data and table rows
  RowRef ref = locate<G>(p, p_begin, slot);
  const uint16_t* src = ref.second ? p.x1 : p.x0;
  uint4 xa = *(const uint4*)(src + (size_t)ref.ri * D + off_a);
  uint4 xb = *(const uint4*)(src + (size_t)ref.ri * D + off_b);
  float4 c0 = make_float4(0.f, 0.f, 0.f, 0.f), c1 = c0, s0 = c0, s1 = c0;
  if (rope_lane) {
    const float* cp = p.cos + (size_t)ref.tok * half + cs_off;
    const float* sp = p.sin + (size_t)ref.tok * half + cs_off;
    c0 = *(const float4*)cp; c1 = *(const float4*)(cp + 4);
    s0 = *(const float4*)sp; s1 = *(const float4*)(sp + 4);
  }

  for (uint32_t pass = p_begin; pass < p_end; ++pass) {
    // ---- issue the next pass's loads
    const bool has_next = pass + 1 < p_end;
    RowRef nref = ref;
    uint4 nxa = xa, nxb = xb;
    float4 nc0 = c0, nc1 = c1, ns0 = s0, ns1 = s1;
    if (has_next) {
      nref = locate<G>(p, pass + 1, slot);
      const uint16_t* nsrc = nref.second ? p.x1 : p.x0;
      nxa = *(const uint4*)(nsrc + (size_t)nref.ri * D + off_a);
      nxb = *(const uint4*)(nsrc + (size_t)nref.ri * D + off_b);
      if (rope_lane && nref.tok != ref.tok) {
        const float* cp = p.cos + (size_t)nref.tok * half + cs_off;
        const float* sp = p.sin + (size_t)nref.tok * half + cs_off;
        nc0 = *(const float4*)cp; nc1 = *(const float4*)(cp + 4);
        ns0 = *(const float4*)sp; ns1 = *(const float4*)(sp + 4);
      }
    }

    // ---- sum of squares: fp64 (exact for these inputs), reduced over the row's lanes
    float xva[8], xvb[8];
    unpack8<DT>(xa, xva);
    unpack8<DT>(xb, xvb);
    double acc = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      acc = __builtin_fma((double)xva[i], (double)xva[i], acc);
      acc = __builtin_fma((double)xvb[i], (double)xvb[i], acc);
    }
    acc = group_sum<L>(acc);
    const float ssq = (float)acc;                // one rounding of the exact sum
    const float ms = ssq * (1.0f / (float)D);    // D is a power of two: equals ssq / D
    const float rstd = rstd_of(ms + p.eps);

    // ---- normalise: (x * rstd) * w, rounded to the input dtype
    float na[8], nb[8];
    const uint64_t sec = __builtin_amdgcn_ballot_w64(ref.second);
    if (sec == 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) { na[i] = (xva[i] * rstd) * w0a[i]; nb[i] = (xvb[i] * rstd) * w0b[i]; }
    } else if (sec == __builtin_amdgcn_ballot_w64(true)) {
#pragma unroll
      for (int i = 0; i < 8; ++i) { na[i] = (xva[i] * rstd) * w1a[i]; nb[i] = (xvb[i] * rstd) * w1b[i]; }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        na[i] = (xva[i] * rstd) * (ref.second ? w1a[i] : w0a[i]);
        nb[i] = (xvb[i] * rstd) * (ref.second ? w1b[i] : w0b[i]);
      }
    }
    uint4 ya = pack8<DT>(na);
    uint4 yb = pack8<DT>(nb);

    // ---- RoPE on the tail: lo' = lo c - hi s, hi' = hi c + lo s, each rounded to dtype
    if (rope_lane) {
      float lo[8], hi[8];
      unpack8<DT>(ya, lo);
      unpack8<DT>(yb, hi);
      const float cc[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      const float ss[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
      float ra[8], rb[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ra[i] = (lo[i] * cc[i]) - (hi[i] * ss[i]);
        rb[i] = (hi[i] * cc[i]) + (lo[i] * ss[i]);
      }
      ya = pack8<DT>(ra);
      yb = pack8<DT>(rb);
    }

    const size_t ebase = (size_t)ref.ri * D;
    if (ref.valid) {
      uint16_t* dst = ref.second ? p.y1 : p.y0;
      if (dst != nullptr) {
        *(uint4*)(dst + ebase + off_a) = ya;
        *(uint4*)(dst + ebase + off_b) = yb;
      }
    }
    if (p.rstd != nullptr && ref.valid && u == 0) p.rstd[ref.row] = rstd;

    if constexpr (QUANT) {
      float va[8], vb[8];
      unpack8<DT>(ya, va);
      unpack8<DT>(yb, vb);
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, fmaxf(fabsf(va[i]), fabsf(vb[i])));
      const float amax = group_max<L>(m);
      const float scale = fmaxf(amax, 1e-4f) / p.fp8_max;
      const float rs = 1.0f / scale;
      const float lim = p.fp8_max;
      float qa[8], qb[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        qa[i] = fminf(fmaxf(div_by_scale(va[i], scale, rs), -lim), lim);
        qb[i] = fminf(fmaxf(div_by_scale(vb[i], scale, rs), -lim), lim);
      }
      uint2 ca, cb;
      ca.x = fp8x4(qa[0], qa[1], qa[2], qa[3]);
      ca.y = fp8x4(qa[4], qa[5], qa[6], qa[7]);
      cb.x = fp8x4(qb[0], qb[1], qb[2], qb[3]);
      cb.y = fp8x4(qb[4], qb[5], qb[6], qb[7]);
      if (ref.valid) {
        uint8_t* cdst = ref.second ? p.c1 : p.c0;
        *(uint2*)(cdst + ebase + off_a) = ca;
        *(uint2*)(cdst + ebase + off_b) = cb;
        if (u == 0) (ref.second ? p.s1 : p.s0)[ref.ri] = scale;
      }
    }

    if (has_next) {
      ref = nref;
      xa = nxa; xb = nxb;
      c0 = nc0; c1 = nc1; s0 = ns0; s1 = ns1;
    }
  }
}

// --------------------------------------------------------------- launcher

template <class DT, bool QUANT>
static hipError_t launch_L(const RowParams& p, int L, dim3 grid, dim3 block, hipStream_t s) {
  switch (L) {
    case 4: hipLaunchKernelGGL((rows_kernel<DT, 4, QUANT>), grid, block, 0, s, p); break;
    case 8: hipLaunchKernelGGL((rows_kernel<DT, 8, QUANT>), grid, block, 0, s, p); break;
    case 16: hipLaunchKernelGGL((rows_kernel<DT, 16, QUANT>), grid, block, 0, s, p); break;
    case 32: hipLaunchKernelGGL((rows_kernel<DT, 32, QUANT>), grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rows(RowParams p, int head_dim, bool bf16, bool quant, hipStream_t stream) {
  const int L = head_dim / 16;
  const uint32_t G = 64u / (uint32_t)L;
  p.passes = (uint32_t)((p.total_rows + G - 1) / G);
  // divisor magic for t = row / heads: shift = 31 + ceil(log2 heads), magic = ceil(2^shift / heads)
  uint32_t lg = 0;
  while ((1u << lg) < p.heads) ++lg;
  p.div_shift = 31 + lg;
  p.div_magic = (uint32_t)((((uint64_t)1 << p.div_shift) + p.heads - 1) / p.heads);

  // passes per wave: spread over ~target waves; keep whole tokens per wave when rows tile tokens
  const uint32_t target = tuning_target_waves();
  uint32_t ppw = (p.passes + target - 1) / target;
  if (ppw == 0) ppw = 1;
  if (p.heads % G == 0 && p.heads0 % G == 0) {
    const uint32_t per_tok = p.heads / G;
    ppw = ((ppw + per_tok - 1) / per_tok) * per_tok;
  }
  if (const uint32_t forced = tuning_passes_per_wave()) ppw = forced;
  p.passes_per_wave = ppw;
  const uint32_t waves = (p.passes + ppw - 1) / ppw;
  const uint32_t wpb = 4;
  dim3 block(64 * wpb);
  dim3 grid((waves + wpb - 1) / wpb);
  if (bf16) {
    return quant ? launch_L<BF16, true>(p, L, grid, block, stream) : launch_L<BF16, false>(p, L, grid, block, stream);
  }
  return quant ? launch_L<F16, true>(p, L, grid, block, stream) : launch_L<F16, false>(p, L, grid, block, stream);
}

}  // namespace rnq
