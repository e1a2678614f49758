// RMSNorm backward for narrow rows (64, 128, 256 or 512 elements: head-sized
// rows), optionally through the partial NeoX RoPE of the last R columns.
//
// Operation: tilelang-tutorial chapter 17 page "rmsnorm_tl.py",
// RMSNormTileLang.backward (xn = x * rstd, g = grad_y * w,
// grad_x = rstd * (g - xn * mean(g * xn)), grad_w = sum over rows of
// grad_y * xn). With RoPE (the tail rotation of the chapter 13 fusion page,
// pair p <-> p + R/2 of the last R columns rotated by (cos, sin) of the row's
// table row), grad_y first goes back through the rotation: the transposed
// rotation, (g_lo c + g_hi s, g_hi c - g_lo s); the two casts to the input
// dtype count as identities, as in the chapter 17 backward.
//
// Mapping: L = N / 8 lanes per row (8 elements, one 16-byte chunk, per lane),
// 64 / L rows per wave, 16 waves per workgroup. Row sums are DPP butterflies
// inside the row's lanes, so no barrier is taken per row. The RoPE partner
// chunk sits R/16 lanes away in the same row and comes over by a lane
// permute. Workgroup b owns a contiguous range of rows (the partition of
// bwd_blocks) and walks it RPI rows at a time, the next step's loads in
// flight while a step is computed; every global access is a buffer access
// relative to the workgroup's first row, so rows past its range fall outside
// the descriptor (read as zero, stores dropped) and nothing is conditional.
// grad_w: each lane keeps its 8 columns' sums in registers (its rows in
// ascending order); at the end the lanes of a column are added in a fixed
// order (an xor butterfly over the wave's row slots, then a pairwise tree
// over the waves) and written to the workspace row b; dw_reduce_kernel adds
// the workspace rows in a fixed order.
#include "rnq_device.h"
#include "rnq_launch.h"

namespace rnq {

constexpr int NB = 1024;      // threads per workgroup
constexpr int NBW = NB / 64;  // waves

// (the fields its first loads need come as leading scalar arguments, 14 dwords
// that gfx950 preloads into scalar registers: x, grad_y, w, cos, sin, M, rows
// per block, the row -> token magic, and its shift with the rope width; a
// struct argument is not preloaded, and every wave would first wait for a load
// of it)
template <class DT, int D, bool ROPE, bool SAVED>
__global__ __launch_bounds__(NB) void narrow_bwd_kernel(const uint16_t* x_in, const uint16_t* gy_in,
                                                        const uint16_t* w_in, const float* cos_in,
                                                        const float* sin_in, uint32_t M, uint32_t rows_per_block,
                                                        uint32_t div_magic, uint32_t shift_rope, WideBwdParams p) {
  constexpr int L = D / 8;      // lanes per row
  constexpr int G = 64 / L;     // rows per wave
  constexpr int RPI = NBW * G;  // rows per step of the workgroup
  constexpr uint32_t kOutOfRange = 0x80000000u;
  constexpr uint32_t row_bytes = 2u * D;
  __shared__ float red[NBW * D];  // per-wave column sums

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const uint32_t ch = lane % L;                    // chunk within the row
  const uint32_t lrow = (tid >> 6) * G + lane / L;  // row within a step
  const uint32_t div_shift = shift_rope & 0xffu, rope = shift_rope >> 8;
  const uint32_t r0 = blockIdx.x * rows_per_block;
  // (bwd_blocks' partition gives every block rows; a block without rows would
  // read nothing and write a zero partial row. No early exit: a branch here
  // would come before the kernel-argument loads, and the compiler issues none
  // past a branch.)
  const uint32_t nrows = r0 < M ? min(rows_per_block, M - r0) : 0u;
  const uint32_t steps = (nrows + RPI - 1) / RPI;
  const uint32_t span = nrows * row_bytes;  // < 2^31 (checked by the caller)
  const rsrc_t rx = make_rsrc(x_in + (size_t)r0 * D, span);
  const rsrc_t rg = make_rsrc(gy_in + (size_t)r0 * D, span);
  // one table row per token: tokens = (M - 1) / rows_per_token + 1
  const uint32_t table_bytes =
      ROPE ? ((uint32_t)(((uint64_t)(M - 1) * div_magic) >> div_shift) + 1u) * (rope / 2) * 4u : 0u;
  const rsrc_t rc = make_rsrc(cos_in, table_bytes);
  const rsrc_t rs = make_rsrc(sin_in, table_bytes);

  // (kept packed and unpacked in each step: a wait for it ahead of the loop
  // would hold back the second step's loads)
  const uint4 w_raw = buf_load16(make_rsrc(w_in, row_bytes), 16u * ch);

  // RoPE geometry of this lane's chunk (row-independent)
  bool tail = false, lo_half = false;
  uint32_t pj = 0;
  int src = (int)lane;
  if constexpr (ROPE) {
    const uint32_t t0 = (D - rope) / 8, hc = rope / 16;
    tail = ch >= t0;
    const uint32_t j = ch - t0;
    lo_half = tail && j < hc;
    pj = lo_half ? j : j - hc;
    src = tail ? (int)lane + (lo_half ? (int)hc : -(int)hc) : (int)lane;
  }
  const uint32_t half = rope / 2;
  // (grad_x and rstd are not preloaded: their descriptors come from the
  // argument struct, loaded while the first step's loads are in flight)
  rsrc_t rdx, rrs;

  struct In {
    uint4 x, g;
    float rs;
    float4 c0, c1, s0, s1;
  };
  auto load = [&](uint32_t step, In& in) {
    const uint32_t lr = step * RPI + lrow;
    const uint32_t off = lr * row_bytes + 16u * ch;
    in.x = buf_load16_nt(rx, off);
    in.g = buf_load16_nt(rg, off);
    if constexpr (ROPE) {
      const uint32_t row = r0 + lr;
      const uint32_t t = (uint32_t)(((uint64_t)row * div_magic) >> div_shift);
      const uint32_t toff = tail ? 4u * (t * half + 8u * pj) : kOutOfRange;
      in.c0 = buf_load16f(rc, toff);
      in.c1 = buf_load16f(rc, toff + 16u);
      in.s0 = buf_load16f(rs, toff);
      in.s1 = buf_load16f(rs, toff + 16u);
    }
    if constexpr (SAVED) in.rs = buf_load4f(rrs, 4u * lr);
  };

  float dw[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) dw[i] = 0.f;

  auto compute = [&](uint32_t step, const In& in) {
    const uint32_t lr = step * RPI + lrow;
    const bool real = lr < nrows;
    float xf[8], gn[8], w[8];
    unpack8<DT>(in.x, xf);
    unpack8<DT>(in.g, gn);
    // (an empty asm keeps the weights' unpacking in the step: hoisted out of
    // the loop it would wait for them before the next step's loads go out)
    uint4 wr = w_raw;
    asm volatile("" : "+v"(wr.x), "+v"(wr.y), "+v"(wr.z), "+v"(wr.w));
    unpack8<DT>(wr, w);
    float rstd;
    if constexpr (SAVED) {
      rstd = in.rs;
    } else {
      double acc = 0.0;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc = __builtin_fma((double)xf[i], (double)xf[i], acc);
      acc = group_sum<L>(acc);
      rstd = rstd_of((float)acc / (float)D + p.eps);
    }
    if constexpr (ROPE) {
      // partner chunk (same lane for columns outside the tail)
      uint4 pg;
      pg.x = (uint32_t)__shfl((int)in.g.x, src, 64);
      pg.y = (uint32_t)__shfl((int)in.g.y, src, 64);
      pg.z = (uint32_t)__shfl((int)in.g.z, src, 64);
      pg.w = (uint32_t)__shfl((int)in.g.w, src, 64);
      float pf[8];
      unpack8<DT>(pg, pf);
      const float cc[8] = {in.c0.x, in.c0.y, in.c0.z, in.c0.w, in.c1.x, in.c1.y, in.c1.z, in.c1.w};
      const float ss[8] = {in.s0.x, in.s0.y, in.s0.z, in.s0.w, in.s1.x, in.s1.y, in.s1.z, in.s1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float own = gn[i] * cc[i];
        const float other = pf[i] * ss[i];
        const float r = lo_half ? own + other : own - other;
        gn[i] = tail ? r : gn[i];
      }
    }
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) dot += (gn[i] * w[i]) * (xf[i] * rstd);
    const float C = group_sum<L>(dot) / (float)D;
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float xn = xf[i] * rstd;
      o[i] = rstd * ((gn[i] * w[i]) - xn * C);
      dw[i] += real ? gn[i] * xn : 0.f;
    }
    // rows past the range are past the descriptor: the store is dropped
    buf_store16_nt(rdx, lr * row_bytes + 16u * ch, pack8<DT>(o));
  };

  In a, b;
  // (the first step's input and table loads need only preloaded arguments; its
  // saved rstd, if any, waits for the argument struct)
  rrs = make_rsrc(p.rstd + r0, SAVED ? 4u * nrows : 0u);
  load(0, a);
  __builtin_amdgcn_sched_barrier(0);
  rdx = make_rsrc(p.gx + (size_t)r0 * D, span);
  uint32_t s = 0;
  for (; s + 2 <= steps; s += 2) {
    load(s + 1, b);
    compute(s, a);
    load(s + 2, a);
    compute(s + 1, b);
  }
  if (s < steps) compute(s, a);

  // column sums: the G row slots of a wave by an xor butterfly (every lane of
  // a column ends with the same sum), then the 16 waves by a fixed pairwise
  // tree in LDS, then one workspace row
#pragma unroll
  for (int m = L; m < 64; m *= 2) {
#pragma unroll
    for (int i = 0; i < 8; ++i) dw[i] += __shfl_xor(dw[i], m, 64);
  }
  if (lane < (uint32_t)L) {
    float4* mine = (float4*)(red + (tid >> 6) * D + 8 * ch);
    mine[0] = make_float4(dw[0], dw[1], dw[2], dw[3]);
    mine[1] = make_float4(dw[4], dw[5], dw[6], dw[7]);
  }
  lds_barrier();
#pragma unroll
  for (int h = NBW / 2; h >= 1; h /= 2) {
    for (uint32_t i = tid; i < (uint32_t)(h * D); i += NB) red[i] += red[i + h * D];
    lds_barrier();
  }
  if (tid < (uint32_t)D) p.partial[(size_t)blockIdx.x * D + tid] = red[tid];
}

// ----------------------------------------------------------------- launcher

bool narrow_bwd_width(int64_t N) { return N == 64 || N == 128 || N == 256 || N == 512; }

template <class DT, int D, bool ROPE>
static void launch_saved(const WideBwdParams& p, hipStream_t s) {
  if (p.rstd != nullptr)
    hipLaunchKernelGGL((narrow_bwd_kernel<DT, D, ROPE, true>), dim3(p.blocks), dim3(NB), 0, s, p.x, p.gy, p.w, p.cos,
                       p.sin, p.M, p.rows_per_block, p.div_magic, p.div_shift | p.rope << 8, p);
  else
    hipLaunchKernelGGL((narrow_bwd_kernel<DT, D, ROPE, false>), dim3(p.blocks), dim3(NB), 0, s, p.x, p.gy, p.w, p.cos,
                       p.sin, p.M, p.rows_per_block, p.div_magic, p.div_shift | p.rope << 8, p);
}

template <class DT, int D>
static void launch_rope(const WideBwdParams& p, hipStream_t s) {
  if (p.rope > 0)
    launch_saved<DT, D, true>(p, s);
  else
    launch_saved<DT, D, false>(p, s);
}

template <class DT>
static hipError_t launch_width(const WideBwdParams& p, hipStream_t s) {
  switch (p.N) {
    case 64: launch_rope<DT, 64>(p, s); break;
    case 128: launch_rope<DT, 128>(p, s); break;
    case 256: launch_rope<DT, 256>(p, s); break;
    case 512: launch_rope<DT, 512>(p, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_narrow_bwd(WideBwdParams p, bool bf16, hipStream_t stream) {
  if (!narrow_bwd_width(p.N) || p.rope > p.N || p.rope % 16 != 0) return hipErrorInvalidValue;
  if (p.rows_per_token == 0) p.rows_per_token = 1;
  // row / rows_per_token by multiply-shift (exact for every row < 2^31)
  div_magic_for(p.rows_per_token, p.div_magic, p.div_shift);
  const hipError_t e = bf16 ? launch_width<BF16>(p, stream) : launch_width<F16>(p, stream);
  if (e != hipSuccess) return e;
  return launch_dw_reduce(p.partial, p.gw, p.blocks, p.N, stream);
}

}  // namespace rnq
