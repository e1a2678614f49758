// RMSNorm backward, one wave per row, for rows of 512 * KC elements (KC = 2,
// 4 or 8: 1024, 2048 or 4096), optionally through the partial NeoX RoPE of
// the last R <= 512 columns.
//
// Operation: tilelang-tutorial chapter 17 page "rmsnorm_tl.py",
// RMSNormTileLang.backward (xn = x * rstd, g = grad_y * w,
// grad_x = rstd * (g - xn * mean(g * xn)), grad_w = sum over rows of
// grad_y * xn); with RoPE, grad_y first goes back through the transposed
// rotation of the chapter 13 fusion page's tail, (g_lo c + g_hi s,
// g_hi c - g_lo s), as in the narrow backward.
//
// Mapping: lane l of a wave owns the 16-byte chunks l, l + 64, ... of a row
// (KC of them), so both row sums are DPP butterflies inside the wave and the
// row loop takes no barrier: each wave walks its own rows with the next row's
// loads in flight while a row is computed (16 KB of input per wave at 4096
// columns). With R <= 512 the tail is the last R / 8 chunks of the row, all in
// the lane's last chunk slot, so the partner chunk of a pair sits R / 16 lanes
// away and comes over by a lane permute. Workgroup b owns the contiguous rows
// of bwd_blocks' partition; wave v takes its rows v, v + 8, ... Every global
// access is a buffer access relative to the workgroup's first row: rows past
// its range are outside the descriptors (read as zero, stores dropped).
// grad_w: each wave keeps its columns' sums in its own LDS area (its rows in
// ascending order; registers hold the two rows in flight); at the end the 8
// areas are added by a fixed pairwise tree and written to the workspace row b,
// which dw_reduce_kernel adds in a fixed order.
#include "rnq_device.h"
#include "rnq_launch.h"

namespace rnq {

namespace {

constexpr int RBW = 8;          // waves per workgroup
constexpr int RBT = 64 * RBW;   // threads per workgroup
constexpr uint32_t kMaxRowBwdRope = 512;

// (the fields its first loads need come as leading scalar arguments, 14 dwords
// that gfx950 preloads into scalar registers: x, grad_y, w, cos, sin, M, rows
// per block, the row -> token magic, and its shift with the rope width)
template <class DT, int KC, bool ROPE, bool SAVED>
__global__ __launch_bounds__(RBT) void row_bwd_kernel(const uint16_t* x_in, const uint16_t* gy_in, const uint16_t* w_in,
                                                     const float* cos_in, const float* sin_in, uint32_t M,
                                                     uint32_t rows_per_block, uint32_t div_magic, uint32_t shift_rope,
                                                     WideBwdParams p) {
  constexpr uint32_t N = 512u * KC;
  constexpr uint32_t row_bytes = 2u * N;
  constexpr uint32_t kOutOfRange = 0x80000000u;
  const uint32_t div_shift = shift_rope & 0xffu, rope = shift_rope >> 8;
  // the weight row as fp32 (read where it is used, twice per row, without
  // unpacking): float4 (2 k + h) * 64 + lane holds columns 8 (lane + 64 k) + 4 h .. + 3
  __shared__ float4 w_f[N / 4];
  // grad_w sums of each wave: float4 (2 k + h) * 64 + lane of wave v holds
  // columns 8 (lane + 64 k) + 4 h .. + 3 (lanes 16 bytes apart)
  __shared__ float4 dw_s[RBW][N / 4];

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const uint32_t wave = (uint32_t)__builtin_amdgcn_readfirstlane((int)(tid >> 6));
  const uint32_t r0 = blockIdx.x * rows_per_block;
  // (bwd_blocks' partition gives every block rows; a wave without rows reads
  // nothing and adds nothing. No early exit: a branch here would come before
  // the kernel-argument loads, and the compiler issues none past a branch.)
  const uint32_t nrows = r0 < M ? min(rows_per_block, M - r0) : 0u;
  const uint32_t mine = nrows > wave ? (nrows - wave + RBW - 1) / RBW : 0u;  // rows of this wave
  const uint32_t span = nrows * row_bytes;  // < 2^31 (checked by the caller)
  const rsrc_t rx = make_rsrc(x_in + (size_t)r0 * N, span);
  const rsrc_t rg = make_rsrc(gy_in + (size_t)r0 * N, span);
  // one table row per token: tokens = (M - 1) / rows_per_token + 1
  const uint32_t table_bytes =
      ROPE ? ((uint32_t)(((uint64_t)(M - 1) * div_magic) >> div_shift) + 1u) * (rope / 2) * 4u : 0u;
  const rsrc_t rc = make_rsrc(cos_in, table_bytes);
  const rsrc_t rs = make_rsrc(sin_in, table_bytes);

  // the weight row: thread t copies chunk t (N / 8 <= 512 chunks)
  const uint4 wc = buf_load16(make_rsrc(w_in, row_bytes), tid < N / 8 ? 16u * tid : kOutOfRange);

  // RoPE geometry of the lane's last chunk (the tail's chunks are lanes
  // 64 - R / 8 .. 63 of slot KC - 1)
  bool tail = false, lo_half = false;
  uint32_t pj = 0;
  int src = (int)lane;
  if constexpr (ROPE) {
    const uint32_t t0 = 64u - rope / 8, hc = rope / 16;
    tail = lane >= t0;
    const uint32_t j = lane - t0;
    lo_half = tail && j < hc;
    pj = lo_half ? j : j - hc;
    src = tail ? (int)lane + (lo_half ? (int)hc : -(int)hc) : (int)lane;
  }
  const uint32_t half = rope / 2;

  struct In {
    uint4 x[KC], g[KC];
    float rs;
    float4 c0, c1, s0, s1;
  };
  auto row_of = [&](uint32_t j) { return wave + RBW * j; };  // local row of the wave's j-th row
  auto load_xg = [&](uint32_t j, In& in) {
    const uint32_t base = row_of(j) * row_bytes + 16u * lane;
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      in.x[k] = buf_load16_nt(rx, base + 1024u * k);
      in.g[k] = buf_load16_nt(rg, base + 1024u * k);
    }
  };
  auto load_tab = [&](uint32_t j, In& in) {
    if constexpr (ROPE) {
      const uint32_t row = r0 + row_of(j);
      const uint32_t t = (uint32_t)(((uint64_t)row * div_magic) >> div_shift);
      const uint32_t toff = tail ? 4u * (t * half + 8u * pj) : kOutOfRange;
      in.c0 = buf_load16f(rc, toff);
      in.c1 = buf_load16f(rc, toff + 16u);
      in.s0 = buf_load16f(rs, toff);
      in.s1 = buf_load16f(rs, toff + 16u);
    }
  };
  // (grad_x and rstd are not preloaded: their descriptors are made after the
  // first row's x, grad_y and table loads are out)
  rsrc_t rdx, rrs;
  auto load_rs = [&](uint32_t j, In& in) {
    if constexpr (SAVED) in.rs = buf_load4f(rrs, 4u * row_of(j));
  };
  auto load = [&](uint32_t j, In& in) {
    load_xg(j, in);
    load_tab(j, in);
    load_rs(j, in);
  };

  float4* dw_w = dw_s[wave];  // this wave's sums (touched by this wave alone until the end)
#pragma unroll
  for (int q = 0; q < 2 * KC; ++q) dw_w[q * 64 + lane] = make_float4(0.f, 0.f, 0.f, 0.f);

  // (the 16-bit values are unpacked again in each pass over the row: an empty
  // asm makes the packed registers opaque between passes, so the compiler
  // cannot keep a pass's 8 * KC unpacked floats live into the next one)
  auto opaque = [](In& in) {
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      asm volatile("" : "+v"(in.x[k].x), "+v"(in.x[k].y), "+v"(in.x[k].z), "+v"(in.x[k].w));
      asm volatile("" : "+v"(in.g[k].x), "+v"(in.g[k].y), "+v"(in.g[k].z), "+v"(in.g[k].w));
    }
  };
  auto wk = [&](int k, float* w) {
    const float4 a = w_f[(2 * k) * 64 + lane], b = w_f[(2 * k + 1) * 64 + lane];
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w; w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  };
  auto compute = [&](uint32_t j, In& in) {
    const uint32_t lr = row_of(j);
    float rstd;
    if constexpr (SAVED) {
      rstd = in.rs;
    } else {
      // (one accumulator per chunk, added pairwise: the chains stay short)
      double part[KC];
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        float xf[8];
        unpack8<DT>(in.x[k], xf);
        part[k] = 0.0;
#pragma unroll
        for (int i = 0; i < 8; ++i) part[k] = __builtin_fma((double)xf[i], (double)xf[i], part[k]);
      }
#pragma unroll
      for (int h = 1; h < KC; h *= 2)
#pragma unroll
        for (int k = 0; k + h < KC; k += 2 * h) part[k] += part[k + h];
      const double acc = group_sum<64>(part[0]);
      rstd = rstd_of((float)acc / (float)N + p.eps);
    }
    opaque(in);
    // the output gradient of the last slot, through the transposed rotation on the tail
    float gl[8];
    unpack8<DT>(in.g[KC - 1], gl);
    if constexpr (ROPE) {
      uint4 pg;
      pg.x = (uint32_t)__shfl((int)in.g[KC - 1].x, src, 64);
      pg.y = (uint32_t)__shfl((int)in.g[KC - 1].y, src, 64);
      pg.z = (uint32_t)__shfl((int)in.g[KC - 1].z, src, 64);
      pg.w = (uint32_t)__shfl((int)in.g[KC - 1].w, src, 64);
      float pf[8];
      unpack8<DT>(pg, pf);
      const float cc[8] = {in.c0.x, in.c0.y, in.c0.z, in.c0.w, in.c1.x, in.c1.y, in.c1.z, in.c1.w};
      const float ss[8] = {in.s0.x, in.s0.y, in.s0.z, in.s0.w, in.s1.x, in.s1.y, in.s1.z, in.s1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float own = gl[i] * cc[i];
        const float other = pf[i] * ss[i];
        const float r = lo_half ? own + other : own - other;
        gl[i] = tail ? r : gl[i];
      }
    }
    auto grad = [&](int k, float* gf) {
      if (k == KC - 1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) gf[i] = gl[i];
      } else {
        unpack8<DT>(in.g[k], gf);
      }
    };
    // C = mean(g * xn): lane-sequential within each chunk, the chunks added
    // pairwise, then the wave's butterfly
    float dot[KC];
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      float xf[8], gf[8], w[8];
      unpack8<DT>(in.x[k], xf);
      grad(k, gf);
      wk(k, w);
      dot[k] = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) dot[k] += (gf[i] * w[i]) * (xf[i] * rstd);
    }
#pragma unroll
    for (int h = 1; h < KC; h *= 2)
#pragma unroll
      for (int k = 0; k + h < KC; k += 2 * h) dot[k] += dot[k + h];
    const float C = group_sum<64>(dot[0]) / (float)N;
    opaque(in);
    const bool real = lr < nrows;  // (a row past the range adds nothing to grad_w)
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      float xf[8], gf[8], w[8], o[8], d[8];
      unpack8<DT>(in.x[k], xf);
      grad(k, gf);
      wk(k, w);
      const float4 d0 = dw_w[(2 * k) * 64 + lane], d1 = dw_w[(2 * k + 1) * 64 + lane];
      d[0] = d0.x; d[1] = d0.y; d[2] = d0.z; d[3] = d0.w;
      d[4] = d1.x; d[5] = d1.y; d[6] = d1.z; d[7] = d1.w;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float xn = xf[i] * rstd;
        o[i] = rstd * ((gf[i] * w[i]) - xn * C);
        d[i] += real ? gf[i] * xn : 0.f;
      }
      dw_w[(2 * k) * 64 + lane] = make_float4(d[0], d[1], d[2], d[3]);
      dw_w[(2 * k + 1) * 64 + lane] = make_float4(d[4], d[5], d[6], d[7]);
      // rows past the range are past the descriptor: the store is dropped
      // (nontemporal: ordinary stores measured no faster once the rotated
      // outputs exceed the Infinity Cache, and slower with RoPE)
      buf_store16_nt(rdx, lr * row_bytes + 16u * lane + 1024u * k, pack8<DT>(o));
    }
  };

  In a, b;
  load_xg(0, a);
  load_tab(0, a);
  __builtin_amdgcn_sched_barrier(0);
  rdx = make_rsrc(p.gx + (size_t)r0 * N, span);
  rrs = make_rsrc(p.rstd + r0, SAVED ? 4u * nrows : 0u);
  load_rs(0, a);
  // the weight row goes to LDS once the first row's loads are out (thread t
  // holds chunk t = lane + 64 k)
  if (tid < N / 8) {
    float wf8[8];
    unpack8<DT>(wc, wf8);
    const uint32_t kk = tid / 64, ll = tid % 64;
    w_f[(2 * kk) * 64 + ll] = make_float4(wf8[0], wf8[1], wf8[2], wf8[3]);
    w_f[(2 * kk + 1) * 64 + ll] = make_float4(wf8[4], wf8[5], wf8[6], wf8[7]);
  }
  lds_barrier();
  uint32_t s = 0;
  for (; s + 2 <= mine; s += 2) {
    load(s + 1, b);
    compute(s, a);
    load(s + 2, a);
    compute(s + 1, b);
  }
  if (s < mine) compute(s, a);

  // the 8 waves' sums by a fixed pairwise tree, ((0 + 1) + (2 + 3)) + ((4 +
  // 5) + (6 + 7)); thread t adds float4 q = t, t + 512, ... of the areas
  lds_barrier();
  const rsrc_t rp = make_rsrc(p.partial + (size_t)blockIdx.x * N, 4u * N);
#pragma unroll
  for (uint32_t q = tid; q < N / 4; q += RBT) {
    float4 v[RBW];
#pragma unroll
    for (int u = 0; u < RBW; ++u) v[u] = dw_s[u][q];
#pragma unroll
    for (int h = 1; h < RBW; h *= 2)
#pragma unroll
      for (int u = 0; u + h < RBW; u += 2 * h) {
        v[u].x += v[u + h].x; v[u].y += v[u + h].y; v[u].z += v[u + h].z; v[u].w += v[u + h].w;
      }
    // float4 q = (2 k + h) * 64 + l holds columns 8 (l + 64 k) + 4 h .. + 3
    const uint32_t l = q % 64, kh = q / 64;
    const uint32_t col = 8u * (l + 64u * (kh / 2)) + 4u * (kh % 2);
    buf_store16(rp, 4u * col, make_uint4(__float_as_uint(v[0].x), __float_as_uint(v[0].y), __float_as_uint(v[0].z),
                                         __float_as_uint(v[0].w)));
  }
}

template <class DT, int KC, bool ROPE>
void launch_saved(const WideBwdParams& p, hipStream_t s) {
  if (p.rstd != nullptr)
    hipLaunchKernelGGL((row_bwd_kernel<DT, KC, ROPE, true>), dim3(p.blocks), dim3(RBT), 0, s, p.x, p.gy, p.w, p.cos,
                       p.sin, p.M, p.rows_per_block, p.div_magic, p.div_shift | p.rope << 8, p);
  else
    hipLaunchKernelGGL((row_bwd_kernel<DT, KC, ROPE, false>), dim3(p.blocks), dim3(RBT), 0, s, p.x, p.gy, p.w, p.cos,
                       p.sin, p.M, p.rows_per_block, p.div_magic, p.div_shift | p.rope << 8, p);
}

template <class DT, int KC>
void launch_rope(const WideBwdParams& p, hipStream_t s) {
  if (p.rope > 0)
    launch_saved<DT, KC, true>(p, s);
  else
    launch_saved<DT, KC, false>(p, s);
}

template <class DT>
hipError_t launch_width(const WideBwdParams& p, hipStream_t s) {
  switch (p.N) {
    case 1024: launch_rope<DT, 2>(p, s); break;
    case 2048: launch_rope<DT, 4>(p, s); break;
    case 4096: launch_rope<DT, 8>(p, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool row_bwd_fits(int64_t N, int64_t rope) {
  return (N == 1024 || N == 2048 || N == 4096) && rope <= (int64_t)kMaxRowBwdRope;
}

hipError_t launch_row_bwd(WideBwdParams p, bool bf16, hipStream_t stream) {
  if (!row_bwd_fits(p.N, p.rope) || p.rope % 16 != 0) return hipErrorInvalidValue;
  if (p.rows_per_token == 0) p.rows_per_token = 1;
  // row / rows_per_token by multiply-shift (exact for every row < 2^31)
  div_magic_for(p.rows_per_token, p.div_magic, p.div_shift);
  const hipError_t e = bf16 ? launch_width<BF16>(p, stream) : launch_width<F16>(p, stream);
  if (e != hipSuccess) return e;
  return launch_dw_reduce(p.partial, p.gw, p.blocks, p.N, stream);
}

}  // namespace rnq
