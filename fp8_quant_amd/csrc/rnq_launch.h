// Kernel parameter blocks and launchers (internal to librnq.so).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

namespace rnq {

// Rows are (token, head) pairs in token-major order: heads [0, heads0) come
// from tensor 0 (q or x), heads [heads0, heads) from tensor 1 (k).
struct RowParams {
  const uint16_t* x0;
  const uint16_t* x1;
  const uint16_t* w0;
  const uint16_t* w1;
  const float* cos;  // [tokens, rope/2], or [max_pos, rope/2] gathered through positions
  const float* sin;
  const int32_t* positions;  // optional [tokens]: table row of each token (ROW_POS)
  uint64_t xs0;  // token strides of x0 / x1 in elements (rows of a token are contiguous)
  uint64_t xs1;
  uint32_t max_pos;  // table rows when positions are given (positions are clamped into range)
  uint8_t* c0;  // codes (quantising kernels)
  uint8_t* c1;
  float* s0;    // scales
  float* s1;
  uint16_t* y0;  // optional y (for both tensors or for neither)
  uint16_t* y1;
  float* rstd;   // optional per-row rstd, flattened row order
  uint32_t total_rows;
  uint32_t heads;
  uint32_t heads0;
  uint32_t rope;
  float eps;
  float fp8_max;
  // filled by the launcher
  float rcp_fp8_max;   // RN(1 / fp8_max)
  float scale_floor;   // RN(1e-4 / fp8_max)
  uint32_t scale_by_rcp;
  uint32_t clamp;       // clamp quotients to +-fp8_max before encoding
  uint32_t code16;      // both code outputs 16-byte aligned: whole 16-byte code stores allowed
  uint32_t passes;      // groups of 64 / (D / 16) consecutive rows
  uint32_t waves;       // waves that take passes (round-robin)
  uint32_t per_wave;    // passes per wave (the last ones repeat the final pass)
  uint32_t div_magic;
  uint32_t div_shift;
  uint32_t tok_shift;  // passes of whole tokens: log2(heads per token)
  uint32_t prio_by_progress;  // every wave resident at once: issue priority by passes done
};

// What a row-kernel launch computes and writes (bit set).
enum RowMode : int {
  ROW_QUANT = 1,  // fp8 codes + per-row scale
  ROW_ROPE = 2,   // rotate the rope tail
  ROW_Y = 4,      // write y (16-bit)
  ROW_RSTD = 8,   // write per-row rstd
  ROW_POS = 16,   // table row of token t is positions[t]
};

hipError_t launch_rows(RowParams p, int head_dim, bool bf16, bool quant, hipStream_t stream);

struct WideFwdParams {
  const uint16_t* x;
  const uint16_t* w;
  uint16_t* y;
  float* rstd;
  uint32_t M;
  uint32_t N;
  float eps;
};

hipError_t launch_wide_fwd(const WideFwdParams& p, bool bf16, hipStream_t stream);

struct WideBwdParams {
  const uint16_t* x;
  const uint16_t* w;
  const uint16_t* gy;
  const float* rstd;  // optional
  uint16_t* gx;
  float* gw;
  float* partial;     // [blocks, N] fp32 workspace
  uint32_t M;
  uint32_t N;
  uint32_t rows_per_block;
  uint32_t blocks;
  float eps;
  // the gradient goes back through the RoPE of the last `rope` columns first
  // (rope == 0: plain RMSNorm backward)
  const float* cos;  // [M / rows_per_token, rope / 2]
  const float* sin;
  uint32_t rope;
  uint32_t rows_per_token;
  uint32_t div_magic;   // row / rows_per_token = (row * div_magic) >> div_shift
  uint32_t div_shift;
  uint32_t table_bytes;  // bytes of one table (cos or sin)
};

// RMSNorm -> partial RoPE -> FP8 with one scale per group of group_size
// consecutive elements, over rows of up to 16384 elements (row r uses table
// row r / rows_per_token).
struct GroupQuantParams {
  const uint16_t* x;
  const uint16_t* w;
  const float* cos;  // [M / rows_per_token, rope / 2], or [max_pos, rope / 2] gathered through positions
  const float* sin;
  uint16_t* y;       // optional when quantising; the output of the no-quantise mode
  uint8_t* codes;    // [M, N] (quantising mode)
  float* scales;     // [M, N / group_size] (quantising mode)
  const int32_t* positions;  // optional [M / rows_per_token]: table row of each token (clamped into range)
  uint64_t xs;       // token stride of x in elements (0: contiguous rows; the launcher sets rows_per_token * N)
  uint32_t max_pos;  // table rows when positions are given (the launcher sets the table's rows otherwise)
  uint32_t M;
  uint32_t N;
  uint32_t rope;
  uint32_t rows_per_token;
  uint32_t group_size;  // 0: no quantisation (RMSNorm + RoPE into y only)
  float eps;
  float fp8_max;
  // filled by the launcher
  float rcp_fp8_max;
  float scale_floor;
  uint32_t scale_by_rcp;
  uint32_t clamp;
  uint32_t div_magic, div_shift;  // row / rows_per_token = (row * div_magic) >> div_shift
};

hipError_t launch_group_quant(GroupQuantParams p, bool bf16, hipStream_t stream);
// RMSNorm + RoPE (no quantisation) over rows of up to 16384 elements, one
// workgroup per row (the grouped kernel's mode that writes y only)
hipError_t launch_wide_norm_rope(GroupQuantParams p, bool bf16, hipStream_t stream);

// row / d for every row < 2^31 as (row * magic) >> shift (64-bit product):
// shift = 31 + lg with 2^lg >= d, magic = ceil(2^shift / d). With e = magic *
// d - 2^shift in [0, d): row * magic / 2^shift = row / d + row * e / (d *
// 2^shift), and the second term is below 2^31 / 2^shift = 2^-lg <= 1 / d,
// too small to carry row / d (fractional part at most (d - 1) / d) past the
// next integer, so the floor is exact.
inline void div_magic_for(uint32_t d, uint32_t& magic, uint32_t& shift) {
  uint32_t lg = 0;
  while ((1u << lg) < d) ++lg;
  shift = 31 + lg;
  magic = (uint32_t)((((uint64_t)1 << shift) + d - 1) / d);
}

// Host side: e4m3fn code magnitude of a positive value below 480 (nearest even).
inline int e4m3_magnitude_host(double v) {
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
inline bool fp8_clamp_needed(float fp8_max) {
  return e4m3_magnitude_host((double)fp8_max * (1.0 + 0x1p-20)) != e4m3_magnitude_host((double)fp8_max);
}

// How a row-kernel launch's passes of G rows sit in the rows: each lane
// locates its own row, a pass lies inside one token of one tensor (both head
// counts multiples of G), or a pass holds whole tokens of one tensor (G a
// multiple of the heads per token, whole passes only, the pass's input span
// below 2^31 bytes, and with positions a cos/sin table below 2^31 bytes, since
// such passes gather table rows at 32-bit offsets). For the last, tok_shift =
// log2(heads per token). Inputs: the token stride xs0 in elements (as the
// launcher fills it), the rope width (0: none) and whether positions are given.
enum RowsAlign : int { ROWS_PER_LANE = 0, ROWS_ONE_TOKEN = 1, ROWS_WHOLE_TOKENS = 2 };
inline int rows_layout(uint32_t G, uint32_t heads, uint32_t heads0, uint32_t total_rows, uint64_t xs0,
                       uint32_t head_dim, uint32_t rope, bool pos, uint32_t max_pos, uint32_t* tok_shift) {
  if (heads % G == 0 && heads0 % G == 0) return ROWS_ONE_TOKEN;
  if (heads0 != heads || G % heads != 0 || total_rows % G != 0) return ROWS_PER_LANE;
  uint32_t sh = 0;
  while ((1u << sh) < heads) ++sh;
  const uint64_t tpp = G >> sh;
  const uint64_t span = 2 * ((tpp - 1) * xs0 + (uint64_t)heads * (uint64_t)head_dim);
  const bool table_ok = !pos || (uint64_t)max_pos * (rope / 2) * 4 < ((uint64_t)1 << 31);
  if (span >= ((uint64_t)1 << 31) || xs0 >= ((uint64_t)1 << 30) || !table_ok) return ROWS_PER_LANE;
  *tok_shift = sh;
  return ROWS_WHOLE_TOKENS;
}

// Measurement baselines (rnq_baselines.hip): steps 2 and 3 of the unfused
// norm -> rope -> quant plan, and the chapter 28 designs (rows_per_block rows
// per workgroup, lookups staged once per workgroup).
hipError_t launch_unfused_rope_quant(const uint16_t* normed, const float* cos, const float* sin, uint16_t* rotated,
                                     uint8_t* codes, float* scales, uint32_t M, uint32_t N, uint32_t R,
                                     uint32_t rows_per_token, float fp8_max, bool bf16, hipStream_t s);
hipError_t launch_design(const RowParams& p, uint32_t rows_per_block, int D, bool bf16, hipStream_t s);
// src_bytes / 2048 blocks of the memory-floor kernel (0: one empty workgroup)
hipError_t launch_stream(const void* src, void* dst, uint32_t blocks, bool device_scope, hipStream_t s);

// Deterministic row partition used by the backward (rope_dim > 0: the RoPE
// backward); the workspace size covers every rope_dim.
uint32_t bwd_blocks(int64_t M, int64_t N, int64_t rope_dim);
hipError_t launch_wide_bwd(WideBwdParams p, bool bf16, hipStream_t stream);
// grad_w[j] = sum over b of partial[b, j] in a fixed order
hipError_t launch_dw_reduce(const float* partial, float* gw, uint32_t blocks, uint32_t N, hipStream_t stream);
// rows of 64, 128, 256 or 512 elements, several per wave; rope optional
bool narrow_bwd_width(int64_t N);
hipError_t launch_narrow_bwd(WideBwdParams p, bool bf16, hipStream_t stream);
// rows of 1024, 2048 or 4096 elements, one wave per row; rope at most 512
bool row_bwd_fits(int64_t N, int64_t rope_dim);
hipError_t launch_row_bwd(WideBwdParams p, bool bf16, hipStream_t stream);

}  // namespace rnq
