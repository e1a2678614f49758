// Launch of one row-kernel mode for every row width and dtype (included by
// the translation units that instantiate the modes).
#pragma once

#include "rnq_rows.h"

namespace rnq {

// (the fields a wave needs before its first input load go first, as scalar
// arguments the hardware preloads; on passes of whole tokens the slots of the
// second tensor, the token strides and the head division carry the weight,
// cos, sin and positions pointers, the token stride and the token shift, as
// RowHot lays out)
#define RNQ_ROWS_HOT(p, mt)                                                                                       \
  (p).x0, (mt) ? (uint64_t)(uintptr_t)(p).w0 : (uint64_t)(uintptr_t)(p).x1,                                       \
      (mt) ? (uint64_t)(uintptr_t)(p).cos : (p).xs0, (mt) ? (uint64_t)(uintptr_t)(p).sin : (p).xs1, (p).waves,     \
      (p).passes, (mt) ? (uint32_t)(uintptr_t)(p).positions : (p).heads,                                           \
      (mt) ? (uint32_t)((uintptr_t)(p).positions >> 32) : (p).heads0, (mt) ? (uint32_t)(p).xs0 : (p).div_magic,    \
      ((mt) ? (p).tok_shift : (p).div_shift) | (p).rope << 8, (p)

template <class DT, int L, int MODE>
static hipError_t launch_shape(const RowParams& p, int align, dim3 grid, hipStream_t s) {
  if (align == ROWS_WHOLE_TOKENS) {
    hipLaunchKernelGGL((rows_kernel<DT, L, MODE, true, true>), grid, dim3(RT), 0, s, RNQ_ROWS_HOT(p, true));
    return hipGetLastError();
  }
  if (align == ROWS_ONE_TOKEN)
    hipLaunchKernelGGL((rows_kernel<DT, L, MODE, true>), grid, dim3(RT), 0, s, RNQ_ROWS_HOT(p, false));
  else if (align == ROWS_PER_LANE)
    hipLaunchKernelGGL((rows_kernel<DT, L, MODE, false>), grid, dim3(RT), 0, s, RNQ_ROWS_HOT(p, false));
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// One 16-byte chunk of each half of a unit per lane: 8 lanes own a 128-wide
// row, so each wave-wide input access covers whole 128-byte spans of 8 rows,
// and each code store whole 128-byte rows (64-byte halves where the rope tail
// does not allow the lane-pair swap).
template <class DT, int MODE>
static hipError_t launch_dt(const RowParams& p, int D, int align, dim3 grid, hipStream_t s) {
  switch (D) {
    case 64: return launch_shape<DT, 4, MODE>(p, align, grid, s);
    case 128: return launch_shape<DT, 8, MODE>(p, align, grid, s);
    case 256: return launch_shape<DT, 16, MODE>(p, align, grid, s);
    case 512: return launch_shape<DT, 32, MODE>(p, align, grid, s);
    default: return hipErrorInvalidValue;
  }
}

template <int MODE>
hipError_t launch_rows_mode(const RowParams& p, int head_dim, bool bf16, int align, dim3 grid, hipStream_t s) {
  return bf16 ? launch_dt<BF16, MODE>(p, head_dim, align, grid, s)
              : launch_dt<F16, MODE>(p, head_dim, align, grid, s);
}

}  // namespace rnq
