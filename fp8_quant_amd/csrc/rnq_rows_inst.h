// Launch of one row-kernel mode for every row width and dtype (included by
// the translation units that instantiate the modes).
#pragma once

#include "rnq_rows.h"

namespace rnq {

template <class DT, int L, int MODE>
static hipError_t launch_shape(const RowParams& p, bool aligned, dim3 grid, hipStream_t s) {
  if (aligned)
    hipLaunchKernelGGL((rows_kernel<DT, L, MODE, true>), grid, dim3(RT), 0, s, p);
  else
    hipLaunchKernelGGL((rows_kernel<DT, L, MODE, false>), grid, dim3(RT), 0, s, p);
  return hipGetLastError();
}

// One 16-byte chunk of each half of a unit per lane: 8 lanes own a 128-wide
// row, so each wave-wide input access covers whole 128-byte spans of 8 rows,
// and each code store whole 128-byte rows (64-byte halves where the rope tail
// does not allow the lane-pair swap).
template <class DT, int MODE>
static hipError_t launch_dt(const RowParams& p, int D, bool aligned, dim3 grid, hipStream_t s) {
  switch (D) {
    case 64: return launch_shape<DT, 4, MODE>(p, aligned, grid, s);
    case 128: return launch_shape<DT, 8, MODE>(p, aligned, grid, s);
    case 256: return launch_shape<DT, 16, MODE>(p, aligned, grid, s);
    case 512: return launch_shape<DT, 32, MODE>(p, aligned, grid, s);
    default: return hipErrorInvalidValue;
  }
}

template <int MODE>
hipError_t launch_rows_mode(const RowParams& p, int head_dim, bool bf16, bool aligned, dim3 grid, hipStream_t s) {
  return bf16 ? launch_dt<BF16, MODE>(p, head_dim, aligned, grid, s)
              : launch_dt<F16, MODE>(p, head_dim, aligned, grid, s);
}

}  // namespace rnq
