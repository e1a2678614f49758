// Row-kernel modes that write fp8 codes (QK-norm + RoPE + FP8).
#include "rnq_rows_inst.h"

namespace rnq {

template hipError_t launch_rows_mode<ROW_QUANT>(const RowParams&, int, bool, int, dim3, hipStream_t);
template hipError_t launch_rows_mode<ROW_QUANT | ROW_ROPE>(const RowParams&, int, bool, int, dim3, hipStream_t);
template hipError_t launch_rows_mode<ROW_QUANT | ROW_Y>(const RowParams&, int, bool, int, dim3, hipStream_t);
template hipError_t launch_rows_mode<ROW_QUANT | ROW_ROPE | ROW_Y>(const RowParams&, int, bool, int, dim3, hipStream_t);

}  // namespace rnq
