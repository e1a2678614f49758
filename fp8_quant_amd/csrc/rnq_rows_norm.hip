// Row-kernel modes without quantisation (RMSNorm, RMSNorm + RoPE).
#include "rnq_rows_inst.h"

namespace rnq {

template hipError_t launch_rows_mode<ROW_Y>(const RowParams&, int, bool, int, dim3, hipStream_t);
template hipError_t launch_rows_mode<ROW_Y | ROW_ROPE>(const RowParams&, int, bool, int, dim3, hipStream_t);
template hipError_t launch_rows_mode<ROW_Y | ROW_RSTD>(const RowParams&, int, bool, int, dim3, hipStream_t);

}  // namespace rnq
