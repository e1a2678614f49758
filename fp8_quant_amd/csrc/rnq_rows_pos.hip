// Row-kernel modes whose cos/sin rows are gathered through a positions index.
#include "rnq_rows_inst.h"

namespace rnq {

template hipError_t launch_rows_mode<ROW_QUANT | ROW_ROPE | ROW_POS>(const RowParams&, int, bool, int, dim3, hipStream_t);
template hipError_t launch_rows_mode<ROW_QUANT | ROW_ROPE | ROW_Y | ROW_POS>(const RowParams&, int, bool, int, dim3,
                                                                          hipStream_t);
template hipError_t launch_rows_mode<ROW_Y | ROW_ROPE | ROW_POS>(const RowParams&, int, bool, int, dim3, hipStream_t);

}  // namespace rnq
