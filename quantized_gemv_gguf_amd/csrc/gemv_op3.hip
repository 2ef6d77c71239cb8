// gemv_op3.hip -- instantiates the GEMV kernels of fused-transform variant
// kOpSilu (every format and team shape); see qgemv_impl.h.
#include "qgemv_impl.h"

namespace qgemv_detail {
template GemvFn pick_op<kOpSilu>(int32_t, Shape);
}  // namespace qgemv_detail
