// gemv_op4.hip -- instantiates the GEMV kernels of fused-transform variant
// kOpGelu (every format and team shape); see qgemv_impl.h.
#include "qgemv_impl.h"

namespace qgemv_detail {
template GemvFn pick_op<kOpGelu>(int32_t, Shape);
}  // namespace qgemv_detail
