// gemv_op0.hip -- instantiates the GEMV kernels of fused-transform variant
// kOpNone (every format and team shape); see qgemv_impl.h.
#include "qgemv_impl.h"

namespace qgemv_detail {
template GemvFn pick_op<kOpNone>(int32_t, Shape);
}  // namespace qgemv_detail
