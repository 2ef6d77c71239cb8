// gemv_op5.hip -- instantiates the GEMV kernels of fused-transform variant
// kOpSwiglu (paired gate/up windows storing silu(gate . x) * (up . x); every format
// and team shape); see qgemv_impl.h.
#include "qgemv_impl.h"

namespace qgemv_detail {
template GemvFn pick_op<kOpSwiglu>(int32_t, Shape);
}  // namespace qgemv_detail
