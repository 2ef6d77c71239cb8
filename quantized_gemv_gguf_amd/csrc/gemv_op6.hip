// gemv_op6.hip -- instantiates the GEMV kernels of fused-transform variant
// kOpRmsSwiglu (paired gate/up windows storing silu(gate . x) * (up . x); every format
// and team shape); see qgemv_impl.h.
#include "qgemv_impl.h"

namespace qgemv_detail {
template GemvFn pick_op<kOpRmsSwiglu>(int32_t, Shape);
}  // namespace qgemv_detail
