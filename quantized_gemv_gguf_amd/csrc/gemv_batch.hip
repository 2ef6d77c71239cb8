// gemv_batch.hip -- instantiates the several-token GEMV kernels (two and four
// tokens per launch, no fused transform; every format, one column per lane);
// see qgemv_impl.h.
#include "qgemv_impl.h"

namespace qgemv_detail {
template GemvFn pick_batch<2>(int32_t, Shape);
template GemvFn pick_batch<4>(int32_t, Shape);
}  // namespace qgemv_detail
