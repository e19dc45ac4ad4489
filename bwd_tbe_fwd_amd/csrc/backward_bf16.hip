// Short-run and long-apply kernels for bf16 weights (see backward_kernels.h).
#include "backward_launch.h"

namespace tbe {
template tbe_status launch_short_and_apply<2>(const tbe_tables*, void*, float*, int, const float*,
                                              const float*, float, float, char*, const BwdLayout&,
                                              int, const Config&, hipStream_t, hipStream_t);
}  // namespace tbe
