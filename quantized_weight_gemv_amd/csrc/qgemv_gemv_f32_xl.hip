// Vector-ALU GEMV kernels: Q4_0 weights, fp32 activations rounded into LDS (1-4 tokens).
#include "qgemv_gemv_impl.h"

namespace qg {
template hipError_t launch_variant<kQ4_0, kModeF32, true>(int, int, int, int, const GemvParams &, dim3, dim3, size_t,
                                                hipStream_t);
}  // namespace qg
