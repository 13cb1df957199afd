// Vector-ALU GEMV kernels: Q4_0 weights against activations quantized to 8-bit blocks in LDS.
#include "qgemv_gemv_impl.h"

namespace qg {
template hipError_t launch_variant<kQ4_0, kModeQ8Act, true>(int, int, int, int, const GemvParams &, dim3, dim3, size_t,
                                                hipStream_t);
}  // namespace qg
