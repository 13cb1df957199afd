// Vector-ALU GEMV kernels: q2w weights against activations quantized to 8-bit blocks in LDS.
#include "qgemv_gemv_impl.h"

namespace qg {
template hipError_t launch_variant<kQ2W, kModeQ8Act, true>(int, int, int, int, const GemvParams &, dim3, dim3, size_t,
                                                hipStream_t);
}  // namespace qg
