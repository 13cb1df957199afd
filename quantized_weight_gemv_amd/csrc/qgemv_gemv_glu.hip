// Vector-ALU GEMV kernels: stacked gate + up Q4_0 table with the SwiGLU epilogue, fp32 activations in registers.
#include "qgemv_gemv_impl.h"

namespace qg {
template hipError_t launch_variant<kQ4_0, kModeGlu, false>(int, int, int, int, const GemvParams &, dim3, dim3, size_t,
                                                hipStream_t);
}  // namespace qg
