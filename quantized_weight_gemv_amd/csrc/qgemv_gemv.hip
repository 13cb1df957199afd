// Dispatch of the vector-ALU GEMV / MoE kernel (qgemv_gemv_impl.h) to the
// instantiated variant of each weight format and activation mode.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "qgemv_internal.h"

namespace qg {

size_t gemv_xl_lds_bytes(int K, int M, int mode)
{
    return (size_t)M * (K / 32 + 1) * (mode == kModeQ8Act ? 48 : 64);
}

hipError_t launch_gemv(int fmt, int M, int G, int J, int R, bool xl, int mode, const GemvParams &p, dim3 grid,
                       dim3 block, hipStream_t stream)
{
    // fp32 activations (and SwiGLU): Q4_0 only; 8-bit activations: Q4_0, q2w
    if (mode != kModeF16 && fmt != kQ4_0 && !(mode == kModeQ8Act && fmt == kQ2W))
        return hipErrorInvalidValue;
    if (xl) {
        // XL: up to 4 tokens with whole rows per wave, activations staged in
        // LDS (per token K/32 blocks of 64 bytes plus a zero block)
        if (M > 4 || p.ksplit != 1)
            return hipErrorInvalidValue;
        const size_t shmem = gemv_xl_lds_bytes(p.K, M, mode);
        if (mode == kModeF32)
            return launch_variant<kQ4_0, kModeF32, true>(M, G, J, R, p, grid, block, shmem, stream);
        if (mode == kModeQ8Act)
            return fmt == kQ2W ? launch_variant<kQ2W, kModeQ8Act, true>(M, G, J, R, p, grid, block, shmem, stream)
                               : launch_variant<kQ4_0, kModeQ8Act, true>(M, G, J, R, p, grid, block, shmem, stream);
        if (mode == kModeGlu)
            return launch_variant<kQ4_0, kModeGlu, true>(M, G, J, R, p, grid, block, shmem, stream);
        if (fmt == kQ4_0)
            return launch_variant<kQ4_0, kModeF16, true>(M, G, J, R, p, grid, block, shmem, stream);
        if (fmt == kQ2W)
            return launch_variant<kQ2W, kModeF16, true>(M, G, J, R, p, grid, block, shmem, stream);
        return launch_variant<kQ8_0, kModeF16, true>(M, G, J, R, p, grid, block, shmem, stream);
    }
    if (mode == kModeQ8Act)
        return hipErrorInvalidValue;   // quantized into LDS: XL only
    if (mode == kModeF32)
        return launch_variant<kQ4_0, kModeF32, false>(M, G, J, R, p, grid, block, 0, stream);
    if (mode == kModeGlu)
        return launch_variant<kQ4_0, kModeGlu, false>(M, G, J, R, p, grid, block, 0, stream);
    if (fmt == kQ4_0)
        return launch_variant<kQ4_0, kModeF16, false>(M, G, J, R, p, grid, block, 0, stream);
    if (fmt == kQ2W)
        return launch_variant<kQ2W, kModeF16, false>(M, G, J, R, p, grid, block, 0, stream);
    return launch_variant<kQ8_0, kModeF16, false>(M, G, J, R, p, grid, block, 0, stream);
}

}  // namespace qg
