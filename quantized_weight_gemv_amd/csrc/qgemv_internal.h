// Internal declarations shared by the kernel and launcher translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace qg {

constexpr int kQ4_0 = 0;
constexpr int kQ8_0 = 1;

constexpr int kMaxWavesPerWg = 8;   // 512 threads
constexpr int kMaxRM = 32;          // rows per group (<= 4) x tokens (<= 8)

// Arguments of the GEMV / MoE kernel (passed by value).
struct GemvParams {
    const uint8_t *W;          // packed matrix, or the expert pool for MoE
    const int32_t *idx;        // MoE: expert index per batch item; nullptr for GEMV
    const uint16_t *x;         // fp16 activations [items][M][K]
    float *y;                  // fp32 outputs [items][M][N]
    int64_t matrix_stride;     // bytes between pool matrices (MoE)
    int64_t scale_offset;      // byte offset of the scale region in one matrix
    int N;
    int K;
    int ksplit;                // waves sharing one row group along K
    int teams_per_wg;          // independent teams per workgroup
};

// Launch with the one-shot timing events armed by qg_time_next_launch, if
// any; otherwise a plain launch.  `args` is the single by-value parameter.
template <typename P>
hipError_t launch_kernel(const void *fn, dim3 grid, dim3 block, size_t shmem, hipStream_t stream, const P &args);

hipError_t launch_raw(const void *fn, dim3 grid, dim3 block, void **args, size_t shmem, hipStream_t stream);

template <typename P>
inline hipError_t launch_kernel(const void *fn, dim3 grid, dim3 block, size_t shmem, hipStream_t stream,
                                const P &args)
{
    void *a[] = {const_cast<P *>(&args)};
    return launch_raw(fn, grid, block, a, shmem, stream);
}

hipError_t launch_gemv(int fmt, int M, int J, int R, bool xl, const GemvParams &p, dim3 grid, dim3 block,
                       hipStream_t stream);

// Few-token GEMV on the matrix cores (qgemv_mfma.hip): `waves` waves split K.
hipError_t launch_gemv_mfma(int fmt, const uint8_t *W, int64_t scale_offset, const uint16_t *x, float *y, int M,
                            int N, int K, int waves, hipStream_t stream);

}  // namespace qg
