// Internal declarations shared by the kernel and launcher translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace qg {

constexpr int kQ4_0 = 0;
constexpr int kQ8_0 = 1;
constexpr int kQ2W = 2;   // plain 2-bit: codes -2..1, one fp16 scale per 32

// Code bytes per 32-weight block of each packed format.
constexpr int code_bytes_per_block(int fmt) { return fmt == kQ4_0 ? 16 : fmt == kQ2W ? 8 : 32; }

constexpr int kMaxWavesPerWg = 8;   // 512 threads
constexpr int kMaxRM = 32;          // rows per group (<= 4) x tokens (<= 8)

// Weight bytes are read once per call, so both GEMV kernels load them
// non-temporal: the stream does not displace the activations from the caches
// (measured on MI355X: 6.5 TB/s against 6.0 TB/s with plain loads on the
// 296 MB 128256 x 4096 matrix).  The loads are buffer loads: a base address
// and extent live in a scalar resource descriptor, each lane adds a 32-bit
// offset, so no vector instruction is spent on 64-bit addresses, and the
// hardware range check returns zeros rather than reading past the matrix.
constexpr int kNtAux = 2;                     // cache policy: non-temporal
constexpr int kRsrcWord3 = 0x00020000;        // raw (untyped) buffer, gfx9 family

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const uint8_t *base, int64_t bytes)
{
    const int n = (int)min(bytes, (int64_t)0x7FFFFFFF);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(base), (short)0, n, kRsrcWord3);
}

__device__ __forceinline__ uint4 stream_load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    const auto t = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNtAux);
    return make_uint4(t[0], t[1], t[2], t[3]);
}

__device__ __forceinline__ uint2 stream_load8(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    const auto t = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kNtAux);
    return make_uint2(t[0], t[1]);
}

__device__ __forceinline__ uint16_t stream_load2(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, kNtAux);
}

// Arguments of the GEMV / MoE kernel (passed by value).
struct GemvParams {
    const uint8_t *W;          // packed matrix, or the expert pool for MoE
    const int32_t *idx;        // MoE: expert index per batch item; nullptr for GEMV
    const uint16_t *x;         // fp16 activations [items][M][K]
    const float *xf;           // fp32 activations [M][K] (fp32-input modes)
    float *y;                  // fp32 outputs [items][M][N]
    int64_t matrix_stride;     // bytes between pool matrices (MoE)
    int64_t pool;              // MoE: matrices in the pool (valid indices 0..pool-1)
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

// Activation modes of the vector-ALU GEMV kernel: fp16 activations; fp32
// activations rounded to binary16 as they are loaded (Q4_0); fp32
// activations and a stacked gate + up table (2N rows) with the SwiGLU
// epilogue y = silu(gate) * up (Q4_0, two row sets: a gate set and the up
// set N rows further); fp16 activations quantized to 8-bit blocks in LDS and
// multiplied with int8 dot products (Q4_0, LDS staging only).
constexpr int kModeF16 = 0;
constexpr int kModeF32 = 1;
constexpr int kModeGlu = 2;
constexpr int kModeQ8Act = 3;

// Which vector-ALU GEMV instantiations exist (G lanes per row, J blocks per
// lane, R row sets per group, xl: activations in LDS).  Register estimate: R *
// J code words and scales in flight twice (ping-pong; 5 registers per Q4_0
// block, 9 per Q8_0 block), without XL J * M resident activation blocks of 16
// registers (counted as 18, 2 of slack), R * M sums and ~36 temporaries; keeping it
// within 256 (and R * J <= 8 / 4, J <= 7, 8 with XL, J * M <= 8) leaves every
// instantiation free of spills.  Rows narrower than a wave (G < 64) are for
// one token; XL uses G = 64 and up to 4 tokens.
constexpr bool gemv_fits(int fmt, int M, int G, int J, int R, bool xl, int mode = 0)
{
    if (G != 16 && G != 32 && G != 64)
        return false;
    if (M != 1 && G != 64)
        return false;
    if (xl && (G != 64 || M > 4))
        return false;
    if (mode == kModeQ8Act && (!xl || fmt == kQ8_0))
        return false;
    if (R * J > (fmt == kQ8_0 ? 4 : 8) || J > (xl ? 8 : 7) || (!xl && J * M > 8))
        return false;
    // fp32 activations (mode != 0) hold 32 raw words per block until they
    // are converted, 16 more than fp16 ones
    const int regs = 2 * R * J * (fmt == kQ4_0 ? 5 : fmt == kQ2W ? 3 : 9) + (xl ? 0 : J * M * (mode ? 34 : 18)) +
                     R * M + 36;
    return regs <= 256 && R * M * (64 / G) <= kMaxRM;
}

// LDS bytes of the XL activation copy of M tokens for rows of K weights
// (per block: 64 bytes of fp16 pairs, or 32 int8 codes and 16 bytes of scale
// and offset with 8-bit activations).
size_t gemv_xl_lds_bytes(int K, int M, int mode);


hipError_t launch_gemv(int fmt, int M, int G, int J, int R, bool xl, int mode, const GemvParams &p, dim3 grid,
                       dim3 block, hipStream_t stream);

// Every launch shape (M tokens, G lanes per row, J blocks per lane, R row
// sets per group) of one vector-ALU kernel variant; defined in
// qgemv_gemv_impl.h and instantiated per variant in qgemv_gemv_*.hip.
template <int FMT, int MODE, bool XL>
hipError_t launch_variant(int M, int G, int J, int R, const GemvParams &p, dim3 grid, dim3 block, size_t shmem,
                          hipStream_t stream);

// Few-token GEMV on the matrix cores (qgemv_mfma.hip), fp16 activations x or
// fp32 activations xf (Q4_0, non-null xf), with glu the SwiGLU of a stacked
// gate + up table (Q4_0, fp32): `waves` waves split K; `teams` teams of
// them per workgroup share one staged copy of the activations (1 or 2; 0:
// two at 1.5-4 tiles of 16 rows per CU, else one); `wgs` persistent
// workgroups (0: as many as fit, at most 2 per CU of `cus` with one team, 1
// with two).
hipError_t launch_gemv_mfma(int fmt, const uint8_t *W, int64_t scale_offset, const uint16_t *x, const float *xf,
                            float *y, int M, int N, int K, int waves, int teams, int64_t wgs, int cus,
                            hipStream_t stream, bool glu = false);

// Prefill for 1..64 tokens on the matrix cores (qgemv_mfma.hip): weights
// streamed once in 16-row tiles, activations held as MFMA operands in
// registers; `wgs` persistent workgroups along N (0: one per CU of `cus`).
hipError_t launch_prefill_skinny(const uint8_t *W, int64_t scale_offset, const uint16_t *X, float *Y, int M, int N,
                                 int K, int cus, int64_t wgs, hipStream_t stream);

// Zero n floats of y (a small fill kernel, no memset: safe inside captured
// graphs) before split work adds its parts into y (qgemv_prefill.hip).
hipError_t launch_zero_fill(float *y, int64_t n, int cus, hipStream_t stream);

// Times-table GEMV for q2w at one token (qgemv_lut.hip): LDS bytes of the
// tables for rows of K weights (64 KB for 32 <= K <= 4096, else SIZE_MAX),
// and the launcher (up to two workgroups per CU of `cus`).
size_t gemv_lut_lds_bytes(int K);
hipError_t launch_gemv_q2w_lut(const uint8_t *W, int64_t scale_offset, const uint16_t *x, float *y, int N, int K,
                               int cus, hipStream_t stream);

}  // namespace qg
