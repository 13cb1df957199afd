// Q4_0 prefill GEMM on the gfx950 matrix cores:
//   Y[m][n] = sum_k X[m][k] * w[n][k],  w = (q - 8) * d
//
// With many tokens the work is a dense contraction, so it belongs on MFMA:
// each workgroup stages a BM x 64 activation tile and a BN x 64 weight tile
// in LDS per step, the weight tile dequantized on the way in (packed codes ->
// fp16 values, the same round-to-nearest-even values qdequant_q4_0 writes),
// and four waves multiply them with v_mfma_f32_32x32x16_f16 into fp32
// accumulators [volta-kernel-bakeoff, "What's in the race" (tc_q4: unpack a
// tile to shared memory, then matrix-core multiply) and "Stage 3" (unpack
// inside the multiply instead of dequantize-to-fp16 followed by a dense GEMM)].
//
// Pipeline per 64-wide K step: the global loads of the next three steps are in
// flight in registers; the MFMAs of step s run out of one of two LDS buffers
// while the next step is dequantized into the other, one barrier per step.  Both tiles are stored in the same permuted
// k order within each 32-element block (the order the nibble unpack produces),
// which leaves the contraction unchanged.  When the output tiles are too few
// to occupy the chip, K is split across workgroups that add their partial
// tiles with fp32 atomics into a zero-filled Y.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "qgemv.h"
#include "qgemv_tuning.h"
#include "qgemv_internal.h"

namespace qg {
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f16x_t __attribute__((ext_vector_type(16)));

constexpr int kBK = 64;          // K per pipeline step: two Q4_0 blocks
constexpr int kDepth = 3;        // K steps of global loads in flight
constexpr int kLdsStride = 72;   // halves per LDS tile row: 64 + 8 padding

__device__ __forceinline__ h2_t as_h2(uint32_t u) { return __builtin_bit_cast(h2_t, u); }
__device__ __forceinline__ uint32_t as_u32(h2_t h) { return __builtin_bit_cast(uint32_t, h); }

__device__ __forceinline__ uint32_t magic_reg()
{
    uint32_t m;
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(m));
    return m;
}

// One Q4_0 block -> 16 words of fp16 pairs (q - 8) * d, rounded to nearest
// even, in the permuted order
//   word 4t+0 = (e[4t], e[4t+2])      word 4t+2 = (e[4t+1], e[4t+3])
//   word 4t+1 = (e[16+4t], e[18+4t])  word 4t+3 = (e[17+4t], e[19+4t])
// (q - 8) is exact in fp16 (1024 + q from the 0x6400 pattern, minus 1032;
// for the high nibbles (1024 + 16 q) / 16 - 72); the product with d is one
// correctly rounded fp16 multiply.
__device__ __forceinline__ void dequant_block_f16(const uint4 c, uint16_t dbits, uint32_t (&o)[16])
{
    const uint32_t kMagic = magic_reg();
    const h2_t kOffLo = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const h2_t kScaleHi = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2_t kOffHi = {(_Float16)-72.0f, (_Float16)-72.0f};
    const _Float16 dh = __builtin_bit_cast(_Float16, dbits);
    const h2_t d2 = {dh, dh};
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint32_t a = w[t];
        const uint32_t b = w[t] >> 8;
        o[4 * t + 0] = as_u32((as_h2((a & 0x000F000Fu) | kMagic) + kOffLo) * d2);
        o[4 * t + 1] = as_u32((as_h2((a & 0x00F000F0u) | kMagic) * kScaleHi + kOffHi) * d2);
        o[4 * t + 2] = as_u32((as_h2((b & 0x000F000Fu) | kMagic) + kOffLo) * d2);
        o[4 * t + 3] = as_u32((as_h2((b & 0x00F000F0u) | kMagic) * kScaleHi + kOffHi) * d2);
    }
}

__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) { return (a & 0xFFFFu) | (b << 16); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }

// 32 activations (natural order, 16 words) -> the permuted order above.
__device__ __forceinline__ void permute_x(const uint32_t (&d)[16], uint32_t (&o)[16])
{
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        o[4 * t + 0] = pair_lo(d[2 * t], d[2 * t + 1]);
        o[4 * t + 2] = pair_hi(d[2 * t], d[2 * t + 1]);
        o[4 * t + 1] = pair_lo(d[8 + 2 * t], d[9 + 2 * t]);
        o[4 * t + 3] = pair_hi(d[8 + 2 * t], d[9 + 2 * t]);
    }
}

struct PrefillParams {
    const uint8_t *W;          // packed Q4_0 matrix
    const uint16_t *X;         // fp16 [M][K]
    float *Y;                  // fp32 [M][N]
    int64_t scale_offset;
    int M, N, K;
    int steps_per_split;       // K steps (of 64) per workgroup along z
    int atomic;                // 1: add partial tiles into Y (split K)
};

// Per-thread staging registers for one K step.
template <int BM, int BN>
struct Stage {
    static constexpr int kXChunks = (BM * 2 + 255) / 256;   // 32-element chunks per thread
    static constexpr int kWBlocks = (BN * 2 + 255) / 256;   // Q4_0 blocks per thread
    uint4 x[kXChunks][4];
    uint4 code[kWBlocks];
    uint16_t scale[kWBlocks];
};

template <int BM, int BN>
__device__ __forceinline__ void load_stage(Stage<BM, BN> &st, const PrefillParams &p, int m0, int n0, int step)
{
    const int tid = threadIdx.x;
    const int KB = p.K >> 5;
    // Every thread issues every load (threads past the tile repeat its last
    // chunk): with no load under a condition the compiler can wait for
    // exactly the stage it needs while the later stages stay in flight.
#pragma unroll
    for (int c = 0; c < Stage<BM, BN>::kXChunks; ++c) {
        const int idx = min(tid + 256 * c, BM * 2 - 1);   // chunk index within the BM x 2 tile
        const int r = idx >> 1, b = idx & 1;
        const int m = min(m0 + r, p.M - 1);
        const int kb = min(step * 2 + b, KB - 1);
        const uint4 *src = reinterpret_cast<const uint4 *>(p.X + (int64_t)m * p.K + (int64_t)kb * 32);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            st.x[c][q] = src[q];
    }
#pragma unroll
    for (int c = 0; c < Stage<BM, BN>::kWBlocks; ++c) {
        const int idx = min(tid + 256 * c, BN * 2 - 1);
        const int r = idx >> 1, b = idx & 1;
        const int64_t n = min(n0 + r, p.N - 1);
        const int kb = min(step * 2 + b, KB - 1);
        const int64_t bi = n * KB + kb;
        typedef unsigned int v4u __attribute__((ext_vector_type(4)));
        const v4u t = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p.W + bi * 16));
        st.code[c] = make_uint4(t.x, t.y, t.z, t.w);
        st.scale[c] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(p.W + p.scale_offset) + bi);
    }
}

template <int BM, int BN>
__device__ __forceinline__ void store_stage(const Stage<BM, BN> &st, const PrefillParams &p, int m0, int n0, int step,
                                            uint16_t (*Xs)[kLdsStride], uint16_t (*Ws)[kLdsStride])
{
    const int tid = threadIdx.x;
    const int KB = p.K >> 5;
    // Threads past the tile store a repeat of its last chunk: the same bytes
    // to the same place, so no store needs a condition either.  Activation
    // rows past M and blocks past K hold clamped copies of real activations
    // and are stored as they are: rows past M only reach output rows that are
    // never written, and blocks past K meet weights whose scale is zeroed
    // below.  (With no select the step body is one basic block.)
#pragma unroll
    for (int c = 0; c < Stage<BM, BN>::kXChunks; ++c) {
        const int idx = min(tid + 256 * c, BM * 2 - 1);
        const int r = idx >> 1, b = idx & 1;
        {
            uint32_t d[16], o[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                d[4 * q + 0] = st.x[c][q].x;
                d[4 * q + 1] = st.x[c][q].y;
                d[4 * q + 2] = st.x[c][q].z;
                d[4 * q + 3] = st.x[c][q].w;
            }
            permute_x(d, o);
            uint4 *dst = reinterpret_cast<uint4 *>(&Xs[r][b * 32]);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                dst[q] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
        }
    }
#pragma unroll
    for (int c = 0; c < Stage<BM, BN>::kWBlocks; ++c) {
        const int idx = min(tid + 256 * c, BN * 2 - 1);
        const int r = idx >> 1, b = idx & 1;
        {
            const bool ok = (n0 + r < p.N) && (step * 2 + b < KB);
            uint32_t o[16];
            dequant_block_f16(st.code[c], ok ? st.scale[c] : (uint16_t)0, o);
            uint4 *dst = reinterpret_cast<uint4 *>(&Ws[r][b * 32]);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                dst[q] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
        }
    }
}

template <int BM, int BN>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillParams p)
{
    constexpr int TM = BM / 64;   // 32 x 32 MFMA tiles per wave along M
    constexpr int TN = BN / 64;   // ... along N
    __shared__ __attribute__((aligned(16))) uint16_t Xs[2][BM][kLdsStride];
    __shared__ __attribute__((aligned(16))) uint16_t Ws[2][BN][kLdsStride];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;   // 2 x 2 waves
    const int n0 = blockIdx.x * BN;
    const int m0 = blockIdx.y * BM;
    const int nsteps = (p.K / 32 + 1) / 2;
    const int s_beg = blockIdx.z * p.steps_per_split;
    const int s_end = min(nsteps, s_beg + p.steps_per_split);

    f16x_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.0f;

    // A ring of kDepth register stages keeps the global loads of the next
    // kDepth K steps in flight.  Each iteration first issues the MFMAs of
    // step s (reading LDS buffer s & 1), then unpacks and stores step s + 1
    // into the other buffer, so the vector-ALU dequantization runs while the
    // matrix cores work; one barrier per step.  The buffer written in
    // iteration s was last read in iteration s - 1, before its barrier.
    //
    // Every stage load is issued unconditionally, also past the workgroup's
    // last step (load_stage clamps to valid blocks; such stages are never
    // multiplied): with the same load order on every path into the loop the
    // compiler waits only for the stage a step consumes, while the later
    // stages stay in flight.
    Stage<BM, BN> st[kDepth];
#pragma unroll
    for (int q = 0; q < kDepth; ++q)
        load_stage<BM, BN>(st[q], p, m0, n0, s_beg + q);
    store_stage<BM, BN>(st[0], p, m0, n0, s_beg, Xs[0], Ws[0]);
    load_stage<BM, BN>(st[0], p, m0, n0, s_beg + kDepth);
    __syncthreads();

    auto multiply = [&](int buf) {
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) {
            const int col = kk * 16 + (lane >> 5) * 8;
            half8_t a[TM], b[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                a[i] = *reinterpret_cast<const half8_t *>(&Xs[buf][wm * (BM / 2) + 32 * i + (lane & 31)][col]);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                b[j] = *reinterpret_cast<const half8_t *>(&Ws[buf][wn * (BN / 2) + 32 * j + (lane & 31)][col]);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    };

    // Steps s0 .. s0 + kDepth - 1 per iteration, ring slot (s - s_beg) %
    // kDepth static once unrolled.  Staging step s + 1 = s_end (last step
    // of the last iteration) fills the unused buffer with data never read.
    int s0 = s_beg;
    for (; s0 + kDepth <= s_end; s0 += kDepth) {
#pragma unroll
        for (int q = 0; q < kDepth; ++q) {
            const int s = s0 + q;
            const int buf = (s - s_beg) & 1;
            multiply(buf);
            const int qn = (q + 1) % kDepth;
            store_stage<BM, BN>(st[qn], p, m0, n0, s + 1, Xs[buf ^ 1], Ws[buf ^ 1]);
            load_stage<BM, BN>(st[qn], p, m0, n0, s + 1 + kDepth);
            __syncthreads();
        }
    }
#pragma unroll
    for (int q = 0; q < kDepth - 1; ++q) {
        const int s = s0 + q;
        if (s < s_end) {
            const int buf = (s - s_beg) & 1;
            multiply(buf);
            if (s + 1 < s_end)
                store_stage<BM, BN>(st[(q + 1) % kDepth], p, m0, n0, s + 1, Xs[buf ^ 1], Ws[buf ^ 1]);
            __syncthreads();
        }
    }

    // D layout of a 32 x 32 tile: lane l, register r -> row 8(r/4) + 4(l/32) + r%4, column l%32
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = n0 + wn * (BN / 2) + 32 * j + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * (BM / 2) + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (m < p.M && n < p.N) {
                    float *dst = p.Y + (int64_t)m * p.N + n;
                    if (p.atomic)
                        unsafeAtomicAdd(dst, acc[i][j][r]);   // hardware fp32 add
                    else
                        *dst = acc[i][j][r];
                }
            }
        }
}

struct FillParams {
    float *Y;
    int64_t n;
};

__global__ __launch_bounds__(256) void zero_fill_kernel(FillParams f)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < f.n; i += stride)
        f.Y[i] = 0.0f;
}

inline bool aligned(const void *ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0; }

thread_local int o_splits = 0, o_bm = 0;   // tuning override (0: built-in)

template <int BM, int BN>
hipError_t launch_prefill(PrefillParams p, int cus, hipStream_t stream)
{
    const int64_t tiles_n = (p.N + BN - 1) / BN;
    const int64_t tiles_m = (p.M + BM - 1) / BM;
    const int nsteps = (p.K / 32 + 1) / 2;
    int splits = 1;
    const int64_t tiles = tiles_n * tiles_m;
    if (tiles < (int64_t)cus * 5 / 8) {
        // Too few output tiles to occupy the chip: split K, about one
        // workgroup per CU in total (three per four CUs with 64-token tiles).
        // Each extra split adds an fp32 atomic per output element and needs a
        // zero-filled Y, so splits stay few (sweeps on MI355X: 6144 x 2048 at
        // 512 tokens 38.6 us unsplit against 47.0 us with 2 splits; 2560 x
        // 6144 at 512 tokens best at 3; 12288 x 2560 at 64 tokens 28.7 us with
        // 2 splits against 31.8 with 4 and more with 3, cycled copies).
        const int64_t target = BM == 64 ? (int64_t)cus * 3 / 4 : (int64_t)cus;
        splits = (int)std::min<int64_t>((target + tiles / 2) / tiles, std::max(1, nsteps / 4));
        splits = std::max(1, std::min(splits, 16));
    }
    if (o_splits > 0)
        splits = std::min(o_splits, nsteps);
    p.steps_per_split = (nsteps + splits - 1) / splits;
    splits = (nsteps + p.steps_per_split - 1) / p.steps_per_split;
    p.atomic = splits > 1;
    if (tiles_m > 65535 || splits > 65535 || tiles_n > INT32_MAX)
        return hipErrorInvalidValue;
    if (p.atomic) {
        FillParams f{p.Y, (int64_t)p.M * p.N};
        void *a[] = {&f};
        const int64_t wgs = std::min<int64_t>((f.n + 255) / 256, (int64_t)cus * 16);
        hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&zero_fill_kernel), dim3((unsigned)wgs),
                                       dim3(256), a, 0, stream);
        if (e != hipSuccess)
            return e;
    }
    return launch_kernel(reinterpret_cast<const void *>(&prefill_kernel<BM, BN>),
                         dim3((unsigned)tiles_n, (unsigned)tiles_m, (unsigned)splits), dim3(256), 0, stream, p);
}

}  // namespace
}  // namespace qg

extern "C" qg_status qgemm_q4_0_prefill(const void *Wp, const uint16_t *X, float *Y, int64_t M, int64_t N, int64_t K,
                                        void *stream)
{
    using namespace qg;
    if (!Wp || !X || !Y)
        return QG_ERR_NULL;
    if (M < 1 || N < 1 || K < 32 || K % 32 != 0 || M > INT32_MAX / 2 || N > INT32_MAX / 2 || K > INT32_MAX / 2 ||
        M * N > ((int64_t)1 << 40))
        return QG_ERR_SHAPE;
    if (!aligned(Wp, 256) || !aligned(X, 16) || !aligned(Y, 4))
        return QG_ERR_ALIGN;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return QG_ERR_DEVICE;
    PrefillParams p;
    p.W = static_cast<const uint8_t *>(Wp);
    p.X = X;
    p.Y = Y;
    p.scale_offset = (int64_t)((N * (K / 32) * 16 + 255) / 256 * 256);
    p.M = (int)M;
    p.N = (int)N;
    p.K = (int)K;
    p.steps_per_split = 0;
    p.atomic = 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool small = o_bm ? (o_bm == 64) : (M <= 64);
    // 128 x 192 tiles where they give every CU exactly one workgroup while
    // 128 x 128 tiles would leave some CUs with two (MI355X: 12288 x 2560 at
    // 512 tokens 79 against 86 us); elsewhere 128 x 128 (with fewer tiles
    // than CUs the wider tile needs more K splits and loses).
    const int64_t tiles_m = (M + 127) / 128;
    const int64_t t128 = (N + 127) / 128 * tiles_m, t192 = (N + 191) / 192 * tiles_m;
    const bool wide = !small && o_bm == 0 && t128 > cus && t192 <= cus && t192 * 8 >= (int64_t)cus * 7;
    hipError_t e = small  ? launch_prefill<64, 128>(p, cus, s)
                   : wide ? launch_prefill<128, 192>(p, cus, s)
                          : launch_prefill<128, 128>(p, cus, s);
    if (e == hipErrorInvalidValue)
        return QG_ERR_SHAPE;
    return e == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
}

// Tuning knob for sweeps: fixes the K split count and the token tile (64 or
// 128) of later qgemm_q4_0_prefill calls from the calling thread; 0 keeps the
// built-in choice.
extern "C" void qg_set_prefill_shape(int splits, int bm)
{
    qg::o_splits = splits;
    qg::o_bm = bm;
}
