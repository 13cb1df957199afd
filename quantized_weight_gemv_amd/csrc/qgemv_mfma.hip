// Few-token GEMV (2..8 tokens) on the gfx950 matrix cores, Q4_0 and Q8_0.
//
// With several tokens the vector-ALU kernel spends M dot products per
// unpacked weight pair and every wave re-reads all M activation rows; here one
// v_mfma_f32_16x16x32_f16 takes exactly one 32-weight block of 16 output rows
// against up to 16 tokens, so the unpack cost per block no longer grows with
// M and each activation fragment serves 16 rows per instruction [volta-kernel-
// bakeoff, "Results", the few-tokens bullet: one activation load should serve
// several rows].
//
// Exactness is kept: the B operand holds the exact integers (q - 8) (or q)
// as fp16, each MFMA sums the 32 exact products of one block into fp32, and
// the block's scale multiplies that sum in fp32 afterwards.
//
// Mapping: a workgroup owns 16 consecutive rows; its `ksplit` waves split K.
// Per step a lane loads 16 code bytes with one 16-byte load: lane l reads row
// n0 + l%16, block b0 + l/16 (Q4_0; four blocks of the 16 rows per
// instruction, 64 contiguous bytes per row).  The 16x16x32 B operand wants
// lane group g to hold word g of one block, so the four words are transposed
// across the four 16-lane groups with v_permlane32_swap and v_permlane16_swap
// (Q8_0 blocks are 32 bytes: two blocks per load, one swap stage, and the k
// order inside a block is permuted the same way in the activations, which
// leaves the contraction unchanged).  Each wave issues all of its code and
// scale loads (one scale per lane per step, broadcast to the row's lane groups
// with the same swaps) before the first MFMA, and stages its activation slice
// in LDS with coalesced 16-byte loads, already in operand order, so an A
// operand is one ds_read_b128.  Partial 16x16 tiles of the waves are summed
// through LDS in a fixed order: results are reproducible.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "qgemv_internal.h"

namespace qg {
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ h2_t as_h2(uint32_t u) { return __builtin_bit_cast(h2_t, u); }
__device__ __forceinline__ uint32_t as_u32(h2_t h) { return __builtin_bit_cast(uint32_t, h); }

__device__ __forceinline__ uint32_t magic_reg()
{
    uint32_t m;
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(m));
    return m;
}

__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) { return (a & 0xFFFFu) | (b << 16); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }

__device__ __forceinline__ half8_t pack8(uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
    const u4_t v = {a, b, c, d};
    return __builtin_bit_cast(half8_t, v);
}

// Swap helpers (16-lane groups r0..r3):
//   swap32(A, B): A <- [A.r0, A.r1, B.r0, B.r1], B <- [A.r2, A.r3, B.r2, B.r3]
//   swap16(A, B): A <- [A.r0, B.r0, A.r2, B.r2], B <- [A.r1, B.r1, A.r3, B.r3]
__device__ __forceinline__ void swap32(uint32_t &a, uint32_t &b)
{
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    a = r[0];
    b = r[1];
}
__device__ __forceinline__ void swap16(uint32_t &a, uint32_t &b)
{
    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    a = r[0];
    b = r[1];
}

constexpr size_t kMaxLds = 131072;   // dynamic LDS cap of the staged activations

struct MfmaParams {
    const uint8_t *W;
    const uint16_t *x;     // fp16 [M][K]
    float *y;              // fp32 [M][N]
    int64_t scale_offset;
    int M, N, K;
    int kw;                // blocks per wave (multiple of 4)
};

// Q4_0 B operand of one block from word g (= lane group) of its codes:
// halves (e[4g], e[4g+2], e[16+4g], e[18+4g], e[4g+1], e[4g+3], e[17+4g], e[19+4g]) - 8
__device__ __forceinline__ half8_t q4_operand(uint32_t w, uint32_t magic)
{
    const h2_t kOffLo = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const h2_t kScaleHi = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2_t kOffHi = {(_Float16)-72.0f, (_Float16)-72.0f};
    const uint32_t b = w >> 8;
    const h2_t p0 = as_h2((w & 0x000F000Fu) | magic) + kOffLo;
    const h2_t p1 = as_h2((w & 0x00F000F0u) | magic) * kScaleHi + kOffHi;
    const h2_t p2 = as_h2((b & 0x000F000Fu) | magic) + kOffLo;
    const h2_t p3 = as_h2((b & 0x00F000F0u) | magic) * kScaleHi + kOffHi;
    return pack8(as_u32(p0), as_u32(p1), as_u32(p2), as_u32(p3));
}

// Q8_0 B operand from two code words t0, t0 + 1:
// halves (e[4t0], e[4t0+2], e[4t0+1], e[4t0+3], e[4t1], e[4t1+2], e[4t1+1], e[4t1+3])
__device__ __forceinline__ half8_t q8_operand(uint32_t w0, uint32_t w1, uint32_t magic)
{
    const h2_t kOff = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    const uint32_t u0 = w0 ^ 0x80808080u, u1 = w1 ^ 0x80808080u;
    const h2_t p0 = as_h2((u0 & 0x00FF00FFu) | magic) + kOff;
    const h2_t p1 = as_h2(((u0 >> 8) & 0x00FF00FFu) | magic) + kOff;
    const h2_t p2 = as_h2((u1 & 0x00FF00FFu) | magic) + kOff;
    const h2_t p3 = as_h2(((u1 >> 8) & 0x00FF00FFu) | magic) + kOff;
    return pack8(as_u32(p0), as_u32(p1), as_u32(p2), as_u32(p3));
}

// Activations of one (token, block): 32 fp16 as 16 words in the pair order
//   word 4t+0 = (x[4t], x[4t+2])      word 4t+2 = (x[4t+1], x[4t+3])
//   word 4t+1 = (x[16+4t], x[18+4t])  word 4t+3 = (x[17+4t], x[19+4t])   (Q4_0)
//   word 2t   = (x[4t], x[4t+2])      word 2t+1 = (x[4t+1], x[4t+3])     (Q8_0)
// so that the 8 halves lane group g feeds to the MFMA are the 16 bytes at
// word 4g (Q4_0) or 4p, p = {0,2,1,3}[g] (Q8_0: the swap pattern below).
template <int FMT>
__device__ __forceinline__ void permute_x(const uint4 (&r)[4], uint4 (&o)[4])
{
    const uint32_t d[16] = {r[0].x, r[0].y, r[0].z, r[0].w, r[1].x, r[1].y, r[1].z, r[1].w,
                            r[2].x, r[2].y, r[2].z, r[2].w, r[3].x, r[3].y, r[3].z, r[3].w};
    uint32_t w[16];
    if constexpr (FMT == kQ4_0) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            w[4 * t + 0] = pair_lo(d[2 * t], d[2 * t + 1]);
            w[4 * t + 1] = pair_lo(d[8 + 2 * t], d[9 + 2 * t]);
            w[4 * t + 2] = pair_hi(d[2 * t], d[2 * t + 1]);
            w[4 * t + 3] = pair_hi(d[8 + 2 * t], d[9 + 2 * t]);
        }
    } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            w[2 * t + 0] = pair_lo(d[2 * t], d[2 * t + 1]);
            w[2 * t + 1] = pair_hi(d[2 * t], d[2 * t + 1]);
        }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
        o[q] = make_uint4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
}

template <int FMT, int KWMAX>
__global__ __launch_bounds__(512) void gemv_mfma_kernel(MfmaParams p)
{
    constexpr int kBlocksPerLoad = (FMT == kQ4_0) ? 4 : 2;   // blocks of 16 rows per 16-byte load step
    constexpr int kSteps = KWMAX / kBlocksPerLoad;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nwaves = blockDim.x >> 6;
    const int g = lane >> 4;          // lane group
    const int c = lane & 15;          // row within the tile / token of the A operand
    const int n0 = blockIdx.x * 16;
    const int KB = p.K >> 5;
    const int kbeg = wave * p.kw;
    const int kend = min(KB, kbeg + p.kw);
    const int nblk = max(0, kend - kbeg);
    const int nsteps = (nblk + kBlocksPerLoad - 1) / kBlocksPerLoad;

    const int row = min(n0 + c, p.N - 1);
    const uint8_t *__restrict__ crow = p.W + (int64_t)row * KB * (FMT == kQ4_0 ? 16 : 32);
    const uint16_t *__restrict__ srow = reinterpret_cast<const uint16_t *>(p.W + p.scale_offset) + (int64_t)row * KB;

    // 1. this wave's activations (M tokens x its blocks, 64 bytes each) with
    //    coalesced 16-byte loads.  They are issued first: loads retire in
    //    order, and these come from cache while the codes come from HBM.
    constexpr int kXPer = 8 * KWMAX / 64;    // (token, block) pairs per lane, M <= 8
    uint4 xr[kXPer][4];
#pragma unroll
    for (int t = 0; t < kXPer; ++t) {
        const int i = lane + 64 * t;
        if (i < p.M * nblk) {
            const int m = i / nblk, b = i - m * nblk;
            const uint4 *src = reinterpret_cast<const uint4 *>(p.x + (int64_t)m * p.K + (int64_t)(kbeg + b) * 32);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                xr[t][q] = src[q];
        }
    }

    // 2. this wave's code and scale loads: one 16-byte code load and one
    //    scale per lane per step (lane group g: block b0 + g, Q4_0; block
    //    b0 + g/2, Q8_0)
    uint4 code[kSteps];
    uint16_t scl[kSteps];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        if (s < nsteps) {
            const int b0 = kbeg + s * kBlocksPerLoad;
            const int bl = (FMT == kQ4_0) ? min(b0 + g, KB - 1) : min(b0 + (g >> 1), KB - 1);
            const int off = (FMT == kQ4_0) ? bl * 16 : bl * 32 + (g & 1) * 16;
            typedef unsigned int v4u __attribute__((ext_vector_type(4)));
            const v4u t = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(crow + (uint32_t)off));
            code[s] = make_uint4(t.x, t.y, t.z, t.w);
            scl[s] = srow[bl];
        }
    }

    // 3. the activations into this wave's own LDS area, in MFMA operand
    //    order; layout [block][token][64 bytes]
    extern __shared__ uint4 xs_dyn[];
    uint4 *xs = xs_dyn + (int64_t)wave * p.kw * p.M * 4;
#pragma unroll
    for (int t = 0; t < kXPer; ++t) {
        const int i = lane + 64 * t;
        if (i < p.M * nblk) {
            const int m = i / nblk, b = i - m * nblk;
            uint4 o[4];
            permute_x<FMT>(xr[t], o);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                xs[(b * p.M + m) * 4 + q] = o[q];
        }
    }
    // the reads below are this wave's own writes: LDS keeps a wave's order

    const uint32_t magic = magic_reg();
    f4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const bool rok = n0 + c < p.N;
    const bool live = c < p.M;
    const int xq = (FMT == kQ4_0) ? g : (((g & 1) << 1) | (g >> 1));
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        if (s < nsteps) {
            const int b0 = kbeg + s * kBlocksPerLoad;
            uint32_t w0 = code[s].x, w1 = code[s].y, w2 = code[s].z, w3 = code[s].w;
            // scale of (row, block b0 + j) to every lane group of the row
            uint32_t sa = scl[s], sb = scl[s];
            swap32(sa, sb);                      // Q4_0: sa = [s0 s1 s0 s1], sb = [s2 s3 s2 s3]
            uint32_t sc[4];
            if constexpr (FMT == kQ4_0) {
                uint32_t sa2 = sa, sb2 = sb;
                swap16(sa, sa2);
                swap16(sb, sb2);
                sc[0] = sa; sc[1] = sa2; sc[2] = sb; sc[3] = sb2;
                // 4 x 4 transpose across lane groups: afterwards register j
                // of lane group g holds word g of block b0 + j
                swap32(w0, w2);
                swap32(w1, w3);
                swap16(w0, w1);
                swap16(w2, w3);
            } else {
                sc[0] = sa; sc[1] = sb; sc[2] = 0; sc[3] = 0;   // Q8_0: [s0 s0 s0 s0], [s1 s1 s1 s1]
                // afterwards (w0, w1) hold block b0 and (w2, w3) block b0 + 1:
                // lane group g has code words 2p, 2p + 1, p = {0, 2, 1, 3}[g]
                swap32(w0, w2);
                swap32(w1, w3);
            }
#pragma unroll
            for (int j = 0; j < kBlocksPerLoad; ++j) {
                const int b = b0 + j;
                const bool bok = b < kend;
                half8_t bop;
                if constexpr (FMT == kQ4_0)
                    bop = q4_operand(j == 0 ? w0 : j == 1 ? w1 : j == 2 ? w2 : w3, magic);
                else
                    bop = (j == 0) ? q8_operand(w0, w1, magic) : q8_operand(w2, w3, magic);
                half8_t aop = pack8(0u, 0u, 0u, 0u);
                if (live && bok) {
                    const uint4 v = xs[((b - kbeg) * p.M + c) * 4 + xq];
                    aop = pack8(v.x, v.y, v.z, v.w);
                }
                const f4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
                const f4_t d = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop, zero, 0, 0, 0);
                // D layout: lane l, register r -> token 4(l/16) + r, row n0 + l%16
                const float scv = (bok && rok) ? (float)__builtin_bit_cast(_Float16, (uint16_t)sc[j]) : 0.0f;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[r] = __builtin_fmaf(scv, d[r], acc[r]);
            }
        }
    }

    // combine the waves' partial tiles in a fixed order and store
    __shared__ f4_t red[kMaxWavesPerWg][64];
    red[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {
        f4_t s = red[0][lane];
        for (int w = 1; w < nwaves; ++w) {
            const f4_t t = red[w][lane];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                s[r] += t[r];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 4 * g + r;
            if (m < p.M && rok)
                p.y[(int64_t)m * p.N + n0 + c] = s[r];
        }
    }
}

template <int FMT, int KWMAX>
hipError_t launch_kw(const MfmaParams &p, int waves, hipStream_t stream)
{
    const void *fn = reinterpret_cast<const void *>(&gemv_mfma_kernel<FMT, KWMAX>);
    // every wave stages M x kw blocks of activations (64 bytes each)
    const size_t shmem = (size_t)waves * p.kw * p.M * 64;
    if (shmem > kMaxLds)
        return hipErrorInvalidValue;
    static bool raised = false;   // allow more than the default dynamic LDS once per kernel
    if (!raised) {
        if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds) != hipSuccess)
            return hipErrorInvalidValue;
        raised = true;
    }
    const dim3 grid((unsigned)((p.N + 15) / 16)), block(64 * waves);
    return launch_kernel(fn, grid, block, shmem, stream, p);
}

template <int FMT>
hipError_t launch_fmt(const MfmaParams &p, int kwmax, int waves, hipStream_t stream)
{
    switch (kwmax) {
    case 8: return launch_kw<FMT, 8>(p, waves, stream);
    case 16: return launch_kw<FMT, 16>(p, waves, stream);
    case 32: return launch_kw<FMT, 32>(p, waves, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

// Launch the matrix-core GEMV: `waves` (1..8) split K; each wave takes
// kw = ceil(K/32 / waves) blocks rounded up to 4, at most 32.
hipError_t launch_gemv_mfma(int fmt, const uint8_t *W, int64_t scale_offset, const uint16_t *x, float *y, int M,
                            int N, int K, int waves, hipStream_t stream)
{
    const int KB = K / 32;
    if (M < 1 || M > 8 || waves < 1 || waves > kMaxWavesPerWg)
        return hipErrorInvalidValue;
    int kw = (KB + waves - 1) / waves;
    kw = (kw + 3) / 4 * 4;
    if (kw > 32)
        return hipErrorInvalidValue;
    const int kwmax = kw <= 8 ? 8 : (kw <= 16 ? 16 : 32);
    MfmaParams p{W, x, y, scale_offset, M, N, K, kw};
    return fmt == kQ4_0 ? launch_fmt<kQ4_0>(p, kwmax, waves, stream) : launch_fmt<kQ8_0>(p, kwmax, waves, stream);
}

}  // namespace qg
