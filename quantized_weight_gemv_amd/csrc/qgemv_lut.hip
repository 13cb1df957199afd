// Times-table GEMV for plain 2-bit weights (q2w), one token, gfx950.
//
// Instead of unpacking codes and multiplying, each pair of activations gets a
// table of the 16 possible sums c_a * x_a + c_b * x_b (c in -2..1), and the
// 4-bit nibble holding the two codes of a weight pair indexes it
// [volta-kernel-bakeoff, "What's in the race": q2_lut / q2w_lut, the "times
// table"; "Results": it lost to unpacking on V100].  In q2w byte j of a block
// holds elements j, j + 8 (low nibble) and j + 16, j + 24 (high nibble), so
// the 16 pairs of a block are (j + 16 h, j + 8 + 16 h), j < 8, h < 2, and
// the table index is u_a + 4 u_b (u = c + 2).
//
// Every workgroup builds the tables of all K / 32 blocks in LDS once, as
// fp16 entries in 256-byte entry rows [pair][entry][128 columns]: lane l of a
// row owns blocks 2l and 2l + 1, so one lookup instruction of a wave reads 64
// different 4-byte banks (no conflicts; the pages' 2-bit kernel lost 1.9x to
// a per-lane stride in shared memory [volta-kernel-bakeoff, "Results", the
// found-on-the-way bullet]), and the byte address of an entry is
// the code nibble in bits 8..11 above the lane's column byte: a single byte
// permute builds it, the pair index rides in the instruction's offset.  For
// K <= 2048 (1024) the row holds two (four) copies of the table and a wave
// pass covers two (four) rows, each row's lanes reading their own copy.  The
// table is 16 * 16 * 256 bytes = 64 KB, so K <= 4096.  Each wave takes one or
// two passes at once, sums entries in pairs with an fp32 dot product against
// (1, 1), scales each block sum once in fp32 and reduces the row.
//
// Accuracy: an entry is the fp32 sum of two exact products rounded to fp16,
// within 2^-11 of |c_a x_a| + |c_b x_b|, so y is within 2^-11 * sum |w x|
// plus fp32 accumulation of the exact q2w GEMV: inside 1e-3 * sum |w x|.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "qgemv_internal.h"

namespace qg {
namespace {

typedef _Float16 lut_h2 __attribute__((ext_vector_type(2)));

struct LutParams {
    const uint8_t *W;      // packed q2w matrix
    int64_t scale_offset;  // byte offset of the scale region
    const uint16_t *x;     // fp16 bits [K]
    float *y;              // fp32 [N]
    int N, K;
};

constexpr int kLutWaves = 8;
constexpr int kLutRowBytes = 256;              // one entry row: 128 fp16 columns
constexpr int kLutBytes = 16 * 16 * kLutRowBytes;
constexpr uint32_t kDeadOffset = 0x7FFFFFF0u;  // beyond every descriptor extent

__device__ __forceinline__ _Float16 lut_entry(const char *lutb, uint32_t off)
{
    return *reinterpret_cast<const _Float16 *>(lutb + off);
}

// Address of the entry for byte BYTE of nib (a word of 4-bit code pairs, one
// per byte) in the lane's column col (< 256): that byte -> bits 8..15, col ->
// bits 0..7 (selector bytes 0-3 pick bytes of col, 4-7 bytes of nib, 12 a
// zero).
template <int BYTE>
__device__ __forceinline__ uint32_t nib_address(uint32_t nib, uint32_t col)
{
    return __builtin_amdgcn_perm(nib, col, 0x0C0C0000u | ((4u + BYTE) << 8));
}

// Sum of the 16 pair entries of one block: byte j of the codes indexes pair
// j with its low nibble and pair 8 + j with its high nibble.
__device__ __forceinline__ float block_lookup(const char *lutb, uint32_t col, uint32_t w0, uint32_t w1)
{
    const lut_h2 one = {(_Float16)1.0f, (_Float16)1.0f};
    const uint32_t lo[2] = {w0 & 0x0F0F0F0Fu, w1 & 0x0F0F0F0Fu};
    const uint32_t hi[2] = {(w0 >> 4) & 0x0F0F0F0Fu, (w1 >> 4) & 0x0F0F0F0Fu};
    float bs = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t a, b;
        switch (j & 3) {
        case 0: a = nib_address<0>(lo[j >> 2], col); b = nib_address<0>(hi[j >> 2], col); break;
        case 1: a = nib_address<1>(lo[j >> 2], col); b = nib_address<1>(hi[j >> 2], col); break;
        case 2: a = nib_address<2>(lo[j >> 2], col); b = nib_address<2>(hi[j >> 2], col); break;
        default: a = nib_address<3>(lo[j >> 2], col); b = nib_address<3>(hi[j >> 2], col); break;
        }
        const lut_h2 v = {lut_entry(lutb, a + j * 16 * kLutRowBytes),
                          lut_entry(lutb, b + (8 + j) * 16 * kLutRowBytes)};
        bs = __builtin_amdgcn_fdot2(v, one, bs, false);
    }
    return bs;
}

// COLS: table columns per copy (a power of two >= K / 32, 32..128); a row is
// COLS / 2 lanes and a pass 128 / COLS rows.  PASSES: row passes per wave
// iteration (their loads are in flight together).
template <int COLS, int PASSES>
__global__ __launch_bounds__(64 * kLutWaves) void gemv_q2w_lut_kernel(LutParams p)
{
    __shared__ __attribute__((aligned(16))) _Float16 lut[kLutBytes / 2];   // static: addresses need no base
    constexpr int LPR = COLS / 2;                 // lanes per row
    constexpr int RPP = 64 / LPR;                 // rows per pass (= copies)
    constexpr int RW = RPP * PASSES;              // rows per wave iteration
    const int KB = p.K >> 5;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sub = lane / LPR;                   // row within the pass
    const int bl = lane % LPR;                    // owns blocks 2 bl, 2 bl + 1
    const bool live0 = 2 * bl < KB, live1 = 2 * bl + 1 < KB;
    const int64_t code_row = (int64_t)KB * 8;
    const int64_t wave_rows = (int64_t)gridDim.x * kLutWaves * RW;

    // First the activation pairs of this thread's table item (one pair, four
    // adjacent columns), then the weights of its first rows: both are in
    // flight together, and loads return in order, so building the tables
    // waits only for the activations.  Items x copies = 16 * COLS / 4 *
    // 128 / COLS = 512, so each thread builds one copy of one item and no
    // branch exists for the compiler to sink a load into; column indices are
    // clamped into range and the values of columns past K / 32 masked to
    // zero.  Thirty-two consecutive threads fill one 256-byte entry row (all
    // its copies), so the 8-byte writes of a half-wave hit 64 banks.
    static_assert(4 * COLS * RPP == 64 * kLutWaves, "one item copy per thread");
    const int q = threadIdx.x % (COLS / 4);                 // columns 4q .. 4q + 3
    const int cp = (int)(threadIdx.x / (COLS / 4)) % RPP;   // table copy
    const int pr = threadIdx.x / 32;                        // pair
    uint32_t xr[4][2];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
        const int b = std::min(4 * q + cc, KB - 1);
        const int ea = b * 32 + (pr & 7) + 16 * (pr >> 3);
        xr[cc][0] = p.x[ea];
        xr[cc][1] = p.x[ea + 8];
    }

    // Loads of the rows n0 .. n0 + RW - 1, branch-free (the compiler's waits
    // then need not cover a path that skipped them).  The extents end at the
    // last real row, so rows past N and dead block slots (an offset far
    // beyond the extent) read zeros without touching memory.  A lane whose
    // second block is past K / 32 takes its first with an 8-byte load; the
    // other lanes' 8-byte loads are dead.
    uint4 c[PASSES];
    uint16_t d0[PASSES], d1[PASSES];
    auto load_rows = [&](int64_t n0) {
        const int64_t rows = std::max<int64_t>(0, std::min<int64_t>(p.N - n0, RW));
        const auto rc = make_rsrc(p.W + n0 * code_row, rows * code_row);
        const auto rs = make_rsrc(p.W + p.scale_offset + n0 * KB * 2, rows * KB * 2);
#pragma unroll
        for (int u = 0; u < PASSES; ++u) {
            const uint32_t blk = (uint32_t)((u * RPP + sub) * KB + 2 * bl);
            const uint4 w = stream_load16(rc, live1 ? blk * 8u : kDeadOffset);
            const uint2 h = stream_load8(rc, live0 && !live1 ? blk * 8u : kDeadOffset);
            c[u] = make_uint4(w.x | h.x, w.y | h.y, w.z, w.w);
            d0[u] = stream_load2(rs, live0 ? blk * 2u : kDeadOffset);
            d1[u] = stream_load2(rs, live1 ? blk * 2u + 2u : kDeadOffset);
        }
    };
    int64_t n0 = ((int64_t)blockIdx.x * kLutWaves + wave) * RW;
    load_rows(n0);

    // tables; columns past K / 32 hold zeros
    float xa[4], xb[4];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
        const uint32_t keep = 4 * q + cc < KB ? 0xFFFFu : 0u;
        xa[cc] = (float)__builtin_bit_cast(_Float16, (uint16_t)(xr[cc][0] & keep));
        xb[cc] = (float)__builtin_bit_cast(_Float16, (uint16_t)(xr[cc][1] & keep));
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float ca = (float)((i & 3) - 2), cb = (float)((i >> 2) - 2);
        uint32_t h[4];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
            h[cc] = __builtin_bit_cast(uint16_t, (_Float16)(ca * xa[cc] + cb * xb[cc]));
        *reinterpret_cast<uint2 *>(&lut[(pr * 16 + i) * (kLutRowBytes / 2) + cp * COLS + 4 * q]) =
            make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
    }
    __syncthreads();

    const char *lutb = reinterpret_cast<const char *>(lut);
    const uint32_t col = (uint32_t)(sub * COLS * 2 + bl * 4);
    while (n0 < p.N) {
        float acc[PASSES];
#pragma unroll
        for (int u = 0; u < PASSES; ++u) {
            const float s0 = block_lookup(lutb, col, c[u].x, c[u].y);
            const float s1 = block_lookup(lutb, col + 2u, c[u].z, c[u].w);
            acc[u] = __builtin_fmaf((float)__builtin_bit_cast(_Float16, d0[u]), s0,
                                    (float)__builtin_bit_cast(_Float16, d1[u]) * s1);
#pragma unroll
            for (int off = LPR / 2; off > 0; off >>= 1)
                acc[u] += __shfl_xor(acc[u], off, 64);
        }
#pragma unroll
        for (int u = 0; u < PASSES; ++u) {
            const int64_t n = n0 + u * RPP + sub;
            if (bl == 0 && n < p.N)
                p.y[n] = acc[u];
        }
        n0 += wave_rows;
        load_rows(n0);
    }
}

}  // namespace

size_t gemv_lut_lds_bytes(int K) { return K >= 32 && K <= 4096 ? (size_t)kLutBytes : (size_t)-1; }

hipError_t launch_gemv_q2w_lut(const uint8_t *W, int64_t scale_offset, const uint16_t *x, float *y, int N, int K,
                               int cus, hipStream_t stream)
{
    if (N < 1 || K < 32 || K % 32 != 0 || K > 4096 || cus < 1)
        return hipErrorInvalidValue;
    LutParams p{W, scale_offset, x, y, N, K};
    const int KB = K / 32;
    const int cols = KB <= 32 ? 32 : (KB <= 64 ? 64 : 128);
    // Up to two workgroups per CU (64 KB of LDS each), each building the
    // table once.  A wave's passes run one after another, and every extra
    // workgroup on a CU builds the table again.  One pass while that needs
    // at most one workgroup per CU (128-column tables) or two (narrower
    // ones, whose rows need half the lookups), else two passes.  Measured on
    // MI355X: 4096 x 4096 at 5.7 us in 256 two-pass workgroups against
    // 7.0 us in 512 one-pass ones; 6144 x 2048 at 5.3 us in 384 one-pass
    // workgroups against 5.6 us in 192 two-pass ones; four passes were
    // slower everywhere.
    const int64_t wgs_max = 2 * (int64_t)cus;
    const int64_t rows_per_pass_wg = (int64_t)kLutWaves * (128 / cols);
    const int passes = N <= (cols == 128 ? 1 : 2) * (int64_t)cus * rows_per_pass_wg ? 1 : 2;
    const int64_t rows_per_wg = rows_per_pass_wg * passes;
    const int64_t wgs = std::min<int64_t>(wgs_max, (N + rows_per_wg - 1) / rows_per_wg);
    const void *fn;
    switch (cols * 4 + passes) {
    case 32 * 4 + 1: fn = reinterpret_cast<const void *>(&gemv_q2w_lut_kernel<32, 1>); break;
    case 32 * 4 + 2: fn = reinterpret_cast<const void *>(&gemv_q2w_lut_kernel<32, 2>); break;
    case 64 * 4 + 1: fn = reinterpret_cast<const void *>(&gemv_q2w_lut_kernel<64, 1>); break;
    case 64 * 4 + 2: fn = reinterpret_cast<const void *>(&gemv_q2w_lut_kernel<64, 2>); break;
    case 128 * 4 + 1: fn = reinterpret_cast<const void *>(&gemv_q2w_lut_kernel<128, 1>); break;
    default: fn = reinterpret_cast<const void *>(&gemv_q2w_lut_kernel<128, 2>); break;
    }
    return launch_kernel(fn, dim3((unsigned)wgs), dim3(64 * kLutWaves), 0, stream, p);
}

}  // namespace qg
