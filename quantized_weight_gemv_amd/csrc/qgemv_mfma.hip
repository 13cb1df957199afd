// Few-token GEMV (2..8 tokens) on the gfx950 matrix cores, Q4_0, Q8_0 and
// plain 2-bit (q2w).
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
// Mapping: a workgroup walks 16-row tiles (tiles w, w + grid, ...: a
// persistent grid, so each workgroup stages its activations once); its
// `ksplit` waves split K.  Per step a lane loads 16 code bytes with one 16-byte load: lane l reads row
// n0 + l%16, block b0 + l/16 (Q4_0; four blocks of the 16 rows per
// instruction, 64 contiguous bytes per row).  The 16x16x32 B operand wants
// lane group g to hold word g of one block, so the four words are transposed
// across the four 16-lane groups with v_permlane32_swap and v_permlane16_swap
// (Q8_0 blocks are 32 bytes: two blocks per load, one swap stage, and the k
// order inside a block is permuted the same way in the activations, which
// leaves the contraction unchanged; q2w blocks are 8 bytes: eight blocks per
// load, and ten swaps give every lane group the word of each block that holds
// its eight elements).  Each wave issues all of a tile's code
// and scale loads (one scale per lane per step, broadcast to the row's lane
// groups with the same swaps) before that tile's first MFMA, and the next
// tile's while it multiplies the current one.  It stages its activation slice
// in LDS once, with coalesced 16-byte loads, already in operand order, so an
// A operand is one ds_read_b128.  Partial 16x16 tiles of the waves are summed
// through LDS in a fixed order: results are reproducible.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <map>
#include <set>
#include <mutex>
#include <tuple>

#include "qgemv_internal.h"

namespace qg {
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

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

// Blocks of 16 rows per 16-byte load step, and code bytes per block.
template <int FMT>
constexpr int blocks_per_load() { return FMT == kQ4_0 ? 4 : (FMT == kQ8_0 ? 2 : 8); }
template <int FMT>
constexpr int mfma_code_bytes() { return FMT == kQ4_0 ? 16 : (FMT == kQ8_0 ? 32 : 8); }

struct MfmaParams {
    const uint8_t *W;
    const uint16_t *x;     // fp16 [M][K] (fp16 input)
    const float *xf;       // fp32 [M][K] (fp32 input, rounded to binary16 at staging)
    float *y;              // fp32 [M][N]
    int64_t scale_offset;
    int M, N, K;
    int kw;                // blocks per wave (multiple of 4)
    int glu;               // 1: stacked gate + up table of 2N rows, y = silu(gate) * up
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

// q2w B operand of one block from the code word holding lane group g's
// elements, already shifted right by 4 (g & 1) so that its bit pairs 0 and 1
// are the block's bit pairs r0 = 2 (g & 1) and r0 + 1.  Byte t' of word
// t = g >> 1 is byte 4t + t' of the block, whose bit pair r is element
// 4t + t' + 8r; halves (for r = r0, then r0 + 1)
//   (e[4t + 8r], e[4t + 2 + 8r], e[4t + 1 + 8r], e[4t + 3 + 8r]) as c = u - 2:
// (u | 0x6400) - 1026 and ((4u) | 0x6400) / 4 - 258, every step exact.
__device__ __forceinline__ half8_t q2_operand(uint32_t w, uint32_t magic)
{
    const h2_t kOff0 = {(_Float16)-1026.0f, (_Float16)-1026.0f};
    const h2_t kScale1 = {(_Float16)0.25f, (_Float16)0.25f};
    const h2_t kOff1 = {(_Float16)-258.0f, (_Float16)-258.0f};
    const uint32_t b = w >> 8;
    const h2_t p0 = as_h2((w & 0x00030003u) | magic) + kOff0;
    const h2_t p1 = as_h2((b & 0x00030003u) | magic) + kOff0;
    const h2_t p2 = as_h2((w & 0x000C000Cu) | magic) * kScale1 + kOff1;
    const h2_t p3 = as_h2((b & 0x000C000Cu) | magic) * kScale1 + kOff1;
    return pack8(as_u32(p0), as_u32(p1), as_u32(p2), as_u32(p3));
}

// Activations of one (token, block): 32 fp16 as 16 words in the pair order
//   word 4t+0 = (x[4t], x[4t+2])      word 4t+2 = (x[4t+1], x[4t+3])
//   word 4t+1 = (x[16+4t], x[18+4t])  word 4t+3 = (x[17+4t], x[19+4t])   (Q4_0)
//   word 2t   = (x[4t], x[4t+2])      word 2t+1 = (x[4t+1], x[4t+3])     (Q8_0)
//   words 4g..4g+3 = the pairs (x[e], x[e+2]), (x[e+1], x[e+3]) for
//   e = 4(g >> 1) + 8 r, r = 2 (g & 1), then r + 1                     (q2w)
// so that the 8 halves lane group g feeds to the MFMA are the 16 bytes at
// word 4g (Q4_0, q2w) or 4p, p = {0,2,1,3}[g] (Q8_0: the swap pattern below).
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
    } else if constexpr (FMT == kQ8_0) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            w[2 * t + 0] = pair_lo(d[2 * t], d[2 * t + 1]);
            w[2 * t + 1] = pair_hi(d[2 * t], d[2 * t + 1]);
        }
    } else {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int e0 = 2 * (g >> 1) + 8 * (g & 1);   // word of x[4(g >> 1) + 8 r0]
            const int e1 = e0 + 4;                       // r0 + 1
            w[4 * g + 0] = pair_lo(d[e0], d[e0 + 1]);
            w[4 * g + 1] = pair_hi(d[e0], d[e0 + 1]);
            w[4 * g + 2] = pair_lo(d[e1], d[e1 + 1]);
            w[4 * g + 3] = pair_hi(d[e1], d[e1 + 1]);
        }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
        o[q] = make_uint4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
}

// One 16-row tile's codes and scales for a wave's K slice (KW blocks per
// wave at most).  Codes: per step one 16-byte load per lane (lane group g:
// block b0 + g, Q4_0; block b0 + g/2, Q8_0; blocks b0 + 2g, b0 + 2g + 1, q2w).  Scales, WS (rows of an even
// number of blocks, so every row's scales are 4-byte aligned): one load per
// lane per tile of the KW/4 scales of row c starting at block kbeg + g*KW/4
// (16 rows x KW*2 bytes per instruction rather than one instruction per step,
// a quarter of the cache requests); otherwise one 2-byte scale per lane per
// step (lane group g: the block its code load covers).
template <int FMT, int KW, bool WS>
struct TileRegs {
    static_assert(FMT != kQ2W || WS, "q2w tiles take their scales per lane group");
    static constexpr int kSteps = KW / blocks_per_load<FMT>();
    static constexpr int kScaleRegs = WS ? KW / 8 : kSteps;
    uint4 code[kSteps];
    uint32_t scl[kScaleRegs];
};

// Issue one tile's loads at the lane's 32-bit offsets coff / soff from the
// tile's first block.  Every load is issued, so the compiler waits for
// exactly one tile's loads while the next tile's are in flight: blocks past
// the wave's slice read neighbouring blocks of the matrix and rows past N
// read zeros (the descriptors end at the matrix), and `compute_tile` drops
// both.  A tile past the last one (the prefetch after a workgroup's final
// tile) gets empty descriptors: its loads return zeros without touching
// memory.
// `row_shift` moves the tile down the table (SwiGLU: the up rows, N below
// the gate rows) and `rows` is the table's row count (N, or 2N for SwiGLU).
template <int FMT, int KW, bool WS>
__device__ __forceinline__ void load_tile(const MfmaParams &p, int tile, int ntiles, int KB, uint32_t coff,
                                          uint32_t soff, TileRegs<FMT, KW, WS> &t, int64_t row_shift, int64_t rows)
{
    constexpr int kBlocksPerLoad = blocks_per_load<FMT>();
    constexpr int CB = mfma_code_bytes<FMT>();
    const int64_t nblocks = rows * KB;
    const bool real = tile < ntiles;
    const int64_t base = real ? ((int64_t)tile * 16 + row_shift) * KB : 0;
    const int64_t left = real ? nblocks - base : 0;
    const auto rc = make_rsrc(p.W + base * CB, left * CB);
    const auto rs = make_rsrc(p.W + p.scale_offset + base * 2, left * 2);
#pragma unroll
    for (int s = 0; s < TileRegs<FMT, KW, WS>::kSteps; ++s)
        t.code[s] = stream_load16(rc, coff + s * kBlocksPerLoad * CB);
    if constexpr (WS) {
        if constexpr (KW == 8) {
            t.scl[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, soff, 0, kNtAux);
        } else if constexpr (KW == 16) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, soff, 0, kNtAux);
            t.scl[0] = v[0];
            t.scl[1] = v[1];
        } else {
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, soff, 0, kNtAux);
            t.scl[0] = v[0];
            t.scl[1] = v[1];
            t.scl[2] = v[2];
            t.scl[3] = v[3];
        }
    } else {
#pragma unroll
        for (int s = 0; s < TileRegs<FMT, KW, WS>::kSteps; ++s)
            t.scl[s] = stream_load2(rs, soff + s * kBlocksPerLoad * 2);
    }
}

__device__ __forceinline__ float half_lo(uint32_t u) { return (float)__builtin_bit_cast(_Float16, (uint16_t)u); }
__device__ __forceinline__ float half_hi(uint32_t u)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16));
}

// The tile's partial 16 x 16 product over this wave's K slice:
// D layout lane l, register r -> token 4(l/16) + r, row l%16 of the tile.
// Lanes whose A row is past the tokens (c >= M) read token `cm` = min(c,
// M - 1): row i of D depends only on row i of A, so those rows are never
// stored and need no masking.  Blocks past the slice (only in the last step)
// are skipped with a wave-uniform branch; rows past N carry zero scales (the
// descriptor returns zeros) and are not stored.
template <int FMT, int KW, bool WS>
__device__ __forceinline__ f4_t compute_tile(TileRegs<FMT, KW, WS> &t, const uint4 *xs, int M, int cm, int xq,
                                             int kbeg, int kend, int nsteps, uint32_t magic)
{
    constexpr int kBlocksPerLoad = blocks_per_load<FMT>();
    constexpr int kSteps = TileRegs<FMT, KW, WS>::kSteps;
    const uint32_t q2_shift = ((threadIdx.x >> 4) & 1u) * 4u;   // q2w: 4 (g & 1)
    // WS: every lane group's scale words to all four groups: bc[d][src] is
    // word d of lane group src (scales of blocks kbeg + src*KW/4 + 2d, +1)
    uint32_t bc[WS ? KW / 8 : 1][4];
    if constexpr (WS) {
#pragma unroll
        for (int d = 0; d < KW / 8; ++d) {
            uint32_t lo = t.scl[d], hi = t.scl[d];
            swap32(lo, hi);                    // lo = [r0 r1 r0 r1], hi = [r2 r3 r2 r3]
            uint32_t lo2 = lo, hi2 = hi;
            swap16(lo, lo2);                   // lo = [r0 x4], lo2 = [r1 x4]
            swap16(hi, hi2);                   // hi = [r2 x4], hi2 = [r3 x4]
            bc[d][0] = lo;
            bc[d][1] = lo2;
            bc[d][2] = hi;
            bc[d][3] = hi2;
        }
    }
    f4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        if (s < nsteps) {
            const int b0 = kbeg + s * kBlocksPerLoad;
            uint32_t w0 = t.code[s].x, w1 = t.code[s].y, w2 = t.code[s].z, w3 = t.code[s].w;
            uint32_t sc[4] = {0u, 0u, 0u, 0u};
            if constexpr (!WS) {
                // scale of (row, block b0 + j) to every lane group of the row
                uint32_t sa = t.scl[s], sb = t.scl[s];
                swap32(sa, sb);                      // Q4_0: sa = [s0 s1 s0 s1], sb = [s2 s3 s2 s3]
                if constexpr (FMT == kQ4_0) {
                    uint32_t sa2 = sa, sb2 = sb;
                    swap16(sa, sa2);
                    swap16(sb, sb2);
                    sc[0] = sa; sc[1] = sa2; sc[2] = sb; sc[3] = sb2;
                } else {
                    sc[0] = sa; sc[1] = sb;          // Q8_0: [s0 s0 s0 s0], [s1 s1 s1 s1]
                }
            }
            uint32_t q2[FMT == kQ2W ? 8 : 1];
            if constexpr (FMT == kQ4_0) {
                // 4 x 4 transpose across lane groups: afterwards register j
                // of lane group g holds word g of block b0 + j
                swap32(w0, w2);
                swap32(w1, w3);
                swap16(w0, w1);
                swap16(w2, w3);
            } else if constexpr (FMT == kQ2W) {
                // lane group h holds (w0, w1) of block b0 + 2h and (w2, w3) of
                // b0 + 2h + 1; afterwards q2[j] of lane group g is word g >> 1
                // of block b0 + j (each word reaches two lane groups)
                swap16(w0, w1);   // w0 = words (0, 1) of blocks 0, 4; w1: blocks 2, 6
                swap16(w2, w3);   // w2: blocks 1, 5; w3: blocks 3, 7
                const uint32_t src[4] = {w0, w1, w2, w3};
                const int first[4] = {0, 2, 1, 3};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    uint32_t a = src[k], b = src[k];
                    swap16(a, b);   // a = [x.r0 x.r0 x.r2 x.r2], b = [x.r1 x.r1 x.r3 x.r3]
                    swap32(a, b);   // a = [x.r0 x.r0 x.r1 x.r1], b = [x.r2 x.r2 x.r3 x.r3]
                    q2[first[k]] = a;
                    q2[first[k] + 4] = b;
                }
            } else {
                // afterwards (w0, w1) hold block b0 and (w2, w3) block b0 + 1:
                // lane group g has code words 2p, 2p + 1, p = {0, 2, 1, 3}[g]
                swap32(w0, w2);
                swap32(w1, w3);
            }
#pragma unroll
            for (int j = 0; j < kBlocksPerLoad; ++j) {
                const int b = b0 + j;
                if (b < kend) {
                    half8_t bop;
                    if constexpr (FMT == kQ4_0)
                        bop = q4_operand(j == 0 ? w0 : j == 1 ? w1 : j == 2 ? w2 : w3, magic);
                    else if constexpr (FMT == kQ8_0)
                        bop = (j == 0) ? q8_operand(w0, w1, magic) : q8_operand(w2, w3, magic);
                    else
                        bop = q2_operand(q2[j] >> q2_shift, magic);
                    const uint4 v = xs[((b - kbeg) * M + cm) * 4 + (xq ^ ((b - kbeg) & 3))];
                    const half8_t aop = pack8(v.x, v.y, v.z, v.w);
                    const f4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
                    const f4_t d = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop, zero, 0, 0, 0);
                    float scv;
                    if constexpr (WS) {
                        constexpr int kPer = KW / 4;          // scales per lane group
                        const int rb = s * kBlocksPerLoad + j;   // block within the slice
                        const uint32_t wsc = bc[(rb % kPer) / 2][rb / kPer];
                        scv = (rb & 1) ? half_hi(wsc) : half_lo(wsc);
                    } else {
                        scv = half_lo(sc[j]);
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[r] = __builtin_fmaf(scv, d[r], acc[r]);
                }
            }
        }
    }
    return acc;
}

// Sum a team's partial tiles in a fixed order (its wave 0 first) and store.
// `red` is double-buffered by tile parity: tile i writes red[i & 1] and one
// barrier per tile separates every write from the reads of the same buffer.
// The reducing wave rotates with the tile so no wave carries all stores.
// A team is `nwaves` waves from wave `wbase`; `kw` is this wave's index in it.
template <int NW>
__device__ __forceinline__ void reduce_store(const MfmaParams &p, f4_t acc, f4_t (*red)[NW][64], int it, int tile,
                                             int wave, int wbase, int kw, int nwaves, int lane, int g, int c)
{
    const int par = it & 1;
    red[par][wave][lane] = acc;
    __syncthreads();
    if (kw == it % nwaves) {
        f4_t s = red[par][wbase][lane];
        for (int w = 1; w < nwaves; ++w) {
            const f4_t t = red[par][wbase + w][lane];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                s[r] += t[r];
        }
        const int n = tile * 16 + c;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 4 * g + r;
            if (m < p.M && n < p.N)
                p.y[(int64_t)m * p.N + n] = s[r];
        }
    }
}

// SwiGLU: the gate and up tiles' partial products, summed like
// reduce_store (gate in red[par], up in red[2 + par]); the storing wave
// writes silu(g) * u, evaluated in fp32 as the vector kernel's epilogue
// does [the CUDA-kernel diary's FFN fusion step: gate, up and SwiGLU in one
// kernel, only the final product written].
template <int NW>
__device__ __forceinline__ void reduce_store_glu(const MfmaParams &p, f4_t accg, f4_t accu, f4_t (*red)[NW][64],
                                                 int it, int tile, int wave, int wbase, int kw, int nwaves, int lane,
                                                 int g, int c)
{
    const int par = it & 1;
    red[par][wave][lane] = accg;
    red[2 + par][wave][lane] = accu;
    __syncthreads();
    if (kw == it % nwaves) {
        f4_t sg = red[par][wbase][lane], su = red[2 + par][wbase][lane];
        for (int w = 1; w < nwaves; ++w) {
            const f4_t tg = red[par][wbase + w][lane], tu = red[2 + par][wbase + w][lane];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sg[r] += tg[r];
                su[r] += tu[r];
            }
        }
        const int n = tile * 16 + c;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 4 * g + r;
            if (m < p.M && n < p.N)
                p.y[(int64_t)m * p.N + n] = sg[r] / (1.0f + expf(-sg[r])) * su[r];
        }
    }
}

// fp32 activations rounded to binary16 (nearest, ties to even: the
// conversion's default mode; beyond binary16's range: infinity), two per
// word in natural order [volta-kernel-bakeoff, "Results": fp32 activations
// in, the conversion inside the kernel].
__device__ __forceinline__ uint32_t half2_bits(float a, float b)
{
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
}

// Persistent over 16-row tiles: a workgroup holds TEAMS teams of waves;
// team t of workgroup w takes tiles TEAMS w + t, + TEAMS grid, ...; a
// team's waves split K and prefetch the next tile's codes and scales while
// the current tile is multiplied.  The activation slices are staged in LDS
// once per workgroup (by team 0) and read by every team: two teams of a
// workgroup share one copy where two workgroups of one team each read their
// own (every copy of x is read from L2; with a few tiles per workgroup the
// copies approach the weight bytes).  Every team runs the same number of
// iterations (one barrier each); a team past the last tile multiplies
// zeros and stores nothing.
// GLU (fp32 input): a tile's gate rows and its up rows, N rows below them,
// are multiplied one after the other, each while the other's loads are in
// flight, and combined when both are summed.

template <int FMT, int KWMAX, bool WS, bool F32, bool GLU, int TEAMS>
__global__ __launch_bounds__(512 * TEAMS) void gemv_mfma_kernel(MfmaParams p)
{
    static_assert(!GLU || (F32 && FMT == kQ4_0), "SwiGLU: Q4_0 with fp32 activations");
    static_assert(TEAMS == 1 || TEAMS == 2, "one or two teams per workgroup");
    constexpr int kBlocksPerLoad = blocks_per_load<FMT>();   // blocks of 16 rows per 16-byte load step
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nwaves = (blockDim.x >> 6) / TEAMS;   // waves per team
    const int team = wave / nwaves;
    const int kwv = wave - team * nwaves;            // this wave's K slice
    const int wbase = team * nwaves;
    const int g = lane >> 4;          // lane group
    const int c = lane & 15;          // row within the tile / token of the A operand
    const int KB = p.K >> 5;
    const int ntiles = (p.N + 15) >> 4;
    const int kbeg = kwv * p.kw;
    const int kend = min(KB, kbeg + p.kw);
    const int nblk = max(0, kend - kbeg);
    const int nsteps = (nblk + kBlocksPerLoad - 1) / kBlocksPerLoad;

    // 1. this wave's activations (M tokens x its blocks), issued first (they
    //    come from cache; loads retire in order).  fp16: each lane loads the
    //    64 bytes of its (token, block) pairs (pair i is (token i / nblk,
    //    block i % nblk); pairs past the slice re-read a valid block).  fp32
    //    (128 bytes a pair): whole lines at a time, lane l of load u taking
    //    16-byte chunk l + 64 u of the token-major slice (a lane per pair put
    //    each lane of an instruction on a different cache line; with fp32
    //    the address unit then bounded the staging: 8 tokens of 14336 x 4096
    //    18.4 -> 16.9 us); chunks past the slice re-read a valid one.
    constexpr int kXPer = 8 * KWMAX / 64;    // (token, block) pairs per lane, M <= 8
    constexpr int kCpt = KWMAX * 8;          // fp32: 16-byte chunks per token row slot
    constexpr int kCPer = F32 ? 8 * kCpt / 64 : 1;   // fp32: chunks per lane
    const int npairs = p.M * nblk;
    uint4 xr[F32 ? 1 : kXPer][4];
    u32x4_t xc[kCPer];
    const bool stager = team == 0;   // wave-uniform
    if (!stager) {
    } else if constexpr (F32) {
#pragma unroll
        for (int u = 0; u < kCPer; ++u) {
            const int f = lane + 64 * u;
            const int m = min(f / kCpt, p.M - 1);
            const int b = min((f % kCpt) >> 3, max(nblk, 1) - 1);
            const int blk = min(kbeg + b, KB - 1);
            xc[u] = reinterpret_cast<const u32x4_t *>(p.xf + (int64_t)m * p.K + (int64_t)blk * 32)[f & 7];
        }
    } else {
#pragma unroll
        for (int t = 0; t < kXPer; ++t) {
            const int i = min(lane + 64 * t, max(npairs, 1) - 1);
            const int m = i / max(nblk, 1), b = i - m * max(nblk, 1);
            const int blk = min(kbeg + b, KB - 1);
            const uint4 *src = reinterpret_cast<const uint4 *>(p.x + (int64_t)m * p.K + (int64_t)blk * 32);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                xr[t][q] = src[q];
        }
    }

    // 2. the first tile's codes and scales; lane offsets from a tile's first
    //    block (row c of the tile, this wave's first block, lane group g)
    const int gb = (FMT == kQ4_0) ? g : (FMT == kQ8_0 ? (g >> 1) : 2 * g);
    const uint32_t coff = (uint32_t)(c * KB + kbeg + gb) * (uint32_t)mfma_code_bytes<FMT>() +
                          ((FMT == kQ8_0) ? (uint32_t)(g & 1) * 16u : 0u);
    const uint32_t soff = WS ? (uint32_t)(c * KB + kbeg + g * (KWMAX / 4)) * 2u : (uint32_t)(c * KB + kbeg + gb) * 2u;
    const int64_t rows = GLU ? 2 * (int64_t)p.N : (int64_t)p.N;   // rows of the packed table
    // The workgroup walks units: tiles blockIdx.x, + grid, ...; with SwiGLU
    // each tile is two units, its gate rows and then its up rows (N further
    // down the table), so one unit's loads are in flight while the other is
    // multiplied, with the registers of the plain kernel.
    const int step = gridDim.x * TEAMS;
    const int first = blockIdx.x * TEAMS + team;
    TileRegs<FMT, KWMAX, WS> ta, tb;
    load_tile<FMT, KWMAX, WS>(p, first, ntiles, KB, coff, soff, ta, 0, rows);
    __builtin_amdgcn_sched_barrier(0);

    // 3. the activations into this wave's own LDS area in MFMA operand
    //    order; layout [block][token][64 bytes], 16-byte chunk q of (block b,
    //    token m) at position q ^ (b & 3) of its slot: consecutive lanes hold
    //    consecutive blocks, whose slots are M * 64 bytes apart (the same
    //    banks for M a multiple of 4), and the swizzle spreads four of them
    //    over different banks.  fp32 first goes in natural order
    //    ([token][block][64 bytes], rounded to binary16 here) and is then
    //    rearranged in place: every lane reads all its pairs before any lane
    //    writes (both layouts cover the same M x nblk slots).  The area is
    //    this wave's own and LDS keeps a wave's order: no barrier.  Lanes
    //    past the slice repeat a valid chunk or pair (the same bytes to the
    //    same place), so no write is conditional.
    extern __shared__ uint4 xs_dyn[];
    uint4 *xs = xs_dyn + (int64_t)kwv * p.kw * p.M * 4;
    uint4 xn[kXPer][4];
    if (!stager) {
    } else if constexpr (F32) {
#pragma unroll
        for (int u = 0; u < kCPer; ++u) {
            const int f = lane + 64 * u;
            const int m = min(f / kCpt, p.M - 1);
            const int b = min((f % kCpt) >> 3, max(nblk, 1) - 1);
            // (each element copied out before the bit cast: this compiler
            // bit-casts an element of a vector-typed value in place as
            // element 0)
            const u32x4_t v = xc[u];
            const u32x2_t h = {half2_bits(__builtin_bit_cast(float, (uint32_t)v[0]), __builtin_bit_cast(float, (uint32_t)v[1])),
                               half2_bits(__builtin_bit_cast(float, (uint32_t)v[2]), __builtin_bit_cast(float, (uint32_t)v[3]))};
            reinterpret_cast<u32x2_t *>(xs)[(m * nblk + b) * 8 + (f & 7)] = h;
        }
        // the two layouts are accessed through different types: keep the
        // compiler from moving the reads above the writes, or the writes
        // below above the reads
        asm volatile("" ::: "memory");
#pragma unroll
        for (int t = 0; t < kXPer; ++t) {
            const int i = min(lane + 64 * t, max(npairs, 1) - 1);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                xn[t][q] = xs[i * 4 + q];
        }
        asm volatile("" ::: "memory");
    } else {
#pragma unroll
        for (int t = 0; t < kXPer; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                xn[t][q] = xr[t][q];
    }
    if (stager) {
#pragma unroll
        for (int t = 0; t < kXPer; ++t) {
            const int i = min(lane + 64 * t, max(npairs, 1) - 1);
            const int m = i / max(nblk, 1), b = i - m * max(nblk, 1);
            uint4 o[4];
            permute_x<FMT>(xn[t], o);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                xs[(b * p.M + m) * 4 + (q ^ (b & 3))] = o[q];
        }
    }
    if constexpr (TEAMS > 1)
        __syncthreads();   // team 0's copy, read by every team

    __shared__ f4_t red[GLU ? 4 : 2][kMaxWavesPerWg * TEAMS][64];
    const uint32_t magic = magic_reg();
    const int cm = min(c, p.M - 1);
    const int xq = (FMT == kQ8_0) ? (((g & 1) << 1) | (g >> 1)) : g;
    const int last = ntiles - 1;
    if constexpr (GLU) {
        // units: gate of tile t in ta, its up rows in tb; while one is
        // multiplied the other's loads (or the next tile's gate) are in flight
        for (int it = 0, tile = first;; ++it, tile += step) {
            load_tile<FMT, KWMAX, WS>(p, tile, ntiles, KB, coff, soff, tb, p.N, rows);
            __builtin_amdgcn_sched_barrier(0);
            const f4_t accg = compute_tile<FMT, KWMAX, WS>(ta, xs, p.M, cm, xq, kbeg, kend, nsteps, magic);
            const int t1 = tile + step;   // past the end: empty loads, never used
            load_tile<FMT, KWMAX, WS>(p, t1, ntiles, KB, coff, soff, ta, 0, rows);
            __builtin_amdgcn_sched_barrier(0);
            const f4_t accu = compute_tile<FMT, KWMAX, WS>(tb, xs, p.M, cm, xq, kbeg, kend, nsteps, magic);
            reduce_store_glu(p, accg, accu, red, it, tile, wave, wbase, kwv, nwaves, lane, g, c);
            if (t1 - team > last)   // team 0's next tile: the same test for every wave
                break;
        }
    } else {
        // (the loop ends on team 0's tiles, the same test for every wave; a
        // team past the last tile gets empty loads and stores nothing)
        for (int it = 0, tile = first;; it += 2) {
            // tile in `ta`; prefetch the next into `tb` (past the end: empty
            // loads, never used)
            const int t1 = tile + step;
            load_tile<FMT, KWMAX, WS>(p, t1, ntiles, KB, coff, soff, tb, 0, rows);
            __builtin_amdgcn_sched_barrier(0);
            f4_t acc = compute_tile<FMT, KWMAX, WS>(ta, xs, p.M, cm, xq, kbeg, kend, nsteps, magic);
            reduce_store(p, acc, red, it, tile, wave, wbase, kwv, nwaves, lane, g, c);
            if (t1 - team > last)
                break;
            const int t2 = t1 + step;
            load_tile<FMT, KWMAX, WS>(p, t2, ntiles, KB, coff, soff, ta, 0, rows);
            __builtin_amdgcn_sched_barrier(0);
            acc = compute_tile<FMT, KWMAX, WS>(tb, xs, p.M, cm, xq, kbeg, kend, nsteps, magic);
            reduce_store(p, acc, red, it + 1, t1, wave, wbase, kwv, nwaves, lane, g, c);
            if (t2 - team > last)
                break;
            tile = t2;
        }
    }
}

// Workgroups of `fn` resident on one CU at once (at least 1), cached per
// kernel, block size and LDS size.
int resident_per_cu(const void *fn, int threads, size_t shmem)
{
    static std::mutex mu;
    static std::map<std::tuple<const void *, int, size_t>, int> cache;
    const auto key = std::make_tuple(fn, threads, shmem);
    std::lock_guard<std::mutex> lock(mu);
    const auto it = cache.find(key);
    if (it != cache.end())
        return it->second;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, threads, shmem) != hipSuccess || n < 1)
        n = 1;
    cache.emplace(key, n);
    return n;
}

template <int FMT, int KWMAX, bool WS, int TEAMS>
const void *mfma_kernel_fn(int variant)
{
    if constexpr (FMT == kQ4_0)
        return variant == 2   ? reinterpret_cast<const void *>(&gemv_mfma_kernel<FMT, KWMAX, WS, true, true, TEAMS>)
               : variant == 1 ? reinterpret_cast<const void *>(&gemv_mfma_kernel<FMT, KWMAX, WS, true, false, TEAMS>)
                              : reinterpret_cast<const void *>(&gemv_mfma_kernel<FMT, KWMAX, WS, false, false, TEAMS>);
    else
        return reinterpret_cast<const void *>(&gemv_mfma_kernel<FMT, KWMAX, WS, false, false, TEAMS>);
}

template <int FMT, int KWMAX, bool WS>
hipError_t launch_kw(const MfmaParams &p, int waves, int teams, int64_t wgs, int cus, hipStream_t stream)
{
    // fp32 activations and SwiGLU: Q4_0 only (their entry points' format)
    int variant = 0;
    if constexpr (FMT == kQ4_0) {
        variant = p.glu ? 2 : (p.xf ? 1 : 0);
        if (p.glu && !p.xf)
            return hipErrorInvalidValue;
    } else {
        if (p.xf || p.glu)
            return hipErrorInvalidValue;
    }
    // two teams: 16 waves, at most 128 VGPRs each (slices of up to 16 blocks)
    if (teams < 1 || teams > 2 || (teams == 2 && (KWMAX > 16 || waves > 8)))
        return hipErrorInvalidValue;
    const void *fn = teams == 2 ? mfma_kernel_fn<FMT, KWMAX, WS, (KWMAX <= 16 ? 2 : 1)>(variant)
                                : mfma_kernel_fn<FMT, KWMAX, WS, 1>(variant);
    // the workgroup stages M x kw blocks of activations per wave of a team
    // (64 bytes each); the partial tiles take (2, SwiGLU 4) x 8 KB per team of
    // static LDS
    const size_t shmem = (size_t)waves * p.kw * p.M * 64;
    const size_t red = (size_t)(p.glu ? 4 : 2) * teams * 8192;
    if (shmem > kMaxLds || shmem + red > kMaxLds + 16384)
        return hipErrorInvalidValue;
    static std::mutex mu;
    static std::set<const void *> raised;   // dynamic LDS beyond the default allowed once per kernel
    {
        std::lock_guard<std::mutex> lock(mu);
        if (!raised.count(fn)) {
            // at most what the static partial-tile buffers leave of 160 KB
            const int cap = (int)std::min<size_t>(kMaxLds, 160 * 1024 - red);
            if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, cap) != hipSuccess) {
                (void)hipGetLastError();   // reported as a shape error, not left for the next runtime call
                return hipErrorInvalidValue;
            }
            raised.insert(fn);
        }
    }
    const int64_t units = ((p.N + 15) / 16 + teams - 1) / teams;   // tiles per team slot
    if (wgs <= 0) {
        // as many workgroups as are resident at once (registers, LDS, wave
        // slots), at most 2 per CU with one team (MI355X, 8 tokens, 28672 x
        // 4096: fp32 activations 25.2 us at two per CU against 26.2 at one)
        // and 1 with two
        wgs = (int64_t)cus * std::min(teams == 2 ? 1 : 2, resident_per_cu(fn, 64 * waves * teams, shmem));
    }
    wgs = std::min(wgs, units);
    const dim3 grid((unsigned)wgs), block(64 * waves * teams);
    return launch_kernel(fn, grid, block, shmem, stream, p);
}

template <int FMT>
hipError_t launch_fmt(const MfmaParams &p, int kwmax, int waves, int teams, int64_t wgs, int cus, hipStream_t stream)
{
    const bool ws = (p.K / 32) % 2 == 0;   // every row's scales 4-byte aligned
    if constexpr (FMT == kQ2W) {
        if (!ws)
            return hipErrorInvalidValue;   // q2w: an even number of blocks per row
        switch (kwmax) {
        case 8: return launch_kw<FMT, 8, true>(p, waves, teams, wgs, cus, stream);
        case 16: return launch_kw<FMT, 16, true>(p, waves, teams, wgs, cus, stream);
        case 32: return launch_kw<FMT, 32, true>(p, waves, teams, wgs, cus, stream);
        }
        return hipErrorInvalidValue;
    } else {
        switch (kwmax) {
        case 8: return ws ? launch_kw<FMT, 8, true>(p, waves, teams, wgs, cus, stream)
                          : launch_kw<FMT, 8, false>(p, waves, teams, wgs, cus, stream);
        case 16: return ws ? launch_kw<FMT, 16, true>(p, waves, teams, wgs, cus, stream)
                           : launch_kw<FMT, 16, false>(p, waves, teams, wgs, cus, stream);
        case 32: return ws ? launch_kw<FMT, 32, true>(p, waves, teams, wgs, cus, stream)
                           : launch_kw<FMT, 32, false>(p, waves, teams, wgs, cus, stream);
        }
        return hipErrorInvalidValue;
    }
}

// ----------------------------------------------------------- skinny prefill
//
// Q4_0 GEMM for 9..64 tokens (Y[m][n] = sum_k X[m][k] w[n][k], w rounded to
// fp16 as in the tiled prefill): the weights are streamed once, in 16-row
// tiles, as the few-token kernel streams them, and each wave keeps its K
// slice of every token's activations in registers as ready MFMA A operands
// for the whole launch [volta-kernel-bakeoff, "Where we lose: prompts" and
// "Stage 3": the unpack inside the matrix multiply].  Per 32-weight block of
// 16 rows the B operand is unpacked once (q4_operand), scaled by the block's
// fp16 scale with one rounding (the values qdequant_q4_0 writes with fp16
// output) and used by one v_mfma_f32_16x16x32_f16 per 16-token group, all
// accumulating into fp32.  The waves' partial 16 x (16 MT) tiles are summed
// through LDS in a fixed order; a launch whose workgroups each cover all of K
// stores every output once (bitwise reproducible), one that splits K over
// workgroups adds the parts with fp32 atomics into a zero-filled Y.

struct SkinnyParams {
    const uint8_t *W;
    const uint16_t *X;     // fp16 [M][K]
    float *Y;              // fp32 [M][N]
    int64_t scale_offset;
    int M, N, K;
    int kw;                // blocks per wave (<= KWA)
    int span;              // blocks per workgroup along K (waves * kw)
    int atomic;            // 1: K split over workgroups (blockIdx.y), parts added into zero-filled Y
};

constexpr int kSkinnyWaves = 8;

// uint4 of LDS before the LDS-held operands: the larger of the staging
// windows (16 tokens x BB blocks per wave, padded rows) and the partial tiles
constexpr int skinny_region_uint4(int MT, int BB)
{
    const int stage = kSkinnyWaves * 16 * (BB * 4 + 1);
    const int red = 2 * kSkinnyWaves * MT * 64;
    return stage > red ? stage : red;
}

template <int MT, int KWA, int KWL>
__global__ __launch_bounds__(512) void skinny_kernel(SkinnyParams p)
{
    // KWA blocks per wave hold their A operands in registers, KWL more in
    // LDS (read back per tile: registers run out first)
    constexpr int KWT = KWA + KWL;
    constexpr int KW = (KWT + 3) / 4 * 4;   // four blocks of 16 rows per 16-byte load step
    constexpr int kSteps = KW / 4;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nwaves = blockDim.x >> 6;
    const int g = lane >> 4;          // lane group
    const int c = lane & 15;          // row of the tile (B) / token of the group (A)
    const int KB = p.K >> 5;
    const int ntiles = (p.N + 15) >> 4;
    const int kbeg = blockIdx.y * p.span + wave * p.kw;
    const int kend = min(KB, kbeg + p.kw);
    const int nblk = max(0, kend - kbeg);
    const int nsteps = (nblk + 3) / 4;

    // the first tile's codes and scales go out first: their HBM latency
    // overlaps the activation staging below (lane: row c, block b0 + g)
    const MfmaParams mp{p.W, nullptr, nullptr, nullptr, p.scale_offset, p.M, p.N, p.K, p.kw, 0};
    const uint32_t coff = (uint32_t)(c * KB + kbeg + g) * 16u;
    const uint32_t soff = (uint32_t)(c * KB + kbeg + g) * 2u;
    TileRegs<kQ4_0, KW, false> ta, tb;
    int tile = blockIdx.x;
    load_tile<kQ4_0, KW, false>(mp, tile, ntiles, KB, coff, soff, ta, 0, p.N);
    __builtin_amdgcn_sched_barrier(0);

    // 1. this wave's activations, every (block, token group), as A operands
    //    in the unpack's pair order: lane group g holds words 4g..4g+3 of the
    //    block's pair-ordered 16 words, i.e. (x[4g], x[4g+2]), (x[16+4g],
    //    x[18+4g]), (x[4g+1], x[4g+3]), (x[17+4g], x[19+4g]) of its token.
    //    Staged through this wave's LDS window eight blocks of 16 tokens at
    //    a time: whole 16-byte chunks of each token's slice read coalesced
    //    (32 lanes per 512-byte token row), then the 8-byte pieces each lane
    //    needs read back (token rows padded by 16 bytes: the 16 tokens of a
    //    read fall on different banks).  Tokens past M read token M - 1 (their
    //    rows of the product are never stored); blocks past the slice read
    //    the last block and are never multiplied.
    // LDS: the staging windows, then (after them) the partial tiles
    // [2][nwaves][MT][64] in the same bytes; the LDS-held operands
    // [wave][KWL][MT][64 lanes] beyond both
    extern __shared__ f4_t red_dyn[];
    constexpr int BB = KWL > 0 ? 4 : 8;     // blocks per staging batch
    constexpr int kRow = BB * 4 + 1;        // uint4 per staged token row: BB blocks x 64 bytes + padding
    constexpr int kRegion = skinny_region_uint4(MT, BB);
    uint4 *stage = reinterpret_cast<uint4 *>(red_dyn) + wave * 16 * kRow;
    half8_t A[KWA][MT];
    uint4 *alds = reinterpret_cast<uint4 *>(red_dyn) + kRegion + wave * KWL * MT * 64;
#pragma unroll
    for (int tg = 0; tg < MT; ++tg) {
#pragma unroll
        for (int bb = 0; bb < KWT; bb += BB) {
            uint4 v[BB];
#pragma unroll
            for (int i = 0; i < BB; ++i) {
                // chunk q: token q / (4 BB), block (q % (4 BB)) / 4, 16-byte part q % 4
                const int q = lane + 64 * i;
                const int t = q / (4 * BB), b = (q % (4 * BB)) >> 2, u = q & 3;
                const int m = min(tg * 16 + t, p.M - 1);
                const int blk = min(kbeg + bb + b, KB - 1);
                v[i] = *reinterpret_cast<const uint4 *>(p.X + (int64_t)m * p.K + (int64_t)blk * 32 + 8 * u);
            }
#pragma unroll
            for (int i = 0; i < BB; ++i) {
                const int q = lane + 64 * i;
                stage[(q / (4 * BB)) * kRow + q % (4 * BB)] = v[i];
            }
            // LDS keeps a wave's order: the reads below see these writes
            const uint2 *st2 = reinterpret_cast<const uint2 *>(stage);
#pragma unroll
            for (int b = 0; b < BB; ++b) {
                if (bb + b < KWT) {
                    const int base = (c * kRow + b * 4) * 2 + (g & 1);   // uint2 units
                    const uint2 lo = st2[base + 2 * (g >> 1)];            // bytes 8g..8g+7: x[4g..4g+3]
                    const uint2 hi = st2[base + 2 * (2 + (g >> 1))];      // bytes 32+8g..: x[16+4g..19+4g]
                    const half8_t f = pack8(pair_lo(lo.x, lo.y), pair_lo(hi.x, hi.y), pair_hi(lo.x, lo.y),
                                            pair_hi(hi.x, hi.y));
                    if (bb + b < KWA)
                        A[(bb + b) < KWA ? bb + b : 0][tg] = f;
                    else
                        alds[((bb + b - KWA) * MT + tg) * 64 + lane] = __builtin_bit_cast(uint4, f);
                }
            }
        }
    }
    __syncthreads();   // the staging windows become the partial-tile buffers

    // 2. tiles w, w + grid, ...: codes and scales of the next tile in flight
    //    while the current one is multiplied
    const int step = gridDim.x;
    const int last = ntiles - 1;
    const uint32_t magic = magic_reg();

    auto compute = [&](const TileRegs<kQ4_0, KW, false> &t, f4_t (&acc)[MT]) {
#pragma unroll
        for (int tg = 0; tg < MT; ++tg)
            acc[tg] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            if (s < nsteps) {
                // scale of (row c, block 4s + j) to every lane group, and the
                // 4 x 4 transpose of the code words (register j of lane group
                // g: word g of block 4s + j), as the few-token kernel does
                uint32_t sa = t.scl[s], sb = t.scl[s];
                swap32(sa, sb);
                uint32_t sa2 = sa, sb2 = sb;
                swap16(sa, sa2);
                swap16(sb, sb2);
                const uint32_t sc[4] = {sa, sa2, sb, sb2};
                uint32_t w0 = t.code[s].x, w1 = t.code[s].y, w2 = t.code[s].z, w3 = t.code[s].w;
                swap32(w0, w2);
                swap32(w1, w3);
                swap16(w0, w1);
                swap16(w2, w3);
                const uint32_t wj[4] = {w0, w1, w2, w3};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int b = 4 * s + j;
                    if (b < KWT && b < nblk) {
                        const _Float16 d = __builtin_bit_cast(_Float16, (uint16_t)(sc[j] & 0xFFFFu));
                        const half8_t dv = {d, d, d, d, d, d, d, d};
                        const half8_t bop = q4_operand(wj[j], magic) * dv;   // (q - 8) d, rounded once
#pragma unroll
                        for (int tg = 0; tg < MT; ++tg) {
                            const half8_t a = b < KWA ? A[b < KWA ? b : 0][tg]
                                                      : __builtin_bit_cast(half8_t,
                                                                           alds[((b - KWA) * MT + tg) * 64 + lane]);
                            acc[tg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bop, acc[tg], 0, 0, 0);
                        }
                    }
                }
            }
        }
    };

    // sum the waves' partial tiles (double-buffered by tile parity, one
    // barrier per tile; token group tg is summed and stored by wave
    // (tg + it) % nwaves, the waves in a fixed order)
    auto reduce_store = [&](const f4_t (&acc)[MT], int it, int tile) {
        const int par = it & 1;
#pragma unroll
        for (int tg = 0; tg < MT; ++tg)
            red_dyn[((par * nwaves + wave) * MT + tg) * 64 + lane] = acc[tg];
        __syncthreads();
#pragma unroll
        for (int tg = 0; tg < MT; ++tg) {
            if (wave == (tg + it) % nwaves) {
                f4_t sum = red_dyn[((par * nwaves) * MT + tg) * 64 + lane];
                for (int w = 1; w < nwaves; ++w) {
                    const f4_t v = red_dyn[((par * nwaves + w) * MT + tg) * 64 + lane];
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        sum[r] += v[r];
                }
                const int n = tile * 16 + c;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = tg * 16 + 4 * g + r;
                    if (m < p.M && n < p.N) {
                        float *dst = p.Y + (int64_t)m * p.N + n;
                        if (p.atomic)
                            unsafeAtomicAdd(dst, sum[r]);
                        else
                            *dst = sum[r];
                    }
                }
            }
        }
    };

    for (int it = 0;; it += 2) {
        f4_t acc[MT];
        const int t1 = tile + step;   // past the end: empty loads, never used
        load_tile<kQ4_0, KW, false>(mp, t1, ntiles, KB, coff, soff, tb, 0, p.N);
        __builtin_amdgcn_sched_barrier(0);
        compute(ta, acc);
        reduce_store(acc, it, tile);
        if (t1 > last)
            break;
        const int t2 = t1 + step;
        load_tile<kQ4_0, KW, false>(mp, t2, ntiles, KB, coff, soff, ta, 0, p.N);
        __builtin_amdgcn_sched_barrier(0);
        compute(tb, acc);
        reduce_store(acc, it + 1, t1);
        if (t2 > last)
            break;
        tile = t2;
    }
}

// The blocks per wave that each token-group count instantiates (their
// activation registers, 4 KWA MT, stay within ~160 so the kernel keeps two
// waves per SIMD without spilling).
template <int MT, int KWA, int KWL = 0>
hipError_t launch_skinny_kwa(const SkinnyParams &p, dim3 grid, dim3 block, size_t shmem, hipStream_t stream)
{
    const void *fn = reinterpret_cast<const void *>(&skinny_kernel<MT, KWA, KWL>);
    static bool raised = false;   // allow the kernel's LDS (at most 160 KB) once
    if (!raised) {
        if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess)
            return hipErrorInvalidValue;
        raised = true;
    }
    if (shmem > 160 * 1024)
        return hipErrorInvalidValue;
    return launch_kernel(fn, grid, block, shmem, stream, p);
}

}  // namespace

// Launch the matrix-core GEMV on fp16 activations x, or on fp32 activations
// xf (Q4_0; x then unused), or with glu the SwiGLU of a stacked 2N-row
// table (Q4_0, fp32 xf; scale_offset is the 2N-row table's, y is [M][N]):
// `waves` (1..8) split K; each wave takes
// kw = ceil(K/32 / waves) blocks rounded up to 4, at most 32; `wgs`
// persistent workgroups walk the 16-row tiles (0: the built-in count).
hipError_t launch_gemv_mfma(int fmt, const uint8_t *W, int64_t scale_offset, const uint16_t *x, const float *xf,
                            float *y, int M, int N, int K, int waves, int teams, int64_t wgs, int cus,
                            hipStream_t stream, bool glu)
{
    const int KB = K / 32;
    if (M < 1 || M > 8 || waves < 1 || waves > kMaxWavesPerWg || teams < 0 || teams > 2)
        return hipErrorInvalidValue;
    int kw = (KB + waves - 1) / waves;
    kw = (kw + 3) / 4 * 4;
    if (kw > 32)
        return hipErrorInvalidValue;
    const int kwmax = kw <= 8 ? 8 : (kw <= 16 ? 16 : 32);
    if (teams == 0) {
        // Two teams where a workgroup sees only a few tiles, so that the
        // per-workgroup copy of x weighs against the weight bytes (1.5 to 4
        // tiles per CU; MI355X, 8 tokens: 14336 x 4096 13.8 -> 13.0 us, fp32
        // input 15.4 -> 13.7, SwiGLU 2 x 14336 x 4096 23.0 -> 21.5 and 24.3 ->
        // 21.0 at 4 tokens, 2 x 6144 x 2048 9.6 -> 8.3; 28672 x 4096, 7 tiles
        // per CU: 20.9 -> 21.8, one team kept).
        const int64_t ntiles = ((int64_t)N + 15) / 16;
        teams = (kwmax <= 16 && 2 * ntiles >= 3LL * cus && ntiles <= 4LL * cus) ? 2 : 1;
    }
    MfmaParams p{W, x, xf, y, scale_offset, M, N, K, kw, glu ? 1 : 0};
    switch (fmt) {
    case kQ4_0: return launch_fmt<kQ4_0>(p, kwmax, waves, teams, wgs, cus, stream);
    case kQ8_0: return launch_fmt<kQ8_0>(p, kwmax, waves, teams, wgs, cus, stream);
    case kQ2W: return launch_fmt<kQ2W>(p, kwmax, waves, teams, wgs, cus, stream);
    }
    return hipErrorInvalidValue;
}


// Skinny prefill launcher (M = 1..64, Q4_0): eight waves per workgroup split
// a workgroup's K range; the blocks per wave (KWA) come from the instantiated
// set of the token-group count, the fewest K ranges first; one workgroup per
// CU (`wgs` overrides the count along N).  With more than one K range Y is
// zero-filled first and the ranges add into it.
hipError_t launch_prefill_skinny(const uint8_t *W, int64_t scale_offset, const uint16_t *X, float *Y, int M, int N,
                                 int K, int cus, int64_t wgs, hipStream_t stream)
{
    if (M < 1 || M > 64 || N < 1 || K < 32 || K % 32 != 0)
        return hipErrorInvalidValue;
    const int MT = (M + 15) / 16;
    const int KB = K / 32;
    constexpr int kWaves = kSkinnyWaves;
    // KWA candidates per token-group count (largest last)
    // (Four token groups: 10 = 7 in registers and 3 in LDS.)
    static const int kwa_set[4][3] = {{8, 16, 32}, {8, 16, 16}, {8, 12, 12}, {8, 10, 10}};
    int kwa = kwa_set[MT - 1][2];
    int S = (KB + kWaves * kwa - 1) / (kWaves * kwa);
    for (int i = 0; i < 3; ++i) {   // the smallest KWA that needs no more K ranges
        const int cand = kwa_set[MT - 1][i];
        if ((KB + kWaves * cand - 1) / (kWaves * cand) == S) {
            kwa = cand;
            break;
        }
    }
    const int kw = (KB + S * kWaves - 1) / (S * kWaves);
    const int64_t ntiles = (N + 15) / 16;
    int64_t gx = wgs > 0 ? wgs : std::max<int64_t>(1, cus / S);
    gx = std::min(gx, ntiles);
    if (S > 1) {
        const hipError_t e = launch_zero_fill(Y, (int64_t)M * N, cus, stream);
        if (e != hipSuccess)
            return e;
    }
    SkinnyParams p{W, X, Y, scale_offset, M, N, K, kw, kw * kWaves, S > 1 ? 1 : 0};
    const dim3 grid((unsigned)gx, (unsigned)S), block(64 * kWaves);
    // the partial tiles, or the activation staging windows (16 tokens x 8
    // blocks per wave, padded rows) before them; then the LDS-held operands
    const bool lds_ops = MT == 4 && kwa == 10;   // 7 blocks in registers, 3 in LDS
    const size_t shmem = (size_t)skinny_region_uint4(MT, lds_ops ? 4 : 8) * 16 +
                         (lds_ops ? (size_t)kWaves * 3 * MT * 64 * 16 : 0);
    switch (MT * 100 + kwa) {
    case 108: return launch_skinny_kwa<1, 8>(p, grid, block, shmem, stream);
    case 116: return launch_skinny_kwa<1, 16>(p, grid, block, shmem, stream);
    case 132: return launch_skinny_kwa<1, 32>(p, grid, block, shmem, stream);
    case 208: return launch_skinny_kwa<2, 8>(p, grid, block, shmem, stream);
    case 216: return launch_skinny_kwa<2, 16>(p, grid, block, shmem, stream);
    case 308: return launch_skinny_kwa<3, 8>(p, grid, block, shmem, stream);
    case 312: return launch_skinny_kwa<3, 12>(p, grid, block, shmem, stream);
    case 408: return launch_skinny_kwa<4, 8>(p, grid, block, shmem, stream);
    case 410: return launch_skinny_kwa<4, 7, 3>(p, grid, block, shmem, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace qg
