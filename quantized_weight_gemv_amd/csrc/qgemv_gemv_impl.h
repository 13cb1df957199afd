// Fused dequantize-and-multiply GEMV kernels (Q4_0, Q8_0, plain 2-bit q2w,
// and the one-launch MoE variant) for gfx950: the vector-ALU path (1..8
// tokens; the library uses it for 1..3 tokens and for rows too long for the
// matrix-core kernel).
//
// The work is bound by streaming the packed weights from HBM once per call
// [volta-kernel-bakeoff, "Why the V100 is interesting here";
//  H100-KERNEL-5X-ROADMAP, "Why the decode gap is bandwidth"], so the design
// goals are: every weight byte read exactly once with 16-byte coalesced loads,
// enough bytes in flight per compute unit to cover HBM latency, and an unpack
// cheap enough that the vector ALUs keep pace with the memory stream.  On
// MI355X the last point is the hard one: at ~7 TB/s a compute unit receives a
// 32-weight block every ~3 cycles, and a wave64 vector instruction occupies
// its SIMD for 4 cycles, so the per-block instruction count decides whether
// the kernel is memory- or ALU-bound.
//
// Mapping (one wave64 = 64 lanes):
//   * A row is spread over G lanes (G = 16, 32 or 64), so a wave works on
//     P = 64 / G rows at once (a "row set").  Lane l serves row l / G of the
//     set and, of that row, the blocks b0 + l % G + G j (j < J), where b0 is
//     the start of the wave's K chunk.  Lanes of one row read consecutive
//     16-byte code words: a load instruction touches P contiguous spans of
//     16 G bytes.
//   * A "team" of `ksplit` waves owns a group of R row sets at a time (wave w
//     of the team covers K chunk w); teams stride over the groups.
//   * Each lane keeps the activations of its blocks in registers for all M
//     tokens, loaded once per team and reused for every row the team visits
//     (one activation load serves many rows [volta-kernel-bakeoff, "Results",
//     the few-tokens bullet]), or, with XL (up to 4 tokens, whole rows per
//     wave), reads them from the workgroup's LDS copy, staged once for all
//     the workgroup's teams.
//   * Two register sets in ping-pong: the next group's loads are in flight
//     while the current group is unpacked and multiplied.
//   * Unpack: a nibble n OR-ed into the binary16 pattern 0x6400 is the half
//     1024 + n exactly [volta-kernel-bakeoff, "What's in the race", the
//     fused_q4_v2 bit trick]; a high nibble left in place gives 1024 + 16 n.
//     One v_and_or_b32 makes two such halves and one v_pk_add_f16 removes the
//     bias from both, exactly: n - 8 and 16 (n - 8).  Q8_0: (q + 128) | 0x6400
//     = q + 1152, placed with one v_perm_b32 per pair, minus 1152 gives q.
//     Products with the activations go through v_dot2_f32_f16 (two exact fp16
//     products summed into fp32) in two chains per block, low + high / 16 =
//     sum (q - 8) x; the block scale multiplies the block sum once.  (Leaving
//     the bias in and starting the chains from -1032 * sum x saves the
//     subtraction, but the chains then run at 1032 |x|: one activation near
//     the binary16 limit against a zero weight rounds them by more than the
//     1e-3 sum |w x| accuracy of the result.)
//   * Reduction over a row's G lanes: DPP within 16-lane rows, then
//     v_permlane16_swap / v_permlane32_swap across them; waves of a team
//     (ksplit > 1) combine through LDS.  No atomics: results are reproducible.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "qgemv_internal.h"

namespace qg {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ h2_t as_h2(uint32_t u) { return __builtin_bit_cast(h2_t, u); }

__device__ __forceinline__ float dot2(h2_t a, h2_t b, float c)
{
    return __builtin_amdgcn_fdot2(a, b, c, false);
}

// The first product of a chain: the three-operand encoding with an inline
// zero writes a fresh register, where the compiler zeroes one with a move and
// then accumulates into it.
__device__ __forceinline__ float dot2_first(h2_t a, h2_t b)
{
    float d;
    asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(d) : "v"(a), "v"(b));
    return d;
}

// ---------------------------------------------------------------- unpacking
//
// Both formats unpack a block into 16 half pairs whose activation partners
// are the pairs X[0..15] built by load_x_block<FMT>.

// The magic constant is pinned in a vector register (once per kernel): with the
// mask in a scalar register, (w & mask) | magic is then a single v_and_or_b32.
__device__ __forceinline__ uint32_t magic_reg()
{
    uint32_t m;
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(m));
    return m;
}

// Q4_0: word t holds bytes 4t..4t+3 = elements 4t..4t+3 (low nibbles) and
// 16+4t..19+4t (high nibbles); with q' = q - 8:
//   lo[2t]   = (q'[4t],    q'[4t+2])          partner X[4t+0]
//   lo[2t+1] = (q'[4t+1],  q'[4t+3])          partner X[4t+2]
//   hi[2t]   = 16 (q'[16+4t], q'[18+4t])      partner X[4t+1]
//   hi[2t+1] = 16 (q'[17+4t], q'[19+4t])      partner X[4t+3]
__device__ __forceinline__ void unpack_q4(const uint4 c, uint32_t kMagic, h2_t (&lo)[8], h2_t (&hi)[8])
{
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    const h2_t kLo = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const h2_t kHi = {(_Float16)-1152.0f, (_Float16)-1152.0f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint32_t a = w[t];
        const uint32_t b = w[t] >> 8;
        lo[2 * t + 0] = as_h2((a & 0x000F000Fu) | kMagic) + kLo;
        hi[2 * t + 0] = as_h2((a & 0x00F000F0u) | kMagic) + kHi;
        lo[2 * t + 1] = as_h2((b & 0x000F000Fu) | kMagic) + kLo;
        hi[2 * t + 1] = as_h2((b & 0x00F000F0u) | kMagic) + kHi;
    }
}

// Q8_0: word t holds int8 elements 4t..4t+3.  Flipping the sign bits gives
// u = q + 128 in 0..255; with 0x64 as the high byte, u is the half 1024 + u =
// q + 1152 exactly.  v_perm_b32 takes bytes 0 and 2 (1 and 3) of u and the
// 0x64 bytes of the magic word in one instruction.
// Subtracting 1152 leaves the codes:
//   v[2t] = (q[4t], q[4t+2])   v[2t+1] = (q[4t+1], q[4t+3])
__device__ __forceinline__ void unpack_q8(const uint4 c0, const uint4 c1, uint32_t kMagic, h2_t (&v)[16])
{
    const uint32_t w[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    const h2_t kBias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const uint32_t u = w[t] ^ 0x80808080u;
        // selector bytes: 0-3 pick bytes of u, 4-7 bytes of the magic word
        v[2 * t + 0] = as_h2(__builtin_amdgcn_perm(kMagic, u, 0x07020500u)) + kBias;
        v[2 * t + 1] = as_h2(__builtin_amdgcn_perm(kMagic, u, 0x07030501u)) + kBias;
    }
}

// q2w: word h (bytes 4h..4h+3) holds in bit pair r of byte 4h+i element
// 4h + i + 8r, stored as u = c + 2.  With a = word, b = word >> 8, the mask
// 0x00030003 << 2r picks bytes 0 and 2 (or 1 and 3) at bit pair r; OR-ed into
// 0x6400 that is 1024 + 4^r u exactly, and one v_pk_fma_f16 (x / 4^r - 1024 /
// 4^r - 2, every step exact) leaves c in -2..1:
//   v[2r]   = (c[4h + 8r],     c[4h + 8r + 2])   partner X[8h + 2r]
//   v[2r+1] = (c[4h + 8r + 1], c[4h + 8r + 3])   partner X[8h + 2r + 1]
// for word 0 into v0 and word 1 into v1.
__device__ __forceinline__ void unpack_q2_word(uint32_t w, uint32_t kMagic, h2_t (&v)[8])
{
    const uint32_t a = w;
    const uint32_t b = w >> 8;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t mask = 0x00030003u << (2 * r);
        const _Float16 sc = (_Float16)(1.0f / (float)(1 << (2 * r)));
        const _Float16 off = (_Float16)(-(1024.0f / (float)(1 << (2 * r))) - 2.0f);
        const h2_t ksc = {sc, sc};
        const h2_t koff = {off, off};
        v[2 * r + 0] = as_h2((a & mask) | kMagic) * ksc + koff;
        v[2 * r + 1] = as_h2((b & mask) | kMagic) * ksc + koff;
    }
}

__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) { return (a & 0xFFFFu) | (b << 16); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }

// The 32 fp16 activations of one block (64 bytes, raw words r) as the 16
// pairs that match unpack_q4 / unpack_q8.
template <int FMT>
__device__ __forceinline__ void pair_x_block(const uint4 (&r)[4], uint32_t (&X)[16])
{
    const uint32_t d[16] = {r[0].x, r[0].y, r[0].z, r[0].w, r[1].x, r[1].y, r[1].z, r[1].w,
                            r[2].x, r[2].y, r[2].z, r[2].w, r[3].x, r[3].y, r[3].z, r[3].w};
    // d[i] = (x[2i], x[2i+1])
    if constexpr (FMT == kQ2W) {
        // X[8h + 2r + s]: elements (4h + 8r + s, 4h + 8r + s + 2)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                X[8 * h + 2 * r + 0] = pair_lo(d[2 * h + 4 * r], d[2 * h + 4 * r + 1]);
                X[8 * h + 2 * r + 1] = pair_hi(d[2 * h + 4 * r], d[2 * h + 4 * r + 1]);
            }
    } else if constexpr (FMT == kQ4_0) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            X[4 * t + 0] = pair_lo(d[2 * t], d[2 * t + 1]);
            X[4 * t + 2] = pair_hi(d[2 * t], d[2 * t + 1]);
            X[4 * t + 1] = pair_lo(d[8 + 2 * t], d[9 + 2 * t]);
            X[4 * t + 3] = pair_hi(d[8 + 2 * t], d[9 + 2 * t]);
        }
    } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            X[2 * t + 0] = pair_lo(d[2 * t], d[2 * t + 1]);
            X[2 * t + 1] = pair_hi(d[2 * t], d[2 * t + 1]);
        }
    }
}

__device__ __forceinline__ void load_x_raw(const uint16_t *p, uint4 (&r)[4])
{
    const uint4 *q = reinterpret_cast<const uint4 *>(p);
#pragma unroll
    for (int u = 0; u < 4; ++u)
        r[u] = q[u];
}

// 32 fp32 activations rounded to binary16 (nearest, ties to even, the
// conversion's default mode; beyond binary16's range: infinity), in the same
// natural-order words load_x_raw returns [volta-kernel-bakeoff, "Results":
// fp32 activations in, the conversion inside the kernel].
__device__ __forceinline__ uint32_t pack_half2(float a, float b)
{
    const uint32_t lo = __builtin_bit_cast(uint16_t, (_Float16)a);
    const uint32_t hi = __builtin_bit_cast(uint16_t, (_Float16)b);
    return lo | (hi << 16);
}

__device__ __forceinline__ void load_x_raw_f32(const float *p, uint4 (&r)[4])
{
    const float4 *q = reinterpret_cast<const float4 *>(p);
    float4 f[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
        f[u] = q[u];
#pragma unroll
    for (int u = 0; u < 4; ++u)
        r[u] = make_uint4(pack_half2(f[2 * u].x, f[2 * u].y), pack_half2(f[2 * u].z, f[2 * u].w),
                          pack_half2(f[2 * u + 1].x, f[2 * u + 1].y), pack_half2(f[2 * u + 1].z, f[2 * u + 1].w));
}

template <int FMT>
__device__ __forceinline__ void load_x_block(const uint16_t *p, uint32_t (&X)[16])
{
    uint4 r[4];
    load_x_raw(p, r);
    pair_x_block<FMT>(r, X);
}

// ---------------------------------------------------------------- reduction

template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over each G-lane segment of the wave; every lane of a segment receives
// its sum.  With 16-lane rows r0..r3: v_permlane16_swap(A, B) gives
// A = [A.r0, B.r0, A.r2, B.r2], B = [A.r1, B.r1, A.r3, B.r3] and
// v_permlane32_swap(A, B) gives A = [A.r0, A.r1, B.r0, B.r1],
// B = [A.r2, A.r3, B.r2, B.r3].
template <int G>
__device__ __forceinline__ float seg_sum(float v)
{
    v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);   // row_half_mirror
    v += dpp<0x140>(v);   // row_mirror: every lane holds its 16-lane row's sum
    if constexpr (G >= 32) {
        const uint32_t u = __builtin_bit_cast(uint32_t, v);
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        v = __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
    }
    if constexpr (G == 64) {
        const uint32_t u = __builtin_bit_cast(uint32_t, v);
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        v = __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
    }
    return v;
}

// ---------------------------------------------------------------- the kernel

template <int FMT>
struct Codes;
template <>
struct Codes<kQ4_0> {
    uint4 c;
};
template <>
struct Codes<kQ8_0> {
    uint4 c0, c1;
};
template <>
struct Codes<kQ2W> {
    uint2 c;
};

template <int FMT, int J, int R>
struct Group {
    Codes<FMT> code[R][J];
    uint16_t scale[R][J];
};

// Issue the loads of one group (R row sets from row rs0).  Each row set's
// first row is wave-uniform and clamped to rmax = N - P, so every lane's row
// rbase + l / G stays inside the matrix; lanes add a 32-bit offset (coff,
// soff: row within the set and block).  Padding lanes of a short K chunk read
// their chunk's last block (their block index is clamped) and have zero
// activations, so they add nothing.
template <int FMT, int G, int J, int R, bool GLU>
__device__ __forceinline__ void load_group(Group<FMT, J, R> &g, const uint8_t *__restrict__ W,
                                           const uint8_t *__restrict__ S, int64_t rs0, int64_t rmax, int KB,
                                           int64_t nblocks, const uint32_t (&coff)[J], const uint32_t (&soff)[J],
                                           int64_t N)
{
    constexpr int P = 64 / G;
    constexpr int CB = code_bytes_per_block(FMT);
#pragma unroll
    for (int i = 0; i < R; ++i) {
        // GLU: row set 0 holds gate rows, row set 1 the up rows N further
        const int64_t rbase = GLU ? min(rs0, rmax) + i * N : min(rs0 + i * P, rmax);
        const int64_t base = rbase * KB;   // first block of the row set
        const auto rc = make_rsrc(W + base * CB, (nblocks - base) * CB);
        const auto rs = make_rsrc(S + base * 2, (nblocks - base) * 2);
#pragma unroll
        for (int j = 0; j < J; ++j) {
            if constexpr (FMT == kQ4_0) {
                g.code[i][j].c = stream_load16(rc, coff[j]);
            } else if constexpr (FMT == kQ2W) {
                g.code[i][j].c = stream_load8(rc, coff[j]);
            } else {
                g.code[i][j].c0 = stream_load16(rc, coff[j]);
                g.code[i][j].c1 = stream_load16(rc, coff[j] + 16u);
            }
            g.scale[i][j] = stream_load2(rs, soff[j]);
        }
    }
}

// One block's unpacked pairs (chain 0 and chain 1, see unpack_q4 / unpack_q8).
template <int FMT>
__device__ __forceinline__ void unpack_block(const Codes<FMT> &c, uint32_t magic, h2_t (&v0)[8], h2_t (&v1)[8])
{
    if constexpr (FMT == kQ4_0) {
        unpack_q4(c.c, magic, v0, v1);
    } else if constexpr (FMT == kQ2W) {
        unpack_q2_word(c.c.x, magic, v0);
        unpack_q2_word(c.c.y, magic, v1);
    } else {
        h2_t v[16];
        unpack_q8(c.c0, c.c1, magic, v);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            v0[t] = v[t];
            v1[t] = v[8 + t];
        }
    }
}

// sum (q - 8) x (Q4_0), sum q x (Q8_0) or sum c x (q2w) of one block against
// one token's 16 activation pairs (q2w and Q8_0 share the pair order: chain 0
// takes pairs 0..7, chain 1 pairs 8..15).
template <int FMT>
__device__ __forceinline__ float block_dot(const h2_t (&v0)[8], const h2_t (&v1)[8], const uint32_t (&xw)[16])
{
    if constexpr (FMT == kQ4_0) {
        float c0 = dot2_first(v0[0], as_h2(xw[0]));
        float c1 = dot2_first(v1[0], as_h2(xw[1]));
        c0 = dot2(v0[1], as_h2(xw[2]), c0);
        c1 = dot2(v1[1], as_h2(xw[3]), c1);
#pragma unroll
        for (int t = 1; t < 4; ++t) {
            c0 = dot2(v0[2 * t], as_h2(xw[4 * t + 0]), c0);
            c1 = dot2(v1[2 * t], as_h2(xw[4 * t + 1]), c1);
            c0 = dot2(v0[2 * t + 1], as_h2(xw[4 * t + 2]), c0);
            c1 = dot2(v1[2 * t + 1], as_h2(xw[4 * t + 3]), c1);
        }
        return __builtin_fmaf(c1, 0.0625f, c0);
    } else {
        float c0 = dot2_first(v0[0], as_h2(xw[0]));
        float c1 = dot2_first(v1[0], as_h2(xw[8]));
#pragma unroll
        for (int t = 1; t < 8; ++t) {
            c0 = dot2(v0[t], as_h2(xw[t]), c0);
            c1 = dot2(v1[t], as_h2(xw[8 + t]), c1);
        }
        return c0 + c1;
    }
}

// Activations come either from registers (X, loaded once per team) or, with
// XL, from the workgroup's LDS copy (xs holds, token after token, every block
// of x in pair order plus one zero block that padding lanes read; xstride =
// one token's share in uint4).  With XL a block's activations are read once
// per group and used by every row set before the next block's are read (read
// per row set, the compiler keeps them all live across row sets instead).
template <int FMT, int M, int J, int R, bool XL, int MODE>
__device__ __forceinline__ void compute_group(const Group<FMT, J, R> &g,
                                              const uint32_t (&X)[XL ? 1 : M][XL ? 1 : J][16],
                                              const uint4 *xs, uint32_t xstride, const uint32_t (&xoff)[J],
                                              uint32_t magic, float (&acc)[R][M])
{
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int m = 0; m < M; ++m)
            acc[i][m] = 0.0f;
    if constexpr (MODE == kModeQ8Act) {
        // 8-bit activations: per block and token 32 int8 codes (natural
        // order) and the binary32 scale and the integer -8 * sum(codes).  The
        // nibbles themselves are the int8 operands (0..15): the block sum
        // starts from the offset term, so it ends at sum (q - 8) qx, exact.
#pragma unroll
        for (int j = 0; j < J; ++j) {
            uint32_t qw[M][8];
            float dxm[M];
            int bias[M];
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const uint4 *q = xs + m * xstride + xoff[j] * 3;
                const uint4 a = q[0], b = q[1], c = q[2];
                qw[m][0] = a.x;
                qw[m][1] = a.y;
                qw[m][2] = a.z;
                qw[m][3] = a.w;
                qw[m][4] = b.x;
                qw[m][5] = b.y;
                qw[m][6] = b.z;
                qw[m][7] = b.w;
                dxm[m] = __builtin_bit_cast(float, c.x);
                bias[m] = (int)c.y;
            }
#pragma unroll
            for (int i = 0; i < R; ++i) {
                const float d = (float)__builtin_bit_cast(_Float16, g.scale[i][j]);
                // the unsigned codes as int8 operands, each word paired with
                // the activation word of the same four elements
                uint32_t ops[8];
                int qi[8];
                if constexpr (FMT == kQ2W) {
                    // word h, bit pair r: elements 4h + 8r .. 4h + 8r + 3
                    const uint32_t w[2] = {g.code[i][j].c.x, g.code[i][j].c.y};
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            ops[4 * h + r] = (w[h] >> (2 * r)) & 0x03030303u;
                            qi[4 * h + r] = 2 * r + h;
                        }
                } else {
                    // word t: elements 4t..4t+3 (low nibbles), 16+4t..19+4t (high)
                    const uint32_t w[4] = {g.code[i][j].c.x, g.code[i][j].c.y, g.code[i][j].c.z,
                                           g.code[i][j].c.w};
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        ops[2 * t] = w[t] & 0x0F0F0F0Fu;
                        qi[2 * t] = t;
                        ops[2 * t + 1] = (w[t] >> 4) & 0x0F0F0F0Fu;
                        qi[2 * t + 1] = 4 + t;
                    }
                }
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    int sum = bias[m];
#pragma unroll
                    for (int t = 0; t < 8; ++t)
                        sum = __builtin_amdgcn_sdot4((int)ops[t], (int)qw[m][qi[t]], sum, false);
                    acc[i][m] = __builtin_fmaf(d, dxm[m] * (float)sum, acc[i][m]);
                }
            }
        }
    } else if constexpr (XL) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            uint32_t xw[M][16];
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const uint4 *q = xs + m * xstride + xoff[j] * 4;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint4 t = q[u];
                    xw[m][4 * u + 0] = t.x;
                    xw[m][4 * u + 1] = t.y;
                    xw[m][4 * u + 2] = t.z;
                    xw[m][4 * u + 3] = t.w;
                }
            }
#pragma unroll
            for (int i = 0; i < R; ++i) {
                const float d = (float)__builtin_bit_cast(_Float16, g.scale[i][j]);
                h2_t v0[8], v1[8];
                unpack_block<FMT>(g.code[i][j], magic, v0, v1);
#pragma unroll
                for (int m = 0; m < M; ++m)
                    acc[i][m] = __builtin_fmaf(d, block_dot<FMT>(v0, v1, xw[m]), acc[i][m]);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < R; ++i) {
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const float d = (float)__builtin_bit_cast(_Float16, g.scale[i][j]);
                h2_t v0[8], v1[8];
                unpack_block<FMT>(g.code[i][j], magic, v0, v1);
#pragma unroll
                for (int m = 0; m < M; ++m)
                    acc[i][m] = __builtin_fmaf(d, block_dot<FMT>(v0, v1, X[m][j]), acc[i][m]);
            }
        }
    }
}

// Reduce one group's partials and store y (ksplit == 1), or combine the
// team's waves through LDS first (ksplit > 1).  A row set whose first row
// was clamped (at the matrix's tail) also holds rows below rs0 + i P that an
// earlier row set stores: only rows in [rs0 + i P, N) are written.
template <int G, int M, int R>
__device__ __forceinline__ void finish_group(const float (&acc)[R][M], float *__restrict__ y, int64_t rs0,
                                             int64_t rmax, int N, int lane, int wave, int team, int kw, int ksplit,
                                             float (&red)[2][kMaxWavesPerWg][kMaxRM], int &buf)
{
    constexpr int P = 64 / G;
    float tot[R][M];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int m = 0; m < M; ++m)
            tot[i][m] = seg_sum<G>(acc[i][m]);

    // rows of row set i: first = min(want, rmax) + lr; stored if first + lr
    // lies in [want, N), i.e. lo <= lr < hi with small uniform bounds
    const int lr = lane / G;
    int lo[R], hi[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int64_t want = rs0 + i * P;
        const int64_t first = min(want, rmax);
        lo[i] = (int)(want - first);
        hi[i] = (int)min((int64_t)N - first, (int64_t)P);
    }
    if (ksplit == 1) {
        if (lane % G == 0) {
#pragma unroll
            for (int i = 0; i < R; ++i) {
                if (lr >= lo[i] && lr < hi[i]) {
                    const int64_t row = min(rs0 + i * P, rmax) + lr;
#pragma unroll
                    for (int m = 0; m < M; ++m)
                        y[(int64_t)m * N + row] = tot[i][m];
                }
            }
        }
    } else {
        if (lane % G == 0) {
#pragma unroll
            for (int i = 0; i < R; ++i)
#pragma unroll
                for (int m = 0; m < M; ++m)
                    red[buf][wave][(i * M + m) * P + lr] = tot[i][m];
        }
        __syncthreads();
        if (kw == 0 && lane < R * M * P) {
            float s = 0.0f;
            for (int w = 0; w < ksplit; ++w)
                s += red[buf][team * ksplit + w][lane];
            const int i = lane / (M * P), m = (lane / P) % M, r = lane % P;
            int loi = 0, hii = 0;
#pragma unroll
            for (int t = 0; t < R; ++t) {
                loi = (i == t) ? lo[t] : loi;
                hii = (i == t) ? hi[t] : hii;
            }
            if (r >= loi && r < hii)
                y[(int64_t)m * N + min(rs0 + i * P, rmax) + r] = s;
        }
        buf ^= 1;
    }
}

// SwiGLU epilogue: silu(gate) * up, evaluated in fp32 on the two row sets'
// reduced sums (gate rows of the group, and the up rows N further)
// [the CUDA-kernel diary's FFN fusion step: gate, up and SwiGLU in one kernel,
// only the final product written].
__device__ __forceinline__ float swiglu(float g, float u) { return g / (1.0f + expf(-g)) * u; }

template <int G, int M>
__device__ __forceinline__ void finish_group_glu(const float (&acc)[2][M], float *__restrict__ y, int64_t rs0,
                                                 int64_t rmax, int N, int lane, int wave, int team, int kw,
                                                 int ksplit, float (&red)[2][kMaxWavesPerWg][kMaxRM], int &buf)
{
    constexpr int P = 64 / G;
    float tot[2][M];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int m = 0; m < M; ++m)
            tot[i][m] = seg_sum<G>(acc[i][m]);
    const int lr = lane / G;
    const int64_t first = min(rs0, rmax);
    const int lo = (int)(rs0 - first);
    const int hi = (int)min((int64_t)N - first, (int64_t)P);
    if (ksplit == 1) {
        if (lane % G == 0 && lr >= lo && lr < hi) {
#pragma unroll
            for (int m = 0; m < M; ++m)
                y[(int64_t)m * N + first + lr] = swiglu(tot[0][m], tot[1][m]);
        }
    } else {
        if (lane % G == 0) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int m = 0; m < M; ++m)
                    red[buf][wave][(i * M + m) * P + lr] = tot[i][m];
        }
        __syncthreads();
        if (kw == 0 && lane < M * P) {
            const int m = lane / P, r = lane % P;
            float gs = 0.0f, us = 0.0f;
            for (int w = 0; w < ksplit; ++w) {
                gs += red[buf][team * ksplit + w][m * P + r];
                us += red[buf][team * ksplit + w][(M + m) * P + r];
            }
            if (r >= lo && r < hi)
                y[(int64_t)m * N + first + r] = swiglu(gs, us);
        }
        buf ^= 1;
    }
}

template <int G, int M, int R, bool GLU>
__device__ __forceinline__ void finish(const float (&acc)[R][M], float *__restrict__ y, int64_t rs0, int64_t rmax,
                                       int N, int lane, int wave, int team, int kw, int ksplit,
                                       float (&red)[2][kMaxWavesPerWg][kMaxRM], int &buf)
{
    if constexpr (GLU)
        finish_group_glu<G, M>(acc, y, rs0, rmax, N, lane, wave, team, kw, ksplit, red, buf);
    else
        finish_group<G, M, R>(acc, y, rs0, rmax, N, lane, wave, team, kw, ksplit, red, buf);
}

template <int FMT, int M, int G, int J, int R, bool XL, int MODE>
__global__ __launch_bounds__(512) void gemv_kernel(GemvParams p)
{
    static_assert(!XL || M <= 4, "LDS-staged activations: up to 4 tokens");
    static_assert(MODE == kModeF16 || FMT == kQ4_0 || (MODE == kModeQ8Act && FMT == kQ2W),
                  "fp32 activations: Q4_0; 8-bit activations: Q4_0 or q2w");
    static_assert(MODE != kModeQ8Act || XL, "8-bit activations are quantized into LDS");
    constexpr bool GLU = MODE == kModeGlu;
    static_assert(!GLU || R == 2, "SwiGLU: one gate and one up row set per group");
    constexpr int P = 64 / G;
    const int lane = threadIdx.x & 63;
    // wave-uniform: everything derived from it (rows, addresses) stays scalar
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kw = wave % p.ksplit;       // this wave's K chunk
    const int team = wave / p.ksplit;     // team within the workgroup
    const int64_t teams_total = (int64_t)gridDim.x * p.teams_per_wg;
    const int64_t team_id = (int64_t)blockIdx.x * p.teams_per_wg + team;
    const int item = blockIdx.y;          // batch item: MoE expert slot

    const uint16_t *__restrict__ x = p.x + (int64_t)item * M * p.K;
    const float *__restrict__ xf = p.xf + (int64_t)item * M * p.K;
    float *__restrict__ y = p.y + (int64_t)item * M * p.N;
    const uint8_t *__restrict__ W = p.W;
    if (p.idx) {
        // MoE: an expert index outside the pool is never followed; the
        // slot's outputs become NaN (written by its first workgroup) and no
        // weight is read.  The condition is uniform over the workgroup.
        const int64_t e = p.idx[item];
        if (e < 0 || e >= p.pool) {
            if (blockIdx.x == 0)
                for (int64_t i = threadIdx.x; i < (int64_t)M * p.N; i += blockDim.x)
                    y[i] = __builtin_nanf("");
            return;
        }
        W += e * p.matrix_stride;
    }
    const uint8_t *__restrict__ S = W + p.scale_offset;

    const int KB = p.K >> 5;
    const int lr = lane / G;
    const int bbeg = kw * G * J;
    const int bend = min(KB, bbeg + G * J);
    uint32_t blk[J], xoff[J], coff[J], soff[J];
    bool ok[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int b = bbeg + lane % G + G * j;
        ok[j] = b < bend;
        blk[j] = (uint32_t)(ok[j] ? b : bend - 1);
        xoff[j] = (uint32_t)(ok[j] ? b : KB);   // LDS block KB is all zeros
        const uint32_t e = (uint32_t)lr * (uint32_t)KB + blk[j];   // block offset from the row set
        coff[j] = e * (uint32_t)code_bytes_per_block(FMT);
        soff[j] = e * 2u;
    }

    // groups of R row sets; a row set's first row is clamped to rmax = N - P
    // (the launcher ensures N >= P)
    // (GLU: a group is P output rows, read as P gate rows and P up rows of
    // the 2N-row table)
    const int64_t rows_per_group = GLU ? P : (int64_t)R * P;
    const int64_t ngroups = ((int64_t)p.N + rows_per_group - 1) / rows_per_group;
    const int64_t rmax = (int64_t)p.N - P;
    const int64_t nblocks = (int64_t)p.N * KB * (GLU ? 2 : 1);
    int64_t g = team_id;

    Group<FMT, J, R> ga, gb;

    // Activations of this lane's blocks, all M tokens, kept for every row.
    // Their loads are issued before the first weight loads: they hit in the
    // cache after the first waves, and queued behind a full round of weight
    // requests they would hold up every wave's first compute.
    uint32_t X[XL ? 1 : M][XL ? 1 : J][16];
    extern __shared__ uint4 xs_dyn[];
    uint4 XR[XL ? 1 : M][XL ? 1 : J][4];   // raw activation words, paired below
    if constexpr (!XL) {
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int j = 0; j < J; ++j)
                if constexpr (MODE == kModeF16)
                    load_x_raw(x + (int64_t)m * p.K + (int64_t)blk[j] * 32, XR[m][j]);
                else
                    load_x_raw_f32(xf + (int64_t)m * p.K + (int64_t)blk[j] * 32, XR[m][j]);
    }
    __builtin_amdgcn_sched_barrier(0);
    // unconditional (a team without groups re-reads a clamped, in-bounds row
    // set): with a conditional load the wait for the activations below would
    // also cover these weights
    load_group<FMT, G, J, R, GLU>(ga, W, S, g * rows_per_group, rmax, KB, nblocks, coff, soff, p.N);
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t xstride = (uint32_t)(KB + 1) * (MODE == kModeQ8Act ? 3u : 4u);
    if constexpr (XL && MODE == kModeQ8Act) {
        // the workgroup quantizes x once, token after token, to 8-bit blocks
        // (each token followed by a zero block): amax = the block's largest
        // |x|, dx = amax / 127 and inv = 127 / amax (binary32 divisions,
        // correctly rounded), codes rint(x * inv) with ties to even; stored
        // as 32 int8 codes, dx and -8 * sum(codes) [sm8x-bench, "our kernel":
        // the activations quantized to 8-bit blocks once]
        for (int i = threadIdx.x; i < M * (KB + 1); i += blockDim.x) {
            const int m = i / (KB + 1);
            const int b = i - m * (KB + 1);
            uint32_t cw[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
            float dq = 0.0f;
            int qsum = 0;
            if (b < KB) {
                uint4 r[4];
                load_x_raw(x + (int64_t)m * p.K + (int64_t)b * 32, r);
                const uint32_t hw[16] = {r[0].x, r[0].y, r[0].z, r[0].w, r[1].x, r[1].y, r[1].z, r[1].w,
                                         r[2].x, r[2].y, r[2].z, r[2].w, r[3].x, r[3].y, r[3].z, r[3].w};
                float v[32];
                float amax = 0.0f;
#pragma unroll
                for (int k = 0; k < 32; ++k) {
                    const uint16_t h = (uint16_t)(hw[k >> 1] >> (16 * (k & 1)));
                    v[k] = (float)__builtin_bit_cast(_Float16, h);
                    amax = fmaxf(amax, fabsf(v[k]));
                }
                float inv = 0.0f;
                if (amax > 0.0f) {
                    dq = amax / 127.0f;
                    inv = 127.0f / amax;
                }
#pragma unroll
                for (int k = 0; k < 32; ++k) {
                    const int q = (int)__builtin_rintf(v[k] * inv);
                    qsum += q;
                    cw[k >> 2] |= ((uint32_t)q & 0xFFu) << (8 * (k & 3));
                }
            }
            xs_dyn[i * 3 + 0] = make_uint4(cw[0], cw[1], cw[2], cw[3]);
            xs_dyn[i * 3 + 1] = make_uint4(cw[4], cw[5], cw[6], cw[7]);
            // the codes' offset times the activation sum: 8 (Q4_0) or 2 (q2w)
            xs_dyn[i * 3 + 2] = make_uint4(__builtin_bit_cast(uint32_t, dq),
                                           (uint32_t)(-(FMT == kQ2W ? 2 : 8) * qsum), 0u, 0u);
        }
        __syncthreads();
    } else if constexpr (XL) {
        // the workgroup stages x once, token after token, in pair order, each
        // token followed by a zero block (fp32 input: rounded here)
        for (int i = threadIdx.x; i < M * (KB + 1); i += blockDim.x) {
            const int m = i / (KB + 1);
            const int b = i - m * (KB + 1);
            uint32_t w16[16];
            if (b < KB) {
                uint4 r[4];
                if constexpr (MODE == kModeF16)
                    load_x_raw(x + (int64_t)m * p.K + (int64_t)b * 32, r);
                else
                    load_x_raw_f32(xf + (int64_t)m * p.K + (int64_t)b * 32, r);
                pair_x_block<FMT>(r, w16);
            } else {
#pragma unroll
                for (int t = 0; t < 16; ++t)
                    w16[t] = 0u;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                xs_dyn[i * 4 + u] = make_uint4(w16[4 * u], w16[4 * u + 1], w16[4 * u + 2], w16[4 * u + 3]);
        }
        __syncthreads();
    } else {
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int j = 0; j < J; ++j) {
                pair_x_block<FMT>(XR[m][j], X[m][j]);
                if (!ok[j]) {
#pragma unroll
                    for (int t = 0; t < 16; ++t)
                        X[m][j][t] = 0u;
                }
            }
    }

    __shared__ float red[2][kMaxWavesPerWg][kMaxRM];
    int buf = 0;
    const uint32_t magic = magic_reg();

    // Groups g, g + T, g + 2T, ... (T = teams_total), n of them.  The loop
    // body computes two groups and prefetches the next two; the last one or
    // two groups are peeled off after it, so no load is ever conditional: on
    // every path the compiler's wait before a compute then covers exactly
    // that group's loads (with a conditional prefetch it also waits for the
    // prefetch, which serializes the two).
    const int64_t n = (g < ngroups) ? (ngroups - g + teams_total - 1) / teams_total : 0;
    int64_t k = 0;
    for (; k + 2 < n; k += 2) {
        float acc[R][M];
        load_group<FMT, G, J, R, GLU>(gb, W, S, (g + teams_total) * rows_per_group, rmax, KB, nblocks, coff, soff, p.N);
        __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of the compute
        compute_group<FMT, M, J, R, XL, MODE>(ga, X, xs_dyn, xstride, xoff, magic, acc);
        finish<G, M, R, GLU>(acc, y, g * rows_per_group, rmax, p.N, lane, wave, team, kw, p.ksplit, red, buf);
        g += teams_total;
        load_group<FMT, G, J, R, GLU>(ga, W, S, (g + teams_total) * rows_per_group, rmax, KB, nblocks, coff, soff, p.N);
        __builtin_amdgcn_sched_barrier(0);
        compute_group<FMT, M, J, R, XL, MODE>(gb, X, xs_dyn, xstride, xoff, magic, acc);
        finish<G, M, R, GLU>(acc, y, g * rows_per_group, rmax, p.N, lane, wave, team, kw, p.ksplit, red, buf);
        g += teams_total;
    }
    if (n - k == 2) {
        float acc[R][M];
        load_group<FMT, G, J, R, GLU>(gb, W, S, (g + teams_total) * rows_per_group, rmax, KB, nblocks, coff, soff, p.N);
        __builtin_amdgcn_sched_barrier(0);
        compute_group<FMT, M, J, R, XL, MODE>(ga, X, xs_dyn, xstride, xoff, magic, acc);
        finish<G, M, R, GLU>(acc, y, g * rows_per_group, rmax, p.N, lane, wave, team, kw, p.ksplit, red, buf);
        g += teams_total;
        compute_group<FMT, M, J, R, XL, MODE>(gb, X, xs_dyn, xstride, xoff, magic, acc);
        finish<G, M, R, GLU>(acc, y, g * rows_per_group, rmax, p.N, lane, wave, team, kw, p.ksplit, red, buf);
    } else if (n - k == 1) {
        float acc[R][M];
        compute_group<FMT, M, J, R, XL, MODE>(ga, X, xs_dyn, xstride, xoff, magic, acc);
        finish<G, M, R, GLU>(acc, y, g * rows_per_group, rmax, p.N, lane, wave, team, kw, p.ksplit, red, buf);
    }
}

// ---------------------------------------------------------------- dispatch

template <int FMT, int M, int G, int J, int R, bool XL, int MODE>
static hipError_t launch_one(const GemvParams &p, dim3 grid, dim3 block, size_t shmem, hipStream_t stream)
{
    return launch_kernel(reinterpret_cast<const void *>(&gemv_kernel<FMT, M, G, J, R, XL, MODE>), grid, block,
                         shmem, stream, p);
}

template <int FMT, int M, int G, int J, bool XL, int MODE>
static hipError_t launch_r(int R, const GemvParams &p, dim3 grid, dim3 block, size_t shmem, hipStream_t stream)
{
    if constexpr (MODE == kModeGlu) {
        if constexpr (gemv_fits(FMT, M, G, J, 2, XL, MODE))
            if (R == 2) return launch_one<FMT, M, G, J, 2, XL, MODE>(p, grid, block, shmem, stream);
        return hipErrorInvalidValue;
    } else {
        if constexpr (gemv_fits(FMT, M, G, J, 1, XL, MODE))
            if (R == 1) return launch_one<FMT, M, G, J, 1, XL, MODE>(p, grid, block, shmem, stream);
        if constexpr (gemv_fits(FMT, M, G, J, 2, XL, MODE))
            if (R == 2) return launch_one<FMT, M, G, J, 2, XL, MODE>(p, grid, block, shmem, stream);
        if constexpr (gemv_fits(FMT, M, G, J, 4, XL, MODE))
            if (R == 4) return launch_one<FMT, M, G, J, 4, XL, MODE>(p, grid, block, shmem, stream);
        return hipErrorInvalidValue;
    }
}

template <int FMT, int M, int G, bool XL, int MODE>
static hipError_t launch_j(int J, int R, const GemvParams &p, dim3 grid, dim3 block, size_t shmem,
                           hipStream_t stream)
{
    switch (J) {
    case 1: return launch_r<FMT, M, G, 1, XL, MODE>(R, p, grid, block, shmem, stream);
    case 2: return launch_r<FMT, M, G, 2, XL, MODE>(R, p, grid, block, shmem, stream);
    case 3: return launch_r<FMT, M, G, 3, XL, MODE>(R, p, grid, block, shmem, stream);
    case 4: return launch_r<FMT, M, G, 4, XL, MODE>(R, p, grid, block, shmem, stream);
    case 5: return launch_r<FMT, M, G, 5, XL, MODE>(R, p, grid, block, shmem, stream);
    case 6: return launch_r<FMT, M, G, 6, XL, MODE>(R, p, grid, block, shmem, stream);
    case 7: return launch_r<FMT, M, G, 7, XL, MODE>(R, p, grid, block, shmem, stream);
    case 8: return launch_r<FMT, M, G, 8, XL, MODE>(R, p, grid, block, shmem, stream);
    }
    return hipErrorInvalidValue;
}

template <int FMT, int M, bool XL, int MODE = kModeF16>
static hipError_t launch_g(int G, int J, int R, const GemvParams &p, dim3 grid, dim3 block, size_t shmem,
                           hipStream_t stream)
{
    // narrow row segments only for one token (the register cost of resident
    // activations grows with M)
    if constexpr (M == 1) {
        if (G == 16) return launch_j<FMT, M, 16, XL, MODE>(J, R, p, grid, block, shmem, stream);
        if (G == 32) return launch_j<FMT, M, 32, XL, MODE>(J, R, p, grid, block, shmem, stream);
    }
    if (G == 64) return launch_j<FMT, M, 64, XL, MODE>(J, R, p, grid, block, shmem, stream);
    return hipErrorInvalidValue;
}

// Every launch shape of one (format, activation mode, staging) variant; each
// variant is instantiated in a translation unit of its own (the builds run
// in parallel).
template <int FMT, int MODE, bool XL>
hipError_t launch_variant(int M, int G, int J, int R, const GemvParams &p, dim3 grid, dim3 block, size_t shmem,
                          hipStream_t stream)
{
    if constexpr (XL) {
        switch (M) {
        case 1: return launch_g<FMT, 1, true, MODE>(G, J, R, p, grid, block, shmem, stream);
        case 2: return launch_g<FMT, 2, true, MODE>(G, J, R, p, grid, block, shmem, stream);
        case 3: return launch_g<FMT, 3, true, MODE>(G, J, R, p, grid, block, shmem, stream);
        case 4: return launch_g<FMT, 4, true, MODE>(G, J, R, p, grid, block, shmem, stream);
        }
    } else {
        switch (M) {
        case 1: return launch_g<FMT, 1, false, MODE>(G, J, R, p, grid, block, 0, stream);
        case 2: return launch_g<FMT, 2, false, MODE>(G, J, R, p, grid, block, 0, stream);
        case 3: return launch_g<FMT, 3, false, MODE>(G, J, R, p, grid, block, 0, stream);
        case 4: return launch_g<FMT, 4, false, MODE>(G, J, R, p, grid, block, 0, stream);
        case 5: return launch_g<FMT, 5, false, MODE>(G, J, R, p, grid, block, 0, stream);
        case 6: return launch_g<FMT, 6, false, MODE>(G, J, R, p, grid, block, 0, stream);
        case 7: return launch_g<FMT, 7, false, MODE>(G, J, R, p, grid, block, 0, stream);
        case 8: return launch_g<FMT, 8, false, MODE>(G, J, R, p, grid, block, 0, stream);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace qg
