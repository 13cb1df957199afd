// Fused dequantize-and-multiply GEMV kernels (Q4_0, Q8_0, and the one-launch
// MoE variant) for gfx950.
//
// The work is bound by streaming the packed weights from HBM once per call
// [volta-kernel-bakeoff, "Why the V100 is interesting here";
//  H100-KERNEL-5X-ROADMAP, "Why the decode gap is bandwidth"], so the design
// goals are: every weight byte read exactly once with 16-byte coalesced loads,
// enough bytes in flight per compute unit to cover HBM latency, and an unpack
// cheap enough that the vector ALUs keep pace with the memory stream.
//
// Mapping (one wave64 = 64 lanes):
//   * A "team" of `ksplit` waves owns a group of R consecutive rows at a time.
//     Wave w of the team covers blocks [w*64J, (w+1)*64J) of every row; lane
//     l of that wave owns blocks w*64J + l + 64j (j < J).  Consecutive lanes
//     read consecutive 16-byte code words: every load instruction of a wave
//     touches one contiguous 1 KiB span (Q4_0).
//   * Each lane keeps the activations of its blocks in registers for all M
//     tokens, loaded once per team and reused for every row the team visits
//     (one activation load serves many rows [volta-kernel-bakeoff, "Results",
//     the few-tokens bullet]).  J*M <= 8 bounds that register cost.
//   * Teams stride over row groups (a persistent grid sized to the chip) and
//     prefetch the next group's codes and scales before computing the current
//     one, so each wave always has a full group of loads in flight.
//   * Unpack: a nibble n OR-ed into the binary16 pattern 0x6400 is the half
//     1024 + n exactly [volta-kernel-bakeoff, "What's in the race", the
//     fused_q4_v2 bit trick]; subtracting 1032 gives n - 8 exactly, two
//     weights per packed-half instruction.  Nibbles in bits 4..7 give
//     1024 + 16 n, and (1024 + 16 n) / 16 - 72 = n - 8, also exact, which
//     saves the shift.  Products with the activations go through
//     v_dot2_f32_f16 (two fp16 products, exact, summed into fp32).  The block
//     scale multiplies the 32-term block sum once.
//   * Reduction of a row's 64 lane partials: DPP within 16-lane rows, then
//     the four row sums are read out with readlane; waves of a team (ksplit
//     > 1) combine through LDS.  No atomics: results are reproducible.
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

// ---------------------------------------------------------------- unpacking
//
// Both formats unpack a block into 16 half pairs v[0..15] whose activation
// partners are the pairs X[0..15] built by load_x_block<FMT>.

// Q4_0: word t holds bytes 4t..4t+3 = elements 4t..4t+3 (low nibbles) and
// 16+4t..19+4t (high nibbles).
//   v[4t+0] = (e[4t],    e[4t+2])      v[4t+2] = (e[4t+1],  e[4t+3])
//   v[4t+1] = (e[16+4t], e[18+4t])     v[4t+3] = (e[17+4t], e[19+4t])
// The magic constant is pinned in a vector register: with the mask in a scalar
// register, (w & mask) | magic is then a single v_and_or_b32.
__device__ __forceinline__ uint32_t magic_reg()
{
    uint32_t m;
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(m));
    return m;
}

__device__ __forceinline__ void unpack_q4(const uint4 c, h2_t (&v)[16])
{
    const uint32_t kMagic = magic_reg();
    const h2_t kOffLo = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const h2_t kScaleHi = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2_t kOffHi = {(_Float16)-72.0f, (_Float16)-72.0f};
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint32_t a = w[t];
        const uint32_t b = w[t] >> 8;
        v[4 * t + 0] = as_h2((a & 0x000F000Fu) | kMagic) + kOffLo;
        v[4 * t + 1] = as_h2((a & 0x00F000F0u) | kMagic) * kScaleHi + kOffHi;
        v[4 * t + 2] = as_h2((b & 0x000F000Fu) | kMagic) + kOffLo;
        v[4 * t + 3] = as_h2((b & 0x00F000F0u) | kMagic) * kScaleHi + kOffHi;
    }
}

// Q8_0: word t holds int8 elements 4t..4t+3.  Flipping the sign bits gives
// u = q + 128 in 1..255; 0x6400 | u is 1024 + u; minus 1152 is q, exactly.
//   v[2t] = (e[4t], e[4t+2])   v[2t+1] = (e[4t+1], e[4t+3])
__device__ __forceinline__ void unpack_q8(const uint4 c0, const uint4 c1, h2_t (&v)[16])
{
    const uint32_t kMagic = magic_reg();
    const h2_t kOff = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    const uint32_t w[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const uint32_t u = w[t] ^ 0x80808080u;
        v[2 * t + 0] = as_h2((u & 0x00FF00FFu) | kMagic) + kOff;
        v[2 * t + 1] = as_h2(((u >> 8) & 0x00FF00FFu) | kMagic) + kOff;
    }
}

__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) { return (a & 0xFFFFu) | (b << 16); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }

// The 32 fp16 activations of one block (64 bytes at p) as the 16 pairs that
// match unpack_q4 / unpack_q8.
template <int FMT>
__device__ __forceinline__ void load_x_block(const uint16_t *p, uint32_t (&X)[16])
{
    const uint4 *q = reinterpret_cast<const uint4 *>(p);
    const uint4 r0 = q[0], r1 = q[1], r2 = q[2], r3 = q[3];
    const uint32_t d[16] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w,
                            r2.x, r2.y, r2.z, r2.w, r3.x, r3.y, r3.z, r3.w};
    // d[i] = (x[2i], x[2i+1])
    if constexpr (FMT == kQ4_0) {
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

// ---------------------------------------------------------------- reduction

template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over the 64 lanes of a wave; the result is wave-uniform.
__device__ __forceinline__ float wave_sum(float v)
{
    v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);   // row_half_mirror
    v += dpp<0x140>(v);   // row_mirror: every lane holds its 16-lane row's sum
    const int b = __builtin_bit_cast(int, v);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
    return (r0 + r1) + (r2 + r3);
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

template <int FMT, int J, int R>
struct Group {
    Codes<FMT> code[R][J];
    uint16_t scale[R][J];
};

// Issue the loads of one row group.  Addresses are always in bounds: rows past
// N are clamped to N - 1 and padding lanes to their chunk's last block; such
// entries get a zero scale (and zero activations) in compute_group, so they
// add nothing.  Each row's base address is wave-uniform (scalar registers);
// lanes add a 32-bit offset.
#ifndef QG_NT_LOADS
#define QG_NT_LOADS 1
#endif

// Weight bytes are read once per call: they are loaded non-temporal so the
// stream does not displace the activations from the caches (measured on
// MI355X: 6.5 TB/s against 6.0 TB/s with plain loads on the 296 MB
// 128256 x 4096 matrix).
__device__ __forceinline__ uint4 stream_load16(const uint8_t *p)
{
#if QG_NT_LOADS
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    const v4u t = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
#else
    return *reinterpret_cast<const uint4 *>(p);
#endif
}

__device__ __forceinline__ uint16_t stream_load2(const uint8_t *p)
{
#if QG_NT_LOADS
    return __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(p));
#else
    return *reinterpret_cast<const uint16_t *>(p);
#endif
}

template <int FMT, int J, int R>
__device__ __forceinline__ void load_group(Group<FMT, J, R> &g, const uint8_t *__restrict__ W,
                                           const uint16_t *__restrict__ S, int64_t row0, int N, int KB,
                                           const uint32_t (&boff)[J])
{
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int64_t row = min(row0 + i, (int64_t)N - 1);
        const int64_t base = row * KB;   // first block of the row
        const uint8_t *__restrict__ srow = reinterpret_cast<const uint8_t *>(S + base);
        const uint8_t *__restrict__ crow = W + base * (FMT == kQ4_0 ? 16 : 32);
#pragma unroll
        for (int j = 0; j < J; ++j) {
            // scalar row base + unsigned 32-bit lane offset
            if constexpr (FMT == kQ4_0) {
                g.code[i][j].c = stream_load16(crow + (uint64_t)(boff[j] * 16u));
            } else {
                g.code[i][j].c0 = stream_load16(crow + (uint64_t)(boff[j] * 32u));
                g.code[i][j].c1 = stream_load16(crow + (uint64_t)(boff[j] * 32u + 16u));
            }
            g.scale[i][j] = stream_load2(srow + (uint64_t)(boff[j] * 2u));
        }
    }
}

// Activations come either from registers (X, loaded once per team) or, with
// XL, from the workgroup's LDS copy (one token; xs holds every block of x in
// pair order plus one zero block that padding lanes read).
template <int FMT, int M, int J, int R, bool XL>
__device__ __forceinline__ void compute_group(const Group<FMT, J, R> &g,
                                              const uint32_t (&X)[XL ? 1 : M][XL ? 1 : J][16],
                                              const uint4 *xs, const uint32_t (&xoff)[J], const bool (&ok)[J],
                                              int64_t row0, int N, float (&acc)[R][M])
{
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const bool rok = row0 + i < N;
#pragma unroll
        for (int m = 0; m < M; ++m)
            acc[i][m] = 0.0f;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            h2_t v[16];
            if constexpr (FMT == kQ4_0)
                unpack_q4(g.code[i][j].c, v);
            else
                unpack_q8(g.code[i][j].c0, g.code[i][j].c1, v);
            const _Float16 dh = __builtin_bit_cast(_Float16, (uint16_t)((rok && ok[j]) ? g.scale[i][j] : 0));
            const float d = (float)dh;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                uint32_t xw[16];
                if constexpr (XL) {
                    const uint4 *q = xs + xoff[j] * 4;
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const uint4 t = q[u];
                        xw[4 * u + 0] = t.x;
                        xw[4 * u + 1] = t.y;
                        xw[4 * u + 2] = t.z;
                        xw[4 * u + 3] = t.w;
                    }
                } else {
#pragma unroll
                    for (int t = 0; t < 16; ++t)
                        xw[t] = X[m][j][t];
                }
                float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
                for (int t = 0; t < 16; t += 2) {
                    s0 = dot2(v[t], as_h2(xw[t]), s0);
                    s1 = dot2(v[t + 1], as_h2(xw[t + 1]), s1);
                }
                acc[i][m] = __builtin_fmaf(d, s0 + s1, acc[i][m]);
            }
        }
    }
}

// Reduce one group's partials and store y (ksplit == 1), or combine the
// team's waves through LDS first (ksplit > 1).
template <int M, int R>
__device__ __forceinline__ void finish_group(const float (&acc)[R][M], float *__restrict__ y, int64_t row0, int N,
                                             int lane, int wave, int team, int kw, int ksplit,
                                             float (&red)[2][kMaxWavesPerWg][kMaxRM], int &buf)
{
    float tot[R * M];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int m = 0; m < M; ++m)
            tot[i * M + m] = wave_sum(acc[i][m]);

    if (ksplit == 1) {
        float out = 0.0f;
#pragma unroll
        for (int t = 0; t < R * M; ++t)
            out = (lane == t) ? tot[t] : out;
        if (lane < R * M) {
            const int i = lane / M, m = lane % M;
            const int64_t row = row0 + i;
            if (row < N)
                y[(int64_t)m * N + row] = out;
        }
    } else {
        if (lane == 0) {
#pragma unroll
            for (int t = 0; t < R * M; ++t)
                red[buf][wave][t] = tot[t];
        }
        __syncthreads();
        if (kw == 0 && lane < R * M) {
            float s = 0.0f;
            for (int w = 0; w < ksplit; ++w)
                s += red[buf][team * ksplit + w][lane];
            const int i = lane / M, m = lane % M;
            const int64_t row = row0 + i;
            if (row < N)
                y[(int64_t)m * N + row] = s;
        }
        buf ^= 1;
    }
}

template <int FMT, int M, int J, int R, bool XL>
__global__ __launch_bounds__(512) void gemv_kernel(GemvParams p)
{
    static_assert(!XL || M == 1, "LDS-staged activations are for one token");
    const int lane = threadIdx.x & 63;
    // wave-uniform: everything derived from it (rows, addresses) stays scalar
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kw = wave % p.ksplit;       // this wave's K chunk
    const int team = wave / p.ksplit;     // team within the workgroup
    const int64_t teams_total = (int64_t)gridDim.x * p.teams_per_wg;
    const int64_t team_id = (int64_t)blockIdx.x * p.teams_per_wg + team;
    const int item = blockIdx.y;          // batch item: MoE expert slot

    const uint8_t *__restrict__ W = p.W;
    if (p.idx)
        W += (int64_t)p.idx[item] * p.matrix_stride;
    const uint16_t *__restrict__ S = reinterpret_cast<const uint16_t *>(W + p.scale_offset);
    const uint16_t *__restrict__ x = p.x + (int64_t)item * M * p.K;
    float *__restrict__ y = p.y + (int64_t)item * M * p.N;

    const int KB = p.K >> 5;
    const int bbeg = kw * 64 * J;
    const int bend = min(KB, bbeg + 64 * J);
    uint32_t blk[J], xoff[J];
    bool ok[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int b = bbeg + lane + 64 * j;
        ok[j] = b < bend;
        blk[j] = (uint32_t)(ok[j] ? b : bend - 1);
        xoff[j] = (uint32_t)(ok[j] ? b : KB);   // LDS block KB is all zeros
    }

    const int64_t ngroups = ((int64_t)p.N + R - 1) / R;
    int64_t g = team_id;

    Group<FMT, J, R> ga, gb;
    if (g < ngroups)
        load_group<FMT, J, R>(ga, W, S, g * R, p.N, KB, blk);

    // activations of this lane's blocks, all M tokens, kept for every row
    uint32_t X[XL ? 1 : M][XL ? 1 : J][16];
    extern __shared__ uint4 xs_dyn[];
    if constexpr (XL) {
        // the workgroup stages x once, in pair order, plus a zero block
        for (int b = threadIdx.x; b <= KB; b += blockDim.x) {
            uint32_t w16[16];
            if (b < KB) {
                load_x_block<FMT>(x + (int64_t)b * 32, w16);
            } else {
#pragma unroll
                for (int t = 0; t < 16; ++t)
                    w16[t] = 0u;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                xs_dyn[b * 4 + u] = make_uint4(w16[4 * u], w16[4 * u + 1], w16[4 * u + 2], w16[4 * u + 3]);
        }
        __syncthreads();
    } else {
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int j = 0; j < J; ++j) {
                load_x_block<FMT>(x + (int64_t)m * p.K + (int64_t)blk[j] * 32, X[m][j]);
                if (!ok[j]) {
#pragma unroll
                    for (int t = 0; t < 16; ++t)
                        X[m][j][t] = 0u;
                }
            }
    }

    __shared__ float red[2][kMaxWavesPerWg][kMaxRM];
    int buf = 0;

    // two register sets in ping-pong: the next group's loads are in flight
    // while the current group is unpacked and multiplied
    while (g < ngroups) {
        float acc[R][M];
        int64_t gn = g + teams_total;
        if (gn < ngroups)
            load_group<FMT, J, R>(gb, W, S, gn * R, p.N, KB, blk);
        compute_group<FMT, M, J, R, XL>(ga, X, xs_dyn, xoff, ok, g * R, p.N, acc);
        finish_group<M, R>(acc, y, g * R, p.N, lane, wave, team, kw, p.ksplit, red, buf);
        g = gn;
        if (g >= ngroups)
            break;
        gn = g + teams_total;
        if (gn < ngroups)
            load_group<FMT, J, R>(ga, W, S, gn * R, p.N, KB, blk);
        compute_group<FMT, M, J, R, XL>(gb, X, xs_dyn, xoff, ok, g * R, p.N, acc);
        finish_group<M, R>(acc, y, g * R, p.N, lane, wave, team, kw, p.ksplit, red, buf);
        g = gn;
    }
}

// ---------------------------------------------------------------- dispatch

template <int FMT, int M, int J, int R, bool XL>
static hipError_t launch_one(const GemvParams &p, dim3 grid, dim3 block, size_t shmem, hipStream_t stream)
{
    return launch_kernel(reinterpret_cast<const void *>(&gemv_kernel<FMT, M, J, R, XL>), grid, block, shmem, stream,
                         p);
}

// Register budget: R * J code words in flight twice (ping-pong) plus, without
// XL, J * M resident activation blocks.  R * J <= 8 (Q4_0) / 4 (Q8_0) and
// J <= 7 (8 with XL) keep every instantiation within 256 registers without
// spilling.
template <int FMT, int J, int R, bool XL>
constexpr bool fits() { return R * J <= (FMT == kQ4_0 ? 8 : 4) && J <= (XL ? 8 : 7); }

template <int FMT, int M, int J, bool XL>
static hipError_t launch_r(int R, const GemvParams &p, dim3 grid, dim3 block, size_t shmem, hipStream_t stream)
{
    if constexpr (fits<FMT, J, 1, XL>())
        if (R == 1) return launch_one<FMT, M, J, 1, XL>(p, grid, block, shmem, stream);
    if constexpr (fits<FMT, J, 2, XL>())
        if (R == 2) return launch_one<FMT, M, J, 2, XL>(p, grid, block, shmem, stream);
    if constexpr (fits<FMT, J, 4, XL>())
        if (R == 4) return launch_one<FMT, M, J, 4, XL>(p, grid, block, shmem, stream);
    return hipErrorInvalidValue;
}

template <int FMT, int M, bool XL>
static hipError_t launch_j(int J, int R, const GemvParams &p, dim3 grid, dim3 block, size_t shmem,
                           hipStream_t stream)
{
    // J * M <= 8 keeps resident activations at <= 128 registers
    if constexpr (M == 1) {
        switch (J) {
        case 1: return launch_r<FMT, 1, 1, XL>(R, p, grid, block, shmem, stream);
        case 2: return launch_r<FMT, 1, 2, XL>(R, p, grid, block, shmem, stream);
        case 3: return launch_r<FMT, 1, 3, XL>(R, p, grid, block, shmem, stream);
        case 4: return launch_r<FMT, 1, 4, XL>(R, p, grid, block, shmem, stream);
        case 5: return launch_r<FMT, 1, 5, XL>(R, p, grid, block, shmem, stream);
        case 6: return launch_r<FMT, 1, 6, XL>(R, p, grid, block, shmem, stream);
        case 7: return launch_r<FMT, 1, 7, XL>(R, p, grid, block, shmem, stream);
        case 8: return launch_r<FMT, 1, 8, XL>(R, p, grid, block, shmem, stream);
        }
    } else if constexpr (M == 2) {
        switch (J) {
        case 1: return launch_r<FMT, 2, 1, false>(R, p, grid, block, shmem, stream);
        case 2: return launch_r<FMT, 2, 2, false>(R, p, grid, block, shmem, stream);
        case 3: return launch_r<FMT, 2, 3, false>(R, p, grid, block, shmem, stream);
        case 4: return launch_r<FMT, 2, 4, false>(R, p, grid, block, shmem, stream);
        }
    } else if constexpr (M <= 4) {
        switch (J) {
        case 1: return launch_r<FMT, M, 1, false>(R, p, grid, block, shmem, stream);
        case 2: return launch_r<FMT, M, 2, false>(R, p, grid, block, shmem, stream);
        }
    } else {
        if (J == 1)
            return launch_r<FMT, M, 1, false>(R, p, grid, block, shmem, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemv(int fmt, int M, int J, int R, bool xl, const GemvParams &p, dim3 grid, dim3 block,
                       hipStream_t stream)
{
    // XL: one token, one wave per row group, activations staged in LDS
    // (K/32 blocks of 64 bytes plus one zero block)
    const size_t shmem = xl ? (size_t)(p.K / 32 + 1) * 64 : 0;
    if (xl) {
        if (M != 1 || p.ksplit != 1)
            return hipErrorInvalidValue;
        return fmt == kQ4_0 ? launch_j<kQ4_0, 1, true>(J, R, p, grid, block, shmem, stream)
                            : launch_j<kQ8_0, 1, true>(J, R, p, grid, block, shmem, stream);
    }
#define QG_CASE_M(FMT)                                                                \
    switch (M) {                                                                      \
    case 1: return launch_j<FMT, 1, false>(J, R, p, grid, block, 0, stream);          \
    case 2: return launch_j<FMT, 2, false>(J, R, p, grid, block, 0, stream);          \
    case 3: return launch_j<FMT, 3, false>(J, R, p, grid, block, 0, stream);          \
    case 4: return launch_j<FMT, 4, false>(J, R, p, grid, block, 0, stream);          \
    case 5: return launch_j<FMT, 5, false>(J, R, p, grid, block, 0, stream);          \
    case 6: return launch_j<FMT, 6, false>(J, R, p, grid, block, 0, stream);          \
    case 7: return launch_j<FMT, 7, false>(J, R, p, grid, block, 0, stream);          \
    case 8: return launch_j<FMT, 8, false>(J, R, p, grid, block, 0, stream);          \
    }
    if (fmt == kQ4_0) {
        QG_CASE_M(kQ4_0)
    } else {
        QG_CASE_M(kQ8_0)
    }
#undef QG_CASE_M
    return hipErrorInvalidValue;
}

}  // namespace qg
