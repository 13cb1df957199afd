// Q4_0 prefill GEMM on the gfx950 matrix cores:
//   Y[m][n] = sum_k X[m][k] * w[n][k],  w = (q - 8) * d
//
// With many tokens the work is a dense contraction, so it belongs on MFMA
// (v_mfma_f32_32x32x16_f16, fp32 accumulators) [volta-kernel-bakeoff, "What's
// in the race" (tc_q4: unpack a tile, then matrix-core multiply) and
// "Stage 3" (unpack inside the multiply instead of dequantize-to-fp16
// followed by a dense GEMM)].
//
// Data path.  A 64-wide K step covers two Q4_0 blocks; four steps (eight
// blocks, 128 code bytes per row) form a group.
//   * Weights: each wave loads its own 32-row tiles a group at a time with
//     whole-line loads (8 lanes per row, 16 bytes each), writes them to a
//     wave-private LDS buffer (16-byte chunks XOR-swizzled by row, so the
//     reads below hit distinct banks) and, per step, lane l reads back the 16
//     code bytes of row l % 32, block 2s + l / 32.  Two v_permlane32_swap
//     then leave every lane the 8 bytes of each block that its MFMA operand
//     needs (the B operand of lane l holds k = 8 (l / 32) .. +7 of row
//     l % 32: low nibbles of bytes 8 (l / 32) .. +7 for the block's first 16
//     k, high nibbles for the last 16), in natural k order.  The nibbles
//     become fp16 through the 0x6400 pattern (1024 + q, exact), the offset
//     is removed exactly and one correctly rounded fp16 multiply by the block
//     scale gives the same values qdequant_q4_0 writes with fp16 output.
//     The eight scales of a row's group are one 16-byte load.  Loading a
//     step's 32 bytes of each of 32 rows directly would touch 32 cache lines
//     per instruction for a quarter line each; the request count, not the
//     bytes, then bounds the kernel.
//   * Activations: each step's X rows go straight from memory into LDS
//     (buffer loads that write LDS: no registers, no copy instructions), in
//     natural k order with the 16-byte chunks of row r at position c ^ ((r /
//     2) % 8) (conflict-free 16-byte reads without padding), and are read
//     back as the A operands.
//   * Each wave owns 32 TM tokens x 32 TN rows of the workgroup's tile (WM
//     waves along M, NW / WM along N, NW = 4 or 8 waves); with WM = 1 no
//     weight is unpacked twice.
//
// Work split (stream-K): the (tile, K step) iterations are numbered tile by
// tile and cut into equal contiguous ranges of whole groups, one per
// workgroup of a persistent grid, so the chip stays busy however few tiles
// there are.  A workgroup whose range covers a whole tile stores it; partial
// tiles are added with fp32 atomics into Y, which a small fill kernel zeroes
// first (last-bit differences between runs, within the accuracy bound).
//
// Pipelining: four LDS activation buffers, one per step of a group.  Between
// the MFMAs of step s go the copy of step s + 3 (into the buffer steps s - 2
// and s - 1 read), the unpacking of step s + 1's B operands and the reads of
// step s + 1's first two k slices (its buffer is complete a step early); the
// weight loads of the next group are in flight in registers while the
// current group is multiplied; one barrier per step.  Every load is
// issued unconditionally (positions past a workgroup's range repeat its last
// one and are never used), so the load counter, which counts them in issue
// order, tells exactly when a step's copy has landed.
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

__device__ __forceinline__ h2_t as_h2(uint32_t u) { return __builtin_bit_cast(h2_t, u); }
__device__ __forceinline__ uint32_t as_u32(h2_t h) { return __builtin_bit_cast(uint32_t, h); }

// An empty asm statement that claims to modify v: the computation of v stays
// before this point (the compiler cannot sink it past a statement with side
// effects).
template <typename V>
__device__ __forceinline__ void pin(V &v)
{
    asm volatile("" : "+v"(v));
}

__device__ __forceinline__ uint32_t magic_reg()
{
    uint32_t m;
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(m));
    return m;
}

// 8 code bytes of one block (p0 = bytes 0-3, p1 = bytes 4-7 of the lane's
// half) -> two B operands in natural k order: lo = the 8 low nibbles (the
// block's first 16 k for this lane's half), hi = the 8 high nibbles, each
// weight (q - 8) * d rounded once to fp16.  One call makes element pair e
// (0..3) of both: the nibbles of bytes 2 e and 2 e + 1.
__device__ __forceinline__ void unpack_pair(uint32_t p0, uint32_t p1, h2_t d2, uint32_t magic, int e, uint32_t &lo,
                                            uint32_t &hi)
{
    const h2_t kOffLo = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const h2_t kScaleHi = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2_t kOffHi = {(_Float16)-72.0f, (_Float16)-72.0f};
    const uint32_t w = (e >> 1) ? p1 : p0;
    const uint32_t nl = w & 0x0F0F0F0Fu;   // low nibbles, one per byte
    const uint32_t nh = w & 0xF0F0F0F0u;   // high nibbles, times 16
    // bytes (n0, 0x64, n1, 0x64) or (n2, 0x64, n3, 0x64) of the word: the
    // halves 1024 + n of two consecutive elements
    const uint32_t sel = (e & 1) ? 0x07030502u : 0x07010500u;
    const uint32_t l = __builtin_amdgcn_perm(magic, nl, sel);
    const uint32_t h = __builtin_amdgcn_perm(magic, nh, sel);
    lo = as_u32((as_h2(l) + kOffLo) * d2);                // (q - 8) * d
    hi = as_u32((as_h2(h) * kScaleHi + kOffHi) * d2);     // (1024 + 16 q) / 16 - 72 = q - 8
}

struct PrefillParams {
    const uint8_t *W;          // packed Q4_0 matrix
    const uint16_t *X;         // fp16 [M][K]
    float *Y;                  // fp32 [M][N]
    int64_t scale_offset;
    int M, N, K;
    int tiles_n;               // output tiles along N
    int steps;                 // K steps per tile: ceil(K / 64) rounded up to a group of 4
    int chunks;                // tiles * steps / 4 (< 2^31 / 4, checked on the host)
};

constexpr int kGroup = 4;      // K steps per weight group (8 blocks)

// Position of an iteration: output tile (tm along M, tn along N, tn
// fastest) and K step s within it.  Advanced one step at a time, with no
// division.
struct Pos {
    int tm, tn, s;
};

__device__ __forceinline__ Pos pos_of(const PrefillParams &p, int it, int S)
{
    const int tile = it / S;
    return Pos{tile / p.tiles_n, tile % p.tiles_n, it % S};
}

__device__ __forceinline__ void advance(Pos &q, const PrefillParams &p, int S)
{
    if (++q.s == S) {
        q.s = 0;
        if (++q.tn == p.tiles_n) {
            q.tn = 0;
            ++q.tm;
        }
    }
}

template <int WM, int TM, int TN, int NW>
struct Tiling {
    static constexpr int WN = NW / WM;
    static constexpr int BM = 32 * TM * WM;   // tokens per tile
    static constexpr int BN = 32 * TN * WN;   // rows per tile
    static constexpr int AC = BM * 8 / (64 * NW);   // 16-byte activation chunks per thread per step
};

// Registers of one group's weights (per row tile: this lane's four 16-byte
// chunks of whole lines, and the eight scales of its row).
template <int TN>
struct WGroup {
    uint4 code[TN][4];
    uint4 scale[TN];
};

// Load cursors hold a position and the per-lane byte offsets of its tile
// (they change only when the tile does); the K step enters as the scalar
// offset of the buffer loads, so a step spends no vector instruction on
// addresses.
//   Activations: lane l of instruction i of wave w writes the i-th kilobyte
//   of the wave's share of the step, i.e. row 8 w + 8 NW i + l / 8 of the tile
//   (clamped to M - 1: rows past M are never stored) at position l % 8, and
//   reads the chunk stored there (`a_swz`) of that row at the step.
//   Weights: instruction i of row tile j (32 rows from row n0 + 32 (wn TN +
//   j)) has lane l read the 16 bytes of row 8 i + l / 8 at block 8 g + l % 8
//   of group g; the scales: lane l reads the eight of row l % 32.  Rows are
//   clamped to N - 1 (their scale is zeroed).
// Blocks past K (padding steps, or the tail of the last group) read the next
// row's bytes or, past the end, zeros; their activations and scales are
// zeroed.
// Position of 16-byte chunk c of activation row r in its LDS row (128
// bytes, 8 chunks): c ^ ((r / 2) % 8).  Rows are 32 banks apart, so rows r
// and r + 2 share banks; the XOR gives each of 16 consecutive rows its own
// four banks, and a 16-lane quarter of an A-operand read (16 rows, one
// chunk each) touches all 64 banks once.
__device__ __forceinline__ int a_swz(int r, int c) { return c ^ ((r >> 1) & 7); }

template <int AC>
struct ACursor {
    Pos ps;
    int it;
    uint32_t off[AC];
};

template <int TN>
struct WCursor {
    Pos ps;                 // first step of the group
    int it;
    uint32_t off[TN][4];    // code byte offsets (block 8 g + l % 8 of row 8 i + l / 8)
    uint32_t soff[TN];      // scale byte offsets (row l % 32, block 0)
};

template <int BM, int AC, int NT>
__device__ __forceinline__ void a_offsets(ACursor<AC> &c, const PrefillParams &p)
{
#pragma unroll
    for (int i = 0; i < AC; ++i) {
        const int idx = (int)threadIdx.x + NT * i;
        const int r = idx >> 3, ch = a_swz(r, idx & 7);
        const int m = min(c.ps.tm * BM + r, p.M - 1);
        c.off[i] = (uint32_t)m * (uint32_t)p.K * 2u + (uint32_t)ch * 16u;
    }
}

template <int BN, int TN>
__device__ __forceinline__ void w_offsets(WCursor<TN> &c, const PrefillParams &p, int KB, int lane, int wn)
{
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int r0 = c.ps.tn * BN + 32 * (wn * TN + j);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = min(r0 + 8 * i + (lane >> 3), p.N - 1);
            c.off[j][i] = ((uint32_t)row * (uint32_t)KB + (uint32_t)(lane & 7)) * 16u;
        }
        const int row = min(r0 + (lane & 31), p.N - 1);
        c.soff[j] = (uint32_t)row * (uint32_t)KB * 2u;
    }
}

// Advance by one step (activations) or one group (weights), up to the
// workgroup's last step (loads past its range repeat the last position).
template <int BM, int AC, int NT>
__device__ __forceinline__ void a_step(ACursor<AC> &c, const PrefillParams &p, int S, int it_end)
{
    if (c.it + 1 < it_end) {
        ++c.it;
        advance(c.ps, p, S);
        if (c.ps.s == 0)
            a_offsets<BM, AC, NT>(c, p);
    }
}

template <int BN, int TN>
__device__ __forceinline__ void w_step(WCursor<TN> &c, const PrefillParams &p, int S, int it_end, int KB, int lane,
                                       int wn)
{
    if (c.it + kGroup < it_end) {
        c.it += kGroup;
#pragma unroll
        for (int q = 0; q < kGroup; ++q)
            advance(c.ps, p, S);
        if (c.ps.s == 0)
            w_offsets<BN>(c, p, KB, lane, wn);
    }
}

struct Rsrc {
    __amdgpu_buffer_rsrc_t x, w, s;
};


// One step's activations straight into the LDS buffer `buf` (BM rows of
// eight 16-byte chunks): no registers and no copy instructions.  Chunks of
// blocks past K get an offset beyond the buffer, whose range check returns
// zeros.
template <int AC, int NT>
__device__ __forceinline__ void dma_a_one(uint4 (*buf)[8], const Rsrc &rs, const ACursor<AC> &c, int KB, int wave,
                                          int i)
{
    const int so = c.ps.s * 128;   // 64 fp16 per step
    const bool full = 2 * c.ps.s + 2 <= KB;   // uniform: both blocks of the step inside K
    uint32_t off = c.off[i];
    if (!full) {
        const int idx = (int)threadIdx.x + NT * i;
        const int r = idx >> 3, ch = a_swz(r, idx & 7);
        if (2 * c.ps.s + (ch >> 2) >= KB)
            off = 0x80000000u;
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs.x, (__attribute__((address_space(3))) void *)&buf[8 * wave + NT / 8 * i][0], 16, off, so, 0, 0);
}

template <int AC, int NT>
__device__ __forceinline__ void dma_a(uint4 (*buf)[8], const Rsrc &rs, const ACursor<AC> &c, int KB, int wave)
{
#pragma unroll
    for (int i = 0; i < AC; ++i)
        dma_a_one<AC, NT>(buf, rs, c, KB, wave, i);
}

// Wait until at most n vector memory operations of this wave are in flight
// (gfx9 encoding of s_waitcnt: vmcnt in bits 3:0 and 15:14; expcnt and
// lgkmcnt left at their maxima, so they are not waited for).
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// SA: rows hold a whole number of groups (K / 32 a multiple of 8), so a
// row's eight scales of a group are one 16-byte load inside the row (4-byte
// aligned); otherwise eight 2-byte loads.  Non-temporal: every weight line is
// used by one load, and the stream must not evict the activations, which
// every workgroup reads, from L2.
template <int TN, bool SA>
__device__ __forceinline__ void load_w(WGroup<TN> &st, const Rsrc &rs, const WCursor<TN> &c)
{
    const int g8 = c.ps.s * 2;   // first block of the group (8 per group)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const auto t = __builtin_amdgcn_raw_buffer_load_b128(rs.w, c.off[j][i], g8 * 16, kNtAux);
            st.code[j][i] = make_uint4(t[0], t[1], t[2], t[3]);
        }
        if constexpr (SA) {
            const auto t = __builtin_amdgcn_raw_buffer_load_b128(rs.s, c.soff[j], g8 * 2, kNtAux);
            st.scale[j] = make_uint4(t[0], t[1], t[2], t[3]);
        } else {
            uint32_t h[8];
#pragma unroll
            for (int b = 0; b < 8; ++b)
                h[b] = __builtin_amdgcn_raw_buffer_load_b16(rs.s, c.soff[j], g8 * 2 + 2 * b, kNtAux);
            st.scale[j] = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                                     h[6] | (h[7] << 16));
        }
    }
}

template <int WM, int TM, int TN, int OCC, bool SA, int NW>
__global__ __launch_bounds__(64 * NW, OCC) void prefill_kernel(PrefillParams p)
{
    using T = Tiling<WM, TM, TN, NW>;
    constexpr int NT = 64 * NW;   // threads
    constexpr int AC = T::AC;
    constexpr int DB = kGroup;   // steps per weight group
    // activations: one swizzled buffer per step of a group, each a variable
    // of its own, so the compiler knows which buffer an A-operand read
    // touches and waits only for the copies into that one (with one array
    // it waits for every load in flight before each read)
    __shared__ uint4 Ad0[T::BM][8], Ad1[T::BM][8], Ad2[T::BM][8], Ad3[T::BM][8];
    auto abuf = [&](int q) -> uint4(*)[8] { return q == 0 ? Ad0 : q == 1 ? Ad1 : q == 2 ? Ad2 : Ad3; };
    __shared__ uint4 Wl[NW][TN][32][8];   // per wave: the current group's code bytes, chunks swizzled by row

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave % WM, wn = wave / WM;
    const int KB = p.K >> 5;
    const int S = p.steps;   // 64-wide K steps per tile, whole groups (steps past K multiply zeros)
    // this workgroup's range: whole groups, so a group never spans two tiles
    const int it_beg = (int)((int64_t)p.chunks * blockIdx.x / gridDim.x) * kGroup;
    const int it_end = (int)((int64_t)p.chunks * (blockIdx.x + 1) / gridDim.x) * kGroup;
    if (it_beg >= it_end)
        return;   // uniform over the workgroup
    const uint32_t magic = magic_reg();

    Rsrc rs;
    rs.x = make_rsrc(reinterpret_cast<const uint8_t *>(p.X), (int64_t)p.M * p.K * 2);
    rs.w = make_rsrc(p.W, (int64_t)p.N * KB * 16);
    rs.s = make_rsrc(p.W + p.scale_offset, (int64_t)p.N * KB * 2);

    f16x_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.0f;

    // Global loads are counted in issue order by one counter, so a wait for
    // one load waits for every load issued before it.  Issue order: the
    // activations of the range's first three steps (into buffers 0-2), then
    // the first weight group.
    const Pos first = pos_of(p, it_beg, S);
    ACursor<AC> la;
    la.ps = first;
    la.it = it_beg;
    a_offsets<T::BM, AC, NT>(la, p);
    WCursor<TN> lw;
    lw.ps = first;
    lw.it = it_beg;
    w_offsets<T::BN>(lw, p, KB, lane, wn);
    WGroup<TN> wg;
    dma_a<AC, NT>(Ad0, rs, la, KB, wave);
    a_step<T::BM, AC, NT>(la, p, S, it_end);
    dma_a<AC, NT>(Ad1, rs, la, KB, wave);
    a_step<T::BM, AC, NT>(la, p, S, it_end);
    dma_a<AC, NT>(Ad2, rs, la, KB, wave);
    a_step<T::BM, AC, NT>(la, p, S, it_end);
    load_w<TN, SA>(wg, rs, lw);
    w_step<T::BN>(lw, p, S, it_end, KB, lane, wn);

    // The weight group in registers -> this wave's LDS buffer: instruction i
    // of row tile j holds row 8 i + l / 8, chunk l % 8, stored at chunk
    // (l % 8) ^ (row % 8).  Wave-private: LDS operations of a wave complete
    // in order, so no barrier is needed between these writes and the reads.
    auto store_w = [&](const WGroup<TN> &g) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 8 * i + (lane >> 3);
                Wl[wave][j][row][(lane & 7) ^ (row & 7)] = g.code[j][i];
            }
    };

    // Scales of the current group, per row tile (row l % 32, blocks 8 g ..
    // 8 g + 7), with those of rows past N zeroed.
    uint4 scl[TN];
    auto take_scales = [&](const WGroup<TN> &g, const Pos &ps) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const bool row_ok = ps.tn * T::BN + 32 * (wn * TN + j) + (lane & 31) < p.N;
            scl[j] = row_ok ? g.scale[j] : make_uint4(0u, 0u, 0u, 0u);
        }
    };

    // The B operands of one step (this wave's row tiles, both blocks, both k
    // halves) in two sets, as words (bw[o][j][b][h][e]: element pair e of
    // row tile j, block b, k half h): the MFMAs of a step read one set while
    // the next step's operands are unpacked into the other.  Lane l takes
    // row l % 32, block 2 q + l / 32 of the group: its 16 code bytes are read
    // from LDS first (wc); the unpacking then rides between the current
    // step's MFMAs: after the first MFMA the lane-half swaps and the scales,
    // then block 0's element pairs after the MFMAs of k slice 1 and block
    // 1's after those of slice 2, one pair per MFMA (two with TM = 2).
    uint32_t bw[2][TN][2][2][4];
    uint4 wc[TN];
    uint32_t wt[TN][2], wu[TN][2];
    h2_t wd[TN][2];
    auto bop = [&](int o, int j, int b, int h) {
        return __builtin_bit_cast(half8_t, make_uint4(bw[o][j][b][h][0], bw[o][j][b][h][1], bw[o][j][b][h][2],
                                                      bw[o][j][b][h][3]));
    };
    auto read_w = [&](int q) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int row = lane & 31;
            wc[j] = Wl[wave][j][row][(2 * q + (lane >> 5)) ^ (row & 7)];
        }
    };
    auto swap_scales = [&](int q, const Pos &ps) {
        const int b0 = 2 * ps.s;   // first block of the step (2 q of the group)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const auto t = __builtin_amdgcn_permlane32_swap(wc[j].x, wc[j].z, false, false);
            const auto u = __builtin_amdgcn_permlane32_swap(wc[j].y, wc[j].w, false, false);
            wt[j][0] = (uint32_t)t[0];
            wt[j][1] = (uint32_t)t[1];
            wu[j][0] = (uint32_t)u[0];
            wu[j][1] = (uint32_t)u[1];
            const uint32_t sw = q == 0 ? scl[j].x : q == 1 ? scl[j].y : q == 2 ? scl[j].z : scl[j].w;
            const uint32_t s0 = b0 < KB ? (sw & 0xFFFFu) : 0u;
            const uint32_t s1 = b0 + 1 < KB ? (sw >> 16) : 0u;
            const _Float16 d0 = __builtin_bit_cast(_Float16, (uint16_t)s0);
            const _Float16 d1 = __builtin_bit_cast(_Float16, (uint16_t)s1);
            wd[j][0] = h2_t{d0, d0};
            wd[j][1] = h2_t{d1, d1};
        }
    };
    // pair c of block b (row tile c / 4, element pair c % 4) into set o;
    // the empty asm keeps it here: left free, the compiler sinks the
    // unpacking to just before the next step's MFMAs, which would then wait
    auto unpack_chunk = [&](int b, int c, int o) {
        const int j = c >> 2, e = c & 3;
        unpack_pair(wt[j][b], wu[j][b], wd[j][b], magic, e, bw[o][j][b][0][e], bw[o][j][b][1][e]);
        pin(bw[o][j][b][0][e]);
        pin(bw[o][j][b][1][e]);
    };
    auto prep = [&](int q, const Pos &ps, int o) {
        read_w(q);
        swap_scales(q, ps);
#pragma unroll
        for (int c = 0; c < 4 * TN; ++c) {
            unpack_chunk(0, c, o);
            unpack_chunk(1, c, o);
        }
    };

    // A operands, k slices 0 and 1 of a step: read in the step before it
    // (its buffer is complete a step early), so each step starts its MFMAs
    // at once and the LDS keeps streaming across the barrier.
    half8_t apre[2][TM];
    auto read_a = [&](int buf, int kk, half8_t (&dst)[TM]) {
        const int col = kk * 16 + (lane >> 5) * 8;   // block kk / 2, k half kk % 2
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int r = wm * 32 * TM + 32 * i + (lane & 31);
            dst[i] = *reinterpret_cast<const half8_t *>(&abuf(buf)[r][a_swz(r, col >> 3)]);
        }
    };

    // The step's MFMAs: A operands of slices 0-1 from apre, of slices 2-3
    // read from LDS buffer `buf` while slices 0-1 multiply; during slices
    // 2-3 the next step's slices 0-1 are read from buffer `nbuf`.  B operands
    // from set o, with part (kk, m) of the next step's unpacking after MFMA m
    // of slice kk (a scheduling barrier after each pair keeps the vector-ALU
    // work where it overlaps the matrix cores, and each read a slice ahead of
    // its MFMAs: left free, the compiler sinks a read to just before its
    // MFMA, which exposes an LDS round trip per MFMA).
    auto mma = [&](int buf, int nbuf, int o, auto &&part) {
        half8_t acur[2][TM];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            if (kk < 2)
                read_a(buf, kk + 2, acur[kk]);
            else
                read_a(nbuf, kk - 2, apre[kk - 2]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const half8_t av = kk < 2 ? apre[kk][i] : acur[kk - 2][i];
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bop(o, j, kk >> 1, kk & 1), acc[i][j], 0,
                                                                       0, 0);
                    part(kk, i * TN + j);
                    __builtin_amdgcn_sched_barrier(0);
                }
        }
    };
    // the next step's unpacking spread over a step's MFMAs: swaps and scales
    // after the first, block 0 over slice 1, block 1 over slice 2
    constexpr int kPer = 4 / TM;   // element-pair chunks per MFMA
    static_assert(TM * kPer == 4, "TM must be 1, 2 or 4");
    auto next_part = [&](int q, const Pos &ps, int o, int kk, int m) {
        if (kk == 0 && m == 0) {
            swap_scales(q, ps);
        } else if (kk == 1 || kk == 2) {
#pragma unroll
            for (int c = kPer * m; c < kPer * (m + 1); ++c)
                unpack_chunk(kk - 1, c, o);
        }
    };

    // D layout of a 32 x 32 tile: lane l, register r -> token 8 (r / 4) +
    // 4 (l / 32) + r % 4, row l % 32.  A whole tile is stored; a part of one
    // is added atomically (Y was zero-filled).  Tiles inside the matrix need
    // no bounds test.
    auto flush = [&](const Pos &ps, bool whole) {
        const int mb = ps.tm * T::BM + wm * 32 * TM + 4 * (lane >> 5);
        const int nb = ps.tn * T::BN + 32 * wn * TN + (lane & 31);
        const bool inside = (ps.tm + 1) * T::BM <= p.M && (ps.tn + 1) * T::BN <= p.N;   // uniform
        float *base = p.Y + (int64_t)mb * p.N + nb;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int dm = 32 * i + 8 * (r >> 2) + (r & 3);
                    const bool ok = inside || (mb + dm < p.M && nb + 32 * j < p.N);
                    float *dst = base + (int64_t)dm * p.N + 32 * j;
                    if (ok) {
                        if (whole)
                            *dst = acc[i][j][r];
                        else
                            unsafeAtomicAdd(dst, acc[i][j][r]);   // hardware fp32 add
                    }
                    acc[i][j][r] = 0.0f;
                }
    };

    // The first group's codes into this wave's LDS buffer (the wait for
    // them also covers the three activation copies issued before them), the
    // next group's loads issued, step 0's B operands unpacked.
    constexpr int nW = TN * (4 + (SA ? 1 : 8));   // loads of one weight group
    constexpr int kDmaGap = 4 * TM * TN / AC;      // MFMAs of a step per copy instruction
    static_assert(kDmaGap >= 2, "every copy instruction needs its own MFMA slot");
    store_w(wg);
    take_scales(wg, first);
    load_w<TN, SA>(wg, rs, lw);
    w_step<T::BN>(lw, p, S, it_end, KB, lane, wn);
    prep(0, first, 0);
    // every wave's copies of steps 0-2 have landed (only the next group's
    // loads may still be in flight), then a bare barrier: the fence of
    // __syncthreads would also wait for those loads; step 0's first two
    // k slices are read after it
    wait_vm<nW>();
    __builtin_amdgcn_s_barrier();
    read_a(0, 0, apre[0]);
    read_a(0, 1, apre[1]);

    // Step s (q = s - it0 within the group) multiplies the A operands of
    // buffer q (slices 0-1 already in registers) with B operands unpacked
    // during step s - 1; between its MFMAs it reads the next step's slices
    // 0-1, unpacks the next step's B operands and issues the copy of step s +
    // 3 into buffer (q + 3) % 4, which steps s - 2 (early reads) and s - 1
    // read.  After the last step of a group the next group's codes go to LDS
    // before the next step's codes are read, and the loads of the group after
    // it are issued after the MFMAs.  Before the barrier that ends the step
    // each wave waits for its part of step s + 2's copy (step s + 1 reads
    // that buffer early): younger than it are the copy of step s + 3 and the
    // weight group of whichever of steps s - 1 and s ended a group (none when
    // q = 1 or 2), a lower bound of what is in flight, so the wait is never
    // short.  The barrier is bare: the fence of __syncthreads would also wait
    // for the younger loads, and nothing else needs one (the buffer a copy
    // overwrites was last read by reads that fed MFMAs before the previous
    // barrier and so had returned; the weight codes in LDS are private to
    // each wave).  A tile is written out after its last group, or after the
    // workgroup's last group.
    Pos cur = first;
    int seg_s0 = first.s;   // first K step of the current tile segment
    for (int it0 = it_beg; it0 < it_end; it0 += DB) {
        const Pos group = cur;
#pragma unroll
        for (int q = 0; q < DB; ++q) {
            Pos nxt = cur;
            advance(nxt, p, S);
            if (q == DB - 1) {
                // the next group's codes to LDS and its scales, before the
                // next step's codes are read
                store_w(wg);
                take_scales(wg, nxt);
            }
            read_w((q + 1) % DB);
            mma(q, (q + 1) % DB, q & 1, [&](int kk, int m) {
                next_part((q + 1) % DB, nxt, (q + 1) & 1, kk, m);
                // the copy of step s + 3, one instruction every kDmaGap MFMAs
                const int g = kk * TM * TN + m;
#pragma unroll
                for (int i = 0; i < AC; ++i)
                    if (g == kDmaGap * i + 1)
                        dma_a_one<AC, NT>(abuf((q + 3) % DB), rs, la, KB, wave, i);
            });
            a_step<T::BM, AC, NT>(la, p, S, it_end);
            if (q == DB - 1) {
                // the loads of the group after it (clamped past the range: never used)
                load_w<TN, SA>(wg, rs, lw);
                w_step<T::BN>(lw, p, S, it_end, KB, lane, wn);
            }
            if (q == 1 || q == 2)
                wait_vm<AC>();
            else
                wait_vm<AC + nW>();
            cur = nxt;
            __builtin_amdgcn_s_barrier();
        }
        if (cur.s == 0 || it0 + DB == it_end) {
            flush(group, seg_s0 == 0 && cur.s == 0);
            seg_s0 = 0;
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

thread_local int o_wgs = 0, o_tile = 0;   // tuning override (0: built-in)

// Whether every workgroup's range of a stream-K split of `chunks` chunks
// (`per_tile` per tile) over `wgs` workgroups starts and ends on tile
// boundaries (then no tile is split).
bool whole_tiles(int64_t chunks, int64_t per_tile, int64_t wgs)
{
    for (int64_t g = 0; g <= wgs; ++g)
        if ((chunks * g / wgs) % per_tile != 0)
            return false;
    return true;
}

template <int WM, int TM, int TN, int OCC, int NW = 4>
hipError_t launch_prefill(PrefillParams p, int cus, hipStream_t stream)
{
    using T = Tiling<WM, TM, TN, NW>;
    const int64_t KB = p.K / 32;
    constexpr int DB = kGroup;
    const int64_t S = ((KB + 1) / 2 + DB - 1) / DB * DB;
    const int64_t tiles_n = (p.N + T::BN - 1) / T::BN;
    const int64_t tiles = tiles_n * ((p.M + T::BM - 1) / T::BM);
    if (tiles * S > INT32_MAX - 64)
        return hipErrorInvalidValue;
    p.tiles_n = (int)tiles_n;
    p.steps = (int)S;
    p.chunks = (int)(tiles * S / DB);
    // Workgroups (sweeps on MI355X, graph-timed calls on cycled copies): one
    // per tile, up to the OCC slots per CU, when the tiles fill at least
    // three quarters of the CUs: whole tiles need no zero-fill and no atomics
    // (64 x 128 tiles, 4096 x 4096 at 512 tokens: 256 workgroups 34.3 us
    // against 38.3 with the tiles split over 512; 128 x 128 tiles, 14336 x
    // 4096 at 256 tokens: 224 workgroups 45.8 against 60.0); with fewer
    // tiles the iterations are split over every slot when each gets at least
    // four groups (2560 x 6144 at 512 tokens, 64 x 128 tiles: 37.9 us
    // against 47.6 with one workgroup per tile), else over one workgroup per
    // CU (12288 x 2560 at 64 tokens: 21.3 us against 27.3 with two per CU).
    const int64_t slots = (int64_t)cus * OCC;
    int64_t wgs;
    if (tiles * 4 >= (int64_t)cus * 3)
        wgs = std::min(tiles, slots);
    else
        wgs = p.chunks >= 4 * slots ? slots : std::min<int64_t>(cus, p.chunks);
    if (o_wgs > 0)
        wgs = std::min<int64_t>(o_wgs, p.chunks);
    if (wgs > INT32_MAX)
        return hipErrorInvalidValue;
    if (!whole_tiles(p.chunks, S / DB, wgs)) {
        const hipError_t e = launch_zero_fill(p.Y, (int64_t)p.M * p.N, cus, stream);
        if (e != hipSuccess)
            return e;
    }
    // a group's eight scales as one 16-byte load where no group crosses a row
    // (nor the end of the scale region)
    const void *fn = KB % 8 == 0 ? reinterpret_cast<const void *>(&prefill_kernel<WM, TM, TN, OCC, true, NW>)
                                 : reinterpret_cast<const void *>(&prefill_kernel<WM, TM, TN, OCC, false, NW>);
    return launch_kernel(fn, dim3((unsigned)wgs), dim3(64 * NW), 0, stream, p);
}

}  // namespace
}  // namespace qg

namespace qg {
hipError_t launch_zero_fill(float *y, int64_t n, int cus, hipStream_t stream)
{
    FillParams f{y, n};
    void *a[] = {&f};
    const int64_t fw = std::min<int64_t>((n + 255) / 256, (int64_t)cus * 16);
    return hipLaunchKernel(reinterpret_cast<const void *>(&zero_fill_kernel), dim3((unsigned)fw), dim3(256), a, 0,
                           stream);
}
}  // namespace qg

extern "C" qg_status qgemm_q4_0_prefill(const void *Wp, const uint16_t *X, float *Y, int64_t M, int64_t N, int64_t K,
                                        void *stream)
{
    using namespace qg;
    if (!Wp || !X || !Y)
        return QG_ERR_NULL;
    // the kernel addresses X and the code region with 32-bit buffer offsets
    if (M < 1 || N < 1 || K < 32 || K % 32 != 0 || M * K * 2 > INT32_MAX - 256 || N * (K / 32) * 16 > INT32_MAX ||
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
    p.tiles_n = 0;
    p.steps = 0;
    p.chunks = 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // Up to 64 tokens the skinny kernel (qgemv_mfma.hip; MI355X, 64 tokens:
    // 12288 x 2560 18.1 against 21.8 us with 64 x 128 tiles, 6144 x 2048
    // 11.9 against 16.2, 2560 x 6144 13.2 against 17.8).  Beyond, the tile
    // (sweeps on MI355X, graph-timed calls): the largest of 128 tokens x 256
    // rows (eight waves; each activation copy serves 256 rows), 128 x 128
    // and 64 x 128 whose count fills three quarters to all of the CUs, each
    // tile then a workgroup of its own on a CU of its own (14336 x 4096 at
    // 256 tokens: 128 x 128 tiles 45.8 us against 51.9 with 448 of 64 x 128;
    // 12288 x 2560 at 128 tokens: 64 x 128 tiles 24.6 against 28.0 split over
    // 256 workgroups); else 128 x 256 where those tiles fill three quarters
    // of the CUs, 128 x 128 where they give every CU its two workgroups, and
    // 64 x 128 otherwise (one wave along M: no weight unpacked twice).
    const int64_t t136 = (M + 127) / 128 * ((N + 255) / 256);
    const int64_t t130 = (M + 127) / 128 * ((N + 127) / 128);
    const int64_t t64 = (M + 63) / 64 * ((N + 127) / 128);
    auto one_each = [&](int64_t t) { return 4 * t >= 3LL * cus && t <= cus; };
    const int tile = o_tile ? o_tile
                            : (M <= 64                   ? 16
                               : one_each(t136)          ? 136
                               : one_each(t130)          ? 130
                               : one_each(t64)           ? 64
                               : t136 * 4 >= 3LL * cus   ? 136
                               : t130 * 2 >= 3LL * cus   ? 130
                                                         : 64);
    hipError_t e;
    switch (tile) {
    case 16:
        e = launch_prefill_skinny(p.W, p.scale_offset, X, Y, (int)M, (int)N, (int)K, cus, o_wgs, s);
        break;
    case 64: e = launch_prefill<1, 2, 1, 2>(p, cus, s); break;
    case 66: e = launch_prefill<1, 2, 2, 2>(p, cus, s); break;
    case 128: e = launch_prefill<1, 4, 2, 1>(p, cus, s); break;
    case 130: e = launch_prefill<1, 4, 1, 2>(p, cus, s); break;
    case 257: e = launch_prefill<2, 4, 1, 1>(p, cus, s); break;
    case 136: e = launch_prefill<1, 4, 1, 1, 8>(p, cus, s); break;
    default: return QG_ERR_SHAPE;
    }
    if (e == hipErrorInvalidValue)
        return QG_ERR_SHAPE;
    return e == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
}

// Tuning knob for sweeps: fixes the number of persistent workgroups (the
// stream-K split) and the token tile (64, 128 or 256) of later
// qgemm_q4_0_prefill calls from the calling thread; 0 keeps the built-in
// choice.
extern "C" void qg_set_prefill_shape(int wgs, int tile)
{
    qg::o_wgs = wgs;
    qg::o_tile = tile;
}
