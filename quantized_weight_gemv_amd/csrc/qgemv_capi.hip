// C-ABI entry points: host-side validation, per-shape launch choice and
// launches on the caller's stream.  Nothing here allocates device memory or
// synchronizes.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>

#include "qgemv.h"
#include "qgemv_tuning.h"
#include "qgemv_internal.h"

namespace qg {

// ---------------------------------------------------------------- timing hook

namespace {
thread_local hipEvent_t t_start = nullptr;
thread_local hipEvent_t t_stop = nullptr;
}  // namespace

hipError_t launch_raw(const void *fn, dim3 grid, dim3 block, void **args, size_t shmem, hipStream_t stream)
{
    if (t_start || t_stop) {
        hipEvent_t a = t_start, b = t_stop;
        t_start = t_stop = nullptr;
        return hipExtLaunchKernel(fn, grid, block, args, shmem, stream, a, b, 0);
    }
    return hipLaunchKernel(fn, grid, block, args, shmem, stream);
}

// ---------------------------------------------------------------- device info

namespace {
constexpr int kMaxDevices = 64;
int g_cus[kMaxDevices] = {0};
std::mutex g_mu;

int device_cus()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return 0;
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            return 0;
        g_cus[dev] = n;
    }
    return g_cus[dev];
}

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

inline size_t round256(size_t v) { return (v + 255) / 256 * 256; }

inline int64_t scale_offset(int fmt, int64_t N, int64_t K)
{
    return static_cast<int64_t>(round256(static_cast<size_t>(N) * static_cast<size_t>(K / 32) *
                                         static_cast<size_t>(code_bytes_per_block(fmt))));
}

// Launch shape for one GEMV / MoE call.
struct GemvShape {
    int G, J, R, ksplit, teams_per_wg;
    int64_t teams;   // teams per batch item
    bool xl;         // one token: activations staged in LDS, not registers
};

// Caller-set override for tuning sweeps (thread-local, zeros = heuristic).
thread_local int o_G = 0, o_J = 0, o_R = 0, o_ksplit = 0, o_teams_per_wg = 0, o_xl = -1, o_engine = -1;
thread_local int64_t o_teams = 0;

bool choose_shape(int fmt, int M, int64_t N, int64_t K, int items, int cus, int mode, GemvShape &s)
{
    const bool glu = mode == kModeGlu;
    const int64_t KB = K / 32;
    // Activations staged in LDS once per workgroup of 8 teams (XL, whole rows
    // per wave): the default for fp32 activations on tables of at least four
    // groups per CU (one-token GEMV: beyond 8192 rows), where every team's own
    // register copy would read 4 M K bytes (up to ~10x the weight bytes at
    // four tokens).  Launch sweeps on MI355X: one token 14336 x 4096 8.1
    // against 10.6 us, four tokens 6144 x 2048 7.3 against 10.4; SwiGLU
    // 14336 x 4096 13.9 against 16.5 at one token, 25.5 against 32.5 at four.
    // With fp16 activations (half the bytes), on smaller tables and at one
    // token up to 8192 rows (4096 x 4096: 5.0 against 4.6 us with 16 lanes per
    // row) the register copy stays faster.
    // 8-bit activations are quantized into LDS: always XL; two row sets per
    // group for one token on tables of 8192 rows and more (rows of at most
    // 256 blocks), one otherwise (launch sweeps on MI355X: 28672 x 4096
    // 11.8 against 12.3 us; 2048 x 6144 at four tokens 6.6 against 7.2).
    bool xl = false;
    int xl_r = glu ? 2 : (M == 1 ? 1 : 2);
    if (mode == kModeQ8Act)
        xl_r = (M == 1 && N >= 8192 && (KB + 63) / 64 <= 4) ? 2 : 1;
    if (o_xl >= 0)
        xl = (o_xl == 1);
    else if (mode == kModeQ8Act)
        xl = true;
    else if (mode != kModeF16 && items == 1)
        xl = (KB + 63) / 64 * xl_r <= 8 && gemv_xl_lds_bytes(static_cast<int>(K), M, mode) <= 65536 &&
             N / (glu ? 1 : xl_r) >= 4LL * cus && (M > 1 || glu || N > 8192);
    const bool xl_auto = xl && o_xl < 0;
    // Lanes per row: one token with rows of 65..128 blocks spreads a row over
    // 16 (up to 4096 rows) or 32 lanes (up to 64K rows; Q4_0 GEMV: up to 8192),
    // so a wave reduces several rows at once; shorter rows take one wave each.
    // (q2w follows the Q4_0 one-token rules: launch sweeps on MI355X,
    // 14336 x 4096 7.2 against 8.1 us, 4096 x 14336 7.6 against 9.3)
    const bool q4_one = (fmt == kQ4_0 || fmt == kQ2W) && M == 1 && items == 1 && !xl;
    int G = 64;
    if (M == 1 && !xl && KB > 64 && KB <= 128) {
        if (N <= 4096 && N >= 4)
            G = 16;
        else if (N <= (q4_one ? 8192 : 65536) && N >= 2)
            G = 32;
    }
    if (o_G)
        G = o_G;
    if (G != 16 && G != 32 && G != 64)
        return false;
    const int P = 64 / G;
    if (N < P)
        return false;
    // One block per lane per row, K split over up to 8 waves; longer rows
    // take more blocks per lane (with XL: one wave per row).
    int J = static_cast<int>(std::max<int64_t>(1, (KB + 8LL * G - 1) / (8LL * G)));
    if (xl)
        J = static_cast<int>((KB + G - 1) / G);
    // Two to four tokens: two blocks per lane where that halves the waves
    // along K without leaving half of the last wave idle (rows a multiple of
    // 128 blocks, or longer than 384).  Measured on MI355X, Q4_0 at two
    // tokens: 4096 x 4096 4.6 against 5.0 us, 14336 x 4096 8.7 against
    // 10.7 us; 2048 x 6144 (192 blocks) stays faster with one block per lane.
    if (M >= 2 && M <= 4 && !xl && J == 1 && KB > 64 && (KB % 128 == 0 || KB > 384))
        J = 2;
    // One token, Q4_0, full-wave rows: a whole row per wave, no K split and
    // no cross-wave reduction (two blocks per lane for 65..128 blocks, up to
    // seven for 257..448).  Timed as back-to-back graph replay on MI355X:
    // 28672 x 4096 12.4 against 13.5 us with K split over four waves,
    // 14336 x 4096 7.6 against 8.0, 4096 x 14336 7.95 against 8.6,
    // 128256 x 4096 45.1 against 46.9.
    if (q4_one && o_G == 0 && G == 64 && ((KB > 64 && KB <= 128) || (KB > 256 && KB <= 448)))
        J = static_cast<int>((KB + 63) / 64);
    int ksplit = static_cast<int>((KB + static_cast<int64_t>(G) * J - 1) / (static_cast<int64_t>(G) * J));
    const int rj = (fmt == kQ8_0) ? 4 : 8;   // R * J budget of the kernel table
    // Two row sets per group, four for full-wave rows beyond 64K rows, and
    // four for several tokens with K split over waves (launch sweeps on
    // MI355X, 256 CUs: Q4_0 2048 x 6144 at six tokens 7.9 against 8.5 us).
    // Q8_0 holds twice the code registers per row set: there four pay only
    // where one group per team then covers all rows (Q8_0 4096 x 14336 at
    // six tokens: 26.0 us with four, 25.2 with two).
    int R = (N > 65536 && G == 64) ? 4 : 2;
    if (q4_one && G == 16)
        R = 4;   // 4096 x 4096: 3.95 against 4.10 us back to back
    if (glu)
        R = 2;   // SwiGLU: one gate and one up row set per group
    if (M >= 2 && J == 1 && ksplit > 1 && !glu &&
        (fmt != kQ8_0 || N <= 4LL * cus * std::max(2, 8 / ksplit)))
        R = 4;
    if (xl_auto)
        R = xl_r;   // one row set per group at one token, two at 2-4 tokens
    while (R * J > rj && R > (glu ? 2 : 1))
        R /= 2;
    // stay within the instantiated kernels (register budget): fewer row sets,
    // then more waves along K
    while (R > (glu ? 2 : 1) && !gemv_fits(fmt, M, G, J, R, xl, mode))
        R /= 2;
    while (glu && R * J > rj && J > 1) {
        --J;
        ksplit = static_cast<int>((KB + static_cast<int64_t>(G) * J - 1) / (static_cast<int64_t>(G) * J));
    }
    while (!xl && !gemv_fits(fmt, M, G, J, R, xl, mode) && ksplit < kMaxWavesPerWg && J > 1) {
        --J;
        ksplit = static_cast<int>((KB + static_cast<int64_t>(G) * J - 1) / (static_cast<int64_t>(G) * J));
    }
    if (ksplit > kMaxWavesPerWg)
        return false;
    int teams_per_wg = xl_auto ? 8 : 1;
    if (o_J) {
        J = o_J;
        ksplit = static_cast<int>((KB + static_cast<int64_t>(G) * J - 1) / (static_cast<int64_t>(G) * J));
        if (ksplit > kMaxWavesPerWg)
            return false;
    }
    if (o_ksplit) {
        ksplit = o_ksplit;
        if (static_cast<int64_t>(ksplit) * G * J < KB || ksplit > kMaxWavesPerWg)
            return false;
    }
    if (o_R && !glu)
        R = o_R;
    if (o_teams_per_wg)
        teams_per_wg = o_teams_per_wg;
    if (xl && (ksplit > 1 || M > 4 || gemv_xl_lds_bytes(static_cast<int>(K), M, mode) > 65536))
        return false;
    if (!gemv_fits(fmt, M, G, J, R, xl, mode))
        return false;
    if (ksplit > 1)
        teams_per_wg = 1;   // a workgroup's waves must walk the same row groups
    if (teams_per_wg * ksplit > kMaxWavesPerWg)
        teams_per_wg = std::max(1, kMaxWavesPerWg / ksplit);
    const int64_t rows_per_group = glu ? P : static_cast<int64_t>(R) * P;   // output rows per group
    const int64_t ngroups = (N + rows_per_group - 1) / rows_per_group;
    // Teams per CU (launch sweeps on MI355X): 8 for one-wave rows; with K
    // split, about 16 waves per CU for one token and 8 for several; beyond
    // 64K rows 64 teams per CU, more than fit at once (the hardware
    // dispatcher then balances the tail).
    int per_cu = (ksplit == 1) ? 8 : (M == 1 ? std::max(4, 16 / ksplit) : std::max(2, 8 / ksplit));
    if (M == 1 && ksplit == 1 && J > 2)
        per_cu = 4;   // long whole rows per wave: 4096 x 14336 7.95 us at 4, 8.9 at 8
    if (N > 65536 && M == 1)
        per_cu = fmt == kQ2W ? 32 : 64;   // q2w 128256 x 4096: 39.6 against 42.4 us
    if (xl_auto)
        per_cu = (M == 1 && !glu) || (glu && KB <= 64) ? 16 : 8;
    if (xl_auto && mode == kModeQ8Act)
        per_cu = (KB + 63) / 64 > 4 ? 8 : 16;   // 4096 x 14336: 8.6 against 9.2 us
    int64_t teams = std::max<int64_t>(1, static_cast<int64_t>(cus) * per_cu / std::max(1, items));
    // Several tokens, two blocks per lane, whole rows per wave: at least two
    // groups per team, so the prefetch of the next group overlaps the current
    // one (4096 x 4096 at two tokens: 1024 teams 4.6 us, 2048 teams 5.1;
    // with one block per lane, 6144 x 2048 prefers 2048 teams, 4.1 against
    // 4.6 us).
    if (M >= 2 && J >= 2 && ksplit == 1 && items == 1 && !xl)
        teams = std::min(teams, std::max<int64_t>(1, (ngroups + 1) / 2));
    if (o_teams)
        teams = o_teams;
    teams = std::min(teams, ngroups);
    s = GemvShape{G, J, R, ksplit, teams_per_wg, teams, xl};
    return true;
}

qg_status run_gemv(int fmt, const void *Wp, const int32_t *idx, int64_t P, const uint16_t *x, float *y, int M,
                   int items, int64_t N, int64_t K, void *stream, int mode = kModeF16, const float *xf = nullptr)
{
    const void *xa = (mode == kModeF16 || mode == kModeQ8Act) ? static_cast<const void *>(x)
                                                               : static_cast<const void *>(xf);
    if (!Wp || !xa || !y)
        return QG_ERR_NULL;
    const int64_t nmax = (mode == kModeGlu) ? INT32_MAX / 2 : INT32_MAX;   // SwiGLU reads 2N rows
    // fp32 activations and SwiGLU: up to 4 tokens on the vector kernel (their
    // raw words stay in registers until converted), 5-8 on the matrix-core
    // kernel; 8-bit activations: up to 4 tokens (the LDS copy)
    const int mmax = (mode == kModeQ8Act) ? 4 : 8;
    if (M < 1 || M > mmax || N < 1 || N > nmax || K < 32 || K % 32 != 0 || K > (1 << 20) || items < 1 ||
        items > 65535)
        return QG_ERR_SHAPE;
    if (!aligned(Wp, 256) || !aligned(xa, 16) || !aligned(y, 4))
        return QG_ERR_ALIGN;
    const int cus = device_cus();
    if (cus <= 0)
        return QG_ERR_DEVICE;
    // Several tokens on short rows (plain GEMV): the matrix-core kernel,
    // whose unpack cost per block does not grow with M.  It wants at least
    // one 16-row tile per CU; the vector kernel stays faster below four
    // tokens, and for Q8_0 (whose vector unpack is cheaper) below six on rows
    // of 128-256 blocks.  Measured on MI355X: Q4_0 8192 x 2048 at 4 tokens 5.5
    // against 6.3 us, at 8 tokens 5.9 against 9.6; 4096 x 8192 at 6 tokens
    // 10.5 against 12.9; Q8_0 14336 x 4096 at 4 tokens 19.0 against 16.3, at
    // 8 tokens 19.9 against 25.0; Q8_0 4096 x 8192 at 6 / 8 tokens 12.6 / 13.1
    // against 14.8 / 17.5; q2w 14336 x 4096 at 4 tokens 10.6 against
    // 13.2, at 8 tokens 11.3 against 23.6, at 2 tokens 10.5 against 9.2.
    // With 2048 rows half the chip idles and only Q4_0 at 8 tokens and q2w
    // from 6 tokens gain (2048 x 6144: Q4_0 9.0 against 9.6 us; q2w 7.8
    // against 7.9 at 6 tokens, 8.0 against 9.7 at 8, 7.4 against 6.2 at 4).
    // q2w needs an even number of blocks per row (its scales are loaded per
    // lane group, 4-byte aligned).  fp32 activations (Q4_0) and SwiGLU
    // follow the Q4_0 rule (N: the rows of one half for SwiGLU; 4 tokens,
    // SwiGLU 2 x 14336 x 4096 23.5 against 26.3 us, 2 x 6144 x 2048 9.6
    // against 10.6, 2 x 4096 x 4096 9.9 against 12.2; 2 x 2048 x 6144 16.0
    // against 11.5 stays on the vector kernel), and take the matrix-core
    // kernel at 5-8 tokens whatever the shape (it rounds them to binary16 as
    // it stages them; the vector kernel holds at most 4 tokens of raw fp32
    // words).
    const int64_t KB = K / 32;
    const bool tiles_fill = N >= 16LL * cus;
    const bool f32_many = (mode == kModeF32 || mode == kModeGlu) && M > 4;
    bool mfma = idx == nullptr && (mode == kModeF16 || mode == kModeF32 || mode == kModeGlu) &&
                (f32_many || (tiles_fill && fmt == kQ4_0 && M >= 4 && KB <= 256) ||
                 (tiles_fill && fmt == kQ8_0 && ((M >= 4 && KB <= 64) || (M >= 6 && KB <= 256))) ||
                 (N >= 8LL * cus && fmt == kQ4_0 && M == 8 && KB <= 256) ||
                 (fmt == kQ2W && KB % 2 == 0 && KB <= 256 &&
                  ((tiles_fill && M >= 4) || (N >= 8LL * cus && M >= 6))));
    if (o_engine >= 0)
        mfma = (o_engine == 1);
    if (f32_many && !mfma)
        return QG_ERR_SHAPE;   // fp32 activations beyond 4 tokens: the matrix-core kernel only
    if (mfma && (!(mode == kModeF16 || ((mode == kModeF32 || mode == kModeGlu) && fmt == kQ4_0)) ||
                 (fmt == kQ2W && KB % 2 != 0)))
        return QG_ERR_SHAPE;   // the matrix-core kernel: fp16 activations, or fp32 (and SwiGLU) with Q4_0;
                               // q2w rows of an even block count
    if (mfma) {
        if (idx != nullptr || KB > 256 || N > INT32_MAX)
            return QG_ERR_SHAPE;
        // about 16 blocks per wave (sweeps: 4 waves for K = 2048, 8 for 4096)
        int waves = static_cast<int>(std::min<int64_t>(8, std::max<int64_t>(1, (KB + 15) / 16)));
        if (o_ksplit)
            waves = o_ksplit;
        const bool f32 = mode == kModeF32 || mode == kModeGlu;
        const bool glu = mode == kModeGlu;   // the packed table holds 2N rows (gate, then up)
        hipError_t e = launch_gemv_mfma(fmt, static_cast<const uint8_t *>(Wp), scale_offset(fmt, glu ? 2 * N : N, K),
                                        f32 ? nullptr : x, f32 ? xf : nullptr, y, M, static_cast<int>(N),
                                        static_cast<int>(K), waves, o_teams_per_wg, o_teams, cus,
                                        static_cast<hipStream_t>(stream), glu);
        if (e == hipErrorInvalidValue)
            return QG_ERR_SHAPE;
        return e == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
    }
    GemvShape s;
    if (!choose_shape(fmt, M, N, K, items, cus, mode, s))
        return QG_ERR_SHAPE;
    const int64_t rows = (mode == kModeGlu) ? 2 * N : N;   // rows of the packed table
    GemvParams p;
    p.W = static_cast<const uint8_t *>(Wp);
    p.idx = idx;
    p.x = x;
    p.xf = xf;
    p.y = y;
    p.matrix_stride = static_cast<int64_t>(fmt == kQ4_0   ? qpacked_bytes_q4_0(rows, K)
                                           : fmt == kQ2W ? qpacked_bytes_q2w(rows, K)
                                                         : qpacked_bytes_q8_0(rows, K));
    p.scale_offset = scale_offset(fmt, rows, K);
    p.N = static_cast<int>(N);
    p.K = static_cast<int>(K);
    p.ksplit = s.ksplit;
    p.teams_per_wg = s.teams_per_wg;
    p.pool = P;
    const int64_t wgs = (s.teams + s.teams_per_wg - 1) / s.teams_per_wg;
    dim3 grid(static_cast<unsigned>(wgs), static_cast<unsigned>(items), 1);
    dim3 block(64 * s.ksplit * s.teams_per_wg, 1, 1);
    hipError_t e = launch_gemv(fmt, M, s.G, s.J, s.R, s.xl, mode, p, grid, block, static_cast<hipStream_t>(stream));
    if (e == hipErrorInvalidValue)
        return QG_ERR_SHAPE;
    return e == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
}

// ---------------------------------------------------------------- dequant

// One thread per block of 32 weights: the exact (q - 8) * d (q * d, c * d) in
// fp32, or that value rounded to nearest-even binary16.
template <int FMT, bool F16>
__device__ __forceinline__ void dequant_kernel(const uint8_t *__restrict__ W, int64_t blocks,
                                                      int64_t scale_off, void *__restrict__ out)
{
    const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= blocks)
        return;
    const float d = (float)__builtin_bit_cast(_Float16, reinterpret_cast<const uint16_t *>(W + scale_off)[b]);
    float v[32];
    if constexpr (FMT == kQ4_0) {
        const uint4 c = reinterpret_cast<const uint4 *>(W)[b];
        const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const uint32_t byte = (w[j >> 2] >> (8 * (j & 3))) & 0xFFu;
            v[j] = (float)((int)(byte & 0xFu) - 8) * d;
            v[j + 16] = (float)((int)(byte >> 4) - 8) * d;
        }
    } else if constexpr (FMT == kQ2W) {
        // c * d is exact in binary16 too; with fp16 output it is formed there
        // (an fp32 product rounded to fp16 is fused by the compiler into
        // fma(c, d, +0), which turns 0 * (negative d) into +0 instead of -0)
        const uint2 c = reinterpret_cast<const uint2 *>(W)[b];
        const _Float16 dh = __builtin_bit_cast(_Float16, reinterpret_cast<const uint16_t *>(W + scale_off)[b]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t byte = ((j < 4 ? c.x : c.y) >> (8 * (j & 3))) & 0xFFu;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int cc = (int)((byte >> (2 * r)) & 3u) - 2;
                if constexpr (F16)
                    v[j + 8 * r] = (float)((_Float16)cc * dh);
                else
                    v[j + 8 * r] = (float)cc * d;
            }
        }
    } else {
        const uint4 *c = reinterpret_cast<const uint4 *>(W + b * 32);
        const uint4 c0 = c[0], c1 = c[1];
        const uint32_t w[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
        for (int j = 0; j < 32; ++j)
            v[j] = (float)(int8_t)((w[j >> 2] >> (8 * (j & 3))) & 0xFFu) * d;
    }
    if constexpr (F16) {
        uint4 *o = reinterpret_cast<uint4 *>(static_cast<uint16_t *>(out) + b * 32);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t u[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint16_t lo = __builtin_bit_cast(uint16_t, (_Float16)v[8 * q + 2 * t]);
                const uint16_t hi = __builtin_bit_cast(uint16_t, (_Float16)v[8 * q + 2 * t + 1]);
                u[t] = (uint32_t)lo | ((uint32_t)hi << 16);
            }
            o[q] = make_uint4(u[0], u[1], u[2], u[3]);
        }
    } else {
        float4 *o = reinterpret_cast<float4 *>(static_cast<float *>(out) + b * 32);
#pragma unroll
        for (int q = 0; q < 8; ++q)
            o[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    }
}

struct DequantArgs {
    const uint8_t *W;
    int64_t blocks;
    int64_t scale_off;
    void *out;
};

template <int FMT, bool F16>
__global__ __launch_bounds__(256) void dequant_entry(DequantArgs a)
{
    dequant_kernel<FMT, F16>(a.W, a.blocks, a.scale_off, a.out);
}

qg_status run_dequant(int fmt, const void *Wp, int64_t N, int64_t K, int out_fp16, void *out, void *stream)
{
    if (!Wp || !out)
        return QG_ERR_NULL;
    if (N < 1 || K < 32 || K % 32 != 0)
        return QG_ERR_SHAPE;
    if (!aligned(Wp, 256) || !aligned(out, 16))
        return QG_ERR_ALIGN;
    DequantArgs a{static_cast<const uint8_t *>(Wp), N * (K / 32), scale_offset(fmt, N, K), out};
    const int64_t wgs = (a.blocks + 255) / 256;
    if (wgs > INT32_MAX)
        return QG_ERR_SHAPE;
    const void *fn;
    if (fmt == kQ4_0)
        fn = out_fp16 ? reinterpret_cast<const void *>(&dequant_entry<kQ4_0, true>)
                      : reinterpret_cast<const void *>(&dequant_entry<kQ4_0, false>);
    else if (fmt == kQ2W)
        fn = out_fp16 ? reinterpret_cast<const void *>(&dequant_entry<kQ2W, true>)
                      : reinterpret_cast<const void *>(&dequant_entry<kQ2W, false>);
    else
        fn = out_fp16 ? reinterpret_cast<const void *>(&dequant_entry<kQ8_0, true>)
                      : reinterpret_cast<const void *>(&dequant_entry<kQ8_0, false>);
    hipError_t e = launch_kernel(fn, dim3(static_cast<unsigned>(wgs)), dim3(256), 0,
                                 static_cast<hipStream_t>(stream), a);
    return e == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
}

}  // namespace
}  // namespace qg

extern "C" {

qg_status qgemv_q4_0(const void *Wp, const uint16_t *x, float *y, int M, int64_t N, int64_t K, void *stream)
{
    return qg::run_gemv(qg::kQ4_0, Wp, nullptr, 1, x, y, M, 1, N, K, stream);
}

qg_status qgemv_q8_0(const void *Wp, const uint16_t *x, float *y, int M, int64_t N, int64_t K, void *stream)
{
    return qg::run_gemv(qg::kQ8_0, Wp, nullptr, 1, x, y, M, 1, N, K, stream);
}

qg_status qgemv_q4_0_f32in(const void *Wp, const float *x, float *y, int M, int64_t N, int64_t K, void *stream)
{
    return qg::run_gemv(qg::kQ4_0, Wp, nullptr, 1, nullptr, y, M, 1, N, K, stream, qg::kModeF32, x);
}

qg_status qgemv_q4_0_swiglu_f32in(const void *Wp, const float *x, float *y, int M, int64_t N, int64_t K,
                                  void *stream)
{
    return qg::run_gemv(qg::kQ4_0, Wp, nullptr, 1, nullptr, y, M, 1, N, K, stream, qg::kModeGlu, x);
}

qg_status qgemv_q4_0_q8act(const void *Wp, const uint16_t *x, float *y, int M, int64_t N, int64_t K, void *stream)
{
    return qg::run_gemv(qg::kQ4_0, Wp, nullptr, 1, x, y, M, 1, N, K, stream, qg::kModeQ8Act);
}

qg_status qgemv_q2w(const void *Wp, const uint16_t *x, float *y, int M, int64_t N, int64_t K, void *stream)
{
    return qg::run_gemv(qg::kQ2W, Wp, nullptr, 1, x, y, M, 1, N, K, stream);
}

qg_status qgemv_q2w_q8act(const void *Wp, const uint16_t *x, float *y, int M, int64_t N, int64_t K, void *stream)
{
    return qg::run_gemv(qg::kQ2W, Wp, nullptr, 1, x, y, M, 1, N, K, stream, qg::kModeQ8Act);
}

qg_status qgemv_q2w_lut(const void *Wp, const uint16_t *x, float *y, int64_t N, int64_t K, void *stream)
{
    if (!Wp || !x || !y)
        return QG_ERR_NULL;
    if (N < 1 || N > INT32_MAX || K < 32 || K % 32 != 0 || qg::gemv_lut_lds_bytes(static_cast<int>(std::min<int64_t>(K, 1 << 20))) > 65536)
        return QG_ERR_SHAPE;
    if (!qg::aligned(Wp, 256) || !qg::aligned(x, 16) || !qg::aligned(y, 4))
        return QG_ERR_ALIGN;
    const int cus = qg::device_cus();
    if (cus <= 0)
        return QG_ERR_DEVICE;
    hipError_t e = qg::launch_gemv_q2w_lut(static_cast<const uint8_t *>(Wp), qg::scale_offset(qg::kQ2W, N, K), x, y,
                                           static_cast<int>(N), static_cast<int>(K), cus,
                                           static_cast<hipStream_t>(stream));
    if (e == hipErrorInvalidValue)
        return QG_ERR_SHAPE;
    return e == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
}

qg_status qdequant_q2w(const void *Wp, int64_t N, int64_t K, int out_fp16, void *out, void *stream)
{
    return qg::run_dequant(qg::kQ2W, Wp, N, K, out_fp16, out, stream);
}

qg_status qmoe_gemv_q4_0(const void *pool, int64_t P, const int32_t *idx, const uint16_t *x, float *y, int E,
                         int64_t N, int64_t K, void *stream)
{
    if (!idx)
        return QG_ERR_NULL;
    if (P < 1 || E < 1)
        return QG_ERR_SHAPE;
    if (!qg::aligned(idx, 4))
        return QG_ERR_ALIGN;
    return qg::run_gemv(qg::kQ4_0, pool, idx, P, x, y, 1, E, N, K, stream);
}

qg_status qdequant_q4_0(const void *Wp, int64_t N, int64_t K, int out_fp16, void *out, void *stream)
{
    return qg::run_dequant(qg::kQ4_0, Wp, N, K, out_fp16, out, stream);
}

qg_status qdequant_q8_0(const void *Wp, int64_t N, int64_t K, int out_fp16, void *out, void *stream)
{
    return qg::run_dequant(qg::kQ8_0, Wp, N, K, out_fp16, out, stream);
}

void qg_time_next_launch(void *start, void *stop)
{
    qg::t_start = static_cast<hipEvent_t>(start);
    qg::t_stop = static_cast<hipEvent_t>(stop);
}

qg_status qg_device_cus(int device, int *cus)
{
    if (!cus)
        return QG_ERR_NULL;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || n <= 0)
        return QG_ERR_DEVICE;
    *cus = n;
    return QG_OK;
}

// Tuning knob for launch-shape sweeps: fixes J (blocks per lane), R (row sets
// per group), ksplit (waves along K), teams per workgroup, total teams, the
// activation staging (xl: -1 built-in, 0 registers, 1 LDS), the engine (-1
// built-in, 0 vector ALU, 1 matrix cores; with the matrix cores ksplit is the
// number of waves along K) and the lanes per row (16, 32 or 64) for the GEMV /
// MoE calls made afterwards from the calling thread.  Zero keeps the built-in
// choice for the other fields.
void qg_set_gemv_shape(int J, int R, int ksplit, int teams_per_wg, int64_t teams, int xl, int engine,
                       int lanes_per_row)
{
    qg::o_xl = xl;
    qg::o_engine = engine;
    qg::o_J = J;
    qg::o_R = R;
    qg::o_ksplit = ksplit;
    qg::o_teams_per_wg = teams_per_wg;
    qg::o_teams = teams;
    qg::o_G = lanes_per_row;
}

}  // extern "C"

// ---------------------------------------------------------------- HBM probe

namespace qg {
namespace {

struct ProbeArgs {
    const uint8_t *p;
    int64_t bytes;     // multiple of 16
    uint32_t *sink;    // >= gridDim.x words
    uint32_t never;    // a fold the data does not produce (the write below keeps the loads live)
};

// Streaming read on the GEMV kernels' own load path: non-temporal 16-byte
// buffer loads from a scalar descriptor.  The buffer is cut into tiles of
// U x 4 KiB handed round-robin to the workgroups (consecutive workgroups read
// consecutive tiles, as consecutive GEMV teams read consecutive rows); each
// lane has U loads of a tile in flight, and those of its next tile are
// issued before the current one is folded (two register sets, as the GEMV
// keeps two groups).  Loads past the end of the buffer fall outside the
// tile's descriptor (or meet an empty one) and return zeros without
// touching memory.  Nothing is reduced across the workgroup: a lane stores
// its fold only if it equals `never`, so the loads cannot be dropped and the
// launch ends with its last load.  [sm8x-bench, methodology: a bandwidth
// probe gives the measured roofline beside the spec]
template <int U>
__device__ __forceinline__ void probe_tile(const ProbeArgs &a, int64_t t, int64_t ntiles, uint4 (&v)[U])
{
    constexpr int64_t kTile = (int64_t)U * 256 * 16;
    const int64_t base = t * kTile;
    const auto r = t < ntiles ? make_rsrc(a.p + base, min(kTile, a.bytes - base)) : make_rsrc(a.p, 0);
#pragma unroll
    for (int u = 0; u < U; ++u)
        v[u] = stream_load16(r, (uint32_t)(threadIdx.x + u * 256) * 16u);
}

template <int U>
__device__ __forceinline__ uint32_t probe_fold(const uint4 (&v)[U])
{
    uint32_t x = 0;
#pragma unroll
    for (int u = 0; u < U; ++u)
        x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    return x;
}

template <int U>
__global__ __launch_bounds__(256) void read_probe_kernel(ProbeArgs a)
{
    constexpr int64_t kTile = (int64_t)U * 256 * 16;
    const int64_t ntiles = (a.bytes + kTile - 1) / kTile;
    const int64_t step = gridDim.x;
    uint32_t acc = 0;
    uint4 va[U], vb[U];
    int64_t t = blockIdx.x;
    probe_tile<U>(a, t, ntiles, va);
    for (;;) {
        probe_tile<U>(a, t + step, ntiles, vb);
        __builtin_amdgcn_sched_barrier(0);   // the next tile's loads stay ahead of the fold
        acc ^= probe_fold<U>(va);
        if (t + step >= ntiles)
            break;
        probe_tile<U>(a, t + 2 * step, ntiles, va);
        __builtin_amdgcn_sched_barrier(0);
        acc ^= probe_fold<U>(vb);
        if (t + 2 * step >= ntiles)
            break;
        t += 2 * step;
    }
    if (acc == a.never)
        a.sink[blockIdx.x] = acc;
}

}  // namespace
}  // namespace qg

extern "C" qg_status qg_read_probe(const void *buf, size_t bytes, uint32_t *sink, int wgs, int loads, void *stream)
{
    if (!buf || !sink)
        return QG_ERR_NULL;
    if (bytes < 16 || wgs < 1 || bytes > ((size_t)1 << 40))
        return QG_ERR_SHAPE;
    if (!qg::aligned(buf, 16) || !qg::aligned(sink, 4))
        return QG_ERR_ALIGN;
    const void *fn;
    switch (loads) {
    case 2: fn = reinterpret_cast<const void *>(&qg::read_probe_kernel<2>); break;
    case 4: fn = reinterpret_cast<const void *>(&qg::read_probe_kernel<4>); break;
    case 8: fn = reinterpret_cast<const void *>(&qg::read_probe_kernel<8>); break;
    case 16: fn = reinterpret_cast<const void *>(&qg::read_probe_kernel<16>); break;
    default: return QG_ERR_SHAPE;
    }
    qg::ProbeArgs a{static_cast<const uint8_t *>(buf), static_cast<int64_t>(bytes / 16 * 16), sink, 0x9E3779B9u};
    hipError_t e = qg::launch_kernel(fn, dim3(wgs), dim3(256), 0, static_cast<hipStream_t>(stream), a);
    return e == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
}
