// Host quantizer / packer for the Q4_0, Q8_0 and q2w packed layouts of qgemv.h.
//
// Runs on the host, once per weight matrix, off the timed path: weights are
// quantized and uploaded once and stay resident on the device
// [H100-KERNEL-5X-ROADMAP, Lever 1].  The block rule (scale from the block's
// absmax, codes on the stored scale's grid) is stated in qgemv.h.
#include <cmath>
#include <cstdint>
#include <cstring>

#include "qgemv.h"

namespace {

constexpr size_t kAlign = 256;

inline size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

size_t packed_bytes(int64_t N, int64_t K, size_t code_bytes_per_block)
{
    if (N <= 0 || K <= 0 || K % 32 != 0)
        return 0;
    const size_t blocks = static_cast<size_t>(N) * static_cast<size_t>(K / 32);
    return round_up(round_up(blocks * code_bytes_per_block) + 2 * blocks);
}

// binary16 bits of the binary32 value `f`, round to nearest even.  The
// compiler's _Float16 conversion is IEEE-correct (subnormals kept).
inline uint16_t f32_to_f16_bits(float f)
{
    _Float16 h = static_cast<_Float16>(f);
    uint16_t bits;
    std::memcpy(&bits, &h, sizeof bits);
    return bits;
}

inline double f16_bits_to_f64(uint16_t bits)
{
    _Float16 h;
    std::memcpy(&h, &bits, sizeof h);
    return static_cast<double>(h);
}

// Quantize one row-major matrix.  kQmax = 7 (Q4_0) or 127 (Q8_0).
template <int kQmax, size_t kCodeBytes>
qg_status quantize(const float *w, int64_t N, int64_t K, void *packed, size_t nbytes)
{
    if (!w || !packed)
        return QG_ERR_NULL;
    const size_t need = packed_bytes(N, K, kCodeBytes);
    if (need == 0)
        return QG_ERR_SHAPE;
    if (nbytes < need)
        return QG_ERR_SIZE;
    auto *out = static_cast<uint8_t *>(packed);
    std::memset(out, 0, need);
    const int64_t kb = K / 32;
    const size_t blocks = static_cast<size_t>(N) * static_cast<size_t>(kb);
    uint8_t *scales = out + round_up(blocks * kCodeBytes);
    // Q4_0 stores round(w/d) + 8 clamped to [0, 15], i.e. multipliers -8..7
    constexpr int kLo = (kQmax == 7) ? -8 : -kQmax;
    qg_status st = QG_OK;

    for (size_t blk = 0; blk < blocks; ++blk) {
        const float *v = w + blk * 32;   // blocks are contiguous in a row-major matrix
        float amax = 0.0f;
        for (int k = 0; k < 32; ++k) {
            if (!std::isfinite(v[k]))
                st = QG_ERR_RANGE;
            amax = std::fmax(amax, std::fabs(v[k]));
        }
        const uint16_t dbits = f32_to_f16_bits(amax / static_cast<float>(kQmax));   // binary32 division
        if ((dbits & 0x7c00u) == 0x7c00u)
            st = QG_ERR_RANGE;
        const double d = f16_bits_to_f64(dbits);
        int mult[32];
        for (int k = 0; k < 32; ++k) {
            int m = 0;
            if (d != 0.0 && std::isfinite(d)) {
                double r = std::round(static_cast<double>(v[k]) / d);   // half away from zero
                r = std::fmin(std::fmax(r, static_cast<double>(kLo)), static_cast<double>(kQmax));
                m = static_cast<int>(r);
            }
            mult[k] = m;
        }
        if constexpr (kQmax == 7) {
            uint8_t *c = out + blk * 16;
            for (int j = 0; j < 16; ++j)
                c[j] = static_cast<uint8_t>((mult[j] + 8) | ((mult[j + 16] + 8) << 4));
        } else {
            int8_t *c = reinterpret_cast<int8_t *>(out + blk * 32);
            for (int k = 0; k < 32; ++k)
                c[k] = static_cast<int8_t>(mult[k]);
        }
        scales[2 * blk] = static_cast<uint8_t>(dbits & 0xffu);
        scales[2 * blk + 1] = static_cast<uint8_t>(dbits >> 8);
    }
    return st;
}

// Plain 2-bit (q2w): m = the block's weight of largest magnitude (the first
// on ties), scale fp16(m / -2), multipliers round(w / d) clamped to -2..1
// (half away from zero), stored as u = c + 2; byte j holds elements j, j + 8,
// j + 16, j + 24 in bits 0-1, 2-3, 4-5, 6-7.
qg_status quantize_q2w(const float *w, int64_t N, int64_t K, void *packed, size_t nbytes)
{
    if (!w || !packed)
        return QG_ERR_NULL;
    const size_t need = packed_bytes(N, K, 8);
    if (need == 0)
        return QG_ERR_SHAPE;
    if (nbytes < need)
        return QG_ERR_SIZE;
    auto *out = static_cast<uint8_t *>(packed);
    std::memset(out, 0, need);
    const size_t blocks = static_cast<size_t>(N) * static_cast<size_t>(K / 32);
    uint8_t *scales = out + round_up(blocks * 8);
    qg_status st = QG_OK;
    for (size_t blk = 0; blk < blocks; ++blk) {
        const float *v = w + blk * 32;
        float m = 0.0f;
        for (int k = 0; k < 32; ++k) {
            if (!std::isfinite(v[k]))
                st = QG_ERR_RANGE;
            if (std::fabs(v[k]) > std::fabs(m))
                m = v[k];
        }
        const uint16_t dbits = f32_to_f16_bits(m / -2.0f);   // binary32 division
        if ((dbits & 0x7c00u) == 0x7c00u)
            st = QG_ERR_RANGE;
        const double d = f16_bits_to_f64(dbits);
        uint8_t u[32];
        for (int k = 0; k < 32; ++k) {
            int c = 0;
            if (d != 0.0 && std::isfinite(d))
                c = static_cast<int>(std::fmin(std::fmax(std::round(static_cast<double>(v[k]) / d), -2.0), 1.0));
            u[k] = static_cast<uint8_t>(c + 2);
        }
        uint8_t *c = out + blk * 8;
        for (int j = 0; j < 8; ++j)
            c[j] = static_cast<uint8_t>(u[j] | (u[j + 8] << 2) | (u[j + 16] << 4) | (u[j + 24] << 6));
        scales[2 * blk] = static_cast<uint8_t>(dbits & 0xffu);
        scales[2 * blk + 1] = static_cast<uint8_t>(dbits >> 8);
    }
    return st;
}

}  // namespace

extern "C" {

size_t qpacked_bytes_q4_0(int64_t N, int64_t K) { return packed_bytes(N, K, 16); }
size_t qpacked_bytes_q8_0(int64_t N, int64_t K) { return packed_bytes(N, K, 32); }
size_t qpacked_bytes_q2w(int64_t N, int64_t K) { return packed_bytes(N, K, 8); }

qg_status qquantize_q2w(const float *w, int64_t N, int64_t K, void *packed, size_t packed_bytes)
{
    return quantize_q2w(w, N, K, packed, packed_bytes);
}

qg_status qquantize_q4_0(const float *w, int64_t N, int64_t K, void *packed, size_t packed_bytes)
{
    return quantize<7, 16>(w, N, K, packed, packed_bytes);
}

qg_status qquantize_q8_0(const float *w, int64_t N, int64_t K, void *packed, size_t packed_bytes)
{
    return quantize<127, 32>(w, N, K, packed, packed_bytes);
}

const char *qg_status_str(qg_status s)
{
    switch (s) {
    case QG_OK: return "ok";
    case QG_ERR_NULL: return "null pointer";
    case QG_ERR_SHAPE: return "shape out of range (N, K, M, E) or K % 32 != 0";
    case QG_ERR_ALIGN: return "misaligned pointer";
    case QG_ERR_RANGE: return "non-finite weight or scale overflows binary16";
    case QG_ERR_SIZE: return "buffer too small";
    case QG_ERR_LAUNCH: return "kernel launch failed";
    case QG_ERR_DEVICE: return "no usable HIP device";
    default: return "unknown status";
    }
}

}  // extern "C"
