/*
 * qgemv.h -- C ABI of a gfx950 (MI355X) library for the fused
 * dequantize-and-multiply of block-quantized LLM weights.
 *
 * Formats (32 weights per block, one binary16 scale d per block):
 *   Q4_0  4-bit codes q in 0..15, weight = (q - 8) * d.  Within a block's 16
 *         code bytes, byte j holds element j in its low nibble and element
 *         j + 16 in its high nibble (GGUF Q4_0, group size 32)
 *         [sm8x-bench, the Q4_0 table and "our kernel";
 *          volta-kernel-bakeoff, "What's in the race"].
 *   Q8_0  int8 codes q (two's complement), weight = q * d
 *         [H100-KERNEL-5X-ROADMAP, Lever 1: int8 codes plus a per-block
 *          scale; the scale is binary16 here].
 *   q2w   plain 2-bit codes c in -2..1 stored as u = c + 2, weight = c * d;
 *         byte j of a block's 8 code bytes holds elements j, j + 8, j + 16,
 *         j + 24 in bits 0-1, 2-3, 4-5, 6-7 (2.5 bits per weight)
 *         [volta-kernel-bakeoff, "What's in the race": q2w, codes -2..1,
 *          one fp16 scale per 32].
 *
 * Packed buffer of one N x K matrix (row-major weights, K % 32 == 0, blocks
 * along K, block index i = n * (K/32) + b):
 *   codes   at byte 0: 16 B (Q4_0), 32 B (Q8_0) or 8 B (q2w) per block,
 *           block i at byte 16 i (32 i, 8 i).
 *   scales  binary16 little-endian, scale i at byte S0 + 2 i, where S0 is the
 *           code-region size rounded up to a multiple of 256.
 *   total   (S0 + 2 N K / 32) rounded up to a multiple of 256, so packed
 *           matrices can be laid end to end (an MoE expert pool) and stay
 *           256-byte aligned.
 *
 * Conventions for every entry point:
 *   - Device pointers are caller-owned device memory; the library allocates
 *     no device memory and keeps no state between calls (the launch-shape
 *     overrides and the timing hook of qgemv_tuning.h are the only state:
 *     per calling thread, and only set by a caller that uses that header).
 *     Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and never synchronized: results are ready when the caller's stream
 *     reaches them.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     non-zero status means nothing was launched.  QG_ERR_LAUNCH reports a
 *     launch the HIP runtime refused.  Faults inside a kernel surface at the
 *     caller's next synchronization, as for any HIP kernel.
 *   - Alignment: packed weights 256 B, fp16 activations 16 B, fp32 outputs
 *     4 B (QG_ERR_ALIGN otherwise).
 *   - Outputs are fp32, accumulated in fp32 from exactly dequantized weights
 *     and fp16 activations (products are exact; only the sums round).  The
 *     GEMV kernels multiply the exact integer multipliers (q - 8, q or c, as
 *     fp16) and scale each block sum once, so the fp32 sums only ever hold
 *     partial sums of the result's own terms: their rounding stays far
 *     inside 1e-3 * sum |w x| for every finite input, and a one-hot
 *     activation returns a weight column exactly.  A block with a non-finite
 *     scale makes its row non-finite (inf or NaN).  Exceptions, each stated
 *     at its entry point: the fp32-input variants round x to binary16 first,
 *     the 8-bit-activation variants quantize x to 8-bit blocks first, and
 *     the times-table GEMV rounds its pair sums to binary16.
 *   - The GEMV / MoE kernels use no atomics: for a fixed shape and launch
 *     their results are bitwise reproducible.  The prefill adds split-K
 *     partial tiles atomically (last-bit differences between runs).
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int qg_status;
enum {
    QG_OK = 0,
    QG_ERR_NULL = 1,    /* a required pointer is NULL */
    QG_ERR_SHAPE = 2,   /* N, K, M or E out of range, or K % 32 != 0 */
    QG_ERR_ALIGN = 3,   /* a pointer breaks the alignment rule above */
    QG_ERR_RANGE = 4,   /* quantizer: non-finite weight or scale overflows binary16 */
    QG_ERR_SIZE = 5,    /* output buffer smaller than required */
    QG_ERR_LAUNCH = 6,  /* the HIP runtime rejected a launch */
    QG_ERR_DEVICE = 7   /* no usable HIP device / device query failed */
};

/* Static, human-readable name of a status code. */
const char *qg_status_str(qg_status s);

/* ------------------------------------------------------------ host side */

/* Bytes of one packed N x K matrix (the layout above); 0 if N <= 0, K <= 0 or
 * K % 32 != 0. */
size_t qpacked_bytes_q4_0(int64_t N, int64_t K);
size_t qpacked_bytes_q8_0(int64_t N, int64_t K);
size_t qpacked_bytes_q2w(int64_t N, int64_t K);

/* Quantize and pack fp32 weights w[N][K] (host memory) into `packed` (host
 * memory, at least qpacked_bytes_*(N, K) bytes; padding bytes are zeroed).
 *   Q4_0: d = fp16(fl32(absmax / 7)), q = clamp(round(w / d) + 8, 0, 15)
 *   Q8_0: d = fp16(fl32(absmax / 127)), q = clamp(round(w / d), -127, 127)
 * where absmax is the block's largest |w|, fl32 an IEEE binary32 division,
 * fp16 round-to-nearest-even to binary16, w / d is taken in binary64 against
 * the stored binary16 d, and round is half away from zero.  A block whose d
 * is 0 stores q = 8 (Q4_0) / 0 (Q8_0).  Returns QG_ERR_RANGE (after writing
 * every block) if a weight is non-finite or a scale overflows binary16.
 * [the block formats of sm8x-bench, "our kernel", and
 *  H100-KERNEL-5X-ROADMAP, Lever 1; quantized once, off the timed path:
 *  H100-KERNEL-5X-ROADMAP, Lever 1, resident device weights] */
qg_status qquantize_q4_0(const float *w, int64_t N, int64_t K, void *packed, size_t packed_bytes);
qg_status qquantize_q8_0(const float *w, int64_t N, int64_t K, void *packed, size_t packed_bytes);

/* The same for q2w: m = the block's weight of largest magnitude (the first
 * on ties), d = fp16(fl32(m / -2)) (so m is exactly code -2),
 * c = clamp(round(w / d), -2, 1) with w / d in binary64 against the stored d
 * and round half away from zero; d = 0 stores c = 0.  The pages give the
 * format, not a quantizer: this rule is the library's.  Returns
 * QG_ERR_RANGE as above.  [volta-kernel-bakeoff, "What's in the race"] */
qg_status qquantize_q2w(const float *w, int64_t N, int64_t K, void *packed, size_t packed_bytes);

/* ----------------------------------------------------------- device side */

/* Fused dequantize-and-multiply, 1 <= M <= 8 tokens:
 *   y[m][n] = sum_k w[n][k] * x[m][k],  w = (q - 8) * d (Q4_0) or q * d (Q8_0)
 * Wp: packed N x K matrix (device); x: fp16 bits [M][K] row-major (device);
 * y: fp32 [M][N] row-major (device, fully overwritten).  1 <= N <= 2^31 - 1,
 * 32 <= K, K % 32 == 0, K <= 16384 * min(floor(8 / M), 7) (Q4_0) or
 * 16384 * min(floor(8 / M), 4) (Q8_0).
 * [volta-kernel-bakeoff, "What's in the race" (fused_q4*, fused_q8: unpack in
 *  registers, fp32 sums) and "Results" (a few tokens at once: one activation
 *  load serves several rows); sm8x-bench, "our kernel" (several rows per
 *  wave for memory-level parallelism, per-shape launch configuration)] */
qg_status qgemv_q4_0(const void *Wp, const uint16_t *x, float *y, int M, int64_t N, int64_t K,
                     void *stream);
qg_status qgemv_q8_0(const void *Wp, const uint16_t *x, float *y, int M, int64_t N, int64_t K,
                     void *stream);

/* The same GEMV for plain 2-bit weights (q2w), 1 <= M <= 8:
 *   y[m][n] = sum_k c[n][k] * d * x[m][k]
 * with the conventions and limits of qgemv_q4_0 (K <= 16384 * min(floor(8 /
 * M), 7)); vector-ALU kernel only.  [volta-kernel-bakeoff, "What's in the
 * race" (q2w_alu: unpack in registers, fp32 sums) and "Results", the 2-bit
 * bullets] */
qg_status qgemv_q2w(const void *Wp, const uint16_t *x, float *y, int M, int64_t N, int64_t K, void *stream);

/* Q4_0 GEMV on fp32 activations, 1 <= M <= 8 tokens: each activation is
 * rounded to binary16 inside the kernel (nearest, ties to even; a magnitude
 * above 65504 becomes infinity, and so does its outputs' sum), then
 *   y[m][n] = sum_k w[n][k] * fp16(x[m][k])
 * with the conventions of qgemv_q4_0.  x: fp32 [M][K] row-major (device,
 * 16-byte aligned); Wp, y and the other limits as for qgemv_q4_0, with
 * K <= 16384 * min(floor(4 / M), 4) for M <= 4 and K <= 8192 for M = 5..8.
 * The conversion is done inside the GEMV launch, not in a separate pass:
 * once per workgroup into LDS on large tables, by each team for the blocks
 * it reads otherwise, and at 5-8 tokens (or 4 on large tables) by the
 * matrix-core kernel as it stages each wave's activation slice.
 * [volta-kernel-bakeoff, "Results", the like-for-like bullets: fp32
 *  activations in, the conversion counted, inside the kernel at 1 token and
 *  at up to 4 tokens on expert-sized tables] */
qg_status qgemv_q4_0_f32in(const void *Wp, const float *x, float *y, int M, int64_t N, int64_t K, void *stream);

/* Gate, up and SwiGLU in one launch, Q4_0, fp32 activations, 1 <= M <= 8:
 * Wp is ONE packed table of 2N rows (the layout above for 2N x K): rows
 * 0..N-1 are the gate rows, rows N..2N-1 the up rows.  With g and u the two
 * GEMVs on fp16(x) (as qgemv_q4_0_f32in),
 *   y[m][n] = silu(g[m][n]) * u[m][n],   silu(v) = v / (1 + e^-v),
 * evaluated in fp32 on the fp32 sums; only y is written.  y: fp32 [M][N].
 * 1 <= N <= 2^30 - 1; K as for qgemv_q4_0_f32in at M tokens, and at 8
 * tokens K <= 7168 (5-8 tokens, and 4 on large tables, run the matrix-core
 * kernel, each workgroup multiplying a tile's gate rows, then its up rows).  Accuracy: g and u meet the GEMV
 * bound, and y is within 1.1 eg (|u| + eu) + |g| eu + 1e-5 |y| of the exact
 * silu(g) u (eg, eu: the GEMV bounds of g and u).
 * [volta-kernel-bakeoff, "Results", the few-tokens bullet: gate and up
 *  stacked into one table, the activations converted once; the FFN fusion
 *  step of the CUDA-kernel diary: gate, up and SwiGLU in one kernel] */
qg_status qgemv_q4_0_swiglu_f32in(const void *Wp, const float *x, float *y, int M, int64_t N, int64_t K,
                                  void *stream);

/* Q4_0 GEMV on activations quantized to 8-bit blocks, 1 <= M <= 4: every
 * 32-block of each token's fp16 activations becomes int8 codes qx and one
 * binary32 scale dx (amax = the block's largest |x|; dx = amax / 127 and
 * inv = 127 / amax, correctly rounded binary32 divisions; qx = rint(x * inv),
 * a binary32 product rounded to nearest, ties to even; an all-zero block has
 * qx = 0, dx = 0), once per workgroup inside the launch; then
 *   y[m][n] = sum_b d[n][b] * dx[m][b] * sum_{k in b} (q - 8) * qx
 * with exact int8 dot products for the block sums.  This is a different
 * result from qgemv_q4_0: the activations are rounded to 8 bits, so y is
 * within sum_k |w[n][k]| * dx / 2 of the fp16 GEMV; against its own
 * definition above it is within 1e-3 * sum_b |d dx| * sum |(q - 8) qx|.
 * x: fp16 bits [M][K], finite (device, 16-byte aligned); Wp, y and N as for
 * qgemv_q4_0; K <= 16384 and M * (K / 32 + 1) * 48 <= 65536 (the LDS copy).
 * [sm8x-bench, "our kernel": the activations quantized to 8-bit blocks
 *  once, then a 4-way int8 multiply-accumulate dot with the nibbles unpacked
 *  by a 0x0F0F0F0F mask; volta-kernel-bakeoff, "Results", the 2-bit bullet:
 *  activations converted to 8-bit integers once, four weights multiplied per
 *  instruction] */
qg_status qgemv_q4_0_q8act(const void *Wp, const uint16_t *x, float *y, int M, int64_t N, int64_t K,
                           void *stream);

/* The same on plain 2-bit weights (q2w): y[m][n] = sum_b d dx sum c * qx,
 * the 2-bit codes used directly as int8 operands (mask 0x03030303 per bit
 * pair, four weights per dot instruction) with the -2 * sum(qx) offset; the
 * same limits and accuracy statement.  [volta-kernel-bakeoff, "Results",
 * the 2-bit bullet: a plain 2-bit format multiplied against activations
 * converted to 8-bit integers once, four weights per instruction] */
qg_status qgemv_q2w_q8act(const void *Wp, const uint16_t *x, float *y, int M, int64_t N, int64_t K,
                          void *stream);

/* Times-table GEMV on q2w weights, one token: every pair of activations
 * (x_a, x_b) gets the 16 sums c_a x_a + c_b x_b (c in -2..1) as fp16 in LDS,
 * and the nibble holding a weight pair's two codes looks its sum up instead
 * of multiplying.  y[n] = sum_b d * sum of the block's 16 looked-up pair sums.
 * The fp16 entries round each pair sum, so y is within 2^-11 sum |w x| plus
 * fp32 accumulation of the exact GEMV (inside 1e-3 sum |w x|).  x: fp16 bits
 * [K] (16-byte aligned), |x| < 16384 (an entry reaches 2 |x_a| + 2 |x_b|;
 * beyond binary16's range it becomes infinity); y: fp32 [N];
 * 1 <= N <= 2^31 - 1, K % 32 == 0, K <= 4096 (the tables fill 64 KB of
 * LDS).  Built to measure the design on gfx950, not as the fast path
 * (qgemv_q2w and qgemv_q2w_q8act are faster).
 * [volta-kernel-bakeoff, "What's in the race": q2_lut / q2w_lut, the "times
 *  table"; "Results": it lost to unpacking on V100] */
qg_status qgemv_q2w_lut(const void *Wp, const uint16_t *x, float *y, int64_t N, int64_t K, void *stream);

/* Mixture-of-experts GEMV in one launch, Q4_0: expert slot e (0 <= e < E)
 * multiplies pool matrix idx[e] by its own token x[e]:
 *   y[e][n] = sum_k w_{idx[e]}[n][k] * x[e][k]
 * pool: P packed N x K matrices end to end, stride qpacked_bytes_q4_0(N, K)
 * (device); idx: int32 [E] (device); x: fp16 bits [E][K]; y: fp32 [E][N].
 * 1 <= E <= 65535, 1 <= P.  Repeated indices are allowed.  An index
 * outside 0 <= idx[e] < P is never followed: no weight of that slot is read
 * and every output of the slot, y[e][0..N-1], is NaN (the indices live in
 * device memory, so the check happens on the device, not as a status).  [volta-kernel-bakeoff, "What's in the race" (moe_*: 8-10
 *  experts, one token each, one launch) and "Results"] */
qg_status qmoe_gemv_q4_0(const void *pool, int64_t P, const int32_t *idx, const uint16_t *x, float *y,
                         int E, int64_t N, int64_t K, void *stream);

/* Prefill (many tokens), Q4_0: Y[m][n] = sum_k w[n][k] * X[m][k] for any
 * M >= 1.  The weights are unpacked to fp16 (round to nearest even, the same
 * values qdequant_q4_0 writes with out_fp16 = 1) straight into the operands
 * of the fp16 matrix cores, with fp32 accumulation: up to 64 tokens with
 * every token's activations held in registers and the weights streamed once
 * in 16-row tiles, beyond that in tiles of 64 or 128 tokens.  Where the work
 * is split along K over workgroups, parts are added with fp32 atomics into Y
 * after a fill kernel zeroes it (results may then differ in the last bits
 * between runs, within the bound).  X: fp16 bits [M][K]; Y: fp32 [M][N].
 * [volta-kernel-bakeoff, "What's in the race" (tc_q4: unpack a tile to
 *  shared memory, then matrix-core multiply) and "Stage 3" (unpack inside
 *  the matrix multiply instead of dequantize-then-GEMM)] */
qg_status qgemm_q4_0_prefill(const void *Wp, const uint16_t *X, float *Y, int64_t M, int64_t N, int64_t K,
                             void *stream);

/* Dequantize a packed matrix to out[N][K]: fp32 (out_fp16 = 0; exact) or fp16
 * bits (out_fp16 = 1; the exact value rounded to nearest even, subnormals
 * kept).  [volta-kernel-bakeoff, "What's in the race": dq4+cublas unpacks to
 *  fp16 before a dense multiply] */
qg_status qdequant_q4_0(const void *Wp, int64_t N, int64_t K, int out_fp16, void *out, void *stream);
qg_status qdequant_q8_0(const void *Wp, int64_t N, int64_t K, int out_fp16, void *out, void *stream);
qg_status qdequant_q2w(const void *Wp, int64_t N, int64_t K, int out_fp16, void *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_H */
