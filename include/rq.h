/*
 * rq.h -- C ABI of librq: the online hot path of rotational W4A4
 * quantisation on AMD Instinct MI355X (gfx950).
 *
 * Pages cited:
 *   [QuaRot]    aicassindra.com, QuaRot explainer.
 *   [RQ]        llms.blog, "Rotational Quantization: How Orthogonal Transforms
 *               and Hadamard Incoherence Enable Outlier-Free Low-Bit
 *               Inference".
 *   [SpinQuant] aicassindra.com, SpinQuant explainer.
 *
 * Conventions shared by every entry point
 *   - Row vectors ([RQ] "The Principle of Computational Invariance"):
 *     X is m x d, one token per row; W is d x k and is stored transposed,
 *     W^T [k][d] (output channel major, the reduction dimension contiguous).
 *   - R = diag(s) H_n / sqrt(n), H_n the +-1 Sylvester matrix in natural
 *     order, s int8 +-1 (Rademacher).  A rotated row is (x * s) H_n / sqrt(n).
 *   - INT4 codes are two's complement, packed two per byte: code 2i in the low
 *     nibble of byte i, code 2i+1 in the high nibble.  A row of n codes is n/2
 *     bytes.  Scales are IEEE binary16 bit patterns (uint16_t).
 *   - Quantiser (symmetric, per row): a = max|x~|, scale = fp16_rne(a / 7)
 *     rounded once from the exact quotient, q = clamp(rne(x~ / scale), -8, 7)
 *     with round half to even; scale == 0 gives all-zero codes; a scale that
 *     overflows fp16 is +inf and gives all-zero codes.
 *   - All pointers are device pointers.  The caller allocates and owns every
 *     buffer; the library allocates nothing, keeps no state between calls and
 *     may be called from several threads.  Work is queued asynchronously on
 *     `stream` (a hipStream_t passed as void*, NULL = the null stream); the
 *     caller keeps buffers alive until the stream has finished.
 *   - Arguments are validated on the host before anything is launched; a
 *     non-zero rq_status is returned and nothing runs.  Row counts of 0 return
 *     RQ_OK without launching.  Non-finite inputs are undefined behaviour.
 *   - Optional debug outputs (x_rot, w_rot, acc) select an instantiation of the
 *     same kernel that also stores the intermediate value; the arithmetic that
 *     produces the primary outputs is unchanged.
 */
#ifndef RQ_H_
#define RQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RQ_OK = 0,
  RQ_ERR_NULL = 1,  /* a required pointer is NULL */
  RQ_ERR_SHAPE = 2, /* a size is negative, not a power of two, or out of range */
  RQ_ERR_ALIGN = 3, /* a pointer is not 16-byte aligned */
  RQ_ERR_DTYPE = 4, /* unknown input dtype */
  RQ_ERR_HIP = 5    /* a HIP launch failed */
} rq_status;

typedef enum { RQ_F16 = 0, RQ_F32 = 1 } rq_dtype;

/* Smallest and largest supported power-of-two rotation length n. */
#define RQ_MIN_N 2
#define RQ_MAX_N 8192
/*
 * The one supported length that is not a power of two: 28 * 512 = 14336, the
 * input width of a Llama-class down projection ([RQ] "Learned Orthogonal
 * Rotations: SpinQuant": fixed Hadamard rotations need power-of-two sizes or
 * products of small Hadamard-compatible sizes).  Its Hadamard factor is
 * H_28 (x) H_512 (element e = 512 b + p), H_28 from Paley's second
 * construction with q = 13 (symmetric, H_28 H_28^T = 28 I).  The 512-point
 * factor runs first (ascending strides), then H_28 in the order of its Paley
 * structure H_28 = C (x) H_2 + I (x) [[1, -1], [-1, -1]], C the conference
 * matrix of order 14.
 */
#define RQ_N_28X512 14336
/*
 * 28 * 1024 = 28672, the down-projection input width of the 8192 -> 28672
 * model: H_28 (x) H_1024 (element e = 1024 b + p), the 1024-point factor first
 * (ascending strides), then H_28 in the same Paley order as for RQ_N_28X512.
 */
#define RQ_N_28X1024 28672
/*
 * Largest reduction length d of the GEMMs: a multiple of 64 up to 32768
 * covers a down projection of width 28672.  Every int32 sum stays exact:
 * the W4A4 MFMA sum is 256 * acc with |acc| <= 64 d (2^29 at d = 32768), the
 * W4A8 sum 16 * acc with |acc| <= 1024 d.
 */
#define RQ_MAX_D 32768

/*
 * rq_fwht_quant -- online rotation fused with per-token INT4 quantisation.
 *
 * [QuaRot] "End-to-end flow" (runtime: an online Hadamard rotates the
 * activation, which is quantised to INT4); [RQ] "Weight Absorption and Online
 * Fast Walsh-Hadamard Transforms", part 2 (the online rotation is a butterfly
 * FWHT of add/sub stages followed by one global scale); [RQ] "Incoherence
 * Processing via Randomized Hadamard Transforms" (R = sign diagonal times
 * Sylvester matrix).
 *
 *   x       [m][n] activations, dtype x_dtype (RQ_F16 or RQ_F32), row major,
 *           16-byte aligned.
 *   m       number of rows (tokens), >= 0.
 *   n       rotation length, a power of two in [RQ_MIN_N, RQ_MAX_N],
 *           RQ_N_28X512 or RQ_N_28X1024.
 *   signs   [n] int8, each +1 or -1; NULL means all +1 (plain H_n/sqrt(n)).
 *   codes   [m][n/2] uint8 output, 16-byte aligned.
 *   scales  [m] fp16 output (one per row).
 *   x_rot   optional [m][n] float32 output of the rotated rows (debug), or
 *           NULL; 16-byte aligned when given.
 *
 * The butterflies are fp32 additions in ascending-stride order; the rotated
 * value is fp32(y * fp32(1/sqrt(n))).  Codes and scales depend only on x,
 * signs and n.
 */
int rq_fwht_quant(const void* x, int x_dtype, int64_t m, int64_t n, const int8_t* signs,
                  uint8_t* codes, uint16_t* scales, float* x_rot, void* stream);

/*
 * rq_fold_weights -- offline fold W~ = R^T W with per-output-channel INT4.
 *
 * [RQ] "Weight Absorption and Online Fast Walsh-Hadamard Transforms", part 1
 * (an input projection's weight is replaced by R^T W once, offline);
 * [QuaRot] "End-to-end flow" (offline: the folded weights are quantised to
 * INT4); [SpinQuant] "The architecture: every piece explained" (INT4 weights
 * with per-channel scales).
 *
 *   wt       W^T [k][d], dtype wt_dtype, 16-byte aligned.  Row j of the folded
 *            W~^T is w_j R = (w_j * s) H_d / sqrt(d): the same row transform
 *            as rq_fwht_quant, with the same signs as the activations.
 *   k        output channels (rows of W^T), >= 0.
 *   d        input width, a power of two in [RQ_MIN_N, RQ_MAX_N],
 *            RQ_N_28X512 or RQ_N_28X1024.
 *   signs    [d] int8 +-1 or NULL.
 *   w_codes  [k][d/2] uint8 output; w_scales [k] fp16 output.
 *   w_rot    optional [k][d] float32 output of W~^T (debug), or NULL.
 */
int rq_fold_weights(const void* wt, int wt_dtype, int64_t k, int64_t d, const int8_t* signs,
                    uint8_t* w_codes, uint16_t* w_scales, float* w_rot, void* stream);

/*
 * rq_w4a4_gemm_workspace_size -- bytes of device workspace rq_w4a4_gemm needs
 * for this shape.  The current kernels need none and return 0.
 */
size_t rq_w4a4_gemm_workspace_size(int64_t m, int64_t k, int64_t d);

/*
 * rq_w4a4_gemm -- W4A4 linear: y = fp16(acc * sa[m] * sw[j]),
 * acc[m][j] = sum_i qa[m][i] * qw[j][i] in int32.
 *
 * [RQ] "Hardware Execution and Serving Economics", part 1 (rotated W4A4
 * layers run integer GEMMs end to end); [QuaRot] "End-to-end flow" (the INT4
 * rotated activation multiplies the INT4 folded weight in a low-bit kernel).
 * INT4 codes are widened to int8 in registers and multiplied with int8 MFMA
 * into int32 accumulators (exact: |acc| <= 64 * d, see RQ_MAX_D); the epilogue is
 * t = fp32(fp32(acc) * sa), then t * sw rounded once to fp16 half to even
 * (from the exact product, with no fp32 rounding in between).
 *
 *   a_codes  [m][d/2] uint8 activation codes (rq_fwht_quant output), 16-byte
 *            aligned; a_scales [m] fp16.
 *   m        tokens, >= 0.
 *   w_codes  [k][d/2] uint8 weight codes (rq_fold_weights output), 16-byte
 *            aligned; w_scales [k] fp16.
 *   k        output channels, >= 1 when m > 0.
 *   d        reduction length, a multiple of 64 in [64, RQ_MAX_D].
 *   y        [m][k] fp16 output.
 *   acc      optional [m][k] int32 output of the accumulators (debug), or NULL.
 *   workspace, workspace_bytes  device scratch of at least
 *            rq_w4a4_gemm_workspace_size(m, k, d) bytes (may be NULL when 0).
 */
int rq_w4a4_gemm(const uint8_t* a_codes, const uint16_t* a_scales, int64_t m,
                 const uint8_t* w_codes, const uint16_t* w_scales, int64_t k, int64_t d,
                 uint16_t* y, int32_t* acc, void* workspace, size_t workspace_bytes,
                 void* stream);

/*
 * rq_pack_f6 -- repack INT4 codes into F6 rows: fp6 E3M2 containers in the
 * operand layout of the 6-bit MFMA, for rq_w4a4_gemm_f6.
 *
 * [RQ] "Hardware Execution and Serving Economics", part 1 (INT4 matrix
 * arithmetic at twice the 8-bit throughput).  gfx950 has no INT4 MFMA, but
 * every code -8..7 is exactly an OCP MX E3M2 value, and its 6-bit MFMA runs
 * faster than the int8 one.  The layout is group-major: the 128-code group
 * c of row r is the 96 bytes at (c * rows + r) * 96; its 32-code block b is a
 * 192-bit little-endian word with code j (of the block) in bits 6j..6j+5,
 * whose bytes 0..15 sit at group byte 16b and bytes 16..23 at group byte
 * 64 + 16 * (b % 2) + 8 * (b / 2).  The E3M2 code of q is sign (bit 5)
 * with |q| = 0, 1, 2, 3, 4, 5, 6, 7, 8 -> 0x00, 0x0C, 0x10, 0x12, 0x14,
 * 0x15, 0x16, 0x17, 0x18.
 *
 *   codes    [rows][d/2] uint8 packed INT4 (code i in nibble i), 16-byte
 *            aligned.
 *   rows     >= 0.
 *   d        codes per row, a multiple of 128 in [128, RQ_MAX_D].
 *   out      [d/128][rows][96] uint8, 16-byte aligned, caller-owned.
 */
int rq_pack_f6(const uint8_t* codes, int64_t rows, int64_t d, uint8_t* out, void* stream);

/*
 * rq_w4a4_gemm_f6 -- rq_w4a4_gemm on F6 rows of both operands, multiplied on
 * v_mfma_f32_16x16x128_f8f6f4.  The fp32 accumulators hold the integer
 * accumulator exactly (products <= 64 in magnitude, sums < 2^24 for
 * d <= RQ_MAX_D), so y and acc equal rq_w4a4_gemm's on the same codes bit
 * for bit; the epilogue is the same.  One persistent workgroup per CU walks
 * 256 x 224 (or 256 x 256) output tiles.
 *
 *   a_f6     [d/128][m][96] rq_pack_f6 of the activation codes, 16-byte aligned;
 *            a_scales [m] fp16.
 *   m        tokens, >= 0.
 *   w_f6     [d/128][k][96] rq_pack_f6 of the weight codes, 16-byte aligned;
 *            w_scales [k] fp16.
 *   k        output channels, >= 1 when m > 0.
 *   d        reduction length, a multiple of 128 in [128, RQ_MAX_D].
 *   y        [m][k] fp16 output.
 *   acc      optional [m][k] int32 output of the accumulators (debug), or NULL.
 */
int rq_w4a4_gemm_f6(const uint8_t* a_f6, const uint16_t* a_scales, int64_t m, const uint8_t* w_f6,
                    const uint16_t* w_scales, int64_t k, int64_t d, uint16_t* y, int32_t* acc,
                    void* stream);

/*
 * rq_kv_rotate_quant -- per-head rotation and INT4 packing of K and V.
 *
 * [QuaRot] "The architecture: every piece explained" (KV-cache rotation) and
 * "End-to-end flow" (keys and values are rotated, then stored in four bits);
 * [RQ] "Hardware Execution and Serving Economics", part 2 (4-bit KV after
 * rotating K and V).
 *
 *   k_in, v_in   fp16 [rows][head_dim]: every (batch, head, position) vector
 *                is one row, 16-byte aligned.
 *   rows         number of vectors in each of K and V, >= 0.
 *   head_dim     must be 128.
 *   signs        [head_dim] int8 +-1, or NULL for the plain H/sqrt(128)
 *                (the same rotation for every head, for K and for V).
 *   k_codes, v_codes    [rows][head_dim/2] uint8, 16-byte aligned.
 *   k_scales, v_scales  [rows] fp16.
 */
int rq_kv_rotate_quant(const uint16_t* k_in, const uint16_t* v_in, int64_t rows, int64_t head_dim,
                       const int8_t* signs, uint8_t* k_codes, uint16_t* k_scales,
                       uint8_t* v_codes, uint16_t* v_scales, void* stream);

/*
 * rq_linear_decode_workspace_size -- bytes of device workspace that
 * rq_linear_decode needs: m * d / 2 + 64 (0 for a shape rq_linear_decode
 * rejects).
 */
size_t rq_linear_decode_workspace_size(int64_t m, int64_t d);

/*
 * rq_linear_decode -- the whole decode-shaped W4A4 linear in one call:
 * rq_fwht_quant of the fp16 tokens, then rq_w4a4_gemm with the folded weights.
 *
 * [SpinQuant] "The architecture: every piece explained" (the online rotation
 * is fused into the low-bit matmul); [QuaRot] "End-to-end flow" (rotate,
 * quantise to INT4, multiply in a low-bit kernel).  For m <= 4 it is one
 * launch: every workgroup of the decode GEMM rotates and quantises the tokens
 * into LDS as its prologue, with the device code of rq_fwht_quant, while its
 * weights stream in.  For 4 < m <= 16 it is rq_fwht_quant into the workspace
 * followed by the decode GEMM.  Either way y is bit-identical to
 * rq_fwht_quant followed by rq_w4a4_gemm on the same arguments.
 *
 *   x          [m][d] fp16 tokens, 16-byte aligned.
 *   m          tokens, 0 <= m <= 16 (m == 0 returns RQ_OK without launching).
 *   d          input width, a power of two in [512, 8192].
 *   signs      [d] int8 +-1 (the ones the weights were folded with), or NULL.
 *   w_codes    [k][d/2] folded weight codes (rq_fold_weights), 16-byte
 *              aligned; w_scales [k] fp16.
 *   k          output channels, >= 1.
 *   y          [m][k] fp16 output.
 *   workspace  device memory of at least rq_linear_decode_workspace_size(m, d)
 *              bytes, 16-byte aligned (any contents).  When m > 4 it receives
 *              the activation codes ([m][d/2] at offset 0) and scales ([m]
 *              fp16 after the codes); calls that may overlap in time need
 *              separate workspaces.
 *   workspace_bytes  size of workspace.
 */
int rq_linear_decode(const uint16_t* x, int64_t m, int64_t d, const int8_t* signs,
                     const uint8_t* w_codes, const uint16_t* w_scales, int64_t k, uint16_t* y,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the device array rq_linear_decode_noalloc works in:
 * 16 tokens x 8192 / 2 code bytes + 64 (codes, then fp16 scales). */
#define RQ_NOALLOC_SCRATCH_BYTES (16 * 8192 / 2 + 64)

/*
 * rq_linear_decode_noalloc -- rq_linear_decode for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops
 * and harnesses that forbid allocation.  Same arguments, kernels and result
 * as rq_linear_decode (y bit-identical), without the workspace: when m > 4
 * the activation codes and scales go to a file-scope device array of
 * RQ_NOALLOC_SCRATCH_BYTES bytes that the library holds on every GPU it has
 * run on until the process ends.  Nothing is allocated by the call (the
 * array's device address is looked up once per device, with that device
 * current).  Calls that overlap in time on one GPU share the array and race;
 * serialise them (one stream, or events).  Shapes beyond the array's size
 * cannot occur within the limits below and would return RQ_ERR_SHAPE.
 *
 *   x, m, d, signs, w_codes, w_scales, k, y, stream: as rq_linear_decode
 *   (0 <= m <= 16, d a power of two in [512, 8192]).
 */
int rq_linear_decode_noalloc(const uint16_t* x, int64_t m, int64_t d, const int8_t* signs,
                             const uint8_t* w_codes, const uint16_t* w_scales, int64_t k,
                             uint16_t* y, void* stream);

/*
 * rq_fwht_quant8 -- online rotation fused with per-token INT8 quantisation,
 * the activation side of the W4A8 variant.
 *
 * [SpinQuant] "The architecture: every piece explained" and "End-to-end
 * flow" (INT4 weights with 8-bit activations: the rotated activation is
 * quantised to INT8 at run time).  The rotation is the one of rq_fwht_quant
 * (same stages, same fp32 rounding); the quantiser is the symmetric per-row
 * rule with 127 in place of 7: scale = fp16_rne(max |x~| / 127) rounded once
 * from the exact quotient, code = rne(x~ / scale) in [-128, 127] (a zero
 * scale gives zero codes).
 *
 *   x       [m][n] fp16 activations, row major, 16-byte aligned.
 *   m       rows (tokens), >= 0.
 *   n       a power of two in [512, RQ_MAX_N].
 *   signs   [n] int8 +-1, or NULL for all +1; 16-byte aligned when given.
 *   codes   [m][n] int8 output (one two's-complement code per element),
 *           16-byte aligned.
 *   scales  [m] fp16 output.
 *   x_rot   optional [m][n] float32 rotated rows, or NULL.
 */
int rq_fwht_quant8(const uint16_t* x, int64_t m, int64_t n, const int8_t* signs, int8_t* codes,
                   uint16_t* scales, float* x_rot, void* stream);

/*
 * rq_w4a8_gemm -- W4A8 linear: INT8 activation codes times packed INT4
 * folded weight codes, y = fp16(acc * sa[m] * sw[j]),
 * acc[m][j] = sum_i qa[m][i] * qw[j][i] in int32.
 *
 * [SpinQuant] "The architecture: every piece explained" (INT4 weights, INT8
 * activations, integer matmul).  The weight codes are widened to 16 * q in
 * int8 lanes and multiplied with the activation bytes by int8 MFMA; the
 * int32 sum is exactly 16 * acc (|16 * acc| <= 2^14 * d < 2^31).  The epilogue is
 * the one of rq_w4a4_gemm.
 *
 *   a_codes  [m][d] int8 activation codes (rq_fwht_quant8), 16-byte aligned;
 *            a_scales [m] fp16.
 *   m        tokens, >= 0.
 *   w_codes  [k][d/2] uint8 weight codes (rq_fold_weights), 16-byte aligned;
 *            w_scales [k] fp16.
 *   k        output channels, >= 1 when m > 0.
 *   d        reduction length, a multiple of 64 in [64, RQ_MAX_D].
 *   y        [m][k] fp16 output; acc optional [m][k] int32 accumulators.
 */
int rq_w4a8_gemm(const int8_t* a_codes, const uint16_t* a_scales, int64_t m,
                 const uint8_t* w_codes, const uint16_t* w_scales, int64_t k, int64_t d,
                 uint16_t* y, int32_t* acc, void* stream);

/*
 * rq_linear_decode_w4a8 -- the decode-shaped W4A8 linear in one launch:
 * rq_fwht_quant8 of the fp16 tokens, then rq_w4a8_gemm with the folded
 * weights.
 *
 * [SpinQuant] "The architecture: every piece explained" (INT4 weights with
 * 8-bit activations, the online rotation fused into the low-bit matmul).
 * Every workgroup of the INT8-activation decode GEMM rotates and quantises
 * the tokens into LDS as its prologue, with the device code of
 * rq_fwht_quant8, while its weights stream in; y is bit-identical to
 * rq_fwht_quant8 followed by rq_w4a8_gemm on the same arguments.  No
 * workspace: the activation codes never leave the workgroup.
 *
 *   x          [m][d] fp16 tokens, 16-byte aligned.
 *   m          tokens, 0 <= m <= 4 (m == 0 returns RQ_OK without launching;
 *              more tokens: rq_fwht_quant8 then rq_w4a8_gemm).
 *   d          input width, a power of two in [512, 8192].
 *   signs      [d] int8 +-1 (the ones the weights were folded with), or NULL;
 *              16-byte aligned when given.
 *   w_codes    [k][d/2] folded weight codes (rq_fold_weights), 16-byte
 *              aligned; w_scales [k] fp16.
 *   k          output channels, >= 1.
 *   y          [m][k] fp16 output.
 */
int rq_linear_decode_w4a8(const uint16_t* x, int64_t m, int64_t d, const int8_t* signs,
                          const uint8_t* w_codes, const uint16_t* w_scales, int64_t k, uint16_t* y,
                          void* stream);

/*
 * rq_fwht_quant_asym -- online rotation fused with asymmetric per-token INT4.
 *
 * [RQ] "The Activation Outlier Bottleneck in Low-Bit Serving" (a uniform
 * b-bit grid whose step spans the whole range, Delta = (max - min) /
 * (2^b - 1)).  The rotation is the one of rq_fwht_quant.  Per row, with lo
 * and hi the row's min and max widened to contain 0 (fp32 rotated values):
 * scale = fp16(fp32(hi - lo) / 15) rounded once, zero = rne(-lo / scale) in
 * [0, 15], code = clamp(rne(x~ / scale) + zero, 0, 15).  A zero or infinite
 * scale gives zero = 0 and all-zero codes.  Dequantisation:
 * x~ ~ scale * (code - zero).
 *
 *   x       [m][n] fp16, 16-byte aligned; n a power of two in [512, RQ_MAX_N].
 *   signs   [n] int8 +-1 or NULL.
 *   codes   [m][n/2] uint8 output: unsigned 4-bit codes, code 2i in the low
 *           nibble of byte i; 16-byte aligned.
 *   scales  [m] fp16 output; zeros [m] uint8 output (0..15).
 *   x_rot   optional [m][n] float32 rotated rows, or NULL.
 */
int rq_fwht_quant_asym(const uint16_t* x, int64_t m, int64_t n, const int8_t* signs,
                       uint8_t* codes, uint16_t* scales, uint8_t* zeros, float* x_rot,
                       void* stream);

/*
 * rq_weight_code_sums -- sums[j] = sum_i qw[j][i] over the signed INT4 codes
 * of each folded weight row (an offline companion of rq_fold_weights that the
 * asymmetric GEMM needs: sum_i (qa_i - z) qw_i = sum_i qa_i qw_i - z sums[j]).
 *
 *   w_codes  [k][d/2] uint8 (rq_fold_weights output), 16-byte aligned.
 *   k        rows, >= 0;  d  a multiple of 64 in [64, RQ_MAX_D].
 *   sums     [k] int32 output.
 */
int rq_weight_code_sums(const uint8_t* w_codes, int64_t k, int64_t d, int32_t* sums,
                        void* stream);

/*
 * rq_w4a4_gemm_asym -- W4A4 linear with asymmetric activations:
 * y = fp16(acc * sa[m] * sw[j]), acc[m][j] = sum_i (qa[m][i] - za[m]) qw[j][i].
 *
 * [RQ] "The Activation Outlier Bottleneck in Low-Bit Serving" (asymmetric
 * step) and "Hardware Execution and Serving Economics", part 1 (integer GEMM).
 * The unsigned activation codes are widened to int8 lanes as they are, the
 * weights to 16 * q; the int32 MFMA sum is 16 * sum qa qw, and the epilogue
 * subtracts za * w_sums[j] before the fp16 scaling of rq_w4a4_gemm.
 *
 *   a_codes  [m][d/2] unsigned codes (rq_fwht_quant_asym), 16-byte aligned;
 *            a_scales [m] fp16; a_zeros [m] uint8.
 *   w_codes  [k][d/2] signed codes (rq_fold_weights), 16-byte aligned;
 *            w_scales [k] fp16; w_sums [k] int32 (rq_weight_code_sums).
 *   m >= 0, k >= 1 when m > 0, d a multiple of 64 in [64, RQ_MAX_D].
 *   y        [m][k] fp16 output; acc optional [m][k] int32 accumulators.
 */
int rq_w4a4_gemm_asym(const uint8_t* a_codes, const uint16_t* a_scales, const uint8_t* a_zeros,
                      int64_t m, const uint8_t* w_codes, const uint16_t* w_scales,
                      const int32_t* w_sums, int64_t k, int64_t d, uint16_t* y, int32_t* acc,
                      void* stream);

/*
 * rq_quantize_groups -- symmetric INT4 with one scale per group of `group`
 * consecutive elements of each fp32 row (per-group weight scales).
 *
 * [SpinQuant] "End-to-end flow" (the rotated weights are mapped to INT4 with
 * per-channel or per-group scales).  Offline use: the rows are the folded
 * weights W~^T that rq_fold_weights writes to w_rot.  Per group: scale =
 * fp16(max |x| / 7) rounded once, code = clamp(rne(x * fp32(1 / scale)),
 * -8, 7); a zero or infinite scale gives zero codes.
 *
 *   x       [rows][n] float32, 16-byte aligned.
 *   group   32, 64, 128 or 256; n a multiple of group, n <= 2^20.
 *   codes   [rows][n/2] uint8 output (packed like rq_fwht_quant), 16-byte
 *           aligned.
 *   scales  [rows][n / group] fp16 output.
 */
int rq_quantize_groups(const float* x, int64_t rows, int64_t n, int64_t group, uint8_t* codes,
                       uint16_t* scales, void* stream);

/*
 * rq_w4a4_gemm_grouped -- W4A4 linear with per-token activation scales and
 * per-group weight scales (group 128):
 * y[m][j] = fp16(sa[m] * sum_g sw[j][g] * acc[m][j][g]),
 * acc[m][j][g] = sum over the 128 codes of group g of qa[m][i] * qw[j][i].
 *
 * [SpinQuant] "The architecture: every piece explained" and "End-to-end
 * flow" (INT4 weights with per-group scales, integer matmul).  Each group's
 * integer dot product is exact in int32 (int8 MFMA on widened codes) and
 * turns into fp32 with its group scale; the sum over groups is fp32.
 *
 *   a_codes         [m][d/2] (rq_fwht_quant), 16-byte aligned; a_scales [m].
 *   w_codes         [k][d/2] (rq_quantize_groups on the folded weights),
 *                   16-byte aligned.
 *   w_group_scales  [k][d / 128] fp16, 2-byte aligned (with 4-byte alignment,
 *                   shapes with m >= 128, k >= 224 and d a multiple of 256
 *                   run on the persistent prefill kernel, which reads scale
 *                   pairs as dwords; otherwise on the tile kernel).
 *   m >= 0; k >= 1 when m > 0; d a multiple of 128 in [128, RQ_MAX_D].
 *   y               [m][k] fp16 output.
 *   acc             optional [m][k][d / 128] int32 output (debug) of every
 *                   group's exact integer sum acc[m][j][g], or NULL; it
 *                   selects an instantiation of the same kernels that also
 *                   stores them.
 */
int rq_w4a4_gemm_grouped(const uint8_t* a_codes, const uint16_t* a_scales, int64_t m,
                         const uint8_t* w_codes, const uint16_t* w_group_scales, int64_t k,
                         int64_t d, uint16_t* y, int32_t* acc, void* stream);

/*
 * rq_decode_attention_workspace_size -- bytes of device workspace that
 * rq_decode_attention needs for this shape on the current device (one
 * fp32 record of 132 values per query head and split of the cache).  When
 * batch * kv_heads is a multiple of the device's CU count, the call runs one
 * workgroup per KV head over the whole sequence and leaves the workspace
 * untouched; it is still required.  Returns 0 for a shape rq_decode_attention
 * rejects or for batch == 0.
 */
size_t rq_decode_attention_workspace_size(int64_t batch, int64_t kv_heads, int64_t group,
                                          int64_t seq);

/*
 * rq_decode_attention -- single-token attention that reads the 4-bit rotated
 * KV cache written by rq_kv_rotate_quant.
 *
 * [QuaRot] "End-to-end flow" (a later token's attention reads the four-bit
 * rotated cache; rotation invariance keeps the scores) and [RQ] "The
 * Principle of Computational Invariance" (q k^T = (q R)(k R)^T).  For batch
 * entry b and query head j (KV head h = j / group):
 *   q~ = q R with the cache's rotation R = diag(signs) H_128 / sqrt(128),
 *   s_t = (q~ . k^_t) * sm_scale for t < len_b, k^_t = code_t * kscale_t,
 *   p = softmax(s), o = (sum_t p_t v^_t) R^T.
 * The scores use f16 MFMA on the exact key codes with the query split into
 * two f16 parts (about 22 significant bits) and fp32 accumulation; the
 * weighted sum, the softmax and the inverse rotation are fp32.  A length of
 * 0 gives a zero output.
 *
 *   q          [batch][kv_heads * group][128] fp16 queries of the new token,
 *              16-byte aligned.
 *   k_codes, v_codes    [batch][kv_heads][seq][64] uint8 (rq_kv_rotate_quant),
 *              16-byte aligned; k_scales, v_scales [batch][kv_heads][seq] fp16,
 *              4-byte aligned (the scales move in pairs of positions).
 *   lengths    optional device int32 [batch] valid positions per entry
 *              (values are clamped to [0, seq]); NULL means seq for all.
 *   batch >= 0; kv_heads >= 1; 1 <= group <= 8; seq even and >= 2 (shorter
 *              sequences use lengths);
 *   batch * kv_heads <= 65535; head_dim must be 128.
 *   signs      the [128] int8 +-1 signs the cache was rotated with, or NULL.
 *   sm_scale   softmax scale (> 0), normally 1 / sqrt(128).
 *   out        [batch][kv_heads * group][128] fp16 output; out_f32 optional
 *              fp32 copy (debug) or NULL.
 *   workspace  device memory of at least rq_decode_attention_workspace_size
 *              bytes, 16-byte aligned (any contents; calls that may overlap
 *              in time need separate workspaces).
 */
int rq_decode_attention(const uint16_t* q, const uint8_t* k_codes, const uint16_t* k_scales,
                        const uint8_t* v_codes, const uint16_t* v_scales, const int32_t* lengths,
                        int64_t batch, int64_t kv_heads, int64_t group, int64_t seq,
                        int64_t head_dim, const int8_t* signs, float sm_scale, uint16_t* out,
                        float* out_f32, void* workspace, size_t workspace_bytes, void* stream);

/* Text for an rq_status value (static storage, never NULL). */
const char* rq_status_string(int status);

/* Library version: major * 10000 + minor * 100 + patch. */
int rq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RQ_H_ */
