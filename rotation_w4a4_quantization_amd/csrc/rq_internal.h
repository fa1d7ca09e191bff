// Internal launch interface between the C-ABI layer (rq_api.hip) and the
// kernel translation units.  Arguments reaching these functions have been
// validated already; they only pick a kernel instantiation and launch it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rq {

// Compute units of the current device (queried once per device).
int cu_count();

// Row-wise (x * s) H_n / sqrt(n) fused with symmetric INT4 quantisation.
// `is_f32` selects the element type of x (fp32 or fp16).
hipError_t launch_fwht_quant(const void* x, bool is_f32, int64_t rows, int n, const int8_t* signs,
                             uint8_t* codes, uint16_t* scales, float* x_rot, hipStream_t stream);

// Row-wise (x * s) H_n / sqrt(n) fused with symmetric per-row INT8
// quantisation (fp16 x, n in 512..8192 a power of two); codes [rows][n].
hipError_t launch_fwht_quant8(const uint16_t* x, int64_t rows, int n, const int8_t* signs,
                              int8_t* codes, uint16_t* scales, float* x_rot, hipStream_t stream);

// Row-wise (x * s) H_n / sqrt(n) fused with the asymmetric per-row INT4
// quantiser (unsigned codes, integer zero points; fp16 x, n in 512..8192).
hipError_t launch_fwht_quant_asym(const uint16_t* x, int64_t rows, int n, const int8_t* signs,
                                  uint8_t* codes, uint16_t* scales, uint8_t* zeros, float* x_rot,
                                  hipStream_t stream);

// Same transform for the two KV tensors (fp16, n = 128) in one launch.
hipError_t launch_kv_rotate_quant(const uint16_t* k_in, const uint16_t* v_in, int64_t rows,
                                  const int8_t* signs, uint8_t* k_codes, uint16_t* k_scales,
                                  uint8_t* v_codes, uint16_t* v_scales, hipStream_t stream);

// y[m][k] = fp16(acc * sa * sw), acc = qa . qw over d.
hipError_t launch_w4a4_gemm(const uint8_t* a_codes, const uint16_t* a_scales, int64_t m,
                            const uint8_t* w_codes, const uint16_t* w_scales, int64_t k, int64_t d,
                            uint16_t* y, int32_t* acc, hipStream_t stream);

// INT4 codes [rows][d/2] -> F6 rows [rows][3d/4] (fp6 E3M2 containers in
// the operand layout of the 6-bit MFMA; d % 128 == 0), and the W4A4 GEMM on
// F6 rows of both operands (same results as launch_w4a4_gemm).
hipError_t launch_pack_f6(const uint8_t* codes, int64_t rows, int64_t d, uint8_t* out,
                          hipStream_t stream);
hipError_t launch_w4a4_gemm_f6(const uint8_t* a6, const uint16_t* a_scales, int64_t m,
                               const uint8_t* w6, const uint16_t* w_scales, int64_t k, int64_t d,
                               uint16_t* y, int32_t* acc, hipStream_t stream);

// W4A8: y[m][k] = fp16(acc * sa * sw), acc = qa . qw over d with INT8
// activation codes qa ([m][d] bytes) and packed INT4 weight codes.
hipError_t launch_w4a8_gemm(const int8_t* a_codes8, const uint16_t* a_scales, int64_t m,
                            const uint8_t* w_codes, const uint16_t* w_scales, int64_t k, int64_t d,
                            uint16_t* y, int32_t* acc, hipStream_t stream);

// Asymmetric activations: y = fp16(acc * sa * sw) with
// acc = sum_i (qa[i] - za) * qw[i]; qa unsigned packed INT4, w_sums[j] = sum_i qw[j][i].
hipError_t launch_w4a4_gemm_asym(const uint8_t* a_codes, const uint16_t* a_scales,
                                 const uint8_t* a_zeros, int64_t m, const uint8_t* w_codes,
                                 const uint16_t* w_scales, const int32_t* w_sums, int64_t k,
                                 int64_t d, uint16_t* y, int32_t* acc, hipStream_t stream);
hipError_t launch_weight_code_sums(const uint8_t* w_codes, int64_t k, int64_t d, int32_t* sums,
                                   hipStream_t stream);

// Per-group INT4 weights: symmetric INT4 with one scale per `group`
// elements of fp32 rows (group 32, 64, 128 or 256), and the W4A4 GEMM with
// per-group weight scales (group 128, wg_scales [k][d / 128]; gacc, when
// not null, receives the int32 sum of every group, [m][k][d / 128]).
hipError_t launch_quantize_groups(const float* x, int64_t rows, int64_t n, int group,
                                  uint8_t* codes, uint16_t* scales, hipStream_t stream);
hipError_t launch_w4a4_gemm_grouped(const uint8_t* a_codes, const uint16_t* a_scales, int64_t m,
                                    const uint8_t* w_codes, const uint16_t* wg_scales, int64_t k,
                                    int64_t d, uint16_t* y, int32_t* gacc, hipStream_t stream);

// Decode attention over the 4-bit rotated KV cache (head_dim 128, G <= 8
// query heads per KV head); the workspace holds one (max, sum, output)
// record per split and query.
size_t decode_attention_workspace_bytes(int64_t batch, int64_t kv_heads, int64_t group,
                                        int64_t seq);
hipError_t launch_decode_attention(const uint16_t* q, const uint8_t* kc, const uint16_t* ks,
                                   const uint8_t* vc, const uint16_t* vs, const int32_t* lengths,
                                   int64_t B, int64_t H, int64_t G, int64_t S,
                                   const int8_t* signs, float sm_scale, uint16_t* out,
                                   float* out_f32, void* workspace, hipStream_t stream);

// Fused decode linear (m <= 16, fp16 x, d in 512..8192 a power of two):
// rotation + INT4 quantisation of x as the prologue of the decode GEMM.
size_t linear_decode_workspace_bytes(int64_t m, int64_t d);
hipError_t launch_linear_decode(const uint16_t* x, int64_t m, int64_t d, const int8_t* signs,
                                const uint8_t* w_codes, const uint16_t* w_scales, int64_t k,
                                uint16_t* y, void* workspace, hipStream_t stream);

// Fused W4A8 decode linear (m <= 4): rotation + per-token INT8 quantisation
// of x as the prologue of the INT8-activation decode GEMM, one launch.
hipError_t launch_linear_decode_w4a8(const uint16_t* x, int64_t m, int64_t d, const int8_t* signs,
                                     const uint8_t* w_codes, const uint16_t* w_scales, int64_t k,
                                     uint16_t* y, hipStream_t stream);

}  // namespace rq
