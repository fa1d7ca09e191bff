// C ABI of librq (declared in include/rq.h): argument validation on the host,
// then one kernel launch per call.  Nothing here allocates, synchronises or
// keeps state between calls.
#include <hip/hip_runtime.h>

#include "../../include/rq.h"
#include "rq_internal.h"

namespace {

constexpr int kVersion = 1 * 10000 + 0 * 100 + 0;

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Rows are limited so that every grid dimension fits its hardware limit.
constexpr int64_t kMaxRows = (int64_t)1 << 31;
// Token rows of the tile GEMM: 128-row tiles in a grid dimension of 65535.
constexpr int64_t kMaxTileRows = (int64_t)65535 * 128;
// Decode attention: one workgroup row per (batch, KV head), grid y <= 65535.
constexpr int64_t kMaxHeads = 65535;

// Shapes rq_decode_attention accepts (checked without overflow: batch and
// kv_heads are bounded before their product is formed).
bool attention_shape_ok(int64_t batch, int64_t kv_heads, int64_t group, int64_t seq) {
  if (batch < 0 || batch > kMaxHeads || kv_heads < 1 || kv_heads > kMaxHeads) return false;
  if (batch * kv_heads > kMaxHeads) return false;
  return group >= 1 && group <= 8 && seq >= 2 && seq % 2 == 0 && seq < kMaxRows;
}

int from_hip(hipError_t e) { return e == hipSuccess ? RQ_OK : RQ_ERR_HIP; }

int check_rotation_args(const void* x, int dtype, int64_t m, int64_t n, const int8_t* signs,
                        const void* codes, const void* scales, const void* rot) {
  if (dtype != RQ_F16 && dtype != RQ_F32) return RQ_ERR_DTYPE;
  if (m < 0 || m >= kMaxRows) return RQ_ERR_SHAPE;
  if (n != RQ_N_28X512 && n != RQ_N_28X1024 && (!is_pow2(n) || n < RQ_MIN_N || n > RQ_MAX_N))
    return RQ_ERR_SHAPE;
  if (m == 0) return RQ_OK;
  if (x == nullptr || codes == nullptr || scales == nullptr) return RQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(codes)) return RQ_ERR_ALIGN;
  if (signs != nullptr && !aligned16(signs)) return RQ_ERR_ALIGN;
  if (rot != nullptr && !aligned16(rot)) return RQ_ERR_ALIGN;
  return RQ_OK;
}

}  // namespace

extern "C" {

int rq_fwht_quant(const void* x, int x_dtype, int64_t m, int64_t n, const int8_t* signs,
                  uint8_t* codes, uint16_t* scales, float* x_rot, void* stream) {
  const int st = check_rotation_args(x, x_dtype, m, n, signs, codes, scales, x_rot);
  if (st != RQ_OK || m == 0) return st;
  return from_hip(rq::launch_fwht_quant(x, x_dtype == RQ_F32, m, (int)n, signs, codes, scales,
                                        x_rot, static_cast<hipStream_t>(stream)));
}

int rq_fold_weights(const void* wt, int wt_dtype, int64_t k, int64_t d, const int8_t* signs,
                    uint8_t* w_codes, uint16_t* w_scales, float* w_rot, void* stream) {
  const int st = check_rotation_args(wt, wt_dtype, k, d, signs, w_codes, w_scales, w_rot);
  if (st != RQ_OK || k == 0) return st;
  return from_hip(rq::launch_fwht_quant(wt, wt_dtype == RQ_F32, k, (int)d, signs, w_codes,
                                        w_scales, w_rot, static_cast<hipStream_t>(stream)));
}

int rq_fwht_quant8(const uint16_t* x, int64_t m, int64_t n, const int8_t* signs, int8_t* codes,
                   uint16_t* scales, float* x_rot, void* stream) {
  if (m < 0 || m >= kMaxRows) return RQ_ERR_SHAPE;
  if (!is_pow2(n) || n < 512 || n > RQ_MAX_N) return RQ_ERR_SHAPE;
  const int st = check_rotation_args(x, RQ_F16, m, n, signs, codes, scales, x_rot);
  if (st != RQ_OK || m == 0) return st;
  return from_hip(rq::launch_fwht_quant8(x, m, (int)n, signs, codes, scales, x_rot,
                                         static_cast<hipStream_t>(stream)));
}

int rq_fwht_quant_asym(const uint16_t* x, int64_t m, int64_t n, const int8_t* signs,
                       uint8_t* codes, uint16_t* scales, uint8_t* zeros, float* x_rot,
                       void* stream) {
  if (m < 0 || m >= kMaxRows) return RQ_ERR_SHAPE;
  if (!is_pow2(n) || n < 512 || n > RQ_MAX_N) return RQ_ERR_SHAPE;
  const int st = check_rotation_args(x, RQ_F16, m, n, signs, codes, scales, x_rot);
  if (st != RQ_OK || m == 0) return st;
  if (zeros == nullptr) return RQ_ERR_NULL;
  return from_hip(rq::launch_fwht_quant_asym(x, m, (int)n, signs, codes, scales, zeros, x_rot,
                                             static_cast<hipStream_t>(stream)));
}

int rq_weight_code_sums(const uint8_t* w_codes, int64_t k, int64_t d, int32_t* sums,
                        void* stream) {
  if (k < 0 || k >= kMaxRows || d < 64 || d > RQ_MAX_D || d % 64 != 0) return RQ_ERR_SHAPE;
  if (k == 0) return RQ_OK;
  if (w_codes == nullptr || sums == nullptr) return RQ_ERR_NULL;
  if (!aligned16(w_codes)) return RQ_ERR_ALIGN;
  return from_hip(rq::launch_weight_code_sums(w_codes, k, d, sums,
                                              static_cast<hipStream_t>(stream)));
}

size_t rq_w4a4_gemm_workspace_size(int64_t m, int64_t k, int64_t d) {
  (void)m;
  (void)k;
  (void)d;
  return 0;
}

int rq_w4a4_gemm(const uint8_t* a_codes, const uint16_t* a_scales, int64_t m,
                 const uint8_t* w_codes, const uint16_t* w_scales, int64_t k, int64_t d,
                 uint16_t* y, int32_t* acc, void* workspace, size_t workspace_bytes,
                 void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (m < 0 || k < 0 || d < 64 || d > RQ_MAX_D || d % 64 != 0) return RQ_ERR_SHAPE;
  if (m > kMaxTileRows) return RQ_ERR_SHAPE;
  if (k >= kMaxRows) return RQ_ERR_SHAPE;
  if (m == 0) return RQ_OK;
  if (k == 0) return RQ_ERR_SHAPE;
  if (a_codes == nullptr || a_scales == nullptr || w_codes == nullptr || w_scales == nullptr ||
      y == nullptr)
    return RQ_ERR_NULL;
  if (!aligned16(a_codes) || !aligned16(w_codes)) return RQ_ERR_ALIGN;
  return from_hip(rq::launch_w4a4_gemm(a_codes, a_scales, m, w_codes, w_scales, k, d, y, acc,
                                       static_cast<hipStream_t>(stream)));
}

int rq_pack_f6(const uint8_t* codes, int64_t rows, int64_t d, uint8_t* out, void* stream) {
  if (rows < 0 || rows >= kMaxRows || d < 128 || d > RQ_MAX_D || d % 128 != 0) return RQ_ERR_SHAPE;
  if (rows == 0) return RQ_OK;
  if (codes == nullptr || out == nullptr) return RQ_ERR_NULL;
  if (!aligned16(codes) || !aligned16(out)) return RQ_ERR_ALIGN;
  return from_hip(rq::launch_pack_f6(codes, rows, d, out, static_cast<hipStream_t>(stream)));
}

int rq_w4a4_gemm_f6(const uint8_t* a_f6, const uint16_t* a_scales, int64_t m, const uint8_t* w_f6,
                    const uint16_t* w_scales, int64_t k, int64_t d, uint16_t* y, int32_t* acc,
                    void* stream) {
  if (m < 0 || k < 0 || d < 128 || d > RQ_MAX_D || d % 128 != 0) return RQ_ERR_SHAPE;
  if (m > kMaxTileRows) return RQ_ERR_SHAPE;
  if (k >= kMaxRows) return RQ_ERR_SHAPE;
  if (m == 0) return RQ_OK;
  if (k == 0) return RQ_ERR_SHAPE;
  if (a_f6 == nullptr || a_scales == nullptr || w_f6 == nullptr || w_scales == nullptr ||
      y == nullptr)
    return RQ_ERR_NULL;
  if (!aligned16(a_f6) || !aligned16(w_f6)) return RQ_ERR_ALIGN;
  return from_hip(rq::launch_w4a4_gemm_f6(a_f6, a_scales, m, w_f6, w_scales, k, d, y, acc,
                                          static_cast<hipStream_t>(stream)));
}

int rq_kv_rotate_quant(const uint16_t* k_in, const uint16_t* v_in, int64_t rows, int64_t head_dim,
                       const int8_t* signs, uint8_t* k_codes, uint16_t* k_scales,
                       uint8_t* v_codes, uint16_t* v_scales, void* stream) {
  if (head_dim != 128) return RQ_ERR_SHAPE;
  if (rows < 0 || rows >= kMaxRows) return RQ_ERR_SHAPE;
  if (rows == 0) return RQ_OK;
  if (k_in == nullptr || v_in == nullptr || k_codes == nullptr || k_scales == nullptr ||
      v_codes == nullptr || v_scales == nullptr)
    return RQ_ERR_NULL;
  if (!aligned16(k_in) || !aligned16(v_in) || !aligned16(k_codes) || !aligned16(v_codes))
    return RQ_ERR_ALIGN;
  if (signs != nullptr && !aligned16(signs)) return RQ_ERR_ALIGN;
  return from_hip(rq::launch_kv_rotate_quant(k_in, v_in, rows, signs, k_codes, k_scales, v_codes,
                                             v_scales, static_cast<hipStream_t>(stream)));
}

int rq_w4a8_gemm(const int8_t* a_codes, const uint16_t* a_scales, int64_t m,
                 const uint8_t* w_codes, const uint16_t* w_scales, int64_t k, int64_t d,
                 uint16_t* y, int32_t* acc, void* stream) {
  if (m < 0 || k < 0 || d < 64 || d > RQ_MAX_D || d % 64 != 0) return RQ_ERR_SHAPE;
  if (m > kMaxTileRows) return RQ_ERR_SHAPE;
  if (k >= kMaxRows) return RQ_ERR_SHAPE;
  if (m == 0) return RQ_OK;
  if (k == 0) return RQ_ERR_SHAPE;
  if (a_codes == nullptr || a_scales == nullptr || w_codes == nullptr || w_scales == nullptr ||
      y == nullptr)
    return RQ_ERR_NULL;
  if (!aligned16(a_codes) || !aligned16(w_codes)) return RQ_ERR_ALIGN;
  return from_hip(rq::launch_w4a8_gemm(a_codes, a_scales, m, w_codes, w_scales, k, d, y, acc,
                                       static_cast<hipStream_t>(stream)));
}

int rq_w4a4_gemm_asym(const uint8_t* a_codes, const uint16_t* a_scales, const uint8_t* a_zeros,
                      int64_t m, const uint8_t* w_codes, const uint16_t* w_scales,
                      const int32_t* w_sums, int64_t k, int64_t d, uint16_t* y, int32_t* acc,
                      void* stream) {
  if (m < 0 || k < 0 || d < 64 || d > RQ_MAX_D || d % 64 != 0) return RQ_ERR_SHAPE;
  if (m > kMaxTileRows) return RQ_ERR_SHAPE;
  if (k >= kMaxRows) return RQ_ERR_SHAPE;
  if (m == 0) return RQ_OK;
  if (k == 0) return RQ_ERR_SHAPE;
  if (a_codes == nullptr || a_scales == nullptr || a_zeros == nullptr || w_codes == nullptr ||
      w_scales == nullptr || w_sums == nullptr || y == nullptr)
    return RQ_ERR_NULL;
  if (!aligned16(a_codes) || !aligned16(w_codes)) return RQ_ERR_ALIGN;
  return from_hip(rq::launch_w4a4_gemm_asym(a_codes, a_scales, a_zeros, m, w_codes, w_scales,
                                            w_sums, k, d, y, acc,
                                            static_cast<hipStream_t>(stream)));
}

int rq_quantize_groups(const float* x, int64_t rows, int64_t n, int64_t group, uint8_t* codes,
                       uint16_t* scales, void* stream) {
  if (group != 32 && group != 64 && group != 128 && group != 256) return RQ_ERR_SHAPE;
  if (rows < 0 || rows >= kMaxRows || n < group || n % group != 0 || n > (1 << 20))
    return RQ_ERR_SHAPE;
  if (rows == 0) return RQ_OK;
  if (x == nullptr || codes == nullptr || scales == nullptr) return RQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(codes)) return RQ_ERR_ALIGN;
  return from_hip(rq::launch_quantize_groups(x, rows, n, (int)group, codes, scales,
                                             static_cast<hipStream_t>(stream)));
}

int rq_w4a4_gemm_grouped(const uint8_t* a_codes, const uint16_t* a_scales, int64_t m,
                         const uint8_t* w_codes, const uint16_t* w_group_scales, int64_t k,
                         int64_t d, uint16_t* y, int32_t* acc, void* stream) {
  if (m < 0 || k < 0 || d < 128 || d > RQ_MAX_D || d % 128 != 0) return RQ_ERR_SHAPE;
  if (m > kMaxTileRows) return RQ_ERR_SHAPE;
  if (k >= kMaxRows) return RQ_ERR_SHAPE;
  if (m == 0) return RQ_OK;
  if (k == 0) return RQ_ERR_SHAPE;
  if (a_codes == nullptr || a_scales == nullptr || w_codes == nullptr ||
      w_group_scales == nullptr || y == nullptr)
    return RQ_ERR_NULL;
  if (!aligned16(a_codes) || !aligned16(w_codes)) return RQ_ERR_ALIGN;
  return from_hip(rq::launch_w4a4_gemm_grouped(a_codes, a_scales, m, w_codes, w_group_scales, k,
                                               d, y, acc, static_cast<hipStream_t>(stream)));
}

size_t rq_linear_decode_workspace_size(int64_t m, int64_t d) {
  if (m < 0 || m > 16 || !is_pow2(d) || d < 512 || d > 8192) return 0;
  return rq::linear_decode_workspace_bytes(m, d);
}

int rq_linear_decode(const uint16_t* x, int64_t m, int64_t d, const int8_t* signs,
                     const uint8_t* w_codes, const uint16_t* w_scales, int64_t k, uint16_t* y,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (m < 0 || m > 16) return RQ_ERR_SHAPE;
  if (!is_pow2(d) || d < 512 || d > 8192) return RQ_ERR_SHAPE;
  if (k < 1 || k >= kMaxRows) return RQ_ERR_SHAPE;
  if (m == 0) return RQ_OK;
  if (x == nullptr || w_codes == nullptr || w_scales == nullptr || y == nullptr ||
      workspace == nullptr)
    return RQ_ERR_NULL;
  if (workspace_bytes < rq::linear_decode_workspace_bytes(m, d)) return RQ_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(w_codes) || !aligned16(workspace)) return RQ_ERR_ALIGN;
  if (signs != nullptr && !aligned16(signs)) return RQ_ERR_ALIGN;
  return from_hip(rq::launch_linear_decode(x, m, d, signs, w_codes, w_scales, k, y, workspace,
                                           static_cast<hipStream_t>(stream)));
}

int rq_linear_decode_w4a8(const uint16_t* x, int64_t m, int64_t d, const int8_t* signs,
                          const uint8_t* w_codes, const uint16_t* w_scales, int64_t k, uint16_t* y,
                          void* stream) {
  if (m < 0 || m > 4) return RQ_ERR_SHAPE;
  if (!is_pow2(d) || d < 512 || d > 8192) return RQ_ERR_SHAPE;
  if (k < 1 || k >= kMaxRows) return RQ_ERR_SHAPE;
  if (m == 0) return RQ_OK;
  if (x == nullptr || w_codes == nullptr || w_scales == nullptr || y == nullptr)
    return RQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_codes)) return RQ_ERR_ALIGN;
  if (signs != nullptr && !aligned16(signs)) return RQ_ERR_ALIGN;
  return from_hip(rq::launch_linear_decode_w4a8(x, m, d, signs, w_codes, w_scales, k, y,
                                                static_cast<hipStream_t>(stream)));
}

size_t rq_decode_attention_workspace_size(int64_t batch, int64_t kv_heads, int64_t group,
                                          int64_t seq) {
  if (batch < 1 || !attention_shape_ok(batch, kv_heads, group, seq)) return 0;
  return rq::decode_attention_workspace_bytes(batch, kv_heads, group, seq);
}

int rq_decode_attention(const uint16_t* q, const uint8_t* k_codes, const uint16_t* k_scales,
                        const uint8_t* v_codes, const uint16_t* v_scales, const int32_t* lengths,
                        int64_t batch, int64_t kv_heads, int64_t group, int64_t seq,
                        int64_t head_dim, const int8_t* signs, float sm_scale, uint16_t* out,
                        float* out_f32, void* workspace, size_t workspace_bytes, void* stream) {
  if (head_dim != 128) return RQ_ERR_SHAPE;
  if (!attention_shape_ok(batch, kv_heads, group, seq)) return RQ_ERR_SHAPE;
  if (!(sm_scale > 0.0f) || sm_scale > 1e30f) return RQ_ERR_SHAPE;
  if (batch == 0) return RQ_OK;
  if (q == nullptr || k_codes == nullptr || k_scales == nullptr || v_codes == nullptr ||
      v_scales == nullptr || out == nullptr || workspace == nullptr)
    return RQ_ERR_NULL;
  if (workspace_bytes < rq::decode_attention_workspace_bytes(batch, kv_heads, group, seq))
    return RQ_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k_codes) || !aligned16(v_codes) || !aligned16(workspace))
    return RQ_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(k_scales) & 3u) || (reinterpret_cast<uintptr_t>(v_scales) & 3u))
    return RQ_ERR_ALIGN;
  return from_hip(rq::launch_decode_attention(q, k_codes, k_scales, v_codes, v_scales, lengths,
                                              batch, kv_heads, group, seq, signs, sm_scale, out,
                                              out_f32, workspace,
                                              static_cast<hipStream_t>(stream)));
}

const char* rq_status_string(int status) {
  switch (status) {
    case RQ_OK: return "ok";
    case RQ_ERR_NULL: return "a required pointer is NULL";
    case RQ_ERR_SHAPE: return "a size is out of range or not a supported power of two";
    case RQ_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case RQ_ERR_DTYPE: return "unknown input dtype";
    case RQ_ERR_HIP: return "a HIP launch failed";
    default: return "unknown status";
  }
}

int rq_version(void) { return kVersion; }

}  // extern "C"
