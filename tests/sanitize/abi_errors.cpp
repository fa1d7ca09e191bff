// Host-side check of the C-ABI validation layer under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Built from csrc/rq_api.hip and csrc/noalloc.hip
// (host code only) with the launch stand-ins of launch_stubs.cpp, so no GPU
// is needed.  Every call below must be rejected (or be a no-op) before any
// launch: the driver checks each status and that no stand-in launcher ran.
// Besides the error paths of tests/test_abi.py it passes the extremes of
// every integer argument (INT64_MIN, INT64_MAX, values next to each limit),
// where an unguarded product or sum in the validation would overflow.
#include <stdint.h>
#include <stdio.h>

#include <cmath>
#include <limits>

#include "../../include/rq.h"

extern int stub_launches;

namespace {

int failures = 0, checks = 0;

void check(int got, int want, const char* what, int line) {
  ++checks;
  if (got != want) {
    ++failures;
    fprintf(stderr, "line %d: %s returned %d, expected %d\n", line, what, got, want);
  }
}
#define CHECK(call, want) check((call), (want), #call, __LINE__)

// Fake device addresses, never dereferenced (every call below stops in
// validation).
void* const A16 = reinterpret_cast<void*>(0x10000);
void* const A16b = reinterpret_cast<void*>(0x20000);
void* const MIS = reinterpret_cast<void*>(0x10008);
template <typename T>
T* p(void* v) { return static_cast<T*>(v); }

constexpr int64_t I64MAX = std::numeric_limits<int64_t>::max();
constexpr int64_t I64MIN = std::numeric_limits<int64_t>::min();
const int64_t kExtremes[] = {I64MIN, I64MIN + 1, -((int64_t)1 << 40), -1, I64MAX - 127, I64MAX};

}  // namespace

int main() {
  // ------------------------------------------------------------ rotation
  auto fq = [](void* x, int dtype, int64_t m, int64_t n, void* signs, void* codes, void* scales,
               void* rot) {
    return rq_fwht_quant(x, dtype, m, n, p<const int8_t>(signs), p<uint8_t>(codes),
                         p<uint16_t>(scales), p<float>(rot), nullptr);
  };
  CHECK(fq(A16, RQ_F16, 0, 256, nullptr, A16b, A16b, nullptr), RQ_OK);
  CHECK(fq(nullptr, RQ_F16, 0, 256, nullptr, A16b, A16b, nullptr), RQ_OK);
  CHECK(fq(nullptr, RQ_F16, 4, 256, nullptr, A16b, A16b, nullptr), RQ_ERR_NULL);
  CHECK(fq(A16, RQ_F16, 4, 256, nullptr, nullptr, A16b, nullptr), RQ_ERR_NULL);
  CHECK(fq(A16, RQ_F16, 4, 3, nullptr, A16b, A16b, nullptr), RQ_ERR_SHAPE);
  CHECK(fq(A16, RQ_F16, 4, 16384, nullptr, A16b, A16b, nullptr), RQ_ERR_SHAPE);
  CHECK(fq(A16, RQ_F16, 4, 28 * 2048, nullptr, A16b, A16b, nullptr), RQ_ERR_SHAPE);
  CHECK(fq(nullptr, RQ_F16, 4, 28672, nullptr, A16b, A16b, nullptr), RQ_ERR_NULL);
  CHECK(fq(A16, 7, 4, 256, nullptr, A16b, A16b, nullptr), RQ_ERR_DTYPE);
  CHECK(fq(MIS, RQ_F16, 4, 256, nullptr, A16b, A16b, nullptr), RQ_ERR_ALIGN);
  CHECK(fq(A16, RQ_F16, 4, 256, MIS, A16b, A16b, nullptr), RQ_ERR_ALIGN);
  CHECK(fq(A16, RQ_F16, 4, 256, nullptr, A16b, A16b, MIS), RQ_ERR_ALIGN);
  CHECK(fq(A16, RQ_F16, (int64_t)1 << 31, 256, nullptr, A16b, A16b, nullptr), RQ_ERR_SHAPE);
  for (int64_t e : kExtremes) {
    CHECK(fq(A16, RQ_F16, e, 256, nullptr, A16b, A16b, nullptr), RQ_ERR_SHAPE);
    CHECK(fq(A16, RQ_F16, 4, e, nullptr, A16b, A16b, nullptr), RQ_ERR_SHAPE);
    CHECK(rq_fold_weights(A16, RQ_F32, e, 4096, nullptr, p<uint8_t>(A16b), p<uint16_t>(A16b),
                          nullptr, nullptr),
          RQ_ERR_SHAPE);
    CHECK(rq_fwht_quant8(p<uint16_t>(A16), e, 4096, nullptr, p<int8_t>(A16b), p<uint16_t>(A16b),
                         nullptr, nullptr),
          RQ_ERR_SHAPE);
    CHECK(rq_fwht_quant8(p<uint16_t>(A16), 4, e, nullptr, p<int8_t>(A16b), p<uint16_t>(A16b),
                         nullptr, nullptr),
          RQ_ERR_SHAPE);
    CHECK(rq_fwht_quant_asym(p<uint16_t>(A16), e, 4096, nullptr, p<uint8_t>(A16b),
                             p<uint16_t>(A16b), p<uint8_t>(A16b), nullptr, nullptr),
          RQ_ERR_SHAPE);
    CHECK(rq_kv_rotate_quant(p<uint16_t>(A16), p<uint16_t>(A16), e, 128, nullptr,
                             p<uint8_t>(A16b), p<uint16_t>(A16b), p<uint8_t>(A16b),
                             p<uint16_t>(A16b), nullptr),
          RQ_ERR_SHAPE);
    CHECK(rq_kv_rotate_quant(p<uint16_t>(A16), p<uint16_t>(A16), 4, e, nullptr, p<uint8_t>(A16b),
                             p<uint16_t>(A16b), p<uint8_t>(A16b), p<uint16_t>(A16b), nullptr),
          RQ_ERR_SHAPE);
  }
  CHECK(rq_fold_weights(nullptr, RQ_F32, 8, 4096, nullptr, p<uint8_t>(A16b), p<uint16_t>(A16b),
                        nullptr, nullptr),
        RQ_ERR_NULL);
  CHECK(rq_fold_weights(A16, 2, 8, 4096, nullptr, p<uint8_t>(A16b), p<uint16_t>(A16b), nullptr,
                        nullptr),
        RQ_ERR_DTYPE);
  CHECK(rq_fwht_quant8(p<uint16_t>(A16), 4, 14336, nullptr, p<int8_t>(A16b), p<uint16_t>(A16b),
                       nullptr, nullptr),
        RQ_ERR_SHAPE);
  CHECK(rq_fwht_quant_asym(p<uint16_t>(A16), 4, 4096, nullptr, p<uint8_t>(A16b),
                           p<uint16_t>(A16b), nullptr, nullptr, nullptr),
        RQ_ERR_NULL);
  CHECK(rq_kv_rotate_quant(p<uint16_t>(MIS), p<uint16_t>(A16), 4, 128, nullptr, p<uint8_t>(A16b),
                           p<uint16_t>(A16b), p<uint8_t>(A16b), p<uint16_t>(A16b), nullptr),
        RQ_ERR_ALIGN);

  // ------------------------------------------------------------ GEMMs
  auto gemm = [](int64_t m, int64_t k, int64_t d, void* a, void* w, void* y) {
    return rq_w4a4_gemm(p<uint8_t>(a), p<uint16_t>(A16b), m, p<uint8_t>(w), p<uint16_t>(A16b), k,
                        d, p<uint16_t>(y), nullptr, nullptr, 0, nullptr);
  };
  auto gemm8 = [](int64_t m, int64_t k, int64_t d) {
    return rq_w4a8_gemm(p<int8_t>(A16), p<uint16_t>(A16b), m, p<uint8_t>(A16), p<uint16_t>(A16b),
                        k, d, p<uint16_t>(A16b), nullptr, nullptr);
  };
  auto gemma = [](int64_t m, int64_t k, int64_t d) {
    return rq_w4a4_gemm_asym(p<uint8_t>(A16), p<uint16_t>(A16b), p<uint8_t>(A16b), m,
                             p<uint8_t>(A16), p<uint16_t>(A16b), p<int32_t>(A16b), k, d,
                             p<uint16_t>(A16b), nullptr, nullptr);
  };
  auto gemm6 = [](int64_t m, int64_t k, int64_t d) {
    return rq_w4a4_gemm_f6(p<uint8_t>(A16), p<uint16_t>(A16b), m, p<uint8_t>(A16),
                           p<uint16_t>(A16b), k, d, p<uint16_t>(A16b), nullptr, nullptr);
  };
  auto pack6 = [](int64_t rows, int64_t d) {
    return rq_pack_f6(p<uint8_t>(A16), rows, d, p<uint8_t>(A16b), nullptr);
  };
  auto gemmg = [](int64_t m, int64_t k, int64_t d) {
    return rq_w4a4_gemm_grouped(p<uint8_t>(A16), p<uint16_t>(A16b), m, p<uint8_t>(A16),
                                p<uint16_t>(A16b), k, d, p<uint16_t>(A16b), nullptr, nullptr);
  };
  CHECK((int)rq_w4a4_gemm_workspace_size(2048, 28672, 8192), 0);
  CHECK(gemm(0, 64, 4096, A16, A16, A16b), RQ_OK);
  CHECK(gemm(4, 64, 4096, nullptr, A16, A16b), RQ_ERR_NULL);
  CHECK(gemm(4, 64, 4096, A16, A16, nullptr), RQ_ERR_NULL);
  CHECK(gemm(4, 64, 96, A16, A16, A16b), RQ_ERR_SHAPE);
  CHECK(gemm(4, 64, 32768 + 64, A16, A16, A16b), RQ_ERR_SHAPE);
  CHECK(gemm(4, 0, 4096, A16, A16, A16b), RQ_ERR_SHAPE);
  CHECK(gemm((int64_t)128 * 65536, 64, 4096, A16, A16, A16b), RQ_ERR_SHAPE);
  CHECK(gemm(4, 64, 4096, MIS, A16, A16b), RQ_ERR_ALIGN);
  CHECK(gemm(4, 64, 4096, A16, MIS, A16b), RQ_ERR_ALIGN);
  for (int64_t e : kExtremes) {
    CHECK(gemm(e, 64, 4096, A16, A16, A16b), RQ_ERR_SHAPE);
    CHECK(gemm(4, e, 4096, A16, A16, A16b), RQ_ERR_SHAPE);
    CHECK(gemm(4, 64, e, A16, A16, A16b), RQ_ERR_SHAPE);
    CHECK(gemm8(e, 64, 4096), RQ_ERR_SHAPE);
    CHECK(gemm8(4, e, 4096), RQ_ERR_SHAPE);
    CHECK(gemm8(4, 64, e), RQ_ERR_SHAPE);
    CHECK(gemma(e, 64, 4096), RQ_ERR_SHAPE);
    CHECK(gemma(4, e, 4096), RQ_ERR_SHAPE);
    CHECK(gemma(4, 64, e), RQ_ERR_SHAPE);
    CHECK(gemm6(e, 64, 4096), RQ_ERR_SHAPE);
    CHECK(gemm6(4, e, 4096), RQ_ERR_SHAPE);
    CHECK(gemm6(4, 64, e), RQ_ERR_SHAPE);
    CHECK(pack6(e, 4096), RQ_ERR_SHAPE);
    CHECK(pack6(4, e), RQ_ERR_SHAPE);
    CHECK(gemmg(e, 64, 4096), RQ_ERR_SHAPE);
    CHECK(gemmg(4, e, 4096), RQ_ERR_SHAPE);
    CHECK(gemmg(4, 64, e), RQ_ERR_SHAPE);
    CHECK(rq_weight_code_sums(p<uint8_t>(A16), e, 4096, p<int32_t>(A16b), nullptr), RQ_ERR_SHAPE);
    CHECK(rq_weight_code_sums(p<uint8_t>(A16), 4, e, p<int32_t>(A16b), nullptr), RQ_ERR_SHAPE);
    CHECK(rq_quantize_groups(p<float>(A16), e, 4096, 128, p<uint8_t>(A16b), p<uint16_t>(A16b),
                             nullptr),
          RQ_ERR_SHAPE);
    CHECK(rq_quantize_groups(p<float>(A16), 4, e, 128, p<uint8_t>(A16b), p<uint16_t>(A16b),
                             nullptr),
          RQ_ERR_SHAPE);
    CHECK(rq_quantize_groups(p<float>(A16), 4, 4096, e, p<uint8_t>(A16b), p<uint16_t>(A16b),
                             nullptr),
          RQ_ERR_SHAPE);
  }
  CHECK(gemm8(4, 64, 96), RQ_ERR_SHAPE);
  CHECK(gemm6(4, 64, 192), RQ_ERR_SHAPE);
  CHECK(gemm6(4, 0, 4096), RQ_ERR_SHAPE);
  CHECK(gemm6(0, 64, 4096), RQ_OK);
  CHECK(pack6(0, 4096), RQ_OK);
  CHECK(pack6(4, 4160), RQ_ERR_SHAPE);
  CHECK(rq_pack_f6(p<uint8_t>(MIS), 4, 4096, p<uint8_t>(A16b), nullptr), RQ_ERR_ALIGN);
  CHECK(rq_pack_f6(p<uint8_t>(A16), 4, 4096, nullptr, nullptr), RQ_ERR_NULL);
  CHECK(gemma(4, 0, 4096), RQ_ERR_SHAPE);
  CHECK(gemmg(4, 64, 192), RQ_ERR_SHAPE);
  CHECK(gemmg(0, 64, 4096), RQ_OK);
  CHECK(rq_weight_code_sums(p<uint8_t>(A16), 0, 4096, p<int32_t>(A16b), nullptr), RQ_OK);
  CHECK(rq_weight_code_sums(p<uint8_t>(MIS), 4, 4096, p<int32_t>(A16b), nullptr), RQ_ERR_ALIGN);
  CHECK(rq_quantize_groups(p<float>(A16), 4, 4000, 128, p<uint8_t>(A16b), p<uint16_t>(A16b),
                           nullptr),
        RQ_ERR_SHAPE);

  // ------------------------------------------------------------ decode linears
  const size_t need = rq_linear_decode_workspace_size(4, 4096);
  CHECK((int)need, 4 * 2048 + 64);
  auto ld = [need](int64_t m, int64_t d, int64_t k, void* ws, size_t nbytes) {
    return rq_linear_decode(p<uint16_t>(A16), m, d, nullptr, p<uint8_t>(A16), p<uint16_t>(A16b),
                            k, p<uint16_t>(A16b), ws, nbytes, nullptr);
  };
  CHECK(ld(0, 4096, 64, A16b, need), RQ_OK);
  CHECK(ld(17, 4096, 64, A16b, need), RQ_ERR_SHAPE);
  CHECK(ld(4, 14336, 64, A16b, need), RQ_ERR_SHAPE);
  CHECK(ld(4, 4096, 64, A16b, need - 1), RQ_ERR_SHAPE);
  CHECK(ld(4, 4096, 64, nullptr, need), RQ_ERR_NULL);
  CHECK(ld(4, 4096, 64, MIS, need), RQ_ERR_ALIGN);
  for (int64_t e : kExtremes) {
    CHECK((int)rq_linear_decode_workspace_size(e, 4096), 0);
    CHECK((int)rq_linear_decode_workspace_size(4, e), 0);
    CHECK(ld(e, 4096, 64, A16b, need), RQ_ERR_SHAPE);
    CHECK(ld(4, e, 64, A16b, need), RQ_ERR_SHAPE);
    CHECK(ld(4, 4096, e, A16b, need), RQ_ERR_SHAPE);
    CHECK(rq_linear_decode_noalloc(p<uint16_t>(A16), e, 4096, nullptr, p<uint8_t>(A16),
                                   p<uint16_t>(A16b), 64, p<uint16_t>(A16b), nullptr),
          RQ_ERR_SHAPE);
    CHECK(rq_linear_decode_noalloc(p<uint16_t>(A16), 4, e, nullptr, p<uint8_t>(A16),
                                   p<uint16_t>(A16b), 64, p<uint16_t>(A16b), nullptr),
          RQ_ERR_SHAPE);
    CHECK(rq_linear_decode_noalloc(p<uint16_t>(A16), 4, 4096, nullptr, p<uint8_t>(A16),
                                   p<uint16_t>(A16b), e, p<uint16_t>(A16b), nullptr),
          RQ_ERR_SHAPE);
    CHECK(rq_linear_decode_w4a8(p<uint16_t>(A16), e, 4096, nullptr, p<uint8_t>(A16),
                                p<uint16_t>(A16b), 64, p<uint16_t>(A16b), nullptr),
          RQ_ERR_SHAPE);
    CHECK(rq_linear_decode_w4a8(p<uint16_t>(A16), 4, e, nullptr, p<uint8_t>(A16),
                                p<uint16_t>(A16b), 64, p<uint16_t>(A16b), nullptr),
          RQ_ERR_SHAPE);
    CHECK(rq_linear_decode_w4a8(p<uint16_t>(A16), 4, 4096, nullptr, p<uint8_t>(A16),
                                p<uint16_t>(A16b), e, p<uint16_t>(A16b), nullptr),
          RQ_ERR_SHAPE);
  }
  CHECK(rq_linear_decode_noalloc(p<uint16_t>(A16), 0, 4096, nullptr, p<uint8_t>(A16),
                                 p<uint16_t>(A16b), 64, p<uint16_t>(A16b), nullptr),
        RQ_OK);
  CHECK(rq_linear_decode_noalloc(nullptr, 4, 4096, nullptr, p<uint8_t>(A16), p<uint16_t>(A16b),
                                 64, p<uint16_t>(A16b), nullptr),
        RQ_ERR_NULL);
  CHECK(rq_linear_decode_noalloc(p<uint16_t>(MIS), 4, 4096, nullptr, p<uint8_t>(A16),
                                 p<uint16_t>(A16b), 64, p<uint16_t>(A16b), nullptr),
        RQ_ERR_ALIGN);
  CHECK(rq_linear_decode_w4a8(p<uint16_t>(A16), 5, 4096, nullptr, p<uint8_t>(A16),
                              p<uint16_t>(A16b), 64, p<uint16_t>(A16b), nullptr),
        RQ_ERR_SHAPE);
  CHECK(rq_linear_decode_w4a8(p<uint16_t>(A16), 4, 4096, p<int8_t>(MIS), p<uint8_t>(A16),
                              p<uint16_t>(A16b), 64, p<uint16_t>(A16b), nullptr),
        RQ_ERR_ALIGN);

  // ------------------------------------------------------------ decode attention
  const size_t wneed = rq_decode_attention_workspace_size(2, 8, 4, 4096);
  CHECK(wneed > 0 && wneed % 16 == 0, 1);
  auto att = [wneed](int64_t B, int64_t H, int64_t G, int64_t S, int64_t D, float sm, void* q,
                     void* ks, size_t nbytes) {
    return rq_decode_attention(p<uint16_t>(q), p<uint8_t>(A16), p<uint16_t>(ks), p<uint8_t>(A16),
                               p<uint16_t>(A16b), nullptr, B, H, G, S, D, nullptr, sm,
                               p<uint16_t>(A16b), nullptr, A16b, nbytes, nullptr);
  };
  CHECK(att(0, 8, 4, 4096, 128, 0.088f, A16, A16b, wneed), RQ_OK);
  CHECK(att(2, 8, 4, 4096, 64, 0.088f, A16, A16b, wneed), RQ_ERR_SHAPE);
  CHECK(att(2, 8, 9, 4096, 128, 0.088f, A16, A16b, wneed), RQ_ERR_SHAPE);
  CHECK(att(2, 8, 4, 4095, 128, 0.088f, A16, A16b, wneed), RQ_ERR_SHAPE);
  CHECK(att(2, 8, 4, 4096, 128, 0.0f, A16, A16b, wneed), RQ_ERR_SHAPE);
  CHECK(att(2, 8, 4, 4096, 128, std::nanf(""), A16, A16b, wneed), RQ_ERR_SHAPE);
  CHECK(att(2, 8, 4, 4096, 128, std::numeric_limits<float>::infinity(), A16, A16b, wneed),
        RQ_ERR_SHAPE);
  CHECK(att(2, 8, 4, 4096, 128, 0.088f, A16, A16b, wneed - 1), RQ_ERR_SHAPE);
  CHECK(att(65536, 1, 4, 4096, 128, 0.088f, A16, A16b, wneed), RQ_ERR_SHAPE);
  CHECK(att(2, 8, 4, 4096, 128, 0.088f, nullptr, A16b, wneed), RQ_ERR_NULL);
  CHECK(att(2, 8, 4, 4096, 128, 0.088f, MIS, A16b, wneed), RQ_ERR_ALIGN);
  CHECK(att(2, 8, 4, 4096, 128, 0.088f, A16, reinterpret_cast<void*>(0x20002), wneed),
        RQ_ERR_ALIGN);
  for (int64_t e : kExtremes) {
    CHECK((int)rq_decode_attention_workspace_size(e, 8, 4, 4096), 0);
    CHECK((int)rq_decode_attention_workspace_size(2, e, 4, 4096), 0);
    CHECK((int)rq_decode_attention_workspace_size(2, 8, e, 4096), 0);
    CHECK((int)rq_decode_attention_workspace_size(2, 8, 4, e), 0);
    CHECK((int)rq_decode_attention_workspace_size(e, e, 4, 4096), 0);
    CHECK(att(e, 8, 4, 4096, 128, 0.088f, A16, A16b, wneed), RQ_ERR_SHAPE);
    CHECK(att(2, e, 4, 4096, 128, 0.088f, A16, A16b, wneed), RQ_ERR_SHAPE);
    CHECK(att(e, e, 4, 4096, 128, 0.088f, A16, A16b, wneed), RQ_ERR_SHAPE);
    CHECK(att(2, 8, e, 4096, 128, 0.088f, A16, A16b, wneed), RQ_ERR_SHAPE);
    CHECK(att(2, 8, 4, e, 128, 0.088f, A16, A16b, wneed), RQ_ERR_SHAPE);
    CHECK(att(2, 8, 4, 4096, e, 0.088f, A16, A16b, wneed), RQ_ERR_SHAPE);
  }
  CHECK((int)rq_decode_attention_workspace_size(65536, 1, 4, 4096), 0);
  CHECK((int)rq_decode_attention_workspace_size(4096, 4096, 4, 4096), 0);

  // ------------------------------------------------------------ strings
  for (int st = -2; st < 8; ++st) CHECK(rq_status_string(st) != nullptr, 1);
  CHECK(rq_version(), 10000);

  CHECK(stub_launches, 0);  // nothing above may reach a launch
  printf("%s: %d checks, %d failures\n", failures ? "FAILED" : "ok", checks, failures);
  return failures ? 1 : 0;
}
