// Stand-ins for the kernel launchers (csrc/*.hip) when the C-ABI layer is
// built alone for the host sanitizers: every launcher counts its call and
// fails, so a call that passes validation shows up in `stub_launches` and
// returns RQ_ERR_HIP.  The two workspace-size helpers compute what the real
// ones compute for the shapes the driver uses.
#include <hip/hip_runtime.h>

#include "../../rotation_w4a4_quantization_amd/csrc/rq_internal.h"

int stub_launches = 0;

namespace rq {

int cu_count() { return 256; }

#define RQ_STUB_LAUNCH \
  {                    \
    ++stub_launches;   \
    return hipErrorInvalidValue; \
  }

hipError_t launch_fwht_quant(const void*, bool, int64_t, int, const int8_t*, uint8_t*, uint16_t*,
                             float*, hipStream_t) RQ_STUB_LAUNCH
hipError_t launch_fwht_quant8(const uint16_t*, int64_t, int, const int8_t*, int8_t*, uint16_t*,
                              float*, hipStream_t) RQ_STUB_LAUNCH
hipError_t launch_fwht_quant_asym(const uint16_t*, int64_t, int, const int8_t*, uint8_t*,
                                  uint16_t*, uint8_t*, float*, hipStream_t) RQ_STUB_LAUNCH
hipError_t launch_kv_rotate_quant(const uint16_t*, const uint16_t*, int64_t, const int8_t*,
                                  uint8_t*, uint16_t*, uint8_t*, uint16_t*, hipStream_t)
    RQ_STUB_LAUNCH
hipError_t launch_w4a4_gemm(const uint8_t*, const uint16_t*, int64_t, const uint8_t*,
                            const uint16_t*, int64_t, int64_t, uint16_t*, int32_t*, hipStream_t)
    RQ_STUB_LAUNCH
hipError_t launch_pack_f6(const uint8_t*, int64_t, int64_t, uint8_t*, hipStream_t) RQ_STUB_LAUNCH
hipError_t launch_w4a4_gemm_f6(const uint8_t*, const uint16_t*, int64_t, const uint8_t*,
                               const uint16_t*, int64_t, int64_t, uint16_t*, int32_t*, hipStream_t)
    RQ_STUB_LAUNCH
hipError_t launch_w4a8_gemm(const int8_t*, const uint16_t*, int64_t, const uint8_t*,
                            const uint16_t*, int64_t, int64_t, uint16_t*, int32_t*, hipStream_t)
    RQ_STUB_LAUNCH
hipError_t launch_w4a4_gemm_asym(const uint8_t*, const uint16_t*, const uint8_t*, int64_t,
                                 const uint8_t*, const uint16_t*, const int32_t*, int64_t, int64_t,
                                 uint16_t*, int32_t*, hipStream_t) RQ_STUB_LAUNCH
hipError_t launch_weight_code_sums(const uint8_t*, int64_t, int64_t, int32_t*, hipStream_t)
    RQ_STUB_LAUNCH
hipError_t launch_quantize_groups(const float*, int64_t, int64_t, int, uint8_t*, uint16_t*,
                                  hipStream_t) RQ_STUB_LAUNCH
hipError_t launch_w4a4_gemm_grouped(const uint8_t*, const uint16_t*, int64_t, const uint8_t*,
                                    const uint16_t*, int64_t, int64_t, uint16_t*, int32_t*,
                                    hipStream_t) RQ_STUB_LAUNCH
hipError_t launch_decode_attention(const uint16_t*, const uint8_t*, const uint16_t*,
                                   const uint8_t*, const uint16_t*, const int32_t*, int64_t,
                                   int64_t, int64_t, int64_t, const int8_t*, float, uint16_t*,
                                   float*, void*, hipStream_t) RQ_STUB_LAUNCH
hipError_t launch_linear_decode(const uint16_t*, int64_t, int64_t, const int8_t*, const uint8_t*,
                                const uint16_t*, int64_t, uint16_t*, void*, hipStream_t)
    RQ_STUB_LAUNCH
hipError_t launch_linear_decode_w4a8(const uint16_t*, int64_t, int64_t, const int8_t*,
                                     const uint8_t*, const uint16_t*, int64_t, uint16_t*,
                                     hipStream_t) RQ_STUB_LAUNCH

size_t linear_decode_workspace_bytes(int64_t m, int64_t d) {
  return (size_t)m * (size_t)(d / 2) + 64;
}
size_t decode_attention_workspace_bytes(int64_t batch, int64_t kv_heads, int64_t group,
                                        int64_t seq) {
  (void)seq;  // one split per KV head in this stand-in
  return (size_t)(batch * kv_heads * group) * 132 * sizeof(float);
}

}  // namespace rq
