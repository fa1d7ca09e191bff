// rq_linear_decode_noalloc: rq_linear_decode for callers that cannot
// allocate device memory (HIP graph capture, tight serving loops, harnesses
// that forbid allocation).  The activation codes and scales that
// rq_linear_decode keeps in its caller's workspace go to a file-scope device
// array instead; its device address is looked up once per device, with that
// device current, and only that address is handed to the kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/rq.h"
#include "rq_internal.h"

// 16 tokens of width 8192: codes, then fp16 scales.  Each GPU holds its own
// copy for the life of the process; every call on that GPU shares it.
static __device__ __align__(256) unsigned char scratch[RQ_NOALLOC_SCRATCH_BYTES];

namespace {

void* scratch_address() {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" int rq_linear_decode_noalloc(const uint16_t* x, int64_t m, int64_t d,
                                        const int8_t* signs, const uint8_t* w_codes,
                                        const uint16_t* w_scales, int64_t k, uint16_t* y,
                                        void* stream) {
  if (m < 0 || m > 16) return RQ_ERR_SHAPE;
  if (!is_pow2(d) || d < 512 || d > 8192) return RQ_ERR_SHAPE;
  if (k < 1 || k >= ((int64_t)1 << 31)) return RQ_ERR_SHAPE;
  if (m == 0) return RQ_OK;
  if (rq::linear_decode_workspace_bytes(m, d) > (size_t)RQ_NOALLOC_SCRATCH_BYTES) return RQ_ERR_SHAPE;
  if (x == nullptr || w_codes == nullptr || w_scales == nullptr || y == nullptr)
    return RQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_codes)) return RQ_ERR_ALIGN;
  if (signs != nullptr && !aligned16(signs)) return RQ_ERR_ALIGN;
  void* ws = scratch_address();
  if (ws == nullptr) return RQ_ERR_HIP;
  const hipError_t e = rq::launch_linear_decode(x, m, d, signs, w_codes, w_scales, k, y, ws,
                                                static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RQ_OK : RQ_ERR_HIP;
}
