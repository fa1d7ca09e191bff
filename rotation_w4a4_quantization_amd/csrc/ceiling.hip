// Ceiling probes of the machine the hot path runs on (declared in
// include/rq_ceiling.h): a read-only stream and a copy with the access
// pattern of the memory-bound kernels (16-byte nontemporal loads, 1 KB per
// wavefront instruction), a loop of int8 MFMAs on register operands, and
// issue-rate loops of the instruction classes the kernels are made of.
// They measure what the hardware delivers at the sizes the hot path moves,
// so every roofline fraction can be set against a practical ceiling as well
// as the published peak.  They compute nothing of the method.
#include <hip/hip_runtime.h>

#include "../../include/rq_ceiling.h"
#include "rq_internal.h"

namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));

// Grid-stride read of n16 16-byte chunks; each workgroup writes one word
// (the xor of everything it read) so the loads cannot be dropped.
__global__ __launch_bounds__(256) void read_stream_kernel(const v4u* __restrict__ src, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  __shared__ uint32_t red[4];
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const v4u a = __builtin_nontemporal_load(src + i);
    const v4u b = __builtin_nontemporal_load(src + i + stride);
    const v4u c = __builtin_nontemporal_load(src + i + 2 * stride);
    const v4u d = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3] ^ c[0] ^ c[1] ^ c[2] ^ c[3] ^
           d[0] ^ d[1] ^ d[2] ^ d[3];
  }
  for (; i < n16; i += stride) {
    const v4u a = __builtin_nontemporal_load(src + i);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

__global__ __launch_bounds__(256) void copy_stream_kernel(const v4u* __restrict__ src,
                                                          v4u* __restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// Each wavefront runs `iters` rounds of 8 independent v_mfma_i32_16x16x64_i8
// (eight accumulator tiles in VGPRs, so consecutive MFMAs never wait on each
// other; the MFMAs are written as one asm block so that the compiler keeps
// the accumulators in place instead of copying them between register files),
// then writes its accumulators.
__global__ __launch_bounds__(256) void mfma_i8_loop_kernel(int32_t* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  v4i a, b;  // 16 int8 operands per lane
  for (int j = 0; j < 4; ++j) {
    a[j] = 0x01020304 * (lane + j + 1);
    b[j] = 0x05060708 ^ (lane * 131 + j);
  }
  v4i c0 = {0, 0, 0, 0}, c1 = c0, c2 = c0, c3 = c0, c4 = c0, c5 = c0, c6 = c0, c7 = c0;
  for (int it = 0; it < iters; ++it) {
    asm volatile(
        "v_mfma_i32_16x16x64_i8 %0, %8, %9, %0\n"
        "v_mfma_i32_16x16x64_i8 %1, %8, %9, %1\n"
        "v_mfma_i32_16x16x64_i8 %2, %8, %9, %2\n"
        "v_mfma_i32_16x16x64_i8 %3, %8, %9, %3\n"
        "v_mfma_i32_16x16x64_i8 %4, %8, %9, %4\n"
        "v_mfma_i32_16x16x64_i8 %5, %8, %9, %5\n"
        "v_mfma_i32_16x16x64_i8 %6, %8, %9, %6\n"
        "v_mfma_i32_16x16x64_i8 %7, %8, %9, %7\n"
        : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3), "+v"(c4), "+v"(c5), "+v"(c6), "+v"(c7)
        : "v"(a), "v"(b));
  }
  // the results are read only after the last MFMA has written them
  asm volatile("s_nop 7\n s_nop 7\n s_nop 7" ::: "memory");
  const v4i s = c0 + c1 + c2 + c3 + c4 + c5 + c6 + c7;
  reinterpret_cast<v4i*>(out)[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// The same loop on the 6-bit matrix unit: 8 independent
// v_mfma_f32_16x16x128_f8f6f4 with E3M2 operands (format 3 for A and B),
// each lane's six operand registers holding 32 random INT4 codes -8..7 as
// E3M2 values (the operand values the F6 GEMM multiplies; the clock the
// matrix unit holds depends on them).
typedef int v6i __attribute__((ext_vector_type(6)));
typedef float v4f __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint32_t loop_hash(uint32_t x) {
  x ^= x >> 16; x *= 0x7feb352du; x ^= x >> 15; x *= 0x846ca68bu; x ^= x >> 16;
  return x;
}
__global__ __launch_bounds__(256) void mfma_f6_loop_kernel(int32_t* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  // E3M2 codes of q = -8..7 (index q + 8)
  constexpr unsigned char kE3M2[16] = {56, 55, 54, 53, 52, 50, 48, 44, 0, 12, 16, 18, 20, 21, 22, 23};
  v6i a = {0, 0, 0, 0, 0, 0}, b = a;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const uint32_t ca = kE3M2[loop_hash(lane * 977u + j * 131u + 17u) & 15u];
    const uint32_t cb = kE3M2[loop_hash(lane * 977u + 62531u + j * 131u) & 15u];
    const int pos = 6 * j;
    a[pos >> 5] |= (int)(ca << (pos & 31));
    b[pos >> 5] |= (int)(cb << (pos & 31));
    if ((pos & 31) > 26) {
      a[(pos >> 5) + 1] |= (int)(ca >> (32 - (pos & 31)));
      b[(pos >> 5) + 1] |= (int)(cb >> (32 - (pos & 31)));
    }
  }
  v4f c0 = {0, 0, 0, 0}, c1 = c0, c2 = c0, c3 = c0, c4 = c0, c5 = c0, c6 = c0, c7 = c0;
  for (int it = 0; it < iters; ++it) {
    asm volatile(
        "v_mfma_f32_16x16x128_f8f6f4 %0, %8, %9, %0 cbsz:3 blgp:3\n"
        "v_mfma_f32_16x16x128_f8f6f4 %1, %8, %9, %1 cbsz:3 blgp:3\n"
        "v_mfma_f32_16x16x128_f8f6f4 %2, %8, %9, %2 cbsz:3 blgp:3\n"
        "v_mfma_f32_16x16x128_f8f6f4 %3, %8, %9, %3 cbsz:3 blgp:3\n"
        "v_mfma_f32_16x16x128_f8f6f4 %4, %8, %9, %4 cbsz:3 blgp:3\n"
        "v_mfma_f32_16x16x128_f8f6f4 %5, %8, %9, %5 cbsz:3 blgp:3\n"
        "v_mfma_f32_16x16x128_f8f6f4 %6, %8, %9, %6 cbsz:3 blgp:3\n"
        "v_mfma_f32_16x16x128_f8f6f4 %7, %8, %9, %7 cbsz:3 blgp:3\n"
        : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3), "+v"(c4), "+v"(c5), "+v"(c6), "+v"(c7)
        : "v"(a), "v"(b));
  }
  // the results are read only after the last MFMA has written them
  asm volatile("s_nop 7\n s_nop 7\n s_nop 7" ::: "memory");
  const v4f s = c0 + c1 + c2 + c3 + c4 + c5 + c6 + c7;
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = (int32_t)(s[0] + s[1] + s[2] + s[3]);
}

// Issue-rate loops: each wavefront runs `iters` rounds of one block of
// register-only instructions, independent of each other inside the round.
//   KIND 0: 8 v_mfma_i32_16x16x64_i8 (eight accumulators);
//   KIND 1: 32 (v_cvt_f32_i32, v_fmac_f32) pairs, the per-group epilogue of
//           the grouped GEMM;
//   KIND 2: both blocks in the same round;
//   KIND 3: 32 v_fmac_f32 (plain fp32, two source registers);
//   KIND 4: 32 v_fmac_f32_dpp quad_perm:[1,0,3,2], the lane-crossing
//           butterfly of the rotation.
// Every wavefront stores one float per lane so nothing is dropped.
template <int KIND>
__global__ __launch_bounds__(256) void issue_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  float f[32];
  int iv[32];
  for (int i = 0; i < 32; ++i) {
    f[i] = (float)(lane + i) * 0.25f;
    iv[i] = lane * 3 + i;
  }
  v4i a, b;
  for (int j = 0; j < 4; ++j) {
    a[j] = 0x01020304 * (lane + j + 1);
    b[j] = 0x05060708 ^ (lane * 131 + j);
  }
  v4i c0 = {0, 0, 0, 0}, c1 = c0, c2 = c0, c3 = c0, c4 = c0, c5 = c0, c6 = c0, c7 = c0;
  const float g = lane & 1 ? -1.0f : 1.0f;
  for (int it = 0; it < iters; ++it) {
    if constexpr (KIND == 0 || KIND == 2) {  // one asm block: the accumulators stay in place
      asm volatile(
          "v_mfma_i32_16x16x64_i8 %0, %8, %9, %0\n"
          "v_mfma_i32_16x16x64_i8 %1, %8, %9, %1\n"
          "v_mfma_i32_16x16x64_i8 %2, %8, %9, %2\n"
          "v_mfma_i32_16x16x64_i8 %3, %8, %9, %3\n"
          "v_mfma_i32_16x16x64_i8 %4, %8, %9, %4\n"
          "v_mfma_i32_16x16x64_i8 %5, %8, %9, %5\n"
          "v_mfma_i32_16x16x64_i8 %6, %8, %9, %6\n"
          "v_mfma_i32_16x16x64_i8 %7, %8, %9, %7\n"
          : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3), "+v"(c4), "+v"(c5), "+v"(c6), "+v"(c7)
          : "v"(a), "v"(b));
    }
    if constexpr (KIND == 1 || KIND == 2) {
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        asm volatile("" : "+v"(iv[j]));  // a fresh integer every round
        f[j] = __builtin_fmaf((float)iv[j], g, f[j]);
      }
    }
    if constexpr (KIND == 3 || KIND == 4) {
#pragma unroll
      for (int q = 0; q < 32; q += 8) {
        if constexpr (KIND == 3) {
          asm volatile(
              "v_fmac_f32 %0, %0, %8\n v_fmac_f32 %1, %1, %8\n v_fmac_f32 %2, %2, %8\n"
              "v_fmac_f32 %3, %3, %8\n v_fmac_f32 %4, %4, %8\n v_fmac_f32 %5, %5, %8\n"
              "v_fmac_f32 %6, %6, %8\n v_fmac_f32 %7, %7, %8"
              : "+v"(f[q]), "+v"(f[q + 1]), "+v"(f[q + 2]), "+v"(f[q + 3]), "+v"(f[q + 4]),
                "+v"(f[q + 5]), "+v"(f[q + 6]), "+v"(f[q + 7])
              : "v"(g));
        } else {
          asm volatile(
              "s_nop 1\n"
              "v_fmac_f32_dpp %0, %0, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n"
              "v_fmac_f32_dpp %1, %1, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n"
              "v_fmac_f32_dpp %2, %2, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n"
              "v_fmac_f32_dpp %3, %3, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n"
              "v_fmac_f32_dpp %4, %4, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n"
              "v_fmac_f32_dpp %5, %5, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n"
              "v_fmac_f32_dpp %6, %6, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n"
              "v_fmac_f32_dpp %7, %7, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
              : "+v"(f[q]), "+v"(f[q + 1]), "+v"(f[q + 2]), "+v"(f[q + 3]), "+v"(f[q + 4]),
                "+v"(f[q + 5]), "+v"(f[q + 6]), "+v"(f[q + 7])
              : "v"(g));
        }
      }
    }
  }
  // the accumulators are read only after the last MFMA has written them
  asm volatile("s_nop 7\n s_nop 7\n s_nop 7" ::: "memory");
  float sum = 0.0f;
  const v4i cs = c0 + c1 + c2 + c3 + c4 + c5 + c6 + c7;
  sum += (float)(cs[0] ^ cs[1] ^ cs[2] ^ cs[3]);
  for (int i = 0; i < 32; ++i) sum += f[i];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = sum;
}

int grid_for(int64_t n16) {
  const int64_t want = (n16 + 255) / 256;
  const int64_t cap = (int64_t)rq::cu_count() * 16;
  return (int)(want < cap ? (want > 0 ? want : 1) : cap);
}

}  // namespace

extern "C" {

size_t rq_ceiling_read_sink_words(void) { return (size_t)rq::cu_count() * 16; }

int rq_ceiling_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (src == nullptr || sink == nullptr) return 1;
  if ((reinterpret_cast<uintptr_t>(src) & 15u) != 0 || bytes % 16 != 0) return 3;
  if (bytes == 0) return 0;
  const int64_t n16 = (int64_t)(bytes / 16);
  hipLaunchKernelGGL(read_stream_kernel, dim3(grid_for(n16)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const v4u*>(src), n16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

int rq_ceiling_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (src == nullptr || dst == nullptr) return 1;
  if ((reinterpret_cast<uintptr_t>(src) & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(dst) & 15u) != 0 || bytes % 16 != 0)
    return 3;
  if (bytes == 0) return 0;
  const int64_t n16 = (int64_t)(bytes / 16);
  hipLaunchKernelGGL(copy_stream_kernel, dim3(grid_for(n16)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const v4u*>(src),
                     static_cast<v4u*>(dst), n16);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

size_t rq_ceiling_mfma_out_words(int64_t waves_per_simd) {
  if (waves_per_simd < 1 || waves_per_simd > 8) return 0;
  return (size_t)rq::cu_count() * (size_t)waves_per_simd * 256 * 4;
}

int64_t rq_ceiling_mfma_i8(int32_t* out, int64_t waves_per_simd, int64_t iters, void* stream) {
  if (out == nullptr) return -1;
  if (waves_per_simd < 1 || waves_per_simd > 8 || iters < 1 || iters > (1 << 24)) return -2;
  const int blocks = rq::cu_count() * (int)waves_per_simd;  // 4 wavefronts per block
  hipLaunchKernelGGL(mfma_i8_loop_kernel, dim3(blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), out, (int)iters);
  if (hipGetLastError() != hipSuccess) return -5;
  // integer operations: 2 * 16 * 16 * 64 per MFMA, 8 MFMAs per round per wavefront
  return (int64_t)blocks * 4 * iters * 8 * (2 * 16 * 16 * 64);
}

int64_t rq_ceiling_mfma_f6(int32_t* out, int64_t waves_per_simd, int64_t iters, void* stream) {
  if (out == nullptr) return -1;
  if (waves_per_simd < 1 || waves_per_simd > 8 || iters < 1 || iters > (1 << 24)) return -2;
  const int blocks = rq::cu_count() * (int)waves_per_simd;  // 4 wavefronts per block
  hipLaunchKernelGGL(mfma_f6_loop_kernel, dim3(blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), out, (int)iters);
  if (hipGetLastError() != hipSuccess) return -5;
  // operations: 2 * 16 * 16 * 128 per MFMA, 8 MFMAs per round per wavefront
  return (int64_t)blocks * 4 * iters * 8 * (2 * 16 * 16 * 128);
}

size_t rq_ceiling_issue_out_words(int64_t waves_per_simd) {
  if (waves_per_simd < 1 || waves_per_simd > 8) return 0;
  return (size_t)rq::cu_count() * (size_t)waves_per_simd * 256;
}

int64_t rq_ceiling_issue(float* out, int64_t kind, int64_t waves_per_simd, int64_t iters,
                         void* stream) {
  if (out == nullptr) return -1;
  if (kind < 0 || kind > 4 || waves_per_simd < 1 || waves_per_simd > 8 || iters < 1 ||
      iters > (1 << 24))
    return -2;
  const int blocks = rq::cu_count() * (int)waves_per_simd;  // 4 wavefronts per block
  const hipStream_t st = static_cast<hipStream_t>(stream);
  switch (kind) {
    case 0: hipLaunchKernelGGL(issue_kernel<0>, dim3(blocks), dim3(256), 0, st, out, (int)iters); break;
    case 1: hipLaunchKernelGGL(issue_kernel<1>, dim3(blocks), dim3(256), 0, st, out, (int)iters); break;
    case 2: hipLaunchKernelGGL(issue_kernel<2>, dim3(blocks), dim3(256), 0, st, out, (int)iters); break;
    case 3: hipLaunchKernelGGL(issue_kernel<3>, dim3(blocks), dim3(256), 0, st, out, (int)iters); break;
    default: hipLaunchKernelGGL(issue_kernel<4>, dim3(blocks), dim3(256), 0, st, out, (int)iters); break;
  }
  if (hipGetLastError() != hipSuccess) return -5;
  return (int64_t)blocks * 4 * iters;  // wavefront rounds
}

}  // extern "C"
