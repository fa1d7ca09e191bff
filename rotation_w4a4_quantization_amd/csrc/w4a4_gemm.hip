// W4A4 linear on CDNA4 (gfx950): packed INT4 codes are widened to int8 in
// registers and multiplied with int8 MFMA into int32 accumulators; the
// epilogue scales by the per-token and per-channel fp16 scales and rounds to
// fp16.
//
// Pages cited:
//   [RQ]     llms.blog, "Rotational Quantization: How Orthogonal Transforms and
//            Hadamard Incoherence Enable Outlier-Free Low-Bit Inference",
//            "Hardware Execution and Serving Economics", part 1 (rotated W4A4
//            layers run end-to-end integer GEMMs).
//   [QuaRot] aicassindra.com, QuaRot explainer, "End-to-end flow" (the INT4
//            rotated activation multiplies the INT4 folded weight).
//
// Widening.  A 32-bit word holds 8 codes, code i in nibble i.  The two
// operations  lo = (w << 4) & 0xF0F0F0F0  and  hi = w & 0xF0F0F0F0  give four
// int8 lanes each, holding 16*q for the even codes (lo) and the odd codes
// (hi).  A and B are widened the same way, so the MFMA pairs equal reduction
// indices and its int32 sum is exactly 256 * acc; acc = sum >> 8.  gfx950 has
// no INT4 MFMA: the arithmetic runs at the int8 rate and INT4 halves the bytes.
//
// The k positions inside one MFMA operand are a lane-group-local choice: any
// assignment works as long as A and B use the same one, which they do.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "rq_internal.h"

namespace rq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4i widen(uint32_t w0, uint32_t w1) {
  v4i r;
  r[0] = (int)((w0 << 4) & 0xF0F0F0F0u);
  r[1] = (int)(w0 & 0xF0F0F0F0u);
  r[2] = (int)((w1 << 4) & 0xF0F0F0F0u);
  r[3] = (int)(w1 & 0xF0F0F0F0u);
  return r;
}

__device__ __forceinline__ float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }
__device__ __forceinline__ uint16_t f2h_rn(float f) { return __half_as_ushort(__float2half_rn(f)); }

__device__ __forceinline__ void epilogue_store(int32_t raw, float sa, float sw, int64_t idx,
                                               uint16_t* __restrict__ y, int32_t* __restrict__ acc) {
  const int32_t a = raw >> 8;  // exact: raw is 256 * acc
  if (acc != nullptr) acc[idx] = a;
  y[idx] = f2h_rn(((float)a * sa) * sw);
}

// ---------------------------------------------------------------- tile GEMM
// 128 x 128 output tile per 256-thread block (2 x 2 waves of 64 x 64), K in
// steps of 64 codes (32 bytes per row), MFMA 16x16x64 i8.
constexpr int TM = 128, TN = 128, TK = 64;
constexpr int ROWB = TK / 2;      // packed bytes per row per step
constexpr int PITCH = ROWB + 8;   // LDS row pitch (bytes), breaks the 32-byte stride

__global__ __launch_bounds__(256) void w4a4_tile_kernel(const uint8_t* __restrict__ a_codes,
                                                        const uint16_t* __restrict__ a_scales,
                                                        const uint8_t* __restrict__ w_codes,
                                                        const uint16_t* __restrict__ w_scales,
                                                        int64_t m, int64_t k, int64_t d,
                                                        uint16_t* __restrict__ y,
                                                        int32_t* __restrict__ acc_out) {
  __shared__ __align__(16) unsigned char sa_tile[TM * PITCH];
  __shared__ __align__(16) unsigned char sb_tile[TN * PITCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * TM;
  const int64_t n0 = (int64_t)blockIdx.x * TN;
  const int64_t rowb = d / 2;

  v4i acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  const int lrow = tid >> 1;   // 0..127: row this thread stages
  const int lhalf = tid & 1;   // which 16-byte half of the 32-byte step
  const bool a_ok = m0 + lrow < m;
  const bool b_ok = n0 + lrow < k;
  const uint8_t* a_src = a_codes + (m0 + lrow) * rowb + 16 * lhalf;
  const uint8_t* b_src = w_codes + (n0 + lrow) * rowb + 16 * lhalf;

  const int g = lane >> 4;     // k group of this lane inside an MFMA operand
  const int r16 = lane & 15;

  for (int64_t kb = 0; kb < rowb; kb += ROWB) {
    const uint4 av = a_ok ? *reinterpret_cast<const uint4*>(a_src + kb) : make_uint4(0, 0, 0, 0);
    const uint4 bv = b_ok ? *reinterpret_cast<const uint4*>(b_src + kb) : make_uint4(0, 0, 0, 0);
    __syncthreads();  // previous step's fragments have been read
    *reinterpret_cast<uint4*>(sa_tile + lrow * PITCH + 16 * lhalf) = av;
    *reinterpret_cast<uint4*>(sb_tile + lrow * PITCH + 16 * lhalf) = bv;
    __syncthreads();
    v4i af[4], bf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint2 p = *reinterpret_cast<const uint2*>(sa_tile + (wm * 64 + i * 16 + r16) * PITCH + 8 * g);
      af[i] = widen(p.x, p.y);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint2 p = *reinterpret_cast<const uint2*>(sb_tile + (wn * 64 + j * 16 + r16) * PITCH + 8 * g);
      bf[j] = widen(p.x, p.y);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
  }

  // C layout of 16x16 MFMA: lane l, element e -> row 4*(l/16) + e, column l % 16
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t row = m0 + wm * 64 + i * 16 + 4 * g + e;
      if (row >= m) continue;
      const float sa = h2f(a_scales[row]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t col = n0 + wn * 64 + j * 16 + r16;
        if (col < k) epilogue_store(acc[i][j][e], sa, h2f(w_scales[col]), row * k + col, y, acc_out);
      }
    }
  }
}

// --------------------------------------------------------------- decode GEMM
// m <= 16.  A 256-thread block owns 16 output channels; its 4 waves split the
// reduction, each lane streaming 16 bytes (32 codes) of one weight row per
// 128-code step, and the partial accumulators are summed through LDS.
constexpr int DEC_WAVES = 4;

__global__ __launch_bounds__(256) void w4a4_decode_kernel(const uint8_t* __restrict__ a_codes,
                                                          const uint16_t* __restrict__ a_scales,
                                                          const uint8_t* __restrict__ w_codes,
                                                          const uint16_t* __restrict__ w_scales,
                                                          int64_t m, int64_t k, int64_t d,
                                                          uint16_t* __restrict__ y,
                                                          int32_t* __restrict__ acc_out) {
  __shared__ v4i partial[DEC_WAVES][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int r16 = lane & 15;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t rowb = d / 2;
  const int64_t steps = (rowb + 63) / 64;  // 64 bytes = 128 codes per step

  const bool a_ok = r16 < m;
  const bool b_ok = n0 + r16 < k;
  const uint8_t* a_src = a_codes + (int64_t)r16 * rowb + 16 * g;
  const uint8_t* b_src = w_codes + (n0 + r16) * rowb + 16 * g;

  v4i acc = {0, 0, 0, 0};
#pragma unroll 4
  for (int64_t s = wave; s < steps; s += DEC_WAVES) {
    const int64_t off = s * 64;
    const bool in_k = off + 16 * g < rowb;
    const uint4 av = (a_ok && in_k) ? *reinterpret_cast<const uint4*>(a_src + off) : make_uint4(0, 0, 0, 0);
    const uint4 bv = (b_ok && in_k) ? *reinterpret_cast<const uint4*>(b_src + off) : make_uint4(0, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(widen(av.x, av.y), widen(bv.x, bv.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(widen(av.z, av.w), widen(bv.z, bv.w), acc, 0, 0, 0);
  }
  partial[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    v4i t = partial[0][lane];
#pragma unroll
    for (int w = 1; w < DEC_WAVES; ++w) t += partial[w][lane];
    const int64_t col = n0 + r16;
    if (col < k) {
      const float sw = h2f(w_scales[col]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t row = 4 * g + e;
        if (row < m) epilogue_store(t[e], h2f(a_scales[row]), sw, row * k + col, y, acc_out);
      }
    }
  }
}

}  // namespace

hipError_t launch_w4a4_gemm(const uint8_t* a_codes, const uint16_t* a_scales, int64_t m,
                            const uint8_t* w_codes, const uint16_t* w_scales, int64_t k, int64_t d,
                            uint16_t* y, int32_t* acc, hipStream_t stream) {
  if (m <= 16) {
    const int64_t blocks = (k + 15) / 16;
    hipLaunchKernelGGL(w4a4_decode_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a_codes,
                       a_scales, w_codes, w_scales, m, k, d, y, acc);
  } else {
    const dim3 grid((unsigned)((k + TN - 1) / TN), (unsigned)((m + TM - 1) / TM));
    hipLaunchKernelGGL(w4a4_tile_kernel, grid, dim3(256), 0, stream, a_codes, a_scales, w_codes,
                       w_scales, m, k, d, y, acc);
  }
  return hipGetLastError();
}

}  // namespace rq
