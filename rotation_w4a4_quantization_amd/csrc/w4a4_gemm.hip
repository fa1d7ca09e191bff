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
// m <= 16: the GEMM streams the weights once, so it is bound by HBM latency
// and bandwidth.  A 512-thread block owns 16 output channels; its 8 waves
// split the reduction into 64-byte (128-code) steps dealt round robin, and
// every lane issues all of its 16-byte weight loads (nontemporal: read once)
// before the first MFMA, so a whole slice of the weight matrix is in flight
// at once.  Partial accumulators are summed through LDS.
constexpr int DEC_WAVES = 8;
constexpr int DEC_BATCH = 4;  // 64-byte steps per lane issued together

typedef unsigned int v4u_g __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(64 * DEC_WAVES) void w4a4_decode_kernel(
    const uint8_t* __restrict__ a_codes, const uint16_t* __restrict__ a_scales,
    const uint8_t* __restrict__ w_codes, const uint16_t* __restrict__ w_scales, int64_t m,
    int64_t k, int64_t d, uint16_t* __restrict__ y, int32_t* __restrict__ acc_out) {
  __shared__ v4i partial[DEC_WAVES][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int r16 = lane & 15;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t rowb = d / 2;
  const int64_t steps = (rowb + 63) / 64;  // the last step may hold only 32 bytes

  const bool a_ok = r16 < m;
  const int64_t wrow = n0 + r16 < k ? n0 + r16 : k - 1;  // rows past k re-read the last one
  const uint8_t* a_src = a_codes + (int64_t)r16 * rowb + 16 * g;
  const uint8_t* b_src = w_codes + wrow * rowb + 16 * g;

  v4i acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
  for (int64_t s0 = wave; s0 < steps; s0 += (int64_t)DEC_WAVES * DEC_BATCH) {
    uint4 av[DEC_BATCH], bv[DEC_BATCH];
#pragma unroll
    for (int q = 0; q < DEC_BATCH; ++q) {
      const int64_t off = (s0 + (int64_t)q * DEC_WAVES) * 64;
      const bool in_k = off + 16 * g < rowb && s0 + (int64_t)q * DEC_WAVES < steps;
      bv[q] = make_uint4(0, 0, 0, 0);
      av[q] = make_uint4(0, 0, 0, 0);
      if (in_k) {
        const v4u_g t = __builtin_nontemporal_load(reinterpret_cast<const v4u_g*>(b_src + off));
        bv[q] = make_uint4(t[0], t[1], t[2], t[3]);
        if (a_ok) av[q] = *reinterpret_cast<const uint4*>(a_src + off);
      }
    }
#pragma unroll
    for (int q = 0; q < DEC_BATCH; ++q) {
      acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(widen(av[q].x, av[q].y), widen(bv[q].x, bv[q].y), acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(widen(av[q].z, av[q].w), widen(bv[q].z, bv[q].w), acc1, 0, 0, 0);
    }
  }
  partial[wave][lane] = acc0 + acc1;
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

// ------------------------------------------------------------ large GEMM
// 256 x 224 output tile per 512-thread block: 8 waves in a 4 x 2 grid of
// 64 x 112 wave tiles (4 x 7 MFMA 16x16x64 tiles, 112 int32 accumulators per
// lane, so two waves fit on each SIMD and cover each other's LDS and global
// latency).  K runs in steps of 128 codes.  Each step's packed A and B tiles
// (64 bytes per row) are loaded into registers one step ahead, widened to
// int8 once, and stored into the other of two LDS buffers (128 bytes per
// row); the MFMA loop only reads 16-byte fragments.  The 16-byte chunk index
// of a row is XORed with bits 1..3 of the row, so both the stores and the
// fragment reads are free of bank conflicts.  For 2048 x 28672 the 256 x 224
// tile gives exactly 1024 tiles, four per CU.
constexpr int LM = 256, LN = 224, LK = 128;        // block tile (codes)
constexpr int LPK = LK / 2;                         // packed bytes per row per step
constexpr int LROW = LK;                            // widened bytes per row per step
constexpr int LBUF = (LM + LN) * LROW;              // one LDS buffer: 60 KB
constexpr int LTHREADS = 512;

__device__ __forceinline__ int tile_off(int row, int chunk) {
  return row * LROW + 16 * (chunk ^ ((row >> 1) & 7));
}

// packed chunk (32 codes) -> two widened 16-byte chunks at chunk positions 2p, 2p+1
__device__ __forceinline__ void stash_chunk(unsigned char* buf, int row, int part, uint4 v) {
  *reinterpret_cast<v4i*>(buf + tile_off(row, 2 * part)) = widen(v.x, v.y);
  *reinterpret_cast<v4i*>(buf + tile_off(row, 2 * part + 1)) = widen(v.z, v.w);
}

__global__ __launch_bounds__(LTHREADS) void w4a4_large_kernel(const uint8_t* __restrict__ a_codes,
                                                              const uint16_t* __restrict__ a_scales,
                                                              const uint8_t* __restrict__ w_codes,
                                                              const uint16_t* __restrict__ w_scales,
                                                              int64_t m, int64_t k, int64_t d,
                                                              int tiles_m,
                                                              uint16_t* __restrict__ y,
                                                              int32_t* __restrict__ acc_out) {
  __shared__ __align__(16) unsigned char lds[2 * LBUF];
  const int64_t m0 = (int64_t)(blockIdx.x % tiles_m) * LM;
  const int64_t n0 = (int64_t)(blockIdx.x / tiles_m) * LN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;  // 4 x 2 waves of 64 x 112
  const int g = lane >> 4, r16 = lane & 15;
  const int64_t rowb = d / 2;

  // staging: thread tid moves the packed 16-byte part tid % 4 of rows
  // tid / 4 and tid / 4 + 128 of the A tile and of the B tile (the second B
  // row exists for rows < 224).  Rows past the matrix edge re-read the last
  // row; their results are never stored.  Tile-relative offsets fit in 32 bits.
  const int srow = tid >> 2, part = tid & 3;
  const uint8_t* a_base = a_codes + m0 * rowb + 16 * part;
  const uint8_t* b_base = w_codes + n0 * rowb + 16 * part;
  const int a_last = (int)(m - 1 - m0), b_last = (int)(k - 1 - n0);
  const int ar0 = (srow < a_last ? srow : a_last) * (int)rowb;
  const int ar1 = (srow + 128 < a_last ? srow + 128 : a_last) * (int)rowb;
  const int br0 = (srow < b_last ? srow : b_last) * (int)rowb;
  const int brl = srow + 128 < LN ? srow + 128 : LN - 1;
  const int br1 = (brl < b_last ? brl : b_last) * (int)rowb;
  const bool b2 = srow + 128 < LN;

  v4i acc[4][7];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 7; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  uint4 ra0, ra1, rb0, rb1 = make_uint4(0, 0, 0, 0);
  const int steps = (int)(rowb / LPK);
  ra0 = *reinterpret_cast<const uint4*>(a_base + ar0);
  ra1 = *reinterpret_cast<const uint4*>(a_base + ar1);
  rb0 = *reinterpret_cast<const uint4*>(b_base + br0);
  if (b2) rb1 = *reinterpret_cast<const uint4*>(b_base + br1);
  stash_chunk(lds, srow, part, ra0);
  stash_chunk(lds, srow + 128, part, ra1);
  stash_chunk(lds + LM * LROW, srow, part, rb0);
  if (b2) stash_chunk(lds + LM * LROW, srow + 128, part, rb1);
  __syncthreads();
  for (int s = 0; s < steps; ++s) {
    const unsigned char* cur = lds + (s & 1) * LBUF;
    unsigned char* nxt = lds + ((s + 1) & 1) * LBUF;
    if (s + 1 < steps) {
      const int64_t kb = (int64_t)(s + 1) * LPK;
      ra0 = *reinterpret_cast<const uint4*>(a_base + ar0 + kb);
      ra1 = *reinterpret_cast<const uint4*>(a_base + ar1 + kb);
      rb0 = *reinterpret_cast<const uint4*>(b_base + br0 + kb);
      if (b2) rb1 = *reinterpret_cast<const uint4*>(b_base + br1 + kb);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v4i bf[7];
#pragma unroll
      for (int j = 0; j < 7; ++j)
        bf[j] = *reinterpret_cast<const v4i*>(cur + LM * LROW + tile_off(wn * 112 + j * 16 + r16, 4 * ks + g));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const v4i af = *reinterpret_cast<const v4i*>(cur + tile_off(wm * 64 + i * 16 + r16, 4 * ks + g));
#pragma unroll
        for (int j = 0; j < 7; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, bf[j], acc[i][j], 0, 0, 0);
      }
    }
    if (s + 1 < steps) {
      stash_chunk(nxt, srow, part, ra0);
      stash_chunk(nxt, srow + 128, part, ra1);
      stash_chunk(nxt + LM * LROW, srow, part, rb0);
      if (b2) stash_chunk(nxt + LM * LROW, srow + 128, part, rb1);
    }
    __syncthreads();
  }

  // epilogue: lane holds rows 4g..4g+3 of every 16-row group, column r16 of
  // every 16-column group
  float swv[7];
#pragma unroll
  for (int j = 0; j < 7; ++j) {
    const int64_t col = n0 + wn * 112 + j * 16 + r16;
    swv[j] = col < k ? h2f(w_scales[col]) : 0.0f;
  }
  const bool full = m0 + LM <= m && n0 + LN <= k;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t row = m0 + wm * 64 + i * 16 + 4 * g + e;
      if (!full && row >= m) continue;
      const float sa = h2f(a_scales[row]);
      const int64_t base = row * k + n0 + wn * 112 + r16;
#pragma unroll
      for (int j = 0; j < 7; ++j) {
        if (full || n0 + wn * 112 + j * 16 + r16 < k)
          epilogue_store(acc[i][j][e], sa, swv[j], base + j * 16, y, acc_out);
      }
    }
  }
}

}  // namespace

hipError_t launch_w4a4_gemm(const uint8_t* a_codes, const uint16_t* a_scales, int64_t m,
                            const uint8_t* w_codes, const uint16_t* w_scales, int64_t k, int64_t d,
                            uint16_t* y, int32_t* acc, hipStream_t stream) {
  if (m >= 128 && k >= 224 && d % LK == 0) {
    const int tiles_m = (int)((m + LM - 1) / LM);
    const int64_t tiles = (int64_t)tiles_m * ((k + LN - 1) / LN);
    hipLaunchKernelGGL(w4a4_large_kernel, dim3((unsigned)tiles), dim3(LTHREADS), 0, stream, a_codes,
                       a_scales, w_codes, w_scales, m, k, d, tiles_m, y, acc);
  } else if (m <= 16) {
    const int64_t blocks = (k + 15) / 16;
    hipLaunchKernelGGL(w4a4_decode_kernel, dim3((unsigned)blocks), dim3(64 * DEC_WAVES), 0, stream, a_codes,
                       a_scales, w_codes, w_scales, m, k, d, y, acc);
  } else {
    const dim3 grid((unsigned)((k + TN - 1) / TN), (unsigned)((m + TM - 1) / TM));
    hipLaunchKernelGGL(w4a4_tile_kernel, grid, dim3(256), 0, stream, a_codes, a_scales, w_codes,
                       w_scales, m, k, d, y, acc);
  }
  return hipGetLastError();
}

}  // namespace rq
