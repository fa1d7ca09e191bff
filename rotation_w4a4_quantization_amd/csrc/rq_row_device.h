// Device code shared by the row rotation kernels and the fused decode linear:
// one fp16 row of 512 <= n <= 8192 elements per wavefront, randomized
// Hadamard rotation in fp32 and symmetric INT4 quantisation.
//
// Pages cited:
//   [RQ]     llms.blog, "Rotational Quantization: How Orthogonal Transforms and
//            Hadamard Incoherence Enable Outlier-Free Low-Bit Inference",
//            "Incoherence Processing via Randomized Hadamard Transforms" and
//            "Weight Absorption and Online Fast Walsh-Hadamard Transforms".
//   [QuaRot] aicassindra.com, QuaRot explainer, "End-to-end flow".
//
// Everything here has internal linkage: each translation unit that includes
// the header gets its own copy.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rq {
namespace {

constexpr int kWave = 64;
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
// fma(v, m, kMagic) = 2^23 + 8 + rne(v*m) for |v*m| < 8: the low 4 bits are
// the offset-binary code (q + 8); bits 4..22 are zero.
constexpr float kMagic = 8388616.0f;
constexpr float kMagicLo = 8388608.0f;   // code -8
constexpr float kMagicHi = 8388623.0f;   // code +7
// The same for INT8 codes: fma(v, m, kMagic8) = 2^23 + 128 + rne(v*m) for
// |v*m| < 128 leaves the offset-binary code q + 128 in the low 8 bits.
constexpr float kMagic8 = 8388736.0f;
constexpr float kMagic8Lo = 8388608.0f;  // code -128
constexpr float kMagic8Hi = 8388863.0f;  // code +127

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v >> 1); }

__device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }
__device__ __forceinline__ uint16_t f2h_rn(float f) { return __half_as_ushort(__float2half_rn(f)); }

// fp16 of the product a * b, rounded once from the exact product (half to
// even): v_fma_mixlo_f16 with a -0 addend (a * b + -0 is a * b, the sign of a
// zero product included).  Measured on gfx950: this is the once-rounded
// product, while v_mul_f32 then v_cvt_f16_f32 rounds twice (to fp32, then to
// fp16).  The compiler emits either form for fp16(a * b) depending on the
// code around it, so the GEMM epilogues name the instruction.  Bits 16-31 of
// the result are unspecified.
__device__ __forceinline__ uint32_t f16_mul_lo(float a, float b) {
  uint32_t r;
  asm("v_fma_mixlo_f16 %0, %1, %2, neg(0)" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// fp16(a0 * b0) in bits 0-15 and fp16(a1 * b1) in bits 16-31, each rounded
// once as above
__device__ __forceinline__ uint32_t f16_mul_pair(float a0, float b0, float a1, float b1) {
  uint32_t r = f16_mul_lo(a0, b0);
  asm("v_fma_mixhi_f16 %0, %1, %2, neg(0)" : "+v"(r) : "v"(a1), "v"(b1));
  return r;
}

// fp16_rne(xm / D) rounded once from the exact quotient (xm >= 0, finite;
// D = 7 for INT4 codes, 127 for INT8).  The fp32 quotient is correctly
// rounded; only when it lands exactly on an fp16 rounding midpoint can a
// second rounding go the wrong way, and then the exact residual xm - D q says
// on which side of the midpoint the true quotient lies.  The residual is a
// multiple of ulp(q) below D ulp(q) in size, so it is representable and the
// fma computes it exactly.
template <int D = 7>
__device__ __forceinline__ uint16_t scale_fp16(float xm) {
  const float q = xm / (float)D;
  uint16_t hb = f2h_rn(q);
  const float back = (hb == 0x7C00u) ? 65536.0f : h2f(hb);
  if (q != back) {
    const uint16_t ob = (back < q) ? (uint16_t)(hb + 1) : (uint16_t)(hb - 1);
    const float other = (ob == 0x7C00u) ? 65536.0f : h2f(ob);
    if (q == 0.5f * (back + other)) {
      const float r = __builtin_fmaf(-(float)D, q, xm);
      if (r > 0.0f) hb = hb > ob ? hb : ob;
      else if (r < 0.0f) hb = hb < ob ? hb : ob;
    }
  }
  return hb;
}

#define RQ_DPP8(CTRL, U, G)                                                        \
  asm volatile("s_nop 1\n"                                                          \
               "v_fmac_f32_dpp %0, %0, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"    \
               "v_fmac_f32_dpp %1, %1, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"    \
               "v_fmac_f32_dpp %2, %2, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"    \
               "v_fmac_f32_dpp %3, %3, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"    \
               "v_fmac_f32_dpp %4, %4, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"    \
               "v_fmac_f32_dpp %5, %5, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"    \
               "v_fmac_f32_dpp %6, %6, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"    \
               "v_fmac_f32_dpp %7, %7, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"    \
               : "+v"((U)[0]), "+v"((U)[1]), "+v"((U)[2]), "+v"((U)[3]), "+v"((U)[4]), \
                 "+v"((U)[5]), "+v"((U)[6]), "+v"((U)[7])                           \
               : "v"(G))

// fp16 pair (lo, hi) -> lo + hi and lo - hi in fp32, one rounding each.
__device__ __forceinline__ float mix_add(uint32_t w) {
  float r;
  asm("v_fma_mix_f32 %0, %1, 1.0, %1 op_sel:[0,0,1] op_sel_hi:[1,0,1]" : "=v"(r) : "v"(w));
  return r;
}
__device__ __forceinline__ float mix_sub(uint32_t w) {
  float r;
  asm("v_fma_mix_f32 %0, %1, 1.0, -%1 op_sel:[0,0,1] op_sel_hi:[1,0,1]" : "=v"(r) : "v"(w));
  return r;
}

// Is lane L the one receiving the sum in DPP stage k (k = 0..3)?
__device__ __forceinline__ bool dpp_lower(int L, int k) {
  const int b0 = L & 1, b1 = (L >> 1) & 1, b2 = (L >> 2) & 1, b3 = (L >> 3) & 1;
  switch (k) {
    case 0: return (b0 ^ b2) == 0;
    case 1: return (b1 ^ b2) == 0;
    case 2: return b2 == 0;
    default: return b3 == 0;
  }
}
__device__ __forceinline__ int dpp_partner(int L, int k) {
  const int m = k == 0 ? 1 : k == 1 ? 2 : k == 2 ? 7 : 8;
  return L ^ m;
}
// sigma after the first k DPP stages: (-1)^(number of stages where L was upper)
__device__ __forceinline__ float dpp_sigma(int L, int k) {
  float s = 1.0f;
  for (int t = 0; t < k; ++t) s = dpp_lower(L, t) ? s : -s;
  return s;
}

template <int R>
__device__ __forceinline__ void butterfly_regs(float (&u)[R], int h) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (!(r & h)) {
      const float a = u[r], b = u[r + h];
      u[r] = a + b;
      u[r + h] = a - b;
    }
  }
}

constexpr int kRowWaves = 4;  // wavefronts per 256-thread workgroup

// Max over the 64 lanes of a wavefront, returned in every lane.  Within each
// 16-lane row: DPP max against lane^1, lane^2, the mirrored half row and the
// mirrored row; across rows: permlane16/32 swaps (each lane sees its own value
// and that of lane^16, then lane^32).
__device__ __forceinline__ float wave_max(float m) {
  asm volatile(
      "s_nop 1\n"
      "v_max_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n"
      "s_nop 1\n"
      "v_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n"
      "s_nop 1\n"
      "v_max_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf\n"
      "s_nop 1\n"
      "v_max_f32_dpp %0, %0, %0 row_mirror row_mask:0xf bank_mask:0xf\n"
      : "+v"(m));
  const auto a = __builtin_amdgcn_permlane16_swap(f2u(m), f2u(m), false, false);
  m = fmaxf(u2f(a[0]), u2f(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(f2u(m), f2u(m), false, false);
  return fmaxf(u2f(b[0]), u2f(b[1]));
}

template <int NI>
__device__ __forceinline__ void load_row(uint4 (&raw)[NI], const __half* xr, int L) {
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const v4u t = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(xr + 512 * i + 8 * L));
    raw[i] = make_uint4(t[0], t[1], t[2], t[3]);
  }
}

// ------------------------------------------------------------------------
// One fp16 row with 512 <= n <= 8192 elements on one wavefront, no LDS
// exchange.
//
// Lane L loads the 16-byte chunks at elements 512*i + 8*L (fully coalesced),
// so register index rho = 8*i + r holds element e = 512*i + 8*L + r:
// element bits 0..2 and 9.. live in registers, bits 3..8 in the lane index.
//   * e0: v_fma_mix_f32 widens the fp16 pair and adds/subtracts in one op
//     (the sign flip is an xor on the packed fp16 pair before it);
//   * e1, e2: in registers;
//   * e3..e6 (lane bits 0..3): v_fmac_f32_dpp, u += g * u[partner], with the
//     partner lane given by the DPP patterns xor 1, xor 2, xor 7 (row half
//     mirror) and xor 8 (row rotate by 8).  These four masks span lane bits
//     0..3, so the butterflies combine the same cosets as the ascending
//     natural-order FWHT; the per-lane factor g = +-1 picks sum or difference
//     and leaves each lane's value multiplied by a known sign sigma(L).  The
//     products are exact, so every result is fp32(a +- b), bit-identical up
//     to sign with the plain butterfly.  Output index bits 3..6 of lane L are
//     j(L) = (L0^L2, L1^L2, L0^L1^L2, L3);
//   * e7, e8 (lane bits 4, 5): v_permlane16_swap / v_permlane32_swap trade
//     them for register bits 2 and 1 (elements e2, e1, already done), then
//     e7, e8 and e9.. run in registers.
// Codes: register bit 0 is still e0, so nibble pairs are formed in
// registers; bytes are staged in LDS and leave as coalesced 16-byte stores.

// Per-lane constants of the row transform.
struct RowLane {
  float g[4];     // DPP factors of stages e3..e6
  float sigma;    // sign carried by this lane's values after e6
  int lane_pair;  // code byte index bits 0..5 of this lane
};

__device__ __forceinline__ RowLane make_row_lane(int L) {
  RowLane rl;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int P = dpp_partner(L & 15, k);
    const float lo = dpp_lower(L & 15, k) ? 1.0f : -1.0f;
    rl.g[k] = lo * dpp_sigma(L & 15, k) * dpp_sigma(P, k);
  }
  rl.sigma = dpp_sigma(L & 15, 4);
  const int L0 = L & 1, L1 = (L >> 1) & 1, L2 = (L >> 2) & 1, L3 = (L >> 3) & 1;
  const int j = (L0 ^ L2) | ((L1 ^ L2) << 1) | ((L0 ^ L1 ^ L2) << 2) | (L3 << 3);
  rl.lane_pair = ((L >> 5) & 1) | (((L >> 4) & 1) << 1) | (j << 2);
  return rl;
}

// Stages e1..e8 of a 512-element FWHT held as one 16-byte chunk per lane
// (lane L owns elements 8L .. 8L + 7 in c[0..7], e0 already applied): the
// same operations as inside row_rotate_quant.  On return element
// p(r) = (r & 1) | (lane_pair << 1) | (((r >> 2) & 1) << 7) | (((r >> 1) & 1) << 8)
// of the block sits in c[r], multiplied by rl.sigma.
__device__ __forceinline__ void chunk512_stages(float (&c)[8], const RowLane& rl) {
  const float(&g)[4] = rl.g;
#pragma unroll
  for (int r = 0; r < 8; ++r) {  // e1
    if (!(r & 2)) { const float x0 = c[r], x1 = c[r + 2]; c[r] = x0 + x1; c[r + 2] = x0 - x1; }
  }
#pragma unroll
  for (int r = 0; r < 8; ++r) {  // e2
    if (!(r & 4)) { const float x0 = c[r], x1 = c[r + 4]; c[r] = x0 + x1; c[r + 4] = x0 - x1; }
  }
  RQ_DPP8("quad_perm:[1,0,3,2]", c, g[0]);  // e3
  RQ_DPP8("quad_perm:[2,3,0,1]", c, g[1]);  // e4
  RQ_DPP8("row_half_mirror", c, g[2]);      // e5
  RQ_DPP8("row_ror:8", c, g[3]);            // e6
  // lane bit 4 (e7) <-> register bit 2 (e2); lane bit 5 (e8) <-> register bit 1 (e1)
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    if (!(r & 4)) {
      const auto sw = __builtin_amdgcn_permlane16_swap(f2u(c[r]), f2u(c[r + 4]), false, false);
      c[r] = u2f(sw[0]);
      c[r + 4] = u2f(sw[1]);
    }
  }
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    if (!(r & 2)) {
      const auto sw = __builtin_amdgcn_permlane32_swap(f2u(c[r]), f2u(c[r + 2]), false, false);
      c[r] = u2f(sw[0]);
      c[r + 2] = u2f(sw[1]);
    }
  }
#pragma unroll
  for (int r = 0; r < 8; ++r) {  // e7
    if (!(r & 4)) { const float x0 = c[r], x1 = c[r + 4]; c[r] = x0 + x1; c[r + 4] = x0 - x1; }
  }
#pragma unroll
  for (int r = 0; r < 8; ++r) {  // e8
    if (!(r & 2)) { const float x0 = c[r], x1 = c[r + 2]; c[r] = x0 + x1; c[r + 2] = x0 - x1; }
  }
}

// Signs and stage e0 of one 16-byte chunk (8 fp16 elements of a lane): the
// sign flip is an xor on each fp16 pair, then v_fma_mix_f32 gives the pair's
// sum and difference in fp32, one rounding each.
template <bool HAS_SIGNS>
__device__ __forceinline__ void chunk_e0(const uint4& raw, uint2 sg, float* c) {
  const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    uint32_t w = w4[p];
    if constexpr (HAS_SIGNS) {
      const uint32_t s2 = p < 2 ? sg.x : sg.y;
      const uint32_t b0 = (2u * p) & 3u;
      const uint32_t sel = 0x0Cu | (b0 << 8) | (0x0Cu << 16) | ((b0 + 1u) << 24);
      w ^= __builtin_amdgcn_perm(0u, s2, sel) & 0x80008000u;  // sign bits of s_2p, s_2p+1
    }
    c[2 * p] = mix_add(w);
    c[2 * p + 1] = mix_sub(w);
  }
}

// Sign bytes 512 i + 8 L .. + 7 of each chunk, loaded before the row so that
// the row's chunks can be waited for one at a time.  The pointer is made
// opaque per row so that the loads are not hoisted into registers held across
// the row loop.
template <int NI>
__device__ __forceinline__ void load_signs(uint2 (&sg)[NI], const int8_t* __restrict__ signs, int L) {
  using gptr = const __attribute__((address_space(1))) uint64_t*;
  gptr sp = (gptr)(signs + 8 * L);
  asm volatile("" : "+v"(sp));
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const uint64_t v = sp[64 * i];
    sg[i] = make_uint2((uint32_t)v, (uint32_t)(v >> 32));
  }
}

// Stages e0 .. e8 of NI chunks (lane L's 16-byte chunk i at register
// 8 i .. 8 i + 7) chunk by chunk in load order, so chunk i is worked on while
// later chunks are in flight.  With PROGRESSIVE the stages between chunks
// (e9 .., chunk j with chunk j + h for h = 1, 2, 4, ...) also run as soon as
// their chunks are done: once chunks i + 1 - 2h .. i have had the stages
// below h, that block's stage for h runs, so little is left once the last
// chunk is in.
template <int NI, bool HAS_SIGNS, bool PROGRESSIVE>
__device__ __forceinline__ void chunk_major_stages(const uint4 (&raw)[NI], const uint2 (&sg)[NI],
                                                   const RowLane& rl, float* u) {
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    float* c = u + 8 * i;
    chunk_e0<HAS_SIGNS>(raw[i], sg[i], c);
    chunk512_stages(*reinterpret_cast<float(*)[8]>(c), rl);
#pragma unroll
    for (int h = 1; h < NI; h <<= 1) {
      if (PROGRESSIVE && (i + 1) % (2 * h) == 0) {
#pragma unroll
        for (int j = i + 1 - 2 * h; j < i + 1 - h; ++j) {
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            const float a = u[8 * j + r], b = u[8 * (j + h) + r];
            u[8 * j + r] = a + b;
            u[8 * (j + h) + r] = a - b;
          }
        }
      }
    }
    // keeps the next chunk's first use (and so its wait) after this chunk
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Rotates and quantises the row whose chunks `raw` holds (loaded by
// load_row, after the sign bytes `sg` were loaded by load_signs; sg is unused
// without signs): lane 0 writes the fp16 scale to *scale_out, the wavefront writes
// the code bytes (n/2 packed INT4 codes, or n INT8 codes for BITS == 8) to
// codes_row through its LDS slice cb (as many bytes), or, with TO_LDS, leaves
// them in cb (codes_row unused), and the fp32 rotated row goes to xrot_row
// when it is not null.
//
// ASYM (INT4 only): the asymmetric quantiser.  The row range [lo, hi] is
// widened to contain 0, the step is fp16(fp32(hi - lo) / 15) rounded once,
// the zero point z = rne(-lo / step) (lane 0 writes it to *zero_out), and the
// codes are the unsigned nibbles clamp(rne(x / step) + z, 0, 15).
template <int N, bool HAS_SIGNS, bool TO_LDS = false, int BITS = 4, bool ASYM = false>
__device__ __forceinline__ void row_rotate_quant(const uint4 (&raw)[N / 512],
                                                 const uint2 (&sg)[N / 512], int L,
                                                 const RowLane& rl, float c32, unsigned char* cb,
                                                 uint8_t* __restrict__ codes_row,
                                                 uint16_t* __restrict__ scale_out,
                                                 float* __restrict__ xrot_row,
                                                 uint8_t* __restrict__ zero_out = nullptr) {
  constexpr int R = N / 64;    // elements per lane
  constexpr int NI = N / 512;  // 16-byte loads per lane
  static_assert(N >= 512 && N <= 8192, "one row per wavefront covers 512..8192");
  const float sigma = rl.sigma;
  const int lane_pair = rl.lane_pair;
  // Opaque per iteration: keeps the compiler from hoisting one address
  // register per stored element out of the loop (they fold into immediate
  // offsets instead).
  int lp = lane_pair;
  asm volatile("" : "+v"(lp));
  // e0: signs, then the fp16 pair's sum and difference.  From n = 4096 on the
  // row is transformed chunk by chunk in load order (e0 .. e8 act within one
  // 16-byte chunk per lane), so chunk i is worked on while later chunks are
  // in flight; below that, stage by stage over all chunks, which schedules
  // better when there are few chunks.  Both orders apply the same butterflies
  // to the same operands.
  constexpr bool kChunked = N >= 4096;
  // e9.. between chunks as soon as their chunks are done (n = 4096; at 8192
  // the compiler spills with it), else after the last chunk.
  constexpr bool kProgressive = kChunked && NI <= 8;
  float u[R];
  if constexpr (kChunked) {
    chunk_major_stages<NI, HAS_SIGNS, kProgressive>(raw, sg, rl, u);
  } else {
#pragma unroll
    for (int i = 0; i < NI; ++i) chunk_e0<HAS_SIGNS>(raw[i], sg[i], u + 8 * i);
    const float(&g)[4] = rl.g;
    butterfly_regs(u, 2);  // e1
    butterfly_regs(u, 4);  // e2
#pragma unroll
    for (int b = 0; b < R; b += 8) RQ_DPP8("quad_perm:[1,0,3,2]", u + b, g[0]);  // e3
#pragma unroll
    for (int b = 0; b < R; b += 8) RQ_DPP8("quad_perm:[2,3,0,1]", u + b, g[1]);  // e4
#pragma unroll
    for (int b = 0; b < R; b += 8) RQ_DPP8("row_half_mirror", u + b, g[2]);      // e5
#pragma unroll
    for (int b = 0; b < R; b += 8) RQ_DPP8("row_ror:8", u + b, g[3]);            // e6
    // lane bit 4 (e7) <-> register bit 2 (e2); lane bit 5 (e8) <-> register bit 1 (e1)
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (!(r & 4)) {
        const auto sw = __builtin_amdgcn_permlane16_swap(f2u(u[r]), f2u(u[r + 4]), false, false);
        u[r] = u2f(sw[0]);
        u[r + 4] = u2f(sw[1]);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (!(r & 2)) {
        const auto sw = __builtin_amdgcn_permlane32_swap(f2u(u[r]), f2u(u[r + 2]), false, false);
        u[r] = u2f(sw[0]);
        u[r + 2] = u2f(sw[1]);
      }
    }
    butterfly_regs(u, 4);  // e7
    butterfly_regs(u, 2);  // e8
  }
  if constexpr (!kProgressive) {
#pragma unroll
    for (int h = 8; h < R; h <<= 1) butterfly_regs(u, h);  // e9..
  }

  static_assert(BITS == 4 || BITS == 8, "INT4 or INT8 codes");
  static_assert(!ASYM || BITS == 4, "the asymmetric quantiser has INT4 codes");
  float kM = BITS == 4 ? kMagic : kMagic8;
  constexpr float kMLo = BITS == 4 ? kMagicLo : kMagic8Lo;
  constexpr float kMHi = BITS == 4 ? kMagicHi : kMagic8Hi;
  uint16_t hb;
  if constexpr (ASYM) {
    // u[r] * sigma is the value: the lane's max and min swap when sigma < 0
    float vmax = 0.0f, vmin = 0.0f;  // the range always contains 0
#pragma unroll
    for (int r = 0; r < R; ++r) {
      vmax = fmaxf(vmax, u[r]);
      vmin = fminf(vmin, u[r]);
    }
    float hi_u = sigma > 0.0f ? vmax : -vmin;
    float nlo_u = sigma > 0.0f ? -vmin : vmax;
    hi_u = wave_max(hi_u);
    nlo_u = wave_max(nlo_u);
    const float hi32 = hi_u * c32, nlo32 = nlo_u * c32;  // fp32 hi and -lo of the rotated row
    hb = scale_fp16<15>(hi32 + nlo32);
    float zf = 0.0f;
    if (hb != 0 && hb != 0x7C00u) zf = fminf(rintf(nlo32 / h2f(hb)), 15.0f);
    if (L == 0) *zero_out = (uint8_t)zf;
    kM = kMagicLo + zf;  // 2^23 + z: the low nibble of the sum is the code
  } else {
    float amax = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) amax = fmaxf(amax, fabsf(u[r]));
    amax = wave_max(amax);
    hb = scale_fp16<BITS == 4 ? 7 : 127>(amax * c32);
  }
  const bool subnormal = hb != 0 && hb < 0x0400u;
  const float mult = (hb == 0 ? 0.0f : c32 / h2f(hb)) * sigma;
  if (L == 0) *scale_out = hb;

  if (xrot_row != nullptr) {
    float* xo = xrot_row;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int e = (r & 1) | (lp << 1) | (((r >> 2) & 1) << 7) | (((r >> 1) & 1) << 8) |
                    ((r >> 3) << 9);
      xo[e] = (u[r] * sigma) * c32;
    }
  }

  float t[R];
#pragma unroll
  for (int r = 0; r < R; ++r) t[r] = __builtin_fmaf(u[r], mult, kM);
  if constexpr (ASYM) {  // codes past 15 (step rounded down) or below 0 clamp
#pragma unroll
    for (int r = 0; r < R; ++r) t[r] = __builtin_amdgcn_fmed3f(t[r], kMagicLo, kMagicLo + 15.0f);
  } else if (subnormal) {  // uniform: the scale is shared by the whole row
#pragma unroll
    for (int r = 0; r < R; ++r) t[r] = fminf(fmaxf(t[r], kMLo), kMHi);
  }
  // The wavefront stages its row's code bytes in its own LDS slice and
  // reads them back as 16-byte chunks; LDS instructions of one wavefront
  // execute in order, so only the compiler needs fencing here.
#pragma unroll
  for (int r = 0; r < R; r += 2) {
    const int p = (((r >> 2) & 1) << 6) | (((r >> 1) & 1) << 7) | ((r >> 3) << 8);
    if constexpr (BITS == 4) {
      const uint32_t byte = (f2u(t[r + 1]) << 4) | f2u(t[r]);  // low byte: (q1+8)<<4 | (q0+8)
      cb[lp + p] = (unsigned char)byte;
    } else {  // elements 2(lp + p) and + 1: bytes (q0+128), (q1+128)
      const uint32_t pair = (f2u(t[r]) & 0xFFu) | ((f2u(t[r + 1]) & 0xFFu) << 8);
      *reinterpret_cast<uint16_t*>(cb + 2 * (lp + p)) = (uint16_t)pair;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  uint8_t* dst = codes_row;
  constexpr int kCodeBytes = BITS == 4 ? N / 2 : N;
#pragma unroll
  for (int c = L; c < kCodeBytes / 16; c += 64) {
    v4u v = *reinterpret_cast<const v4u*>(cb + 16 * c);
    if constexpr (!ASYM) v ^= BITS == 4 ? 0x88888888u : 0x80808080u;  // to two's complement
    if constexpr (TO_LDS)
      *reinterpret_cast<v4u*>(cb + 16 * c) = v;
    else
      __builtin_nontemporal_store(v, reinterpret_cast<v4u*>(dst + 16 * c));
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace
}  // namespace rq
