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
#include "rq_row_device.h"

namespace rq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Per-group weight scales: one fp16 scale per WG consecutive codes of a
// weight row, stored [k][d / WG].
constexpr int WG = 128;

// Activation code formats: packed signed INT4 (W4A4), INT8 bytes (W4A8), and
// packed unsigned INT4 with a per-row zero point (asymmetric activations).
constexpr int kA4 = 0, kA8 = 1, kAU4 = 2;

// 16 INT8 activation codes (natural order) rearranged into the k order that
// widen() gives the weight codes: (0,2,4,6), (1,3,5,7), (8,10,12,14), (9,...).
__device__ __forceinline__ v4i order_a8(const uint4& q) {
  v4i r;
  r[0] = (int)__builtin_amdgcn_perm(q.y, q.x, 0x06040200u);
  r[1] = (int)__builtin_amdgcn_perm(q.y, q.x, 0x07050301u);
  r[2] = (int)__builtin_amdgcn_perm(q.w, q.z, 0x06040200u);
  r[3] = (int)__builtin_amdgcn_perm(q.w, q.z, 0x07050301u);
  return r;
}

// Unsigned nibbles widened as q itself (0..15 fits a signed byte), in the
// same k order as widen(); against 16 * q weights the MFMA sum is 16 * acc.
__device__ __forceinline__ v4i widen_u(uint32_t w0, uint32_t w1) {
  v4i r;
  r[0] = (int)(w0 & 0x0F0F0F0Fu);
  r[1] = (int)((w0 >> 4) & 0x0F0F0F0Fu);
  r[2] = (int)(w1 & 0x0F0F0F0Fu);
  r[3] = (int)((w1 >> 4) & 0x0F0F0F0Fu);
  return r;
}

__device__ __forceinline__ v4i widen(uint32_t w0, uint32_t w1) {
  v4i r;
  r[0] = (int)((w0 << 4) & 0xF0F0F0F0u);
  r[1] = (int)(w0 & 0xF0F0F0F0u);
  r[2] = (int)((w1 << 4) & 0xF0F0F0F0u);
  r[3] = (int)(w1 & 0xF0F0F0F0u);
  return r;
}


// raw is 256 * acc for INT4 activations (both operands widened to 16 q) and
// 16 * acc for INT8 and unsigned INT4 activations (SHIFT 4): the shift is
// exact.  zsum = z * sum_i qw[j][i] turns the unsigned sum into the
// accumulator of (qa - z) * qw (asymmetric activations; 0 otherwise).
template <int SHIFT = 8>
__device__ __forceinline__ void epilogue_store(int32_t raw, float sa, float sw, int64_t idx,
                                               uint16_t* __restrict__ y, int32_t* __restrict__ acc,
                                               int32_t zsum = 0) {
  const int32_t a = (raw >> SHIFT) - zsum;
  if (acc != nullptr) acc[idx] = a;
  y[idx] = (uint16_t)f16_mul_lo((float)a * sa, sw);
}

// ---------------------------------------------------------------- tile GEMM
// 128 x 128 output tile per 256-thread block (2 x 2 waves of 64 x 64), K in
// steps of 64 codes (32 bytes per row), MFMA 16x16x64 i8.
constexpr int TM = 128, TN = 128, TK = 64;
constexpr int ROWB = TK / 2;      // packed bytes per row per step
constexpr int PITCH = ROWB + 8;   // LDS row pitch (bytes), breaks the 32-byte stride
constexpr int PITCH8 = TK + 16;   // INT8 activation rows (64 bytes per step), 16-byte aligned

// AM: the activation code format (kA4, kA8: INT8 bytes [m][d], kAU4:
// unsigned INT4 with zero points a_zeros and weight code sums w_sums).
// GROUPED (with kA4): w_scales holds per-group scales [k][d / WG]; every
// two 64-code steps (one group) the int32 tile turns into fp32 with its
// group scale, and (debug) acc_out [m][k][d / WG] receives the group sums.
template <int AM = kA4, bool GROUPED = false>
__global__ __launch_bounds__(256) void w4a4_tile_kernel(const uint8_t* __restrict__ a_codes,
                                                        const uint16_t* __restrict__ a_scales,
                                                        const uint8_t* __restrict__ w_codes,
                                                        const uint16_t* __restrict__ w_scales,
                                                        int64_t m, int64_t k, int64_t d,
                                                        uint16_t* __restrict__ y,
                                                        int32_t* __restrict__ acc_out,
                                                        const uint8_t* __restrict__ a_zeros,
                                                        const int32_t* __restrict__ w_sums) {
  constexpr bool A8 = AM == kA8;
  constexpr int AW = A8 ? 2 : 1;  // activation bytes per weight byte
  constexpr int APITCH = A8 ? PITCH8 : PITCH;
  __shared__ __align__(16) unsigned char sa_tile[TM * APITCH];
  __shared__ __align__(16) unsigned char sb_tile[TN * PITCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * TM;
  const int64_t n0 = (int64_t)blockIdx.x * TN;
  const int64_t rowb = d / 2;

  v4i acc[4][4];
  v4f facc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[i][j] = v4i{0, 0, 0, 0};
      facc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    }
  const int64_t ngroups = d / WG;

  const int lrow = tid >> 1;   // 0..127: row this thread stages
  const int lhalf = tid & 1;   // which 16-byte half of the 32-byte step
  const bool a_ok = m0 + lrow < m;
  const bool b_ok = n0 + lrow < k;
  const uint8_t* a_src = a_codes + (m0 + lrow) * rowb * AW + 16 * AW * lhalf;
  const uint8_t* b_src = w_codes + (n0 + lrow) * rowb + 16 * lhalf;

  const int g = lane >> 4;     // k group of this lane inside an MFMA operand
  const int r16 = lane & 15;

  for (int64_t kb = 0; kb < rowb; kb += ROWB) {
    uint4 av[AW];
#pragma unroll
    for (int u = 0; u < AW; ++u)
      av[u] = a_ok ? *reinterpret_cast<const uint4*>(a_src + AW * kb + 16 * u)
                   : make_uint4(0, 0, 0, 0);
    const uint4 bv = b_ok ? *reinterpret_cast<const uint4*>(b_src + kb) : make_uint4(0, 0, 0, 0);
    __syncthreads();  // previous step's fragments have been read
#pragma unroll
    for (int u = 0; u < AW; ++u)
      *reinterpret_cast<uint4*>(sa_tile + lrow * APITCH + 16 * (AW * lhalf + u)) = av[u];
    *reinterpret_cast<uint4*>(sb_tile + lrow * PITCH + 16 * lhalf) = bv;
    __syncthreads();
    v4i af[4], bf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const unsigned char* ap = sa_tile + (wm * 64 + i * 16 + r16) * APITCH;
      if constexpr (A8) {
        af[i] = order_a8(*reinterpret_cast<const uint4*>(ap + 16 * g));
      } else {
        const uint2 p = *reinterpret_cast<const uint2*>(ap + 8 * g);
        af[i] = AM == kAU4 ? widen_u(p.x, p.y) : widen(p.x, p.y);
      }
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
    if constexpr (GROUPED) {
      if ((kb / ROWB) & 1) {  // the step that completes group kb / (WG / 2)
        const int64_t grp = kb / (WG / 2);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t col = n0 + wn * 64 + j * 16 + r16;
          const float sg = h2f(w_scales[(col < k ? col : k - 1) * ngroups + grp]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (acc_out != nullptr) {  // debug: the exact int32 group sums
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int64_t row = m0 + wm * 64 + i * 16 + 4 * g + e;
                if (row < m && col < k) acc_out[(row * k + col) * ngroups + grp] = acc[i][j][e] >> 8;
              }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) facc[i][j][e] = __builtin_fmaf((float)acc[i][j][e], sg, facc[i][j][e]);
            acc[i][j] = v4i{0, 0, 0, 0};
          }
        }
      }
    }
  }

  // C layout of 16x16 MFMA: lane l, element e -> row 4*(l/16) + e, column l % 16
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t row = m0 + wm * 64 + i * 16 + 4 * g + e;
      if (row >= m) continue;
      const float sa = h2f(a_scales[row]);
      const int32_t z = AM == kAU4 ? (int32_t)a_zeros[row] : 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t col = n0 + wn * 64 + j * 16 + r16;
        if (col >= k) continue;
        if constexpr (GROUPED)
          y[row * k + col] = (uint16_t)f16_mul_lo(facc[i][j][e] * (1.0f / 256.0f), sa);
        else
          epilogue_store<AM == kA4 ? 8 : 4>(acc[i][j][e], sa, h2f(w_scales[col]), row * k + col,
                                            y, acc_out, AM == kAU4 ? z * w_sums[col] : 0);
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

// One 8-row DMA load: lane L's 16 bytes go to LDS byte m0 + 16 L.
#define RQ_DMA(M0, ADDR)                                                           \
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"     \
               :                                                                   \
               : "v"(ADDR), "s"(M0)                                                \
               : "memory", "m0")
// One dword per lane: lane L's 4 bytes land at M0 + 4 L.
#define RQ_DMA_D(M0, ADDR)                                                         \
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"      \
               :                                                                   \
               : "v"(ADDR), "s"(M0)                                                \
               : "memory", "m0")
// The same with the nontemporal hint, for data read exactly once.
#define RQ_DMA_NT(M0, ADDR)                                                        \
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"  \
               :                                                                   \
               : "v"(ADDR), "s"(M0)                                                \
               : "memory", "m0")

// m <= 16 and d % 256 == 0: the same work split, but the weights go straight
// from global memory into LDS, one load instruction per 8 rows x 128 bytes,
// so that every instruction reads whole cache lines (a lane-per-row pattern
// of 16 rows x 64 bytes splits each line between two instructions of
// different waves and costs about a fifth more time at the same bytes).
// A row is cut into 128-byte segments; wave w loads segments 2w and 2w + 1 of
// each 2 KB chunk of the block's 16 RG rows and is also the only wave that reads
// them, so the chunk needs no workgroup barrier.  LDS holds [segment][row][128
// bytes], with the 16-byte part p of row r at position p ^ (r & 7) (the
// fragment reads of one 8-lane phase hit 8 different bank groups).
constexpr int DSEG = 128;                 // bytes per row segment
constexpr int DCHUNK = 2 * DEC_WAVES;     // segments per chunk (2 KB per row)

// Per-lane state of an LDS-staged decode tile of 16 RG weight rows.
template <int RG>
struct DecLane {
  const uint8_t* wsrc[2 * RG];  // DMA source of each 8-row load
  uint32_t wl_base;             // LDS byte address of the weight staging buffer
  int wave, lane, g, r16;
  int64_t n0, nseg;
};

template <int RG>
__device__ __forceinline__ DecLane<RG> dec_lane(const uint8_t* __restrict__ w_codes, int64_t k,
                                                int64_t rowb, unsigned char* wl) {
  DecLane<RG> t;
  const int tid = threadIdx.x;
  t.lane = tid & 63;
  t.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  t.g = t.lane >> 4;
  t.r16 = t.lane & 15;
  t.n0 = (int64_t)blockIdx.x * 16 * RG;
  t.nseg = rowb / DSEG;
  t.wl_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)wl;
  // lane L of the load of rows 8 h .. 8 h + 7 fetches part (L % 8) ^ (L / 8)
  // of row 8 h + L / 8 (rows past k re-read the last one)
#pragma unroll
  for (int h = 0; h < 2 * RG; ++h) {
    const int64_t row = t.n0 + 8 * h + (t.lane >> 3);
    t.wsrc[h] = w_codes + (row < k ? row : k - 1) * rowb + 16 * ((t.lane & 7) ^ (t.lane >> 3));
  }
  return t;
}

// Loads of this wave's two segments of the chunk that starts at segment c0.
template <int RG>
__device__ __forceinline__ void dec_issue_w(const DecLane<RG>& t, int64_t c0) {
  constexpr int SEGB = 16 * RG * DSEG;  // LDS bytes per segment
#pragma unroll
  for (int sl = 0; sl < 2; ++sl) {
    const int64_t seg = c0 + 2 * t.wave + sl;
    if (seg < t.nseg) {
      const uint32_t m0_ = t.wl_base + (uint32_t)((2 * t.wave + sl) * SEGB);
#pragma unroll
      for (int h = 0; h < 2 * RG; ++h) RQ_DMA_NT(m0_ + 8 * h * DSEG, t.wsrc[h] + seg * DSEG);
    }
  }
}

// Activation fragments of this wave's two parts of the chunk that starts at
// segment c0 (16 bytes per lane and half: a 32-code part; A8: two loads, the
// INT8 codes of the same 32 positions).  Every load is unconditional, from a
// clamped address that is always valid: rows past m re-read row 0 (a_src)
// and feed only outputs that are not stored, segments past the end re-read
// the last one and are skipped by the MFMAs.  A register refilled by a load
// under a branch would get a wait for every load in flight (the weight DMA
// included, which the compiler cannot see).
template <int AM = kA4>
__device__ __forceinline__ void dec_load_act(int wave, int64_t nseg, const uint8_t* a_src,
                                             int64_t c0, uint4 (&av)[2][2][AM == kA8 ? 2 : 1]) {
  constexpr int AW = AM == kA8 ? 2 : 1;
#pragma unroll
  for (int sl = 0; sl < 2; ++sl) {
    const int64_t seg = c0 + 2 * wave + sl;
    const int64_t segc = seg < nseg ? seg : nseg - 1;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int u = 0; u < AW; ++u)
        av[sl][h][u] = *reinterpret_cast<const uint4*>(a_src + AW * (segc * DSEG + 64 * h) + 16 * u);
  }
}

// Wait for the chunk's activation fragments (av) and weights, then the
// MFMAs; this wave's LDS reads are back on return (before its next loads may
// overwrite them).  A8: the activations are INT8 codes, two 16-byte loads per
// 32-code part, put in widen's k order.
template <int RG, int AM = kA4>
__device__ __forceinline__ void dec_mma_loaded(const DecLane<RG>& t, const unsigned char* wl,
                                               uint4 (&av)[2][2][AM == kA8 ? 2 : 1], int64_t c0,
                                               v4i (&acc0)[RG], v4i (&acc1)[RG]) {
  constexpr int SEGB = 16 * RG * DSEG;
  constexpr bool A8 = AM == kA8;
  constexpr int AW = A8 ? 2 : 1;
  // The loads read kernel arguments the compiler treats as invariant, so it
  // may sink them past the wait below into their uses: an empty asm that
  // takes every loaded value keeps them issued before the wait.
#pragma unroll
  for (int sl = 0; sl < 2; ++sl)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int u = 0; u < AW; ++u)
        asm volatile("" ::"v"(av[sl][h][u].x), "v"(av[sl][h][u].y), "v"(av[sl][h][u].z),
                     "v"(av[sl][h][u].w));
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
  for (int sl = 0; sl < 2; ++sl) {
    if (c0 + 2 * t.wave + sl >= t.nseg) continue;  // uniform per wave
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v4i a0, a1;
      if constexpr (A8) {
        a0 = order_a8(av[sl][h][0]);
        a1 = order_a8(av[sl][h][AW - 1]);
      } else if constexpr (AM == kAU4) {
        a0 = widen_u(av[sl][h][0].x, av[sl][h][0].y);
        a1 = widen_u(av[sl][h][0].z, av[sl][h][0].w);
      } else {
        a0 = widen(av[sl][h][0].x, av[sl][h][0].y);
        a1 = widen(av[sl][h][0].z, av[sl][h][0].w);
      }
#pragma unroll
      for (int q = 0; q < RG; ++q) {
        const uint4 w = *reinterpret_cast<const uint4*>(
            wl + (2 * t.wave + sl) * SEGB + (16 * q + t.r16) * DSEG +
            16 * ((4 * h + t.g) ^ (t.r16 & 7)));
        acc0[q] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, widen(w.x, w.y), acc0[q], 0, 0, 0);
        acc1[q] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, widen(w.z, w.w), acc1[q], 0, 0, 0);
      }
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// The same with the activation fragments read here from a_src (the fused
// decode linear: its token codes are in LDS), after the chunk's weight loads.
template <int RG, int AM = kA4>
__device__ __forceinline__ void dec_mma_chunk(const DecLane<RG>& t, const unsigned char* wl,
                                              const uint8_t* a_src, bool a_ok, int64_t c0,
                                              v4i (&acc0)[RG], v4i (&acc1)[RG]) {
  constexpr int AW = AM == kA8 ? 2 : 1;
  uint4 av[2][2][AW];
#pragma unroll
  for (int sl = 0; sl < 2; ++sl) {
    const int64_t seg = c0 + 2 * t.wave + sl;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int u = 0; u < AW; ++u) {
        av[sl][h][u] = make_uint4(0, 0, 0, 0);
        if (a_ok && seg < t.nseg)
          av[sl][h][u] =
              *reinterpret_cast<const uint4*>(a_src + AW * (seg * DSEG + 64 * h) + 16 * u);
      }
  }
  dec_mma_loaded<RG, AM>(t, wl, av, c0, acc0, acc1);
}

// Epilogue operands of the waves that finish a 16-row group (waves < RG):
// the column's weight scale (and code sum) and the activation scales (and
// zero points) of the lane's four rows, loaded with the first chunk, before
// its wait, from clamped (always valid) addresses.
struct DecEpi {
  float sw = 0.0f, sa[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  int32_t ws = 0, za[4] = {0, 0, 0, 0};
};

template <int RG>
__device__ __forceinline__ DecEpi dec_load_epi(const DecLane<RG>& t, int64_t m, int64_t k,
                                               const uint16_t* __restrict__ a_scales,
                                               const uint16_t* __restrict__ w_scales,
                                               const uint8_t* __restrict__ a_zeros,
                                               const int32_t* __restrict__ w_sums) {
  DecEpi e;
  if (t.wave < RG) {  // uniform per wave
    const int64_t col = t.n0 + 16 * t.wave + t.r16;
    const int64_t colc = col < k ? col : k - 1;
    const uint32_t swb = w_scales[colc];
    const int32_t wsv = w_sums != nullptr ? w_sums[colc] : 0;
    uint32_t sab[4], zab[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = 4 * t.g + i;
      const int64_t rowc = row < m ? row : m - 1;
      sab[i] = a_scales[rowc];
      zab[i] = a_zeros != nullptr ? a_zeros[rowc] : 0u;
    }
    // (the loads all issue here; taking their values waits for them, and
    // everything issued before them, at once)
    asm volatile("" ::"v"(swb), "v"(wsv));
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" ::"v"(sab[i]), "v"(zab[i]));
    e.sw = h2f((uint16_t)swb);
    e.ws = wsv;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      e.sa[i] = h2f((uint16_t)sab[i]);
      e.za[i] = (int32_t)zab[i];
    }
  }
  return e;
}

// Partial sums of the 8 waves meet in LDS (wave w's RG x 64 sums start at
// partial + w * pitch); waves 0..RG-1 finish one 16-row group each.  Row r's
// activation scale is a_scales[r * sa_stride] (or epi's).
template <int RG, int SHIFT = 8>
__device__ __forceinline__ void dec_reduce_store(const DecLane<RG>& t, v4i* partial, int pitch,
                                                 const v4i (&acc0)[RG], const v4i (&acc1)[RG],
                                                 int64_t m, int64_t k,
                                                 const uint16_t* __restrict__ a_scales,
                                                 const uint16_t* __restrict__ w_scales,
                                                 uint16_t* __restrict__ y,
                                                 int32_t* __restrict__ acc_out,
                                                 const uint8_t* __restrict__ a_zeros = nullptr,
                                                 const int32_t* __restrict__ w_sums = nullptr,
                                                 const DecEpi* epi = nullptr,
                                                 int64_t sa_stride = 1) {
#pragma unroll
  for (int q = 0; q < RG; ++q) partial[t.wave * pitch + q * 64 + t.lane] = acc0[q] + acc1[q];
  __syncthreads();
  if (t.wave < RG) {
    v4i s = partial[t.wave * 64 + t.lane];
#pragma unroll
    for (int w = 1; w < DEC_WAVES; ++w) s += partial[w * pitch + t.wave * 64 + t.lane];
    const int64_t col = t.n0 + 16 * t.wave + t.r16;
    if (col < k) {
      const float sw = epi != nullptr ? epi->sw : h2f(w_scales[col]);
      const int32_t ws = epi != nullptr ? epi->ws : (w_sums != nullptr ? w_sums[col] : 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t row = 4 * t.g + e;
        if (row < m) {
          const float sa = epi != nullptr ? epi->sa[e] : h2f(a_scales[row * sa_stride]);
          const int32_t z = epi != nullptr ? epi->za[e] : (a_zeros != nullptr ? (int32_t)a_zeros[row] : 0);
          epilogue_store<SHIFT>(s[e], sa, sw, row * k + col, y, acc_out, z * ws);
        }
      }
    }
  }
}

// RG 16-row groups of weights per workgroup share each activation fragment.
// AM: activation code format, kA8 (INT8 codes [m][d] bytes, W4A8) or kAU4
// (unsigned INT4 with zero points a_zeros and weight code sums w_sums); for
// both the MFMA sum is 16 * acc.
template <int RG, int AM = kA4>
__global__ __launch_bounds__(64 * DEC_WAVES) void w4a4_decode_lds_kernel(
    const uint8_t* __restrict__ a_codes, const uint16_t* __restrict__ a_scales,
    const uint8_t* __restrict__ w_codes, const uint16_t* __restrict__ w_scales, int64_t m,
    int64_t k, int64_t d, uint16_t* __restrict__ y, int32_t* __restrict__ acc_out,
    const uint8_t* __restrict__ a_zeros, const int32_t* __restrict__ w_sums) {
  constexpr bool A8 = AM == kA8;
  __shared__ __align__(16) unsigned char wl[DCHUNK * 16 * RG * DSEG];  // 32 KB per row group
  __shared__ v4i partial[DEC_WAVES][RG][64];
  const int64_t rowb = d / 2;
  const DecLane<RG> t = dec_lane<RG>(w_codes, k, rowb, wl);
  const bool a_ok = t.r16 < m;
  constexpr int AW = A8 ? 2 : 1;  // activation bytes per weight byte
  const uint8_t* a_src = a_codes + (int64_t)(a_ok ? t.r16 : 0) * rowb * AW + 16 * AW * t.g;

  v4i acc0[RG], acc1[RG];
#pragma unroll
  for (int q = 0; q < RG; ++q) acc0[q] = acc1[q] = v4i{0, 0, 0, 0};
  DecEpi epi;
  for (int64_t c0 = 0; c0 < t.nseg; c0 += DCHUNK) {
    // the activation fragments (L2-resident, read by every workgroup) go out
    // ahead of the chunk's weights, and the epilogue's scales with the first
    // chunk, so neither adds a memory round trip after the weights are in
    uint4 av[2][2][AW];
    dec_load_act<AM>(t.wave, t.nseg, a_src, c0, av);
    dec_issue_w(t, c0);
    if (c0 == 0)
      epi = dec_load_epi(t, m, k, a_scales, w_scales, AM == kAU4 ? a_zeros : nullptr,
                         AM == kAU4 ? w_sums : nullptr);
    dec_mma_loaded<RG, AM>(t, wl, av, c0, acc0, acc1);
  }
  dec_reduce_store<RG, AM == kA4 ? 8 : 4>(t, &partial[0][0][0], RG * 64, acc0, acc1, m, k,
                                          a_scales, w_scales, y, acc_out,
                                          AM == kAU4 ? a_zeros : nullptr,
                                          AM == kAU4 ? w_sums : nullptr, &epi);
}

// ------------------------------------------- decode GEMM, per-group scales
// A wave's part (segment seg, half h) of the decode tile is the 128 codes
// 256 seg + 128 h ... + 127, i.e. exactly weight group 2 seg + h: the two
// MFMAs of the part give the group's integer dot product (times 256), which
// turns into fp32 with the group's scale.  The scales load with the
// activation fragments, before the chunk's wait.
template <int RG>
struct DecGroupedLoads {
  uint4 av[2][2];
  uint16_t sc[2][2][RG];
};

template <int RG>
__device__ __forceinline__ void dec_load_grouped(const DecLane<RG>& t, const uint8_t* a_src,
                                                 int64_t c0, const uint16_t* __restrict__ wg_scales,
                                                 int64_t ngroups, int64_t k, DecGroupedLoads<RG>& l) {
  // Every load is unconditional, from a clamped address that is always
  // valid: rows past m re-read row 0 (a_src) and feed only outputs that are
  // not stored, and parts past the end are skipped below.  A zeroed register
  // refilled by a load under a branch would get a wait for every load in
  // flight (the weight stream included, which the compiler cannot see).
#pragma unroll
  for (int sl = 0; sl < 2; ++sl) {
    const int64_t seg = c0 + 2 * t.wave + sl;
    const int64_t segc = seg < t.nseg ? seg : t.nseg - 1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      l.av[sl][h] = *reinterpret_cast<const uint4*>(a_src + segc * DSEG + 64 * h);
#pragma unroll
      for (int q = 0; q < RG; ++q) {
        const int64_t col = t.n0 + 16 * q + t.r16;
        l.sc[sl][h][q] = wg_scales[(col < k ? col : k - 1) * ngroups + 2 * segc + h];
      }
    }
  }
}

template <int RG, bool GACC = false>
__device__ __forceinline__ void dec_mma_grouped(const DecLane<RG>& t, const unsigned char* wl,
                                                DecGroupedLoads<RG>& l, int64_t c0,
                                                v4f (&facc)[RG], int64_t m = 0, int64_t k = 0,
                                                int64_t ngroups = 0, int32_t* gacc = nullptr) {
  constexpr int SEGB = 16 * RG * DSEG;
  // The loads read kernel arguments the compiler treats as invariant, so it
  // may sink them past the wait below into their uses (each then pays a
  // memory latency of its own): an empty asm that takes every loaded value
  // keeps them issued before the wait.
#pragma unroll
  for (int sl = 0; sl < 2; ++sl)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      asm volatile("" ::"v"(l.av[sl][h].x), "v"(l.av[sl][h].y), "v"(l.av[sl][h].z), "v"(l.av[sl][h].w));
#pragma unroll
      for (int q = 0; q < RG; ++q) asm volatile("" ::"v"(l.sc[sl][h][q]));
    }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
  for (int sl = 0; sl < 2; ++sl) {
    if (c0 + 2 * t.wave + sl >= t.nseg) continue;  // uniform per wave
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const v4i a0 = widen(l.av[sl][h].x, l.av[sl][h].y), a1 = widen(l.av[sl][h].z, l.av[sl][h].w);
#pragma unroll
      for (int q = 0; q < RG; ++q) {
        const uint4 w = *reinterpret_cast<const uint4*>(
            wl + (2 * t.wave + sl) * SEGB + (16 * q + t.r16) * DSEG +
            16 * ((4 * h + t.g) ^ (t.r16 & 7)));
        v4i pg = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, widen(w.x, w.y), v4i{0, 0, 0, 0}, 0, 0, 0);
        pg = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, widen(w.z, w.w), pg, 0, 0, 0);
        if constexpr (GACC) {  // debug: the exact int32 sum of group 2 seg + h
          const int64_t col = t.n0 + 16 * q + t.r16;
          const int64_t grp = 2 * (c0 + 2 * t.wave + sl) + h;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int64_t row = 4 * t.g + e;
            if (row < m && col < k) gacc[(row * k + col) * ngroups + grp] = pg[e] >> 8;
          }
        }
        const float sg = h2f(l.sc[sl][h][q]);
#pragma unroll
        for (int e = 0; e < 4; ++e) facc[q][e] = __builtin_fmaf((float)pg[e], sg, facc[q][e]);
      }
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

template <int RG, bool GACC = false>
__global__ __launch_bounds__(64 * DEC_WAVES) void w4a4_decode_grouped_kernel(
    const uint8_t* __restrict__ a_codes, const uint16_t* __restrict__ a_scales,
    const uint8_t* __restrict__ w_codes, const uint16_t* __restrict__ wg_scales, int64_t m,
    int64_t k, int64_t d, uint16_t* __restrict__ y, int32_t* __restrict__ gacc) {
  __shared__ __align__(16) unsigned char wl[DCHUNK * 16 * RG * DSEG];
  __shared__ v4f partial[DEC_WAVES][RG][64];
  const int64_t rowb = d / 2;
  const DecLane<RG> t = dec_lane<RG>(w_codes, k, rowb, wl);
  const bool a_ok = t.r16 < m;
  const uint8_t* a_src = a_codes + (int64_t)(a_ok ? t.r16 : 0) * rowb + 16 * t.g;
  const int64_t ngroups = d / WG;

  v4f facc[RG];
#pragma unroll
  for (int q = 0; q < RG; ++q) facc[q] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  DecEpi epi;
  for (int64_t c0 = 0; c0 < t.nseg; c0 += DCHUNK) {
    // activation fragments and group scales ahead of the chunk's weights,
    // the epilogue's activation scales with the first chunk
    DecGroupedLoads<RG> l;
    dec_load_grouped<RG>(t, a_src, c0, wg_scales, ngroups, k, l);
    dec_issue_w(t, c0);
    if (c0 == 0) epi = dec_load_epi(t, m, k, a_scales, wg_scales, nullptr, nullptr);
    dec_mma_grouped<RG, GACC>(t, wl, l, c0, facc, m, k, ngroups, gacc);
  }
#pragma unroll
  for (int q = 0; q < RG; ++q) partial[t.wave][q][t.lane] = facc[q];
  __syncthreads();
  if (t.wave < RG) {
    v4f sum = partial[0][t.wave][t.lane];
#pragma unroll
    for (int w = 1; w < DEC_WAVES; ++w) sum += partial[w][t.wave][t.lane];
    const int64_t col = t.n0 + 16 * t.wave + t.r16;
    if (col < k) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t row = 4 * t.g + e;
        if (row < m) y[row * k + col] = (uint16_t)f16_mul_lo(sum[e] * (1.0f / 256.0f), epi.sa[e]);
      }
    }
  }
}

// ------------------------------------------------------- fused decode linear
// y = W4A4(rotate+quantise(x)) for m <= LD_FUSED_M tokens in one launch: the
// rotation of the activations runs as the GEMM's prologue ([SpinQuant] "The
// architecture: every piece explained": the online rotation fused into the
// low-bit matmul; [QuaRot] "End-to-end flow").
//
// Every workgroup first puts the weights of its first chunk in flight, then
// its waves 0..m-1 each rotate and quantise one token with the device code of
// rq_fwht_quant, into LDS.  The GEMM then reads its activation fragments from
// LDS.  Each workgroup repeats the (small) rotation instead of exchanging it
// with the others: a hand-over between workgroups on different XCDs needs
// agent-scope release/acquire (an L2 write-back and invalidation per XCD) and
// a wait, which measured 3x slower than two launches.  The rotation overlaps
// the weight stream, which the decode GEMM waits for anyway.
constexpr int LD_FUSED_M = 4;

// MW > 0 (8 or 4): every token is rotated by MW wavefronts together (m <= 8 / MW):
// wavefront w takes token w / MW, chunks (w % MW) * CPW .. + CPW - 1 of its
// row, runs e0 .. e8 on each and the stages between its own chunks, and
// writes the values (sign sigma taken out) to an fp32 row in LDS in element
// order.  After a barrier the token's 64 MW threads take pairs of adjacent
// positions q = 2a, 2a + 1 of one local chunk lc and finish the stages
// between wavefronts (chunks lc + CPW j, j = 0 .. MW - 1, in ascending
// order), then the absmax (wave max, then across the token's wavefronts
// through LDS), the scale and the codes.  Every butterfly has the same
// operands as in the one-wavefront rotation, up to the exact sign sigma,
// and fma(u sigma, c / s, M) = fma(u, (c / s) sigma, M): codes and scales are
// bit-identical to it.  MW = 0: one wavefront per token (row_rotate_quant).
//
// BITS = 8: the W4A8 linear (rq_fwht_quant8's per-token INT8 quantiser,
// codes [token][n] bytes in LDS, then the INT8-activation MFMA path of the
// decode GEMM with its epilogue); y is bit-identical to rq_fwht_quant8
// followed by rq_w4a8_gemm.
template <int N, bool HAS_SIGNS, int RG, int MW = 0, int BITS = 4>
__global__ __launch_bounds__(64 * DEC_WAVES) void w4a4_linear_decode_kernel(
    const __half* __restrict__ x, int64_t m, const int8_t* __restrict__ signs, float c32,
    const uint8_t* __restrict__ w_codes, const uint16_t* __restrict__ w_scales, int64_t k,
    uint16_t* __restrict__ y) {
  static_assert(BITS == 4 || BITS == 8, "INT4 or INT8 activation codes");
  constexpr int AM = BITS == 8 ? kA8 : kA4;
  constexpr int AW = BITS == 8 ? 2 : 1;  // activation code bytes per weight code byte
  // wl also takes the partial sums: each wave's RG x 64 sums go into the
  // staging segments that only that wave reads, once its MFMAs are done
  __shared__ __align__(16) unsigned char wl[DCHUNK * 16 * RG * DSEG];
  __shared__ __align__(16) unsigned char acodes[LD_FUSED_M][AW * N / 2];
  constexpr int kWavePitch = 2 * 16 * RG * DSEG / (int)sizeof(v4i);  // v4i per wave's two segments
  static_assert(kWavePitch >= RG * 64 + 1, "the partial sums and a scale fit in a wave's segments");
  // A token's fp16 scale stays in a register of the wavefront that finished
  // its quantisation (lane 0) until that wavefront's MFMAs are done; it then
  // goes into the wavefront's own staging segments, after its partial sums,
  // and the epilogue reads it there after the reduction's barrier.  (A
  // separate LDS array would take the kernel 8 bytes past 80 KB at n = 4096
  // with INT8 codes and two 16-row groups, and two workgroups would no
  // longer fit on a CU.)
  constexpr int kScaleStride = (MW > 0 ? MW : 1) * kWavePitch * (int)(sizeof(v4i) / 2);
  uint16_t* const scale_lds = reinterpret_cast<uint16_t*>(wl + RG * 64 * sizeof(v4i));
  bool scale_writer = false;  // uniform per wavefront
  uint16_t my_scale = 0;      // lane 0 of a writer
  constexpr int64_t rowb = N / 2;
  const DecLane<RG> t = dec_lane<RG>(w_codes, k, rowb, wl);

  // The first chunk's weights stream while the tokens are rotated.  A wave
  // that rotates a token loads it (and its sign bytes) before its weights:
  // loads return in order, so the token does not wait behind the weight
  // stream.
  if constexpr (MW > 0) {
    constexpr int NI = N / 512, CPW = NI / MW, RW = 8 * CPW;
    static_assert(NI % MW == 0 && DEC_WAVES % MW == 0, "whole chunks and tokens per wavefront");
    __shared__ __align__(16) float xb[DEC_WAVES / MW][N];  // one fp32 row per token (m <= 8 / MW)
    __shared__ float wmax[DEC_WAVES];
    const int L = t.lane;
    const int tok = t.wave / MW, part = t.wave % MW;
    const bool rot = tok < m;  // uniform per wavefront
    uint2 sg[CPW];
    uint4 raw[CPW];
    if (rot) {
      if constexpr (HAS_SIGNS) {
        const int8_t* sp = signs + 512 * CPW * part + 8 * L;
#pragma unroll
        for (int i = 0; i < CPW; ++i) sg[i] = *reinterpret_cast<const uint2*>(sp + 512 * i);
      }
      load_row(raw, x + (int64_t)tok * N + 512 * CPW * part, L);
    }
    dec_issue_w(t, 0);
    const RowLane rl = make_row_lane(L);
    if (rot) {
      float u[RW];
#pragma unroll
      for (int i = 0; i < CPW; ++i) {
        chunk_e0<HAS_SIGNS>(raw[i], sg[i], u + 8 * i);
        chunk512_stages(*reinterpret_cast<float(*)[8]>(u + 8 * i), rl);
      }
#pragma unroll
      for (int h = 8; h < RW; h <<= 1) butterfly_regs(u, h);  // chunk bits inside the wavefront
      // element 512 chunk + p of register r: p = (r & 1) | (lane_pair << 1) |
      // (r bit 2) << 7 | (r bit 1) << 8, chunk = part CPW + r / 8
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        const int e = 512 * (CPW * part + (r >> 3)) + ((r & 1) | (rl.lane_pair << 1) |
                                                      (((r >> 2) & 1) << 7) | (((r >> 1) & 1) << 8));
        xb[tok][e] = u[r] * rl.sigma;
      }
    }
    __syncthreads();
    constexpr int PG = 256 * CPW;           // position pairs of a token (per local chunk)
    constexpr int TT = 64 * MW;             // threads per token
    constexpr int PGT = (PG + TT - 1) / TT; // pairs per thread (MW = 8: half the threads)
    const int th = 64 * part + L;
    float v[PGT][2][MW];
    float amax = 0.0f;
    if (rot) {
#pragma unroll
      for (int gi = 0; gi < PGT; ++gi) {
        const int G = th + TT * gi;
        if (G >= PG) continue;
        const int a = G % 256, lc = G / 256;
#pragma unroll
        for (int sd = 0; sd < 2; ++sd) {
#pragma unroll
          for (int j = 0; j < MW; ++j) v[gi][sd][j] = xb[tok][512 * (lc + CPW * j) + 2 * a + sd];
#pragma unroll
          for (int h = 1; h < MW; h <<= 1) {  // chunk bits across wavefronts, ascending
#pragma unroll
            for (int j = 0; j < MW; ++j) {
              if (!(j & h)) {
                const float p0 = v[gi][sd][j], p1 = v[gi][sd][j + h];
                v[gi][sd][j] = p0 + p1;
                v[gi][sd][j + h] = p0 - p1;
              }
            }
          }
#pragma unroll
          for (int j = 0; j < MW; ++j) amax = fmaxf(amax, fabsf(v[gi][sd][j]));
        }
      }
    }
    amax = wave_max(amax);
    if (L == 0) wmax[t.wave] = amax;
    __syncthreads();
    if (rot) {
      float tmax = 0.0f;
#pragma unroll
      for (int w = 0; w < MW; ++w) tmax = fmaxf(tmax, wmax[MW * tok + w]);
      constexpr float kM = BITS == 4 ? kMagic : kMagic8;
      constexpr float kMLo = BITS == 4 ? kMagicLo : kMagic8Lo;
      constexpr float kMHi = BITS == 4 ? kMagicHi : kMagic8Hi;
      const uint16_t hb = scale_fp16<BITS == 4 ? 7 : 127>(tmax * c32);
      const bool subnormal = hb != 0 && hb < 0x0400u;
      const float mult = hb == 0 ? 0.0f : c32 / h2f(hb);
      scale_writer = part == 0;
      my_scale = hb;
#pragma unroll
      for (int gi = 0; gi < PGT; ++gi) {
        const int G = th + TT * gi;
        if (G >= PG) continue;
        const int a = G % 256, lc = G / 256;
#pragma unroll
        for (int j = 0; j < MW; ++j) {
          float t0 = __builtin_fmaf(v[gi][0][j], mult, kM);
          float t1 = __builtin_fmaf(v[gi][1][j], mult, kM);
          if (subnormal) {  // uniform: the scale is shared by the whole row
            t0 = fminf(fmaxf(t0, kMLo), kMHi);
            t1 = fminf(fmaxf(t1, kMLo), kMHi);
          }
          if constexpr (BITS == 4) {
            // (q1 + 8) << 4 | (q0 + 8), flipped to two's complement nibbles
            acodes[tok][256 * (lc + CPW * j) + a] =
                (unsigned char)(((f2u(t1) << 4) | (f2u(t0) & 0xFu)) ^ 0x88u);
          } else {
            // bytes q0 + 128, q1 + 128 of elements 2a, 2a + 1, flipped to
            // two's complement
            *reinterpret_cast<uint16_t*>(&acodes[tok][512 * (lc + CPW * j) + 2 * a]) =
                (uint16_t)(((f2u(t0) & 0xFFu) | ((f2u(t1) & 0xFFu) << 8)) ^ 0x8080u);
          }
        }
      }
    }
  } else if (t.wave < m) {
    uint2 sg[N / 512];
    if constexpr (HAS_SIGNS) load_signs(sg, signs, t.lane);
    uint4 raw[N / 512];
    load_row(raw, x + (int64_t)t.wave * N, t.lane);
    dec_issue_w(t, 0);
    row_rotate_quant<N, HAS_SIGNS, true, BITS>(raw, sg, t.lane, make_row_lane(t.lane), c32,
                                               acodes[t.wave], nullptr, &my_scale, nullptr);
    scale_writer = true;
  } else {
    dec_issue_w(t, 0);
  }
  __syncthreads();

  const bool a_ok = t.r16 < m;
  const unsigned char* a_src = acodes[a_ok ? t.r16 : 0] + 16 * AW * t.g;
  v4i acc0[RG], acc1[RG];
#pragma unroll
  for (int q = 0; q < RG; ++q) acc0[q] = acc1[q] = v4i{0, 0, 0, 0};
  dec_mma_chunk<RG, AM>(t, wl, a_src, a_ok, 0, acc0, acc1);
  for (int64_t c0 = DCHUNK; c0 < t.nseg; c0 += DCHUNK) {
    dec_issue_w(t, c0);
    dec_mma_chunk<RG, AM>(t, wl, a_src, a_ok, c0, acc0, acc1);
  }
  // (this wavefront's LDS reads are back: its segments are free)
  if (scale_writer && t.lane == 0) scale_lds[(int64_t)t.wave * kWavePitch * (sizeof(v4i) / 2)] = my_scale;
  dec_reduce_store<RG, BITS == 4 ? 8 : 4>(t, reinterpret_cast<v4i*>(wl), kWavePitch, acc0, acc1,
                                          m, k, scale_lds, w_scales, y, nullptr, nullptr, nullptr,
                                          nullptr, kScaleStride);
}
#undef RQ_DMA_NT

// ------------------------------------------------------------ large GEMM
// 256 x 224 output tile per 512-thread block: 8 waves in a 4 x 2 grid of
// 64 x 112 wave tiles (4 x 7 MFMA 16x16x64 tiles, 112 int32 accumulators per
// lane).  K runs in steps of 256 codes (128 packed bytes per row).
//
// Loads go straight from global memory into LDS (global_load_lds_dwordx4: no
// staging registers) one step ahead into the other of two 60 KB buffers, and
// the tiles stay packed in LDS.  Each wave issues four 8-row A loads and
// waves 0..6 four 8-row B loads per step; a wave waits for its loads only at
// the end of the step, so each load has a whole step of MFMA work to arrive,
// and the block meets at one barrier per 256 codes.
//
// LDS layout per buffer: 256 A rows then 224 B rows, 128 bytes each; the
// 16-byte part p of row r sits at part position p ^ (r & 7), so the 8-lane
// phases of the 16-byte fragment reads hit 8 different bank groups.  A DMA
// load writes lane L's 16 bytes at M0 + 16 L, so lane L of the load of rows
// r0..r0+7 fetches the global part that belongs at position L & 7 of row
// r0 + L / 8.
//
// Fragments: a step is two halves of 128 codes; in half u, lane
// (g = lane / 16, r = lane % 16) reads part 4u + g of its row (16 bytes = 32
// codes) and feeds the first 16 codes to one MFMA and the last 16 to the next.
// A and B use the same assignment, so every code meets its partner exactly
// once.  For 2048 x 28672 the tile gives exactly 1024 tiles, four per CU.
constexpr int LM = 256, LN = 224, LK = 256;  // block tile (codes)
constexpr int LN_WIDE = 256;                  // the wider tile (see wide_tiles)
constexpr int LPK = LK / 2;                   // packed bytes per row per step
constexpr int LTHREADS = 512;
static_assert(LN % 32 == 0 && LN_WIDE % 32 == 0 && LN_WIDE <= LM, "32-row B DMA slices, one per wave");
static_assert(LM == 32 * (LTHREADS / 64), "one 32-row A DMA slice per wave");

__device__ __forceinline__ int part_pos(int row, int p) { return p ^ (row & 7); }


// The grid holds at most one workgroup per CU and each workgroup walks its
// tiles in turn.  During the last K step of a tile it already loads step 0 of
// its next tile, and the finished tile leaves through the buffer that step
// does not use, so the next tile starts without a load ramp.
// AM = kAU4: unsigned activation nibbles with zero points a_zeros and the
// weight code sums w_sums (asymmetric activations); the MFMA sum is then
// 16 * sum qa qw and the epilogue subtracts z * w_sums[col].
// AM = kA8: INT8 activation bytes [m][d] (W4A8).  A step is then 128 codes:
// A rows stay 128 bytes per step, B rows are 64 bytes (part p of row r at
// part position p ^ ((r >> 1) & 3) of its 16-row group, so the 8-lane phases
// of the fragment reads hit distinct bank groups), each lane reads two A
// parts (order_a8 puts their bytes in widen's k order), the MFMA sum is
// 16 * sum qa qw, and the output tile is staged in its own LDS region (a
// 47 KB step buffer cannot hold a 59 KB half tile).
// GROUPED (with kA4): w_scales holds per-group scales [k][d / 128], and a
// half step (128 codes) is one group.  Each step's buffer also takes the two
// group scales of its B rows (4 bytes a row, dword DMA by waves 0..3); per
// half step every (i, j) tile's int32 sum over the group is two MFMAs from
// zero, and it turns into fp32 with its column's group scale.
template <int AM = kA4, bool GROUPED = false, bool GACC = false, int TN = LN>
__global__ __launch_bounds__(LTHREADS) void w4a4_large_kernel(const uint8_t* __restrict__ a_codes,
                                                              const uint16_t* __restrict__ a_scales,
                                                              const uint8_t* __restrict__ w_codes,
                                                              const uint16_t* __restrict__ w_scales,
                                                              int64_t m, int64_t k, int64_t d,
                                                              int tiles_m, int tiles, bool wide_store,
                                                              uint16_t* __restrict__ y,
                                                              int32_t* __restrict__ acc_out,
                                                              const uint8_t* __restrict__ a_zeros,
                                                              const int32_t* __restrict__ w_sums) {
  static_assert(AM == kA4 || AM == kAU4 || AM == kA8, "activation format");
  static_assert(!GROUPED || AM == kA4, "group scales with symmetric INT4 activations");
  static_assert(!GACC || GROUPED, "group sums are an output of the grouped GEMM");
  constexpr bool A8 = AM == kA8;
  constexpr int SHIFT = AM == kA4 ? 8 : 4;
  constexpr int KSTEP = A8 ? LK / 2 : LK;       // codes per step
  constexpr int APK = A8 ? KSTEP : KSTEP / 2;   // A bytes per row per step (128)
  constexpr int BPK = KSTEP / 2;                // B bytes per row per step
  constexpr int JT = TN / 32;                   // 16-column MFMA tiles per wave
  constexpr int WNC = TN / 2;                   // columns per wave
  constexpr int BUF = LM * APK + TN * BPK;      // codes of one step
  constexpr int BUFS = BUF + (GROUPED ? 4 * 256 : 0);  // + group scales: one buffer
  constexpr int OP = 2 * TN + 16;               // LDS row pitch of the output tile (bytes)
  // output rows go through LDS in NH passes of HR rows (GPP 16-row groups of
  // every wave per pass): two passes when half the tile fits, else four
  constexpr int NH = (A8 ? 2 * BUF + (LM / 2) * OP <= 160 * 1024 : (LM / 2) * OP <= BUF) ? 2 : 4;
  constexpr int HR = LM / NH, GPP = 4 / NH;
  constexpr int STAGE = A8 ? 2 * BUF : 0;       // A8: the staging region after both buffers
  static_assert(APK == LPK, "A rows are 128 bytes per step");
  static_assert(A8 ? 2 * BUF + HR * OP <= 160 * 1024 : HR * OP <= BUF, "the output staging fits");
  __shared__ __align__(16) unsigned char lds[A8 ? 2 * BUF + HR * OP : 2 * BUFS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;  // 4 x 2 waves of 64 x TN / 2
  const int g = lane >> 4, r16 = lane & 15;
  const int64_t rowa = A8 ? d : d / 2, rowb = d / 2;
  const int steps = (int)(d / KSTEP);
  const uint32_t lds_base =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)lds;

  // Tile order.  Workgroups go to the 8 XCDs round-robin (workgroup b to XCD
  // b % 8).  When both counts allow it, XCD x owns the contiguous tiles
  // [x T / 8, (x + 1) T / 8) and its workgroups take them in turn, so the CUs
  // of one XCD work on neighbouring tiles at the same time and share their A
  // and B slices in that XCD's L2.
  const int nb = (int)gridDim.x, b = (int)blockIdx.x;
  const bool by_xcd = tiles % 8 == 0 && nb % 8 == 0;
  const int per_xcd = tiles / 8, xcd_base = (b % 8) * per_xcd, xcd_stride = nb / 8;
#define RQ_TILE_OK(R) (by_xcd ? b / 8 + xcd_stride * (R) < per_xcd : b + nb * (R) < tiles)
#define RQ_TILE(R) (by_xcd ? xcd_base + b / 8 + xcd_stride * (R) : b + nb * (R))
  if (!RQ_TILE_OK(0)) return;  // uniform per workgroup
  int64_t m0 = (int64_t)(RQ_TILE(0) % tiles_m) * LM;
  int64_t n0 = (int64_t)(RQ_TILE(0) / tiles_m) * TN;

  // DMA rows of this lane: row 32 wave + 8 t + lane / 8 (t = 0..3) of the A
  // tile and (waves 0..6) of the B tile, 16-byte part drp of it; rows past the
  // matrix edge re-read the last row (their results are never stored).  With
  // 64-byte B rows (A8) one DMA covers 16 B rows: row 32 wave + 16 t + lane / 4
  // (t = 0, 1), part dbp.
  constexpr int NBT = A8 ? 2 : 4;  // B DMA instructions per wave and step
  const int dr0 = 32 * wave + (lane >> 3);
  const int drp = 16 * part_pos(lane >> 3, lane & 7);  // (dr0 + 8 t) & 7 == (lane >> 3)
  const int db0 = A8 ? 32 * wave + (lane >> 2) : dr0;
  const int dbp = A8 ? 16 * ((lane & 3) ^ ((lane >> 3) & 3)) : drp;  // ((lane >> 2) >> 1) & 3
  const uint8_t* asrc[4];
  const uint8_t* bsrc[NBT];
  // GROUPED: group scales of B row 64 wave + lane (waves 0..3), from group 0
  const int64_t gpitch = GROUPED ? d / WG * 2 : 0;  // bytes per row of group scales
  const uint8_t* gsrc = nullptr;
#define RQ_GSRC(N0_)                                                                \
  (GROUPED ? reinterpret_cast<const uint8_t*>(w_scales) +                           \
                 ((N0_) + 64 * wave + lane < k ? (N0_) + 64 * wave + lane : k - 1) * gpitch \
           : nullptr)
#define RQ_SET_SRC(M0_, N0_)                                                        \
  _Pragma("unroll") for (int t = 0; t < 4; ++t) {                                   \
    const int64_t ar_ = (M0_) + dr0 + 8 * t;                                        \
    asrc[t] = a_codes + (ar_ < m ? ar_ : m - 1) * rowa + drp;                       \
  }                                                                                 \
  _Pragma("unroll") for (int t = 0; t < NBT; ++t) {                                 \
    const int64_t br_ = (N0_) + db0 + (A8 ? 16 : 8) * t;                            \
    bsrc[t] = w_codes + (br_ < k ? br_ : k - 1) * rowb + dbp;                       \
  }                                                                                 \
  gsrc = RQ_GSRC(N0_);
  // loads of step S (codes S * KSTEP ..) into buffer BI_ (GROUPED: and the
  // step's two group scales of every B row, from G_)
#define RQ_ISSUE_FROM(BI_, A_, B_, G_, S)                                           \
  do {                                                                              \
    const uint32_t buf_ = lds_base + (uint32_t)((BI_) * BUFS);                      \
    if (GROUPED && wave < 4) RQ_DMA_D(buf_ + (uint32_t)(BUF + 256 * wave), (G_) + 4 * (S)); \
    const int64_t ka_ = (int64_t)(S) * APK, kb_ = (int64_t)(S) * BPK;               \
    _Pragma("unroll") for (int t = 0; t < 4; ++t)                                   \
      RQ_DMA(buf_ + (uint32_t)((32 * wave + 8 * t) * APK), (A_)[t] + ka_);          \
    if (wave < TN / 32) {                                                           \
      _Pragma("unroll") for (int t = 0; t < NBT; ++t)                               \
        RQ_DMA(buf_ + (uint32_t)(LM * APK + (32 * wave + (A8 ? 16 : 8) * t) * BPK), \
               (B_)[t] + kb_);                                                      \
    }                                                                               \
  } while (0)
  RQ_SET_SRC(m0, n0);

  // fragment offsets of this lane inside a 16-row group, halves 0 and 1
  // (A4 / AU4: the same for A and B); A8: A parts 2g and 2g + 1, B part g
  const int frag_off0 = r16 * LPK + 16 * part_pos(r16, A8 ? 2 * g : g);
  const int frag_off1 = r16 * LPK + 16 * part_pos(r16, A8 ? 2 * g + 1 : 4 + g);
  const int frag_b8 = r16 * BPK + 16 * (g ^ ((r16 >> 1) & 3));

  int par = 0;  // buffer of the current step
  RQ_ISSUE_FROM(0, asrc, bsrc, gsrc, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  for (int r = 0;; ++r) {
    const bool has_next = RQ_TILE_OK(r + 1);
    const int tn = has_next ? RQ_TILE(r + 1) : 0;
    const int64_t m0n = (int64_t)(tn % tiles_m) * LM, n0n = (int64_t)(tn / tiles_m) * TN;

    v4i acc[4][JT];
    v4f facc[4][JT];  // GROUPED: 256 * sum over groups of the group scale times its int32 sum
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < JT; ++j) {
        acc[i][j] = v4i{0, 0, 0, 0};
        facc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
      }

    for (int s = 0; s < steps; ++s) {
      // The next step's loads go out at the start of the step's second half:
      // issued together with the first half's fragment reads, their LDS
      // writes slowed those reads (measured 2-4% on the 2048 x 8192 -> 28672
      // prefill).  They still have half a step to land.  A8 (one half per
      // step) issues them after its first column tile (376 -> 364-368 us on
      // the same prefill), and so does GROUPED, in the first half (491 -> 476
      // us; at the second half it would spill 244 bytes and run 2.5x slower).
      constexpr bool kLateIssue = !A8 && !GROUPED;
      auto issue_next = [&]() {
        if (s + 1 < steps) {
          RQ_ISSUE_FROM(par ^ 1, asrc, bsrc, gsrc, s + 1);
        } else if (has_next) {
          const uint8_t* an[4];
          const uint8_t* bn[NBT];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int64_t ar = m0n + dr0 + 8 * t;
            an[t] = a_codes + (ar < m ? ar : m - 1) * rowa + drp;
          }
#pragma unroll
          for (int t = 0; t < NBT; ++t) {
            const int64_t br = n0n + db0 + (A8 ? 16 : 8) * t;
            bn[t] = w_codes + (br < k ? br : k - 1) * rowb + dbp;
          }
          RQ_ISSUE_FROM(par ^ 1, an, bn, RQ_GSRC(n0n), 0);
        }
      };
      const unsigned char* cur = lds + par * BUFS;
      uint32_t sgw[JT];  // GROUPED: the step's two group scales of column j
      if constexpr (GROUPED) {
#pragma unroll
        for (int j = 0; j < JT; ++j)
          sgw[j] = *reinterpret_cast<const uint32_t*>(cur + BUF + 4 * (wn * WNC + j * 16 + r16));
      }
#pragma unroll
      for (int u = 0; u < (A8 ? 1 : 2); ++u) {
        if (kLateIssue && u == 1) issue_next();
        const int fo = u ? frag_off1 : frag_off0;
        v4i af[2][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const unsigned char* ar = cur + (wm * 64 + i * 16) * APK;
          if constexpr (A8) {
            af[0][i] = order_a8(*reinterpret_cast<const uint4*>(ar + frag_off0));
            af[1][i] = order_a8(*reinterpret_cast<const uint4*>(ar + frag_off1));
          } else {
            const uint4 q = *reinterpret_cast<const uint4*>(ar + fo);
            if constexpr (AM == kAU4) {
              af[0][i] = widen_u(q.x, q.y);
              af[1][i] = widen_u(q.z, q.w);
            } else {
              af[0][i] = widen(q.x, q.y);
              af[1][i] = widen(q.z, q.w);
            }
          }
        }
#pragma unroll
        for (int j = 0; j < JT; ++j) {
          if constexpr (A8 || GROUPED) {
            if (u == 0 && j == 1) issue_next();
          }
          const uint4 q = *reinterpret_cast<const uint4*>(cur + LM * APK + (wn * WNC + j * 16) * BPK +
                                                          (A8 ? frag_b8 : fo));
          const v4i b0 = widen(q.x, q.y), b1 = widen(q.z, q.w);
          if constexpr (GROUPED) {
            const float sg = h2f((uint16_t)(u ? sgw[j] >> 16 : sgw[j]));  // group 2s + u
            v4i t[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
              t[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[0][i], b0, v4i{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i)
              t[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[1][i], b1, t[i], 0, 0, 0);
            if constexpr (GACC) {  // debug: the exact int32 sum of group 2 s + u
              const int64_t col = n0 + wn * WNC + j * 16 + r16;
              const int64_t ng = d / WG, grp = 2 * (int64_t)s + u;
#pragma unroll
              for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const int64_t row = m0 + wm * 64 + i * 16 + 4 * g + e;
                  if (row < m && col < k) acc_out[(row * k + col) * ng + grp] = t[i][e] >> 8;
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int e = 0; e < 4; ++e) facc[i][j][e] = __builtin_fmaf((float)t[i][e], sg, facc[i][j][e]);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[0][i], b0, acc[i][j], 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[1][i], b1, acc[i][j], 0, 0, 0);
          }
        }
      }
      // This wave's loads into buffer par ^ 1 have landed and its reads of
      // buffer par have returned (an asm barrier orders memory operations
      // only, so the LDS reads are waited for explicitly); after the barrier
      // the same holds for every wave, so buffer par may be refilled.
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      par ^= 1;
    }

    // Epilogue: lane holds rows 4g..4g+3 of every 16-row group, column r16 of
    // every 16-column group.  Buffer par holds step 0 of the next tile;
    // buffer par ^ 1 is free.  The lane indices are re-derived from an opaque
    // copy so that the compiler does not hoist one address register per store
    // out of the tile loop.
    int tid_o = tid;
    asm volatile("" : "+v"(tid_o));
    const int g = (tid_o & 63) >> 4, r16 = tid_o & 15;
    // Every scale, zero point and code sum the epilogue needs is loaded here,
    // unconditionally, from a clamped row or column that is always valid (past
    // m or k the value is dropped): a load under a branch gets a wait of its
    // own, and loads issued after the first stores would wait for those
    // (vector-memory counts drain in issue order), so one batch means one
    // memory round trip per tile instead of one per load.
    float sav[4][4];
    int32_t zv[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t arow = m0 + wm * 64 + i * 16 + 4 * g + e;
        const int64_t arowc = arow < m ? arow : m - 1;
        sav[i][e] = h2f(a_scales[arowc]);
        zv[i][e] = AM == kAU4 ? (int32_t)a_zeros[arowc] : 0;
      }
    }
    float swv[JT];
    int32_t wsv[JT];  // weight code sums (asymmetric activations only)
#pragma unroll
    for (int j = 0; j < JT; ++j) {
      const int64_t col = n0 + wn * WNC + j * 16 + r16;
      const int64_t colc = col < k ? col : k - 1;
      const float sw = GROUPED ? 0.0f : h2f(w_scales[colc]);
      const int32_t ws = AM == kAU4 ? w_sums[colc] : 0;
      swv[j] = col < k ? sw : 0.0f;
      wsv[j] = col < k ? ws : 0;
    }
    const bool full = m0 + LM <= m && n0 + TN <= k;
    if (full && wide_store) {
      // The fp16 tile goes through the free buffer (A8: its own region) in
      // NH passes of HR rows (OP-byte rows) and leaves as coalesced 16-byte
      // stores.  Pass h holds row groups GPP h .. GPP h + GPP - 1 of every
      // wave: staging row tr is tile row (tr / (16 GPP)) * 64 + 16 GPP h +
      // tr % (16 GPP).
      unsigned char* stg = lds + (A8 ? STAGE : (par ^ 1) * BUFS);
#pragma unroll
      for (int h = 0; h < NH; ++h) {
#pragma unroll
        for (int i2 = 0; i2 < GPP; ++i2) {
          const int i = GPP * h + i2;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int tr = wm * 16 * GPP + i2 * 16 + 4 * g + e;
            const float sa = sav[i][e];
            const int32_t z = zv[i][e];
#pragma unroll
            for (int j = 0; j < JT; ++j) {
              // exact: the MFMA sum is 2^SHIFT * sum qa qw
              const int32_t a = (acc[i][j][e] >> SHIFT) - z * wsv[j];
              *reinterpret_cast<uint16_t*>(stg + tr * OP + 2 * (wn * WNC + j * 16 + r16)) =
                  (uint16_t)(GROUPED ? f16_mul_lo(facc[i][j][e] * (1.0f / 256.0f), sa)
                                     : f16_mul_lo((float)a * sa, swv[j]));
            }
          }
        }
        __syncthreads();
        constexpr int CPR = TN * 2 / 16;  // 16-byte chunks per output row
        static_assert(HR * CPR % LTHREADS == 0, "whole store rounds");
#pragma unroll
        for (int q = 0; q < HR * CPR / LTHREADS; ++q) {
          const int c = tid_o + LTHREADS * q;
          const int tr = c / CPR, ch = c % CPR;
          const v4u_g v = *reinterpret_cast<const v4u_g*>(stg + tr * OP + 16 * ch);
          const int row = (tr / (16 * GPP)) * 64 + 16 * GPP * h + tr % (16 * GPP);
          __builtin_nontemporal_store(v, reinterpret_cast<v4u_g*>(y + (m0 + row) * k + n0 + 8 * ch));
        }
        __syncthreads();
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t row = m0 + wm * 64 + i * 16 + 4 * g + e;
          if (!full && row >= m) continue;
          const float sa = sav[i][e];
          const int32_t z = zv[i][e];
          const int64_t base = row * k + n0 + wn * WNC + r16;
#pragma unroll
          for (int j = 0; j < JT; ++j) {
            if (full || n0 + wn * WNC + j * 16 + r16 < k) {
              if constexpr (GROUPED)
                y[base + j * 16] = (uint16_t)f16_mul_lo(facc[i][j][e] * (1.0f / 256.0f), sa);
              else
                epilogue_store<SHIFT>(acc[i][j][e], sa, swv[j], base + j * 16, y, acc_out,
                                      z * wsv[j]);
            }
          }
        }
      }
    }
    if (!has_next) break;
    m0 = m0n;
    n0 = n0n;
    RQ_SET_SRC(m0, n0);
  }
#undef RQ_TILE_OK
#undef RQ_TILE
#undef RQ_GSRC
#undef RQ_SET_SRC
#undef RQ_ISSUE_FROM
}
#undef RQ_DMA

// Symmetric INT4 with one scale per group of G elements of fp32 rows: each
// thread owns 32 consecutive elements, the G / 32 threads of a group meet
// in a max across neighbouring lanes, and every thread writes its 16 code
// bytes.  scale = fp16(max / 7) rounded once, code = clamp(rne(x * fp32(1 /
// scale)), -8, 7).
template <int G>
__global__ __launch_bounds__(256) void quantize_groups_kernel(const float* __restrict__ x,
                                                              int64_t chunks, int64_t n,
                                                              uint8_t* __restrict__ codes,
                                                              uint16_t* __restrict__ scales) {
  constexpr int TPG = G / 32;  // threads per group
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  // every lane of a wavefront runs the same number of iterations (the
  // cross-lane max needs all of them): chunks is padded up to the stride
  const int64_t trips = (chunks + stride - 1) / stride;
  for (int64_t it = 0; it < trips; ++it) {
    const int64_t c = it * stride + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool live = c < chunks;
    const int64_t cc = live ? c : chunks - 1;
    float v[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 f = *reinterpret_cast<const float4*>(x + cc * 32 + 4 * i);
      v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
    for (int off = 1; off < TPG; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    const uint16_t hb = scale_fp16<7>(amax);
    const float mult = (hb == 0 || hb == 0x7C00u) ? 0.0f : 1.0f / h2f(hb);
    uint32_t wv[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float t = __builtin_amdgcn_fmed3f(__builtin_fmaf(v[i], mult, kMagic), kMagicLo, kMagicHi);
      wv[i / 8] |= ((f2u(t) & 15u) ^ 8u) << (4 * (i % 8));
    }
    if (live) {
      *reinterpret_cast<uint4*>(codes + cc * 16) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
      if (cc % TPG == 0) scales[cc / TPG] = hb;
    }
  }
}

// sums[j] = sum_i qw[j][i] over the packed signed INT4 codes of weight row j
// (one wavefront per row; an offline companion of the folded weights).
__global__ __launch_bounds__(256) void weight_code_sums_kernel(const uint8_t* __restrict__ w_codes,
                                                               int64_t k, int64_t rowb,
                                                               int32_t* __restrict__ sums) {
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (blockDim.x / 64);
  for (int64_t j = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6); j < k;
       j += waves) {
    int32_t acc = 0;
    for (int64_t c = lane; c < rowb / 16; c += 64) {
      const uint4 v = *reinterpret_cast<const uint4*>(w_codes + j * rowb + 16 * c);
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          const int32_t nib = (int32_t)((w4[q] >> (4 * b)) & 15u);
          acc += nib - ((nib & 8) << 1);  // sign-extend the nibble
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (lane == 0) sums[j] = acc;
  }
}

}  // namespace

hipError_t launch_quantize_groups(const float* x, int64_t rows, int64_t n, int group,
                                  uint8_t* codes, uint16_t* scales, hipStream_t stream) {
  const int64_t chunks = rows * (n / 32);
  const int64_t blocks = (chunks + 255) / 256;
  const int64_t cap = (int64_t)cu_count() * 16;
  const dim3 grid((unsigned)(blocks < cap ? blocks : cap));
  switch (group) {
    case 32: hipLaunchKernelGGL(quantize_groups_kernel<32>, grid, dim3(256), 0, stream, x, chunks, n, codes, scales); break;
    case 64: hipLaunchKernelGGL(quantize_groups_kernel<64>, grid, dim3(256), 0, stream, x, chunks, n, codes, scales); break;
    case 128: hipLaunchKernelGGL(quantize_groups_kernel<128>, grid, dim3(256), 0, stream, x, chunks, n, codes, scales); break;
    case 256: hipLaunchKernelGGL(quantize_groups_kernel<256>, grid, dim3(256), 0, stream, x, chunks, n, codes, scales); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_weight_code_sums(const uint8_t* w_codes, int64_t k, int64_t d, int32_t* sums,
                                   hipStream_t stream) {
  const int64_t blocks = (k + 3) / 4;
  const int64_t cap = (int64_t)cu_count() * 8;
  hipLaunchKernelGGL(weight_code_sums_kernel, dim3((unsigned)(blocks < cap ? blocks : cap)),
                     dim3(256), 0, stream, w_codes, k, d / 2, sums);
  return hipGetLastError();
}

// Shapes the persistent prefill kernel takes (d: whole 256-code steps).
bool large_shape(int64_t m, int64_t k, int64_t d) { return m >= 128 && k >= 224 && d % LK == 0; }

template <int AM, bool GROUPED, bool GACC, int TN>
hipError_t launch_large_tn(const uint8_t* a_codes, const uint16_t* a_scales, const uint8_t* a_zeros,
                           int64_t m, const uint8_t* w_codes, const uint16_t* w_scales,
                           const int32_t* w_sums, int64_t k, int64_t d, uint16_t* y, int32_t* acc,
                           hipStream_t stream) {
  const int tiles_m = (int)((m + LM - 1) / LM);
  const int64_t tiles = (int64_t)tiles_m * ((k + TN - 1) / TN);
  if (tiles > INT32_MAX) return hipErrorInvalidValue;
  const int64_t grid = tiles < cu_count() ? tiles : cu_count();  // one workgroup per CU
  // 16-byte output stores need 16-byte aligned rows and no int32 output
  const bool wide_store = acc == nullptr && k % 8 == 0 && ((uintptr_t)y & 15) == 0;
  hipLaunchKernelGGL((w4a4_large_kernel<AM, GROUPED, GACC, TN>), dim3((unsigned)grid),
                     dim3(LTHREADS), 0, stream, a_codes, a_scales, w_codes, w_scales, m, k, d,
                     tiles_m, (int)tiles, wide_store, y, acc, a_zeros, w_sums);
  return hipGetLastError();
}

// Tile width: 224 columns, or 256 where that takes fewer tile rounds on the
// CUs for the same work (rounds x width): k = 8192 gives 296 tiles of 224,
// two rounds, but 256 tiles of 256, one round; k = 28672 gives exactly four
// rounds of 224.  The 256-wide tile holds 128 int32 accumulators per lane;
// the W4A8 and per-group instantiations have no registers left for it.
bool wide_tiles(int64_t m, int64_t k) {
  const int64_t tiles_m = (m + LM - 1) / LM, cus = cu_count();
  const int64_t r224 = (tiles_m * ((k + LN - 1) / LN) + cus - 1) / cus;
  const int64_t r256 = (tiles_m * ((k + LN_WIDE - 1) / LN_WIDE) + cus - 1) / cus;
  return r256 * LN_WIDE < r224 * LN;
}

template <int AM, bool GROUPED = false, bool GACC = false>
hipError_t launch_large(const uint8_t* a_codes, const uint16_t* a_scales, const uint8_t* a_zeros,
                        int64_t m, const uint8_t* w_codes, const uint16_t* w_scales,
                        const int32_t* w_sums, int64_t k, int64_t d, uint16_t* y, int32_t* acc,
                        hipStream_t stream) {
  if constexpr (AM != kA8 && !GROUPED) {
    if (wide_tiles(m, k))
      return launch_large_tn<AM, GROUPED, GACC, LN_WIDE>(a_codes, a_scales, a_zeros, m, w_codes,
                                                         w_scales, w_sums, k, d, y, acc, stream);
  }
  return launch_large_tn<AM, GROUPED, GACC, LN>(a_codes, a_scales, a_zeros, m, w_codes, w_scales,
                                                w_sums, k, d, y, acc, stream);
}

hipError_t launch_w4a4_gemm(const uint8_t* a_codes, const uint16_t* a_scales, int64_t m,
                            const uint8_t* w_codes, const uint16_t* w_scales, int64_t k, int64_t d,
                            uint16_t* y, int32_t* acc, hipStream_t stream) {
  if (large_shape(m, k, d)) {
    return launch_large<kA4>(a_codes, a_scales, nullptr, m, w_codes, w_scales, nullptr, k, d, y,
                             acc, stream);
  } else if (m <= 16) {
    const int64_t blocks = (k + 15) / 16;
    if (d % (2 * DSEG) == 0) {
      // Two 16-row groups per workgroup halve the activation reads per weight
      // byte; worth it for many activation rows when the grid still covers
      // the CUs one and a half times.
      if (m > 4 && (k + 31) / 32 >= (int64_t)cu_count() * 3 / 2)
        hipLaunchKernelGGL(w4a4_decode_lds_kernel<2>, dim3((unsigned)((k + 31) / 32)),
                           dim3(64 * DEC_WAVES), 0, stream, a_codes, a_scales, w_codes, w_scales, m,
                           k, d, y, acc, nullptr, nullptr);
      else
        hipLaunchKernelGGL(w4a4_decode_lds_kernel<1>, dim3((unsigned)blocks), dim3(64 * DEC_WAVES),
                           0, stream, a_codes, a_scales, w_codes, w_scales, m, k, d, y, acc,
                           nullptr, nullptr);
    }
    else
      hipLaunchKernelGGL(w4a4_decode_kernel, dim3((unsigned)blocks), dim3(64 * DEC_WAVES), 0, stream,
                         a_codes, a_scales, w_codes, w_scales, m, k, d, y, acc);
  } else {
    const dim3 grid((unsigned)((k + TN - 1) / TN), (unsigned)((m + TM - 1) / TM));
    hipLaunchKernelGGL(w4a4_tile_kernel<kA4>, grid, dim3(256), 0, stream, a_codes, a_scales,
                       w_codes, w_scales, m, k, d, y, acc, nullptr, nullptr);
  }
  return hipGetLastError();
}

// The decode kernel (m <= 16, d % 256 == 0) or the tile kernel, for the
// activation format AM.
template <int AM>
hipError_t launch_gemm_variant(const uint8_t* a, const uint16_t* a_scales, const uint8_t* a_zeros,
                               int64_t m, const uint8_t* w_codes, const uint16_t* w_scales,
                               const int32_t* w_sums, int64_t k, int64_t d, uint16_t* y,
                               int32_t* acc, hipStream_t stream) {
  if (m <= 16 && d % (2 * DSEG) == 0) {
    if (m > 4 && (k + 31) / 32 >= (int64_t)cu_count() * 3 / 2)
      hipLaunchKernelGGL((w4a4_decode_lds_kernel<2, AM>), dim3((unsigned)((k + 31) / 32)),
                         dim3(64 * DEC_WAVES), 0, stream, a, a_scales, w_codes, w_scales, m, k, d,
                         y, acc, a_zeros, w_sums);
    else
      hipLaunchKernelGGL((w4a4_decode_lds_kernel<1, AM>), dim3((unsigned)((k + 15) / 16)),
                         dim3(64 * DEC_WAVES), 0, stream, a, a_scales, w_codes, w_scales, m, k, d,
                         y, acc, a_zeros, w_sums);
  } else {
    const dim3 grid((unsigned)((k + TN - 1) / TN), (unsigned)((m + TM - 1) / TM));
    hipLaunchKernelGGL(w4a4_tile_kernel<AM>, grid, dim3(256), 0, stream, a, a_scales, w_codes,
                       w_scales, m, k, d, y, acc, a_zeros, w_sums);
  }
  return hipGetLastError();
}

hipError_t launch_w4a4_gemm_grouped(const uint8_t* a_codes, const uint16_t* a_scales, int64_t m,
                                    const uint8_t* w_codes, const uint16_t* wg_scales, int64_t k,
                                    int64_t d, uint16_t* y, int32_t* gacc, hipStream_t stream) {
  // the persistent prefill kernel (a half step is one group) reads each row's
  // two group scales of a step as one dword: 4-byte aligned scales only
  if (large_shape(m, k, d) && (reinterpret_cast<uintptr_t>(wg_scales) & 3u) == 0)
    return gacc != nullptr
               ? launch_large<kA4, true, true>(a_codes, a_scales, nullptr, m, w_codes, wg_scales,
                                               nullptr, k, d, y, gacc, stream)
               : launch_large<kA4, true>(a_codes, a_scales, nullptr, m, w_codes, wg_scales,
                                         nullptr, k, d, y, nullptr, stream);
  if (m <= 16 && d % (2 * DSEG) == 0) {
    const bool rg2 = m > 4 && (k + 31) / 32 >= (int64_t)cu_count() * 3 / 2;
    const dim3 grid((unsigned)(rg2 ? (k + 31) / 32 : (k + 15) / 16));
    if (rg2 && gacc != nullptr)
      hipLaunchKernelGGL((w4a4_decode_grouped_kernel<2, true>), grid, dim3(64 * DEC_WAVES), 0,
                         stream, a_codes, a_scales, w_codes, wg_scales, m, k, d, y, gacc);
    else if (rg2)
      hipLaunchKernelGGL((w4a4_decode_grouped_kernel<2>), grid, dim3(64 * DEC_WAVES), 0, stream,
                         a_codes, a_scales, w_codes, wg_scales, m, k, d, y, nullptr);
    else if (gacc != nullptr)
      hipLaunchKernelGGL((w4a4_decode_grouped_kernel<1, true>), grid, dim3(64 * DEC_WAVES), 0,
                         stream, a_codes, a_scales, w_codes, wg_scales, m, k, d, y, gacc);
    else
      hipLaunchKernelGGL((w4a4_decode_grouped_kernel<1>), grid, dim3(64 * DEC_WAVES), 0, stream,
                         a_codes, a_scales, w_codes, wg_scales, m, k, d, y, nullptr);
  } else {
    const dim3 grid((unsigned)((k + TN - 1) / TN), (unsigned)((m + TM - 1) / TM));
    hipLaunchKernelGGL((w4a4_tile_kernel<kA4, true>), grid, dim3(256), 0, stream, a_codes,
                       a_scales, w_codes, wg_scales, m, k, d, y, gacc, nullptr, nullptr);
  }
  return hipGetLastError();
}

hipError_t launch_w4a8_gemm(const int8_t* a_codes8, const uint16_t* a_scales, int64_t m,
                            const uint8_t* w_codes, const uint16_t* w_scales, int64_t k, int64_t d,
                            uint16_t* y, int32_t* acc, hipStream_t stream) {
  const uint8_t* a8 = reinterpret_cast<const uint8_t*>(a_codes8);
  if (large_shape(m, k, d))  // the persistent prefill kernel, 128-code steps
    return launch_large<kA8>(a8, a_scales, nullptr, m, w_codes, w_scales, nullptr, k, d, y, acc,
                             stream);
  return launch_gemm_variant<kA8>(a8, a_scales, nullptr, m, w_codes, w_scales, nullptr, k, d, y,
                                  acc, stream);
}

hipError_t launch_w4a4_gemm_asym(const uint8_t* a_codes, const uint16_t* a_scales,
                                 const uint8_t* a_zeros, int64_t m, const uint8_t* w_codes,
                                 const uint16_t* w_scales, const int32_t* w_sums, int64_t k,
                                 int64_t d, uint16_t* y, int32_t* acc, hipStream_t stream) {
  if (large_shape(m, k, d))  // the persistent prefill kernel
    return launch_large<kAU4>(a_codes, a_scales, a_zeros, m, w_codes, w_scales, w_sums, k, d, y,
                              acc, stream);
  return launch_gemm_variant<kAU4>(a_codes, a_scales, a_zeros, m, w_codes, w_scales, w_sums, k,
                                   d, y, acc, stream);
}


size_t linear_decode_workspace_bytes(int64_t m, int64_t d) {
  return (size_t)m * (size_t)(d / 2) + 64;  // codes, then the fp16 scales
}

namespace {
template <int N, bool HAS_SIGNS, int RG, int MW, int BITS>
hipError_t launch_ld(const uint16_t* x, int64_t m, const int8_t* signs, const uint8_t* w_codes,
                     const uint16_t* w_scales, int64_t k, uint16_t* y, hipStream_t stream) {
  const float c32 = (float)(1.0 / __builtin_sqrt((double)N));
  const int64_t grid = (k + 16 * RG - 1) / (16 * RG);
  if (MW > 0 && m > DEC_WAVES / (MW > 0 ? MW : 1)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((w4a4_linear_decode_kernel<N, HAS_SIGNS, RG, MW, BITS>), dim3((unsigned)grid),
                     dim3(64 * DEC_WAVES), 0, stream, reinterpret_cast<const __half*>(x), m, signs,
                     c32, w_codes, w_scales, k, y);
  return hipGetLastError();
}

template <int N, int BITS>
hipError_t launch_ld_n(const uint16_t* x, int64_t m, const int8_t* signs, const uint8_t* w_codes,
                       const uint16_t* w_scales, int64_t k, uint16_t* y, hipStream_t stream) {
  // Two 16-row weight groups per workgroup when that still gives every CU a
  // workgroup: the kernel holds a whole row rotation, so fewer of its
  // workgroups fit on a CU than of the plain decode kernel.
  const bool rg2 = (k + 31) / 32 >= (int64_t)cu_count();
  // n = 4096 with one workgroup per CU at most: one token is rotated by all
  // 8 wavefronts, two tokens by 4 each (measured: 6.1 -> 5.2 us and 6.05 ->
  // 5.9 us for k = 4096).  With 3 or 4 tokens, 2 wavefronts a token lost to
  // one (the exchange and the finishing work outweigh the halved butterflies
  // once two such wavefronts share a SIMD).  The fp32 rows this takes (16 KB
  // a token) fit beside one 16-row weight group.
  const bool sg = signs != nullptr;
  if constexpr (N == 4096) {
    if (!rg2 && m <= 2 && (k + 15) / 16 <= (int64_t)cu_count()) {
      if (m == 1)
        return sg ? launch_ld<N, true, 1, 8, BITS>(x, m, signs, w_codes, w_scales, k, y, stream)
                  : launch_ld<N, false, 1, 8, BITS>(x, m, signs, w_codes, w_scales, k, y, stream);
      return sg ? launch_ld<N, true, 1, 4, BITS>(x, m, signs, w_codes, w_scales, k, y, stream)
                : launch_ld<N, false, 1, 4, BITS>(x, m, signs, w_codes, w_scales, k, y, stream);
    }
  }
  if (sg)
    return rg2 ? launch_ld<N, true, 2, 0, BITS>(x, m, signs, w_codes, w_scales, k, y, stream)
               : launch_ld<N, true, 1, 0, BITS>(x, m, signs, w_codes, w_scales, k, y, stream);
  return rg2 ? launch_ld<N, false, 2, 0, BITS>(x, m, signs, w_codes, w_scales, k, y, stream)
             : launch_ld<N, false, 1, 0, BITS>(x, m, signs, w_codes, w_scales, k, y, stream);
}

template <int BITS>
hipError_t launch_ld_d(const uint16_t* x, int64_t m, int64_t d, const int8_t* signs,
                       const uint8_t* w_codes, const uint16_t* w_scales, int64_t k, uint16_t* y,
                       hipStream_t stream) {
  switch (d) {
    case 512: return launch_ld_n<512, BITS>(x, m, signs, w_codes, w_scales, k, y, stream);
    case 1024: return launch_ld_n<1024, BITS>(x, m, signs, w_codes, w_scales, k, y, stream);
    case 2048: return launch_ld_n<2048, BITS>(x, m, signs, w_codes, w_scales, k, y, stream);
    case 4096: return launch_ld_n<4096, BITS>(x, m, signs, w_codes, w_scales, k, y, stream);
    case 8192: return launch_ld_n<8192, BITS>(x, m, signs, w_codes, w_scales, k, y, stream);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

hipError_t launch_linear_decode(const uint16_t* x, int64_t m, int64_t d, const int8_t* signs,
                                const uint8_t* w_codes, const uint16_t* w_scales, int64_t k,
                                uint16_t* y, void* workspace, hipStream_t stream) {
  if (m > LD_FUSED_M) {
    // More tokens than the prologue rotates cheaply: the rotation kernel
    // writes codes and scales into the workspace, then the decode GEMM.
    uint8_t* codes = static_cast<uint8_t*>(workspace);
    uint16_t* scales = reinterpret_cast<uint16_t*>(codes + m * (d / 2));
    const hipError_t e =
        launch_fwht_quant(x, false, m, (int)d, signs, codes, scales, nullptr, stream);
    if (e != hipSuccess) return e;
    return launch_w4a4_gemm(codes, scales, m, w_codes, w_scales, k, d, y, nullptr, stream);
  }
  return launch_ld_d<4>(x, m, d, signs, w_codes, w_scales, k, y, stream);
}

hipError_t launch_linear_decode_w4a8(const uint16_t* x, int64_t m, int64_t d, const int8_t* signs,
                                     const uint8_t* w_codes, const uint16_t* w_scales, int64_t k,
                                     uint16_t* y, hipStream_t stream) {
  if (m > LD_FUSED_M) return hipErrorInvalidValue;
  return launch_ld_d<8>(x, m, d, signs, w_codes, w_scales, k, y, stream);
}

}  // namespace rq
