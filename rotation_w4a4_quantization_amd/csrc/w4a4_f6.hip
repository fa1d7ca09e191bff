// W4A4 prefill GEMM on the 6-bit matrix-core path of CDNA4 (gfx950): the
// INT4 codes travel in fp6 E3M2 containers and multiply on
// v_mfma_f32_16x16x128_f8f6f4.
//
// Pages cited:
//   [RQ]     llms.blog, "Rotational Quantization: How Orthogonal Transforms and
//            Hadamard Incoherence Enable Outlier-Free Low-Bit Inference",
//            "Hardware Execution and Serving Economics", part 1 (rotated W4A4
//            layers run integer GEMMs end to end, and 4-bit matrix arithmetic
//            has twice the throughput of 8-bit).
//   [QuaRot] aicassindra.com, QuaRot explainer, "End-to-end flow" (the INT4
//            rotated activation multiplies the INT4 folded weight).
//
// Why it is exact.  gfx950 has no INT4 MFMA, but every INT4 code -8..7 is a
// value of the OCP MX E3M2 float (sign, 3 exponent bits with bias 3, 2
// mantissa bits): 1 = 2^0, 2 = 2^1, 3 = 1.5 * 2^1, 4..7 = (1 + m/4) * 2^2,
// 8 = 2^3.  Products are integers of magnitude <= 64, and every partial sum
// of a dot product over d <= 2^18 codes stays below 2^24, so the fp32
// accumulators hold the int32 accumulator exactly, whatever order the
// hardware adds in.  In an issue loop with random codes the 6-bit MFMA does
// 7.4-7.5 POP/s against 4.3-4.5 for the int8 MFMA on the same values widened
// to bytes: 1.66x.
//
// F6 layout.  A matrix of R rows of d codes (d % 128 == 0) takes 3Rd/4
// bytes, group-major: the 128-code group c of row r is the 96 bytes at
// (c R + r) * 96, so one K step of a tile of rows is one contiguous run of
// whole cache lines.  The group's 32-code block b (codes
// 128c + 32b + j, j = 0..31) is one 192-bit little-endian word with code j
// in bits 6j..6j+5, which is exactly one lane's MFMA operand (six
// registers).  The word's first 16 bytes sit at group byte 16b, its last 8
// bytes at group byte 64 + 16 (b % 2) + 8 (b / 2): tail unit 4 holds the
// tails of blocks 0 and 2, unit 5 those of blocks 1 and 3.  A lane reads its
// operand as two 16-byte LDS reads, its block's head and its tail unit,
// keeping the half that is its own.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "rq_internal.h"
#include "rq_row_device.h"

namespace rq {
namespace {

typedef int v8i6 __attribute__((ext_vector_type(8)));
typedef float v4f6 __attribute__((ext_vector_type(4)));
typedef unsigned int v4u6 __attribute__((ext_vector_type(4)));

// E3M2 code of the INT4 code in nibble n (two's complement): entries 0..9
// in LO, 10..15 in HI, 6 bits each.  0 -> 0, 1 -> 0x0C (2^0), 2 -> 0x10,
// 3 -> 0x12, 4 -> 0x14, 5 -> 0x15, 6 -> 0x16, 7 -> 0x17, -8 -> 0x38
// (sign | 2^3), -7 -> 0x37, ..., -1 -> 0x2C.
__device__ __forceinline__ uint32_t e3m2_of_nibble(uint32_t n) {
  constexpr uint64_t LO = 0x0DF85D6554490300ull, HI = 0xB30CB4D76ull;
  return (uint32_t)((n < 10 ? LO >> (6 * n) : HI >> (6 * (n - 10))) & 63u);
}

// One thread per 32-code block: 16 bytes of packed INT4 codes (code i in
// nibble i) in, one 24-byte F6 word out.
__global__ __launch_bounds__(256) void pack_f6_kernel(const uint8_t* __restrict__ codes,
                                                      int64_t rows, int64_t d,
                                                      uint8_t* __restrict__ out) {
  const int64_t nb = d / 32, total = rows * nb;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / nb, blk = i - r * nb;
    const uint4 q = *reinterpret_cast<const uint4*>(codes + r * (d / 2) + 16 * blk);
    const uint32_t in[4] = {q.x, q.y, q.z, q.w};
    uint32_t w[6] = {0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const uint32_t c = e3m2_of_nibble((in[j >> 3] >> (4 * (j & 7))) & 15u);
      const int pos = 6 * j;
      w[pos >> 5] |= c << (pos & 31);
      if ((pos & 31) > 26) w[(pos >> 5) + 1] |= c >> (32 - (pos & 31));
    }
    uint8_t* grp = out + ((blk >> 2) * rows + r) * 96;
    const int b = (int)(blk & 3);
    *reinterpret_cast<uint4*>(grp + 16 * b) = make_uint4(w[0], w[1], w[2], w[3]);
    *reinterpret_cast<uint2*>(grp + 64 + 16 * (b & 1) + 8 * (b >> 1)) = make_uint2(w[4], w[5]);
  }
}

// One DMA load: lane L's 16 bytes go to LDS byte m0 + 16 L.
#define RQF6_DMA(M0, ADDR)                                                         \
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"     \
               :                                                                   \
               : "v"(ADDR), "s"(M0)                                                \
               : "memory", "m0")

// ------------------------------------------------------------ the kernel
// 256 x TN output tile per 512-thread block: 8 waves in a 4 x 2 grid of
// 64 x TN/2 wave tiles (4 x TN/32 MFMA tiles of 16 x 16, fp32 accumulators).
// K runs in steps of 128 codes (96 bytes per row); loads go global -> LDS
// (global_load_lds_dwordx4) one step ahead into the other of two buffers.
//
// LDS layout of a step: 256 A rows then TN B rows, 96 bytes (six 16-byte
// slots) each; row r keeps its unit u (units 0..3: block heads, 4 and 5:
// tails of blocks 0,2 and 1,3) in slot u ^ flip(r), flip(r) = (r / 4) % 2.
// Every fragment read is 16 bytes.  Lane (g, r) reads head g and tail unit
// 4 + g % 2 of row r; an LDS read probe on gfx950 (ds_read_b128 throughput
// for lane -> address patterns) found both read kinds as fast as a linear
// 1 KB read with this placement.  Other placements measured 1.7x slower
// reads: a per-row rotation of the units, flip(r) = (r / 8) % 2, tail units
// shared by blocks (0,1) and (2,3) (lanes g and g + 16 then read one
// address), and tails read as 8-byte halves, single or merged by the
// compiler into ds_read2st64_b64.
//
// One DMA instruction fills 64 consecutive slots, so a wave's three cover 32
// rows: slot s (0..191) of wave w is row 32 w + s / 6, slot s % 6 of it,
// which holds unit (s % 6) ^ flip(row).
constexpr int FM = 256, FN = 224, FN_WIDE = 256, FK = 128, FROW = 96, FTHREADS = 512;

__device__ __forceinline__ int f6_flip(int r) { return (r >> 2) & 1; }

template <int TN>
__global__ __launch_bounds__(FTHREADS) void w4a4_f6_kernel(const uint8_t* __restrict__ a6,
                                                           const uint16_t* __restrict__ a_scales,
                                                           const uint8_t* __restrict__ w6,
                                                           const uint16_t* __restrict__ w_scales,
                                                           int64_t m, int64_t k, int64_t d,
                                                           int tiles_m, int tiles, bool wide_store,
                                                           uint16_t* __restrict__ y,
                                                           int32_t* __restrict__ acc_out) {
  constexpr int JT = TN / 32;   // 16-column MFMA tiles per wave
  constexpr int WNC = TN / 2;   // columns per wave
  constexpr int BUF = (FM + TN) * FROW;
  constexpr int OP = 2 * TN + 16;  // LDS row pitch of the staged output tile (bytes)
  constexpr int NH = (FM / 2) * OP <= BUF ? 2 : 4;
  constexpr int HR = FM / NH, GPP = 4 / NH;
  static_assert(HR * OP <= BUF, "the output staging fits a step buffer");
  static_assert(FM == 32 * (FTHREADS / 64) && TN % 32 == 0 && TN <= FM, "32 DMA rows per wave");
  __shared__ __align__(16) unsigned char lds[2 * BUF];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 4, r16 = lane & 15;
  const int64_t astep = m * FROW, bstep = k * FROW;  // bytes from one K step to the next
  const int steps = (int)(d / FK);
  const uint32_t lds_base =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)lds;

  // Tile order: workgroup b runs on XCD b % 8; when the counts allow, XCD x
  // owns the contiguous tiles [x T / 8, (x + 1) T / 8), so the CUs of one XCD
  // share A and B slices in its L2.
  const int nb = (int)gridDim.x, b = (int)blockIdx.x;
  const bool by_xcd = tiles % 8 == 0 && nb % 8 == 0;
  const int per_xcd = tiles / 8, xcd_base = (b % 8) * per_xcd, xcd_stride = nb / 8;
#define RQF6_TILE_OK(R) (by_xcd ? b / 8 + xcd_stride * (R) < per_xcd : b + nb * (R) < tiles)
#define RQF6_TILE(R) (by_xcd ? xcd_base + b / 8 + xcd_stride * (R) : b + nb * (R))
  if (!RQF6_TILE_OK(0)) return;  // uniform per workgroup
  int64_t m0 = (int64_t)(RQF6_TILE(0) % tiles_m) * FM;
  int64_t n0 = (int64_t)(RQF6_TILE(0) / tiles_m) * TN;

  // This lane's DMA rows and units (rows past the matrix edge re-read the
  // last row; their results are never stored).
  int drow[3], dunit[3];
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    const int s = 64 * t + lane, rr = s / 6, p = s - 6 * rr;
    drow[t] = 32 * wave + rr;                      // (32 wave + rr) % 16 == rr % 16
    dunit[t] = p ^ f6_flip(rr);
  }
  const uint8_t* asrc[3];
  const uint8_t* bsrc[3];
#define RQF6_SET_SRC(A_, B_, M0_, N0_)                                              \
  _Pragma("unroll") for (int t = 0; t < 3; ++t) {                                   \
    const int64_t ar_ = (M0_) + drow[t], br_ = (N0_) + drow[t];                     \
    (A_)[t] = a6 + (ar_ < m ? ar_ : m - 1) * FROW + 16 * dunit[t];                  \
    (B_)[t] = w6 + (br_ < k ? br_ : k - 1) * FROW + 16 * dunit[t];                  \
  }
#define RQF6_ISSUE(BI_, A_, B_, S)                                                  \
  do {                                                                              \
    const uint32_t buf_ = lds_base + (uint32_t)((BI_) * BUF);                       \
    const int64_t ka_ = (int64_t)(S) * astep, kb_ = (int64_t)(S) * bstep;           \
    _Pragma("unroll") for (int t = 0; t < 3; ++t)                                   \
      RQF6_DMA(buf_ + (uint32_t)(3072 * wave + 1024 * t), (A_)[t] + ka_);           \
    if (wave < TN / 32) {                                                           \
      _Pragma("unroll") for (int t = 0; t < 3; ++t)                                 \
        RQF6_DMA(buf_ + (uint32_t)(FM * FROW + 3072 * wave + 1024 * t), (B_)[t] + kb_); \
    }                                                                               \
  } while (0)
  RQF6_SET_SRC(asrc, bsrc, m0, n0);

  // fragment offsets of this lane inside a 16-row group: its block g's head
  // and tail unit 4 + g % 2, of which it keeps half g / 2
  const int flip = f6_flip(r16);
  const int head_off = 16 * (6 * r16 + (g ^ flip));
  const int tail_off = 16 * (6 * r16 + ((4 + (g & 1)) ^ flip));
  const bool tail_hi = (g >> 1) != 0;

  int par = 0;  // buffer of the current step
  RQF6_ISSUE(0, asrc, bsrc, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  for (int r = 0;; ++r) {
    const bool has_next = RQF6_TILE_OK(r + 1);
    const int tn = has_next ? RQF6_TILE(r + 1) : 0;
    const int64_t m0n = (int64_t)(tn % tiles_m) * FM, n0n = (int64_t)(tn / tiles_m) * TN;

    v4f6 acc[4][JT];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < JT; ++j) acc[i][j] = v4f6{0.0f, 0.0f, 0.0f, 0.0f};

    for (int s = 0; s < steps; ++s) {
      const unsigned char* cur = lds + par * BUF;
      // The next step's loads (or the next tile's first) go out before this
      // step's fragment reads, so they have the whole step to land (A/B on
      // the 2048 x 8192 -> 28672 prefill: 274 us, against 288 us when they
      // went out after the first column tile).
      if (s + 1 < steps) {
        RQF6_ISSUE(par ^ 1, asrc, bsrc, s + 1);
      } else if (has_next) {
        const uint8_t* an[3];
        const uint8_t* bn[3];
        RQF6_SET_SRC(an, bn, m0n, n0n);
        RQF6_ISSUE(par ^ 1, an, bn, 0);
      }
      v8i6 af[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const unsigned char* ar = cur + (wm * 64 + i * 16) * FROW;
        const uint4 h = *reinterpret_cast<const uint4*>(ar + head_off);
        const uint4 t = *reinterpret_cast<const uint4*>(ar + tail_off);
        af[i] = v8i6{(int)h.x, (int)h.y, (int)h.z, (int)h.w, (int)(tail_hi ? t.z : t.x),
                     (int)(tail_hi ? t.w : t.y), 0, 0};
      }
#pragma unroll
      for (int j = 0; j < JT; ++j) {
        const unsigned char* br = cur + (FM + wn * WNC + j * 16) * FROW;
        const uint4 h = *reinterpret_cast<const uint4*>(br + head_off);
        const uint4 t = *reinterpret_cast<const uint4*>(br + tail_off);
        const v8i6 bf = v8i6{(int)h.x, (int)h.y, (int)h.z, (int)h.w, (int)(tail_hi ? t.z : t.x),
                             (int)(tail_hi ? t.w : t.y), 0, 0};
#pragma unroll
        for (int i = 0; i < 4; ++i)  // format 3 = E3M2 for both operands; no block scales
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bf, acc[i][j], 3, 3,
                                                                         0, 0, 0, 0);
      }
      // This wave's loads into buffer par ^ 1 have landed and its reads of
      // buffer par have returned; after the barrier the same holds for every
      // wave, so buffer par may be refilled.
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      par ^= 1;
    }

    // Epilogue: lane holds rows 4g..4g+3 of every 16-row group, column r16 of
    // every 16-column group; acc is the exact integer sum, so
    // y = fp16(fp32(acc * sa) * sw) rounded once, as in the int8 path.
    int tid_o = tid;
    asm volatile("" : "+v"(tid_o));
    const int g = (tid_o & 63) >> 4, r16 = tid_o & 15;
    float sav[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t arow = m0 + wm * 64 + i * 16 + 4 * g + e;
        sav[i][e] = h2f(a_scales[arow < m ? arow : m - 1]);
      }
    float swv[JT];
#pragma unroll
    for (int j = 0; j < JT; ++j) {
      const int64_t col = n0 + wn * WNC + j * 16 + r16;
      const float sw = h2f(w_scales[col < k ? col : k - 1]);
      swv[j] = col < k ? sw : 0.0f;
    }
    const bool full = m0 + FM <= m && n0 + TN <= k;
    if (full && wide_store) {
      // the fp16 tile leaves through the free buffer in NH passes of HR rows
      // as coalesced 16-byte stores; staging row tr is tile row
      // (tr / (16 GPP)) * 64 + 16 GPP h + tr % (16 GPP)
      unsigned char* stg = lds + (par ^ 1) * BUF;
#pragma unroll
      for (int h = 0; h < NH; ++h) {
#pragma unroll
        for (int i2 = 0; i2 < GPP; ++i2) {
          const int i = GPP * h + i2;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int tr = wm * 16 * GPP + i2 * 16 + 4 * g + e;
#pragma unroll
            for (int j = 0; j < JT; ++j)
              *reinterpret_cast<uint16_t*>(stg + tr * OP + 2 * (wn * WNC + j * 16 + r16)) =
                  (uint16_t)f16_mul_lo(acc[i][j][e] * sav[i][e], swv[j]);
          }
        }
        __syncthreads();
        constexpr int CPR = TN * 2 / 16;  // 16-byte chunks per output row
#pragma unroll
        for (int q = 0; q < (HR * CPR + FTHREADS - 1) / FTHREADS; ++q) {
          const int c = tid_o + FTHREADS * q;
          if (HR * CPR % FTHREADS != 0 && c >= HR * CPR) break;  // last round of 224-wide tiles
          const int tr = c / CPR, ch = c % CPR;
          const v4u6 v = *reinterpret_cast<const v4u6*>(stg + tr * OP + 16 * ch);
          const int row = (tr / (16 * GPP)) * 64 + 16 * GPP * h + tr % (16 * GPP);
          __builtin_nontemporal_store(v, reinterpret_cast<v4u6*>(y + (m0 + row) * k + n0 + 8 * ch));
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
          const int64_t base = row * k + n0 + wn * WNC + r16;
#pragma unroll
          for (int j = 0; j < JT; ++j) {
            if (full || n0 + wn * WNC + j * 16 + r16 < k) {
              if (acc_out != nullptr) acc_out[base + j * 16] = (int32_t)acc[i][j][e];
              y[base + j * 16] = (uint16_t)f16_mul_lo(acc[i][j][e] * sav[i][e], swv[j]);
            }
          }
        }
      }
    }
    if (!has_next) break;
    m0 = m0n;
    n0 = n0n;
    RQF6_SET_SRC(asrc, bsrc, m0, n0);
  }
#undef RQF6_TILE_OK
#undef RQF6_TILE
#undef RQF6_SET_SRC
#undef RQF6_ISSUE
}
#undef RQF6_DMA

template <int TN>
hipError_t launch_f6_tn(const uint8_t* a6, const uint16_t* a_scales, int64_t m, const uint8_t* w6,
                        const uint16_t* w_scales, int64_t k, int64_t d, uint16_t* y, int32_t* acc,
                        hipStream_t stream) {
  const int tiles_m = (int)((m + FM - 1) / FM);
  const int64_t tiles = (int64_t)tiles_m * ((k + TN - 1) / TN);
  if (tiles > INT32_MAX) return hipErrorInvalidValue;
  const int64_t grid = tiles < cu_count() ? tiles : cu_count();  // one workgroup per CU
  const bool wide_store = acc == nullptr && k % 8 == 0 && ((uintptr_t)y & 15) == 0;
  hipLaunchKernelGGL((w4a4_f6_kernel<TN>), dim3((unsigned)grid), dim3(FTHREADS), 0, stream, a6,
                     a_scales, w6, w_scales, m, k, d, tiles_m, (int)tiles, wide_store, y, acc);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack_f6(const uint8_t* codes, int64_t rows, int64_t d, uint8_t* out,
                          hipStream_t stream) {
  const int64_t blocks = (rows * (d / 32) + 255) / 256;
  const int64_t cap = (int64_t)cu_count() * 16;
  hipLaunchKernelGGL(pack_f6_kernel, dim3((unsigned)(blocks < cap ? blocks : cap)), dim3(256), 0,
                     stream, codes, rows, d, out);
  return hipGetLastError();
}

// Tile width 224, or 256 where that takes fewer rounds of tiles on the CUs
// for the same work (rounds x width).
hipError_t launch_w4a4_gemm_f6(const uint8_t* a6, const uint16_t* a_scales, int64_t m,
                               const uint8_t* w6, const uint16_t* w_scales, int64_t k, int64_t d,
                               uint16_t* y, int32_t* acc, hipStream_t stream) {
  const int64_t tiles_m = (m + FM - 1) / FM, cus = cu_count();
  const int64_t r224 = (tiles_m * ((k + FN - 1) / FN) + cus - 1) / cus;
  const int64_t r256 = (tiles_m * ((k + FN_WIDE - 1) / FN_WIDE) + cus - 1) / cus;
  if (r256 * FN_WIDE < r224 * FN)
    return launch_f6_tn<FN_WIDE>(a6, a_scales, m, w6, w_scales, k, d, y, acc, stream);
  return launch_f6_tn<FN>(a6, a_scales, m, w6, w_scales, k, d, y, acc, stream);
}

}  // namespace rq
