// Row-wise randomized Hadamard rotation fused with symmetric INT4
// quantisation, for CDNA4 (gfx950).  One kernel family serves the online
// activation rotation, the offline weight fold (the same row transform applied
// to the rows of W^T) and the per-head KV-cache rotation.
//
// Pages cited:
//   [RQ]     llms.blog, "Rotational Quantization: How Orthogonal Transforms and
//            Hadamard Incoherence Enable Outlier-Free Low-Bit Inference".
//   [QuaRot] aicassindra.com, QuaRot explainer.
//
// What a row goes through ([RQ] "Incoherence Processing via Randomized
// Hadamard Transforms": R = sign diagonal times Sylvester matrix; [RQ] "Weight
// Absorption and Online Fast Walsh-Hadamard Transforms", part 2: add/sub
// butterflies and one global scale at the end; [QuaRot] "End-to-end flow":
// the rotated activation is quantised to INT4):
//   u = x * s                      exact (sign flip of the fp32 value)
//   y = H_n u                      fp32 add/sub, strides 1, 2, ..., n/2
//   x~ = fp32(y * fp32(1/sqrt n))  only stored in debug mode
//   a = max|x~| = fp32(max|y| * c) (rounding is monotone)
//   scale = fp16_rne(a / 7)        rounded once from the exact quotient
//   q = rne(y * m), m = fp32(c / scale), clamped to [-8, 7] only when the
//       scale is an fp16 subnormal (a normal scale bounds |x~/scale| by 7.004)
//
// Work layout.  A row of n elements is spread over LANES = n / E lanes of one
// wavefront, E elements per lane (all of a row in one lane for n <= 128).
//   load   : the wave's block of rows is copied global -> LDS with coalesced
//            16-byte loads (XOR-swizzled 16-byte chunks, so the per-lane
//            reads below hit distinct banks).
//   phase 1: each lane reads E consecutive elements: the butterflies of the
//            low log2(E) index bits run in registers.
//   phase 2: (LANES > 1) an fp32 exchange through LDS gives each lane the
//            elements whose low log2(LANES) index bits equal its lane index;
//            the remaining butterflies (index bits log2(E) .. log2(n) - 1) run
//            in registers.  Stage order stays ascending, so y is bit-identical
//            to an ascending-stride fp32 FWHT.
//   absmax : in-lane max, then an xor-shuffle across the row's lanes.
//   codes  : fma(y, m, 2^23 + 8) leaves rne(y*m) + 8 in the low mantissa bits;
//            bytes go through LDS and are packed into nibbles on the way out
//            (LANES > 1), or packed in registers (LANES == 1).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <atomic>

#include "rq_internal.h"
#include "rq_row_device.h"

namespace rq {
namespace {

template <int N, int E, int TSIZE>
struct Geo {
  static constexpr int LANES = N / E;
  static constexpr int RW = kWave / LANES;  // rows per wave
  static constexpr int LOG_N = ilog2(N);
  static constexpr int LOG_E = ilog2(E);
  static constexpr int LOG_L = LOG_N - LOG_E;
  static constexpr int SEG_BYTES = E * TSIZE;          // raw bytes owned by one lane
  static constexpr int CPL = SEG_BYTES / 16;           // 16-byte chunks per lane (0: < 16 B)
  static constexpr int ROW_BYTES = N * TSIZE;
  static constexpr int BLOCK_BYTES = RW * ROW_BYTES;   // = 64 * SEG_BYTES
  static constexpr int P = E + 4;                      // exchange pitch per lane segment (floats)
  static constexpr int ROWP = LANES * P;               // exchange pitch per row (floats)
  static constexpr int RAW_LDS = BLOCK_BYTES;
  static constexpr int EXCH_LDS = LANES > 1 ? RW * ROWP * 4 : 0;
  static constexpr int CODE_LDS = LANES > 1 ? RW * N : 0;
  static constexpr int LDS = RAW_LDS > EXCH_LDS ? (RAW_LDS > CODE_LDS ? RAW_LDS : CODE_LDS)
                                                 : (EXCH_LDS > CODE_LDS ? EXCH_LDS : CODE_LDS);
  // XOR swizzle of the 16-byte chunk index inside a lane segment: the 16
  // lanes served by one LDS pass land on 16 different 16-byte bank groups.
  static constexpr int SW_SHIFT = CPL >= 16 ? 0 : ilog2(16 / (CPL > 0 ? CPL : 1));
  static_assert(E >= LANES, "two register phases must cover every index bit");
  static_assert(LANES <= kWave, "a row must fit in one wavefront");
};

template <class G>
__device__ __forceinline__ int raw_phys(int c) {
  if constexpr (G::CPL <= 1) {
    return c;
  } else {
    const int s = c / G::CPL;
    const int i = c % G::CPL;
    return s * G::CPL + (i ^ ((s >> G::SW_SHIFT) & (G::CPL - 1)));
  }
}

struct FQOut {
  const void* x;
  uint8_t* codes;
  uint16_t* scales;
  float* xrot;
  uint8_t* zeros;  // asymmetric quantiser only: per-row zero points
};

template <typename T>
__device__ __forceinline__ void widen16(const uint4& v, float* out);

template <>
__device__ __forceinline__ void widen16<__half>(const uint4& v, float* out) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = h2f((uint16_t)(w[i] & 0xFFFFu));
    out[2 * i + 1] = h2f((uint16_t)(w[i] >> 16));
  }
}

template <>
__device__ __forceinline__ void widen16<float>(const uint4& v, float* out) {
  out[0] = u2f(v.x);
  out[1] = u2f(v.y);
  out[2] = u2f(v.z);
  out[3] = u2f(v.w);
}

template <typename T>
__device__ __forceinline__ float load_elem(const unsigned char* p) {
  if constexpr (sizeof(T) == 2) {
    return h2f(*reinterpret_cast<const uint16_t*>(p));
  } else {
    return *reinterpret_cast<const float*>(p);
  }
}

template <typename T, int N, int E, bool HAS_SIGNS>
__global__ __launch_bounds__(64) void fwht_quant_kernel(FQOut o0, FQOut o1, int64_t rows,
                                                       const int8_t* __restrict__ signs,
                                                       float c32) {
  using G = Geo<N, E, (int)sizeof(T)>;
  constexpr int LANES = G::LANES;
  constexpr int RW = G::RW;
  __shared__ __align__(16) unsigned char smem[G::LDS];

  const FQOut o = blockIdx.y ? o1 : o0;
  const int lane = threadIdx.x;
  const int64_t row0 = (int64_t)blockIdx.x * RW;
  const int rows_valid = (int)((rows - row0) < RW ? (rows - row0) : RW);

  // ---- global -> LDS, coalesced 16-byte chunks
  {
    const int64_t valid_bytes = (int64_t)rows_valid * G::ROW_BYTES;
    const unsigned char* src = reinterpret_cast<const unsigned char*>(o.x) + row0 * G::ROW_BYTES;
    constexpr int CHUNKS = G::BLOCK_BYTES / 16;
#pragma unroll
    for (int c = lane; c < CHUNKS; c += kWave) {
      const int64_t off = (int64_t)c * 16;
      if (off + 16 <= valid_bytes) {
        *reinterpret_cast<uint4*>(smem + raw_phys<G>(c) * 16) =
            *reinterpret_cast<const uint4*>(src + off);
      } else if (off < valid_bytes) {
        for (int b = 0; b < 16; ++b)
          if (off + b < valid_bytes) smem[raw_phys<G>(c) * 16 + b] = src[off + b];
      }
    }
  }
  __syncthreads();

  // ---- phase 1: this lane's E consecutive elements (segment = lane)
  const int rho = lane / LANES;  // row inside the block
  const int j = lane % LANES;    // lane inside the row
  float u[E];
  if constexpr (G::CPL >= 1) {
#pragma unroll
    for (int i = 0; i < G::CPL; ++i) {
      const uint4 v = *reinterpret_cast<const uint4*>(smem + raw_phys<G>(lane * G::CPL + i) * 16);
      widen16<T>(v, u + i * (16 / (int)sizeof(T)));
    }
  } else {
#pragma unroll
    for (int r = 0; r < E; ++r) u[r] = load_elem<T>(smem + (lane * E + r) * (int)sizeof(T));
  }

  if constexpr (HAS_SIGNS) {
    const int8_t* sg = signs + j * E;
    if constexpr (E >= 16) {
#pragma unroll
      for (int i = 0; i < E / 16; ++i) {
        const uint4 sv = *reinterpret_cast<const uint4*>(sg + 16 * i);
        const uint32_t w[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t bit = (w[r >> 2] << (24 - 8 * (r & 3))) & 0x80000000u;
          u[16 * i + r] = u2f(f2u(u[16 * i + r]) ^ bit);
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < E; ++r)
        u[r] = u2f(f2u(u[r]) ^ (((uint32_t)(uint8_t)sg[r] & 0x80u) << 24));
    }
  }

#pragma unroll
  for (int h = 1; h < E; h <<= 1) {
#pragma unroll
    for (int r = 0; r < E; ++r) {
      if (!(r & h)) {
        const float a = u[r], b = u[r + h];
        u[r] = a + b;
        u[r + h] = a - b;
      }
    }
  }

  // ---- phase 2: lane j now holds elements r' * LANES + j
  if constexpr (LANES > 1) {
    float* ex = reinterpret_cast<float*>(smem);
    __syncthreads();  // every raw read has completed before the region is reused
    float* wb = ex + rho * G::ROWP + j * G::P;
#pragma unroll
    for (int r = 0; r < E; r += 4)
      *reinterpret_cast<float4*>(wb + r) = make_float4(u[r], u[r + 1], u[r + 2], u[r + 3]);
    __syncthreads();
    const float* rb = ex + rho * G::ROWP + j;
#pragma unroll
    for (int r = 0; r < E; ++r) {
      const int owner = (r * LANES) / E;
      const int pos = (r * LANES) % E;
      u[r] = rb[owner * G::P + pos];
    }
#pragma unroll
    for (int t = G::LOG_E; t < G::LOG_N; ++t) {
      const int h = 1 << (t - G::LOG_L);
#pragma unroll
      for (int r = 0; r < E; ++r) {
        if (!(r & h)) {
          const float a = u[r], b = u[r + h];
          u[r] = a + b;
          u[r + h] = a - b;
        }
      }
    }
  }

  // ---- absmax over the row
  float amax = 0.0f;
#pragma unroll
  for (int r = 0; r < E; ++r) amax = fmaxf(amax, fabsf(u[r]));
#pragma unroll
  for (int off = 1; off < LANES; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));

  const uint16_t hb = scale_fp16(amax * c32);
  const bool subnormal = hb != 0 && hb < 0x0400u;
  const float mult = hb == 0 ? 0.0f : c32 / h2f(hb);  // +inf scale -> 0
  const bool row_ok = rho < rows_valid;
  const int64_t grow = row0 + rho;

  if (o.xrot != nullptr && row_ok) {
    float* xr = o.xrot + grow * N;
    if constexpr (LANES > 1) {
#pragma unroll
      for (int r = 0; r < E; ++r) xr[r * LANES + j] = u[r] * c32;
    } else {
#pragma unroll
      for (int r = 0; r < E; ++r) xr[r] = u[r] * c32;
    }
  }
  if (j == 0 && row_ok) o.scales[grow] = hb;

  float t[E];
#pragma unroll
  for (int r = 0; r < E; ++r) t[r] = __builtin_fmaf(u[r], mult, kMagic);
  if (__ballot(subnormal) != 0) {
    // only reachable with a subnormal fp16 scale; harmless for normal scales
#pragma unroll
    for (int r = 0; r < E; ++r) t[r] = fminf(fmaxf(t[r], kMagicLo), kMagicHi);
  }

  if constexpr (LANES > 1) {
    unsigned char* cb = smem;
    __syncthreads();  // exchange reads done
#pragma unroll
    for (int r = 0; r < E; ++r) cb[rho * N + r * LANES + j] = (unsigned char)f2u(t[r]);
    __syncthreads();
    constexpr int OUT_CHUNKS = RW * N / 32;  // 16 output bytes = 32 codes
    const int64_t valid_bytes = (int64_t)rows_valid * (N / 2);
    uint8_t* dst = o.codes + row0 * (N / 2);
#pragma unroll
    for (int c = lane; c < OUT_CHUNKS; c += kWave) {
      if ((int64_t)c * 16 < valid_bytes) {
        const uint4* s = reinterpret_cast<const uint4*>(cb + c * 32);
        const uint4 lo = s[0], hi = s[1];
        const uint32_t b[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t p0 = b[2 * i] | (b[2 * i] >> 4);
          const uint32_t p1 = b[2 * i + 1] | (b[2 * i + 1] >> 4);
          w[i] = __builtin_amdgcn_perm(p1, p0, 0x06040200u) ^ 0x88888888u;
        }
        *reinterpret_cast<uint4*>(dst + (int64_t)c * 16) = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  } else {
    if (row_ok) {
      uint8_t* dst = o.codes + grow * (N / 2);
      if constexpr (N >= 8) {
        uint32_t w[N / 8];
#pragma unroll
        for (int g = 0; g < N / 8; ++g) {
          uint32_t acc = 0;
#pragma unroll
          for (int i = 0; i < 8; ++i) acc |= ((f2u(t[8 * g + i]) & 0xFu) ^ 0x8u) << (4 * i);
          w[g] = acc;
        }
        if constexpr (N / 2 >= 16) {
#pragma unroll
          for (int g = 0; g < N / 8; g += 4)
            *reinterpret_cast<uint4*>(dst + 4 * g) = make_uint4(w[g], w[g + 1], w[g + 2], w[g + 3]);
        } else if constexpr (N / 2 == 8) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
        } else {
          *reinterpret_cast<uint32_t*>(dst) = w[0];
        }
      } else {
#pragma unroll
        for (int p = 0; p < N / 2; ++p) {
          const uint32_t lo = (f2u(t[2 * p]) & 0xFu) ^ 0x8u;
          const uint32_t hi = (f2u(t[2 * p + 1]) & 0xFu) ^ 0x8u;
          dst[p] = (uint8_t)(lo | (hi << 4));
        }
      }
    }
  }
}

// Each wavefront walks rows w, w + W, w + 2W, ... (W = wavefronts in the
// grid, sized to four resident wavefronts per SIMD).  For n <= 4096 the kernel
// stays within 128 VGPRs so that four wavefronts share each SIMD: while one
// waits for its row, the others keep the VALU busy.  Sign bytes are re-read
// per row (L1/L2 hits) rather than held in registers for the same reason.
template <int N, bool HAS_SIGNS, int BITS = 4, bool ASYM = false>
__global__ __launch_bounds__(64 * kRowWaves, N <= 4096 ? 4 : 2) void fwht_row_kernel(FQOut o, int64_t rows,
                                                                 const int8_t* __restrict__ signs,
                                                                 float c32) {
  constexpr int NI = N / 512;  // 16-byte loads per lane
  constexpr int kCodeBytes = BITS == 4 ? N / 2 : N;
  __shared__ __align__(16) unsigned char cb_all[kRowWaves][kCodeBytes];

  const int L = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  unsigned char* cb = cb_all[wave];
  const int64_t stride = (int64_t)gridDim.x * kRowWaves;
  int64_t row = (int64_t)blockIdx.x * kRowWaves + wave;
  if (row >= rows) return;  // uniform per wavefront
  const RowLane rl = make_row_lane(L);

  for (;;) {
    // The sign loads issue ahead of the row, except at n = 1024, where the
    // row's two chunks came back sooner when issued first (measured).
    constexpr bool kSignsFirst = N != 1024;
    uint2 sg[NI];
    if constexpr (HAS_SIGNS && kSignsFirst) load_signs(sg, signs, L);
    __builtin_amdgcn_sched_barrier(0);
    uint4 raw[NI];
    load_row(raw, static_cast<const __half*>(o.x) + row * N, L);
    if constexpr (HAS_SIGNS && !kSignsFirst) load_signs(sg, signs, L);
    __builtin_amdgcn_sched_barrier(0);  // every load issues before the first wait
    row_rotate_quant<N, HAS_SIGNS, false, BITS, ASYM>(
        raw, sg, L, rl, c32, cb, o.codes + row * kCodeBytes, o.scales + row,
        o.xrot != nullptr ? o.xrot + row * N : nullptr, ASYM ? o.zeros + row : nullptr);
    const int64_t next = row + stride;
    if (next >= rows) break;
    row = next;
  }
}

// ------------------------------------------------------------------------
// n = 28 * P with P = 512 (14336, the width of a Llama-class down projection
// input, 4096 -> 14336) or P = 1024 (28672, the same for the 8192 -> 28672
// model): H_n = H_28 (x) H_P, H_28 by Paley's second construction with
// q = 13 ([RQ] "Learned Orthogonal Rotations: SpinQuant": fixed Hadamard
// rotations need power-of-two sizes or products of small Hadamard-compatible
// sizes; [RQ] "Weight Absorption and Online Fast Walsh-Hadamard Transforms",
// part 2: the down projection's input needs an online rotation).  Element
// e = P b + p: block b of 28, position p of P.
//
// One row per P-thread workgroup at a time (P / 64 wavefronts).  Wave w
// rotates blocks w, w + P/64, ... with the P-point FWHT: each 512-element
// sub-block is one 16-byte chunk per lane through the 512-point stages of the
// row kernel, and for P = 1024 the last stage (stride 512) combines the two
// sub-blocks in registers.  The block goes, sign-corrected, to an fp32 LDS
// row; the next row's chunks are loaded during the P-point stages (P = 1024)
// or right after them, and arrive while the rest of the row runs.
// After a barrier, thread t takes position t and applies H_28 across the 28
// blocks in an order the Paley structure H_28 = C (x) H_2 + I (x) J_2 gives
// (C the order-14 conference matrix, J_2 = [[1, -1], [-1, -1]]):
// a_i = t_2i + t_2i+1, d_i = t_2i - t_2i+1, y_2j = (C a)_j + d_j and
// y_2j+1 = (C d)_j - a_j.  Row 1 + x of C is +1 at column 0 and at the
// columns 1 + (x - r) mod 13 for the six quadratic residues r of 13, and -1
// at the other twelve off-diagonal ones; with S = v_1 + ... + v_13 and T_x
// the sum over those six columns, (C v)_0 = S and (C v)_(1+x) = 2 T_x +
// ((v_0 - S) + v_(1+x)).  In fp32: S left to right, w = v_0 - S, T_x left to
// right over the residues in ascending order, y_0 = S_a + d_0,
// y_1 = S_d - a_0, and for j = 1 + x y_2j = fma(T_x(a), 2, w_a + (a_j + d_j))
// and y_2j+1 = fma(T_x(d), 2, w_d + (d_j - a_j)) (2 T is exact, so the fma is
// the rounded sum).  That is 264 operations per position, against 392 for
// the thirteen-term row sums and 756 for the dense product.

// Quadratic character modulo 13 by Euler's criterion, a^6 mod 13.
constexpr int paley_chi13(int a) {
  a = ((a % 13) + 13) % 13;
  if (a == 0) return 0;
  int r = 1;
  for (int i = 0; i < 6; ++i) r = (r * a) % 13;
  return r == 1 ? 1 : -1;
}
// Conference matrix of order 14: 0 on the diagonal, ones in the first row and
// column, the Jacobsthal matrix chi(a - b) elsewhere.
constexpr int paley_conf14(int j, int i) {
  return j == i ? 0 : (j == 0 || i == 0) ? 1 : paley_chi13((j - 1) - (i - 1));
}

// The quadratic residues of 13, ascending: 1, 3, 4, 9, 10, 12.
constexpr int paley_residue13(int k) {
  int found = -1;
  for (int r = 1; r < 13; ++r) {
    if (paley_chi13(r) > 0 && ++found == k) return r;
  }
  return -1;
}

// Row 1 + x of the conference matrix is +1 exactly at column 0 and at the
// columns 1 + (x - r) mod 13, r a quadratic residue: the evaluation below
// rests on this.
constexpr bool paley_rows_are_residue_sums() {
  for (int x = 0; x < 13; ++x) {
    if (paley_conf14(1 + x, 0) != 1) return false;
    for (int y = 0; y < 13; ++y) {
      if (y == x) continue;
      bool at_residue = false;
      for (int k = 0; k < 6; ++k) at_residue |= (x - paley_residue13(k) + 13) % 13 == y;
      if (paley_conf14(1 + x, 1 + y) != (at_residue ? 1 : -1)) return false;
    }
  }
  return paley_residue13(5) == 12 && paley_residue13(6) == -1;
}
static_assert(paley_rows_are_residue_sums(), "the conference matrix rows are the residue sums");

constexpr int kN28 = 28 * 512;
constexpr int kN28x1024 = 28 * 1024;

template <typename T>
struct Chunk28 {
  v4u w[sizeof(T) / 2];
};

template <typename T>
__device__ __forceinline__ Chunk28<T> load_chunk28(const T* xr, int e0) {
  Chunk28<T> c;
#pragma unroll
  for (int h = 0; h < (int)(sizeof(T) / 2); ++h)
    c.w[h] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(xr + e0 + 8 / (int)(sizeof(T) / 2) * h));
  return c;
}

// Signs, then e0 of the 512-point transform on one chunk.
template <typename T, bool HAS_SIGNS>
__device__ __forceinline__ void chunk28_e0(const Chunk28<T>& raw, const int8_t* signs, int e0,
                                           float (&c)[8]) {
  uint2 sg = make_uint2(0u, 0u);
  if constexpr (HAS_SIGNS) sg = *reinterpret_cast<const uint2*>(signs + e0);
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t w = raw.w[0][q];
      if constexpr (HAS_SIGNS) {
        const uint32_t s2 = q < 2 ? sg.x : sg.y;
        const uint32_t b0 = (2u * q) & 3u;
        const uint32_t sel = 0x0Cu | (b0 << 8) | (0x0Cu << 16) | ((b0 + 1u) << 24);
        w ^= __builtin_amdgcn_perm(0u, s2, sel) & 0x80008000u;
      }
      c[2 * q] = mix_add(w);
      c[2 * q + 1] = mix_sub(w);
    }
  } else {
    float v[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) v[r] = u2f(raw.w[r >> 2][r & 3]);
    if constexpr (HAS_SIGNS) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const uint32_t sbyte = (r < 4 ? sg.x : sg.y) >> (8 * (r & 3));
        v[r] = u2f(f2u(v[r]) ^ ((sbyte & 0x80u) << 24));
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      c[2 * q] = v[2 * q] + v[2 * q + 1];
      c[2 * q + 1] = v[2 * q] - v[2 * q + 1];
    }
  }
}

template <typename T, bool HAS_SIGNS, int P>
__global__ __launch_bounds__(P) void fwht28_kernel(FQOut o, int64_t rows,
                                                   const int8_t* __restrict__ signs, float c32) {
  constexpr int NB = 28, W = P / 64, N = NB * P;
  constexpr int BPW = (NB + W - 1) / W;  // blocks per wave
  constexpr int SUB = P / 512;           // 512-element sub-blocks (chunks) per block
  static_assert(P == 512 || P == 1024, "blocks of 512 or 1024 elements");
  __shared__ __align__(16) float xb[NB][P];  // the row in fp32
  // the row's code bytes, apart from xb: the next row's fp32 stores into xb
  // need no barrier after the codes are packed (its own code bytes are
  // written only after its absmax barrier, which every wave reaches after
  // packing this row)
  __shared__ __align__(16) unsigned char cbuf[NB * P];
  __shared__ float amx[W];
  const int tid = threadIdx.x, L = tid & 63, wave = tid >> 6;
  const RowLane rl = make_row_lane(L);

  int64_t row = blockIdx.x;
  if (row >= rows) return;  // uniform per workgroup
  // wave w owns blocks w, w + W, ...; sub-block j of block b starts at P b + 512 j
  Chunk28<T> raw[BPW][SUB];
#pragma unroll
  for (int i = 0; i < BPW; ++i)
#pragma unroll
    for (int j = 0; j < SUB; ++j)
      if (wave + W * i < NB)
        raw[i][j] = load_chunk28(static_cast<const T*>(o.x) + row * N,
                                 P * (wave + W * i) + 512 * j + 8 * L);

  for (;;) {
    // P = 1024 with fp16 input (one workgroup per CU, nothing else to hide
    // the loads behind): the next row's chunk goes out as soon as this row's
    // is consumed, so it is in flight during the rest of this row (55.0 ->
    // 53.8 us at 2048 x 28672).  Otherwise it is loaded after the P-point
    // stages: at P = 512 the CU's second workgroup already overlaps it (no
    // gain measured), and the fp32 fold would spill.
    constexpr bool kEarlyLoad = sizeof(T) == 2 && P == 1024;
    const int64_t next = row + gridDim.x;
    const bool more = next < rows;
    // 1. the P-point stages of this wave's blocks, sign-corrected into LDS
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int b = wave + W * i;
      if (b >= NB) continue;  // uniform per wave
      float c[SUB][8];
#pragma unroll
      for (int j = 0; j < SUB; ++j) {
        chunk28_e0<T, HAS_SIGNS>(raw[i][j], signs, P * b + 512 * j + 8 * L, c[j]);
        if (kEarlyLoad && more)
          raw[i][j] = load_chunk28(static_cast<const T*>(o.x) + next * N, P * b + 512 * j + 8 * L);
        chunk512_stages(c[j], rl);
      }
      if constexpr (SUB == 2) {  // stride 512: sub-block 0 with sub-block 1
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const float x0 = c[0][r], x1 = c[1][r];
          c[0][r] = x0 + x1;
          c[1][r] = x0 - x1;
        }
      }
#pragma unroll
      for (int j = 0; j < SUB; ++j)
#pragma unroll
        for (int r = 0; r < 8; r += 2) {
          const int p = 512 * j + ((rl.lane_pair << 1) | (((r >> 2) & 1) << 7) | (((r >> 1) & 1) << 8));
          *reinterpret_cast<float2*>(&xb[b][p]) = make_float2(c[j][r] * rl.sigma, c[j][r + 1] * rl.sigma);
        }
    }
    if (!kEarlyLoad && more) {
#pragma unroll
      for (int i = 0; i < BPW; ++i)
#pragma unroll
        for (int j = 0; j < SUB; ++j)
          if (wave + W * i < NB)
            raw[i][j] = load_chunk28(static_cast<const T*>(o.x) + next * N,
                                     P * (wave + W * i) + 512 * j + 8 * L);
    }
    __syncthreads();

    // 2. H_28 across the blocks for position tid
    float y[NB];
    {
      float a[14], d[14];
#pragma unroll
      for (int i = 0; i < 14; ++i) {
        const float t0 = xb[2 * i][tid], t1 = xb[2 * i + 1][tid];
        a[i] = t0 + t1;
        d[i] = t0 - t1;
      }
      float s_a = a[1], s_d = d[1];
#pragma unroll
      for (int i = 2; i < 14; ++i) {
        s_a += a[i];
        s_d += d[i];
      }
      const float w_a = a[0] - s_a, w_d = d[0] - s_d;
      y[0] = s_a + d[0];
      y[1] = s_d - a[0];
#pragma unroll
      for (int x = 0; x < 13; ++x) {
        constexpr int kR = 6;  // quadratic residues of 13
        float ta = a[1 + (x - paley_residue13(0) + 13) % 13];
        float td = d[1 + (x - paley_residue13(0) + 13) % 13];
#pragma unroll
        for (int k = 1; k < kR; ++k) {
          ta += a[1 + (x - paley_residue13(k) + 13) % 13];
          td += d[1 + (x - paley_residue13(k) + 13) % 13];
        }
        const int j = 1 + x;
        y[2 * j] = __builtin_fmaf(ta, 2.0f, w_a + (a[j] + d[j]));
        y[2 * j + 1] = __builtin_fmaf(td, 2.0f, w_d + (d[j] - a[j]));
      }
    }

    // 3. absmax over the row
    float amax = 0.0f;
#pragma unroll
    for (int b = 0; b < NB; ++b) amax = fmaxf(amax, fabsf(y[b]));
    amax = wave_max(amax);
    if (L == 0) amx[wave] = amax;
    __syncthreads();  // also: every thread has read xb
#pragma unroll
    for (int w = 0; w < W; ++w) amax = fmaxf(amax, amx[w]);
    const uint16_t hb = scale_fp16(amax * c32);
    const bool subnormal = hb != 0 && hb < 0x0400u;
    const float mult = hb == 0 ? 0.0f : c32 / h2f(hb);
    if (tid == 0) o.scales[row] = hb;
    if (o.xrot != nullptr) {
      float* xo = o.xrot + row * N;
#pragma unroll
      for (int b = 0; b < NB; ++b) xo[P * b + tid] = y[b] * c32;
    }

    // 4. codes.  Every thread writes its 28 offset-binary codes (q + 8) as
    // bytes, element P b + tid at byte P b + tid: the low byte of fma(y, m, 2^23 + 8) is exactly
    // the code, its bits 4..7 are zero.  After a barrier each thread packs 32
    // consecutive code bytes into 16 bytes of nibble pairs (element e is
    // nibble e & 1 of byte e / 2) and stores them.  The scale is the row's,
    // so the subnormal clamp is a uniform branch.
    float q[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) q[b] = __builtin_fmaf(y[b], mult, kMagic);
    if (__builtin_amdgcn_readfirstlane((int)subnormal)) {
#pragma unroll
      for (int b = 0; b < NB; ++b) q[b] = fminf(fmaxf(q[b], kMagicLo), kMagicHi);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) cbuf[P * b + tid] = (unsigned char)f2u(q[b]);
    __syncthreads();
    uint8_t* dst = o.codes + row * (N / 2);
    for (int c = tid; c < N / 32; c += P) {
      const v4u lo = *reinterpret_cast<const v4u*>(cbuf + 32 * c);
      const v4u hi = *reinterpret_cast<const v4u*>(cbuf + 32 * c + 16);
      // bytes c0..c3 of d0 and c4..c7 of d1: d | d >> 4 holds the pairs
      // (c0, c1), (c2, c3) in its bytes 0 and 2; one byte permute joins them
      const auto pack8 = [](uint32_t d0, uint32_t d1) {
        return __builtin_amdgcn_perm(d1 | (d1 >> 4), d0 | (d0 >> 4), 0x06040200u);
      };
      v4u out;
      out[0] = pack8(lo[0], lo[1]);
      out[1] = pack8(lo[2], lo[3]);
      out[2] = pack8(hi[0], hi[1]);
      out[3] = pack8(hi[2], hi[3]);
      out ^= 0x88888888u;  // offset binary to two's complement nibbles
      __builtin_nontemporal_store(out, reinterpret_cast<v4u*>(dst + 16 * c));
    }
    if (!more) break;
    row = next;
  }
}

template <typename T, bool HAS_SIGNS, int P>
hipError_t launch_28(FQOut o, int64_t rows, const int8_t* signs, hipStream_t stream) {
  const float c32 = (float)(1.0 / __builtin_sqrt((double)(28 * P)));
  // workgroups resident per CU: two of 56 KB (P = 512) or one of 112 KB
  const int64_t cap = (int64_t)cu_count() * (P == 512 ? 2 : 1);
  const int64_t blocks = rows < cap ? rows : cap;
  hipLaunchKernelGGL((fwht28_kernel<T, HAS_SIGNS, P>), dim3((unsigned)blocks), dim3(P), 0, stream,
                     o, rows, signs, c32);
  return hipGetLastError();
}

// ------------------------------------------------------------------------
// fp16 rows with n = 128 (the per-head KV rotation): four lanes per row,
// sixteen rows per wavefront, 32 elements per lane, no LDS.
//
// Lane l (row l/4, quarter q = l%4) loads the 16-byte chunks q + 4i, i = 0..3,
// so register index rho = 8i + r holds element e = 32i + 8q + r: element bits
// 0..2 and 5..6 live in registers, bits 3..4 in the quarter index.  e0 uses
// v_fma_mix_f32 (widen + add/sub), e1, e2, e5, e6 run in registers and e3, e4
// use v_fmac_f32_dpp with quad_perm partners (xor 1, xor 2).  The DPP factor
// g = +-1 leaves the values multiplied by sigma(q) = g0 * g1, which is folded
// into the quantisation multiplier.  Output order is natural.
template <bool HAS_SIGNS>
__global__ __launch_bounds__(256) void fwht128_quad_kernel(FQOut o0, FQOut o1, int64_t rows,
                                                          const int8_t* __restrict__ signs,
                                                          float c32) {
  constexpr int N = 128;
  const FQOut o = blockIdx.y ? o1 : o0;
  const int L = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int q = L & 3;
  const int64_t row_id = ((int64_t)blockIdx.x * 4 + wave) * 16 + (L >> 2);
  const bool row_ok = row_id < rows;
  const int64_t row = row_ok ? row_id : rows - 1;
  const __half* xr = static_cast<const __half*>(o.x) + row * N;

  uint4 raw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const v4u t = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(xr + 8 * (q + 4 * i)));
    raw[i] = make_uint4(t[0], t[1], t[2], t[3]);
  }
  uint2 sg[4];
  if constexpr (HAS_SIGNS) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sg[i] = *reinterpret_cast<const uint2*>(signs + 8 * (q + 4 * i));
  }
  const float g0 = (q & 1) ? -1.0f : 1.0f;
  const float g1 = (q & 2) ? -1.0f : 1.0f;
  const float sigma = g0 * g1;

  float u[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w4[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t w = w4[p];
      if constexpr (HAS_SIGNS) {
        const uint32_t s2 = p < 2 ? sg[i].x : sg[i].y;
        const uint32_t b0 = (2u * p) & 3u;
        const uint32_t sel = 0x0Cu | (b0 << 8) | (0x0Cu << 16) | ((b0 + 1u) << 24);
        w ^= __builtin_amdgcn_perm(0u, s2, sel) & 0x80008000u;
      }
      u[8 * i + 2 * p] = mix_add(w);
      u[8 * i + 2 * p + 1] = mix_sub(w);
    }
  }
  butterfly_regs(u, 2);  // e1
  butterfly_regs(u, 4);  // e2
#pragma unroll
  for (int b = 0; b < 32; b += 8) RQ_DPP8("quad_perm:[1,0,3,2]", u + b, g0);  // e3
#pragma unroll
  for (int b = 0; b < 32; b += 8) RQ_DPP8("quad_perm:[2,3,0,1]", u + b, g1);  // e4
  butterfly_regs(u, 8);   // e5
  butterfly_regs(u, 16);  // e6

  float amax = 0.0f;
#pragma unroll
  for (int r = 0; r < 32; ++r) amax = fmaxf(amax, fabsf(u[r]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));

  const uint16_t hb = scale_fp16(amax * c32);
  const bool subnormal = hb != 0 && hb < 0x0400u;
  const float mult = (hb == 0 ? 0.0f : c32 / h2f(hb)) * sigma;
  if (q == 0 && row_ok) o.scales[row] = hb;
  if (o.xrot != nullptr && row_ok) {
    float* xo = o.xrot + row * N;
#pragma unroll
    for (int r = 0; r < 32; ++r) xo[32 * (r >> 3) + 8 * q + (r & 7)] = (u[r] * sigma) * c32;
  }

  float t[32];
#pragma unroll
  for (int r = 0; r < 32; ++r) t[r] = __builtin_fmaf(u[r], mult, kMagic);
  if (__ballot(subnormal) != 0) {
#pragma unroll
    for (int r = 0; r < 32; ++r) t[r] = fminf(fmaxf(t[r], kMagicLo), kMagicHi);
  }
  // The wavefront's 16 rows of codes (1 KB, contiguous in memory) are staged
  // in its own LDS slice and leave as one 16-byte store per lane.
  __shared__ __align__(16) uint32_t kcb[4][16 * 16];
  uint32_t* cw = kcb[wave] + (L >> 2) * 16;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // 8 offset-binary codes -> one word of two's-complement nibbles
    uint32_t b[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) b[p] = (f2u(t[8 * i + 2 * p + 1]) << 4) | f2u(t[8 * i + 2 * p]);
    const uint32_t lo = __builtin_amdgcn_perm(b[1], b[0], 0x0C0C0400u);  // bytes b0.0, b1.0
    const uint32_t hi = __builtin_amdgcn_perm(b[3], b[2], 0x04000C0Cu);  // bytes b2.0, b3.0 at 2, 3
    // codes of elements 32i + 8q .. +7 are bytes 16i + 4q .. +3 of the row
    cw[4 * i + q] = (lo | hi) ^ 0x88888888u;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const v4u cv = *reinterpret_cast<const v4u*>(kcb[wave] + 4 * L);  // row L / 4, bytes 16 q..
  if (row_ok)
    __builtin_nontemporal_store(cv, reinterpret_cast<v4u*>(o.codes + row * (N / 2) + 16 * q));
}

template <bool HAS_SIGNS>
hipError_t launch_quad(FQOut o0, FQOut o1, int pairs, int64_t rows, const int8_t* signs,
                       hipStream_t stream) {
  const float c32 = (float)(1.0 / __builtin_sqrt(128.0));
  const int64_t blocks = (rows + 63) / 64;
  hipLaunchKernelGGL((fwht128_quad_kernel<HAS_SIGNS>), dim3((unsigned)blocks, pairs), dim3(256), 0,
                     stream, o0, o1, rows, signs, c32);
  return hipGetLastError();
}


// Resident wavefronts per SIMD the row kernel is sized for (its VGPR budget).
template <int N>
constexpr int row_waves_per_simd() { return N <= 4096 ? 4 : 2; }

template <int N, bool HAS_SIGNS, int BITS = 4, bool ASYM = false>
hipError_t launch_row(FQOut o, int64_t rows, const int8_t* signs, hipStream_t stream) {
  const float c32 = (float)(1.0 / __builtin_sqrt((double)N));
  const int64_t max_waves = (int64_t)cu_count() * 4 * row_waves_per_simd<N>();
  int64_t waves = rows < max_waves ? rows : max_waves;
  const int64_t per_wave = (rows + waves - 1) / waves;  // rows per wavefront, balanced
  waves = (rows + per_wave - 1) / per_wave;
  const int64_t blocks = (waves + kRowWaves - 1) / kRowWaves;
  hipLaunchKernelGGL((fwht_row_kernel<N, HAS_SIGNS, BITS, ASYM>), dim3((unsigned)blocks), dim3(kWave * kRowWaves),
                     0, stream, o, rows, signs, c32);
  return hipGetLastError();
}

template <bool HAS_SIGNS>
hipError_t dispatch_row(FQOut o, int64_t rows, int n, const int8_t* signs, hipStream_t stream) {
  switch (n) {
    case 512: return launch_row<512, HAS_SIGNS>(o, rows, signs, stream);
    case 1024: return launch_row<1024, HAS_SIGNS>(o, rows, signs, stream);
    case 2048: return launch_row<2048, HAS_SIGNS>(o, rows, signs, stream);
    case 4096: return launch_row<4096, HAS_SIGNS>(o, rows, signs, stream);
    case 8192: return launch_row<8192, HAS_SIGNS>(o, rows, signs, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int N, int E, bool HAS_SIGNS>
hipError_t launch_one(FQOut o0, FQOut o1, int pairs, int64_t rows, const int8_t* signs,
                      hipStream_t stream) {
  using G = Geo<N, E, (int)sizeof(T)>;
  const int64_t blocks = (rows + G::RW - 1) / G::RW;
  const float c32 = (float)(1.0 / __builtin_sqrt((double)N));
  hipLaunchKernelGGL((fwht_quant_kernel<T, N, E, HAS_SIGNS>), dim3((unsigned)blocks, pairs),
                     dim3(kWave), 0, stream, o0, o1, rows, signs, c32);
  return hipGetLastError();
}

template <typename T, bool HAS_SIGNS>
hipError_t dispatch_n(FQOut o0, FQOut o1, int pairs, int64_t rows, int n, const int8_t* signs,
                      hipStream_t stream) {
  switch (n) {
    case 2: return launch_one<T, 2, 2, HAS_SIGNS>(o0, o1, pairs, rows, signs, stream);
    case 4: return launch_one<T, 4, 4, HAS_SIGNS>(o0, o1, pairs, rows, signs, stream);
    case 8: return launch_one<T, 8, 8, HAS_SIGNS>(o0, o1, pairs, rows, signs, stream);
    case 16: return launch_one<T, 16, 16, HAS_SIGNS>(o0, o1, pairs, rows, signs, stream);
    case 32: return launch_one<T, 32, 32, HAS_SIGNS>(o0, o1, pairs, rows, signs, stream);
    case 64: return launch_one<T, 64, 64, HAS_SIGNS>(o0, o1, pairs, rows, signs, stream);
    case 128: return launch_one<T, 128, 128, HAS_SIGNS>(o0, o1, pairs, rows, signs, stream);
    case 256: return launch_one<T, 256, 64, HAS_SIGNS>(o0, o1, pairs, rows, signs, stream);
    case 512: return launch_one<T, 512, 64, HAS_SIGNS>(o0, o1, pairs, rows, signs, stream);
    case 1024: return launch_one<T, 1024, 64, HAS_SIGNS>(o0, o1, pairs, rows, signs, stream);
    case 2048: return launch_one<T, 2048, 64, HAS_SIGNS>(o0, o1, pairs, rows, signs, stream);
    case 4096: return launch_one<T, 4096, 64, HAS_SIGNS>(o0, o1, pairs, rows, signs, stream);
    case 8192: return launch_one<T, 8192, 128, HAS_SIGNS>(o0, o1, pairs, rows, signs, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Compute units of the current device (queried once per device).
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}


hipError_t launch_fwht_quant(const void* x, bool is_f32, int64_t rows, int n, const int8_t* signs,
                             uint8_t* codes, uint16_t* scales, float* x_rot, hipStream_t stream) {
  const FQOut o{x, codes, scales, x_rot};
  if (n == kN28) {
    if (is_f32)
      return signs ? launch_28<float, true, 512>(o, rows, signs, stream)
                   : launch_28<float, false, 512>(o, rows, signs, stream);
    return signs ? launch_28<__half, true, 512>(o, rows, signs, stream)
                 : launch_28<__half, false, 512>(o, rows, signs, stream);
  }
  if (n == kN28x1024) {
    if (is_f32)
      return signs ? launch_28<float, true, 1024>(o, rows, signs, stream)
                   : launch_28<float, false, 1024>(o, rows, signs, stream);
    return signs ? launch_28<__half, true, 1024>(o, rows, signs, stream)
                 : launch_28<__half, false, 1024>(o, rows, signs, stream);
  }
  if (is_f32) {
    return signs ? dispatch_n<float, true>(o, o, 1, rows, n, signs, stream)
                 : dispatch_n<float, false>(o, o, 1, rows, n, signs, stream);
  }
  if (n >= 512) {
    return signs ? dispatch_row<true>(o, rows, n, signs, stream)
                 : dispatch_row<false>(o, rows, n, signs, stream);
  }
  if (n == 128) {
    return signs ? launch_quad<true>(o, o, 1, rows, signs, stream)
                 : launch_quad<false>(o, o, 1, rows, signs, stream);
  }
  return signs ? dispatch_n<__half, true>(o, o, 1, rows, n, signs, stream)
               : dispatch_n<__half, false>(o, o, 1, rows, n, signs, stream);
}

template <bool HAS_SIGNS>
hipError_t dispatch_row8(FQOut o, int64_t rows, int n, const int8_t* signs, hipStream_t stream) {
  switch (n) {
    case 512: return launch_row<512, HAS_SIGNS, 8>(o, rows, signs, stream);
    case 1024: return launch_row<1024, HAS_SIGNS, 8>(o, rows, signs, stream);
    case 2048: return launch_row<2048, HAS_SIGNS, 8>(o, rows, signs, stream);
    case 4096: return launch_row<4096, HAS_SIGNS, 8>(o, rows, signs, stream);
    case 8192: return launch_row<8192, HAS_SIGNS, 8>(o, rows, signs, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fwht_quant8(const uint16_t* x, int64_t rows, int n, const int8_t* signs,
                              int8_t* codes, uint16_t* scales, float* x_rot, hipStream_t stream) {
  const FQOut o{x, reinterpret_cast<uint8_t*>(codes), scales, x_rot};
  return signs ? dispatch_row8<true>(o, rows, n, signs, stream)
               : dispatch_row8<false>(o, rows, n, signs, stream);
}

template <bool HAS_SIGNS>
hipError_t dispatch_row_asym(FQOut o, int64_t rows, int n, const int8_t* signs,
                             hipStream_t stream) {
  switch (n) {
    case 512: return launch_row<512, HAS_SIGNS, 4, true>(o, rows, signs, stream);
    case 1024: return launch_row<1024, HAS_SIGNS, 4, true>(o, rows, signs, stream);
    case 2048: return launch_row<2048, HAS_SIGNS, 4, true>(o, rows, signs, stream);
    case 4096: return launch_row<4096, HAS_SIGNS, 4, true>(o, rows, signs, stream);
    case 8192: return launch_row<8192, HAS_SIGNS, 4, true>(o, rows, signs, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fwht_quant_asym(const uint16_t* x, int64_t rows, int n, const int8_t* signs,
                                  uint8_t* codes, uint16_t* scales, uint8_t* zeros, float* x_rot,
                                  hipStream_t stream) {
  const FQOut o{x, codes, scales, x_rot, zeros};
  return signs ? dispatch_row_asym<true>(o, rows, n, signs, stream)
               : dispatch_row_asym<false>(o, rows, n, signs, stream);
}

hipError_t launch_kv_rotate_quant(const uint16_t* k_in, const uint16_t* v_in, int64_t rows,
                                  const int8_t* signs, uint8_t* k_codes, uint16_t* k_scales,
                                  uint8_t* v_codes, uint16_t* v_scales, hipStream_t stream) {
  const FQOut ok{k_in, k_codes, k_scales, nullptr};
  const FQOut ov{v_in, v_codes, v_scales, nullptr};
  return signs ? launch_quad<true>(ok, ov, 2, rows, signs, stream)
               : launch_quad<false>(ok, ov, 2, rows, signs, stream);
}

}  // namespace rq
