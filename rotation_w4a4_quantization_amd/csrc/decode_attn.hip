// Decode attention that reads the 4-bit rotated KV cache on CDNA4 (gfx950).
//
// Pages cited:
//   [QuaRot] aicassindra.com, QuaRot explainer, "End-to-end flow" (the KV
//            cache is rotated and stored in four bits; a later token's
//            attention reads the four-bit rotated cache, and rotation
//            invariance keeps the attention scores).
//   [RQ]     llms.blog, "Rotational Quantization: ...", "The Principle of
//            Computational Invariance" (q k^T = (q R)(k R)^T, R R^T = I).
//
// What is computed, per batch entry b and query head j (KV head h = j / G):
//   q~ = q R (the cache's rotation, n = 128), scores s_t = q~ . k^_t * scale
//   over the dequantised rotated keys k^_t = code_t * kscale_t, t < len_b,
//   p = softmax(s), o~ = sum_t p_t v^_t, o = o~ R^T.
//
// Work split (flash-decoding): workgroup (split, b*H + h) covers one chunk of
// positions for the G query heads of KV head h; its 4 wavefronts take 16-
// position tiles in turn and keep their own running max / sums / output.
//   * Codes become f16 operands exactly, as the subnormals code * 2^-24
//     (two masks, v_perm and a packed f16 subtraction per 8 codes); the MFMA
//     keeps subnormal products exact, and the 2^-24 comes out per query.
//   * Scores: S^T = K Q~^T on the f16 MFMA 16x16x32.  A key row (64 bytes)
//     is contiguous, so a lane loads 16 bytes for 4 k-steps.  The query, with
//     the softmax scale and log2(e), is split into f16 hi + lo (about 22
//     significant bits); both products accumulate in fp32.
//   * Output: o~^T = V^T (p vscale)^T on the f16 MFMA 16x16x16.  The value
//     tile goes to LDS as f16 rows; ds_read_b64_tr_b16 reads it transposed
//     (positions along k), and the weights p * vscale (hi + lo) are the other
//     operand straight from the score layout.  The running output is
//     rescaled only when some running max moved.
// A second kernel merges the splits' (max, sum, output) records and applies
// the inverse rotation.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "rq_internal.h"
#include "rq_row_device.h"

namespace rq {
namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef float v4f_a __attribute__((ext_vector_type(4)));

constexpr int AD = 128;          // head dimension
constexpr int AW = 4;            // wavefronts per workgroup
constexpr int AT = 16;           // positions per wavefront step
constexpr int PREC = AD + 4;     // floats per split record: m, l, 2 pad, o~[128]
// f16 row pitch of the value tile: 288 bytes = 72 dwords, so the four rows
// one 16-lane group of a transposing read touches start 8 banks apart and the
// group's 16 x 8 bytes cover all 32 banks once
constexpr int VPITCH = AD + 16;
constexpr float kNegInf = -__builtin_inff();

// Sum / max with the lane 16 and lane 32 apart (lane bits 4 and 5).
__device__ __forceinline__ float pair16_add(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(f2u(x), f2u(x), false, false);
  return u2f(a[0]) + u2f(a[1]);
}
__device__ __forceinline__ float pair32_add(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
  return u2f(a[0]) + u2f(a[1]);
}
__device__ __forceinline__ float pair16_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(f2u(x), f2u(x), false, false);
  return fmaxf(u2f(a[0]), u2f(a[1]));
}
__device__ __forceinline__ float pair32_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
  return fmaxf(u2f(a[0]), u2f(a[1]));
}

// 8 two's-complement nibbles (dims 0..7 of a word, in order) as the exact
// f16 subnormals code * 2^-24.  lo / hi hold the even / odd nibbles plus 8
// as bytes; v_perm interleaves them with zero bytes into the f16 bit
// patterns 0x00nn = (code + 8) * 2^-24, and a packed f16 subtraction of
// 8 * 2^-24 (exact: f16 denormals are kept) leaves code * 2^-24.  The MFMA
// products are exact for subnormal inputs as well; the kernel takes the 2^-24
// out per query.
__device__ __forceinline__ v8h nibbles_f16(uint32_t w) {
  const uint32_t x = w ^ 0x88888888u;
  const uint32_t lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;
  const _Float16 eight = __builtin_bit_cast(_Float16, (uint16_t)8);  // 8 * 2^-24
  v8h r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const v2h h = __builtin_bit_cast(v2h, __builtin_amdgcn_perm(hi, lo, 0x0C040C00u + 0x00010001u * k)) -
                  v2h{eight, eight};
    r[2 * k] = h[0];
    r[2 * k + 1] = h[1];
  }
  return r;
}
constexpr float kTwo24 = 16777216.0f;

// The same without the subtraction: (code + 8) * 2^-24.  Used for the keys,
// whose MFMA sum is reset every tile: q~.k = 2^24 C - 8 sum q~ costs one fp32
// rounding of a sum about twice the score, where the values' running output
// would carry the offset's rounding across the whole sequence.
__device__ __forceinline__ v8h nibbles_f16_offset(uint32_t w) {
  const uint32_t x = w ^ 0x88888888u;
  const uint32_t lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;
  uint32_t r[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) r[k] = __builtin_amdgcn_perm(hi, lo, 0x0C040C00u + 0x00010001u * k);
  return __builtin_bit_cast(v8h, make_uint4(r[0], r[1], r[2], r[3]));
}

// Head dimension of element e of a k-step-t operand in lane group g.
__device__ __forceinline__ int qk_dim(int g, int t, int e) { return 32 * g + 8 * t + e; }

// Direct-to-LDS loads (the data never passes through VGPRs): lane L writes
// its 16 (x4) or 4 (dword) bytes at LDS address m0 + 16 L (4 L).  The
// compiler does not see these as loads; the kernel waits for them with
// explicit s_waitcnt vmcnt(n), and the "memory" clobbers keep LDS reads after
// the waits.
// Addresses are a 32-bit per-lane byte offset against a 64-bit base in SGPRs.
#define RQA_DMA16(M0, OFF, BASE)                                                 \
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %2"    \
               :                                                                 \
               : "v"(OFF), "s"(M0), "s"(BASE)                                    \
               : "memory", "m0")
// The scales use a 64-bit per-lane address (lanes pick the key or the value
// scales).
#define RQA_DMA4(M0, ADDR)                                                       \
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"     \
               :                                                                 \
               : "v"(ADDR), "s"(M0)                                              \
               : "memory", "m0")
#define RQA_WAIT_VM(N) asm volatile("s_waitcnt vmcnt(" #N ")" ::: "memory")

// One tile slot of a wavefront's LDS ring: 16 key rows, 16 value rows (64
// bytes of codes each, row-major) and the 16 key then 16 value scales.
constexpr int SLOT_K = 0, SLOT_V = AT * 64, SLOT_S = 2 * AT * 64;
constexpr int SLOT = SLOT_S + 64;
constexpr int NSLOT = 4;  // default ring depth: the tile in use and three in flight

// The three DMA instructions of the tile at P into the slot at LDS address
// slot: rows from p1 on re-read the split's last valid row (an L2 hit; their
// weights are zero), so every call issues exactly three loads.  DMA lane L
// fetches part (L + (L >> 3)) & 3 of row L / 4 (L >> 3 = r >> 1 for row r),
// which puts part p of row r at 16-byte slot 4 r + ((p - (r >> 1)) & 3): the
// eight lanes of one b128 read phase (rows r .. r + 7, one part) then hit
// eight different bank groups.
// The scales travel as 4-byte pairs of positions (S even keeps them aligned).
// kb / vb / ksb / vsb are wave-uniform bases; offsets are 32-bit bytes.
__device__ __forceinline__ void issue_tile(uint32_t slot, const uint8_t* kb, const uint8_t* vb,
                                           const uint16_t* ksb, const uint16_t* vsb, int64_t P,
                                           int64_t last, int lane) {
  const int64_t r = P + (lane >> 2);
  const uint32_t row = (uint32_t)(r < last ? r : last);
  const uint32_t off = row * (AD / 2) + 16u * (uint32_t)((lane + (lane >> 3)) & 3);
  RQA_DMA16(slot + SLOT_K, off, kb);
  RQA_DMA16(slot + SLOT_V, off, vb);
  if (lane < 16) {
    const int64_t pos = P + 2 * (lane & 7);
    const int64_t lst = last & ~(int64_t)1;
    const uint16_t* src = lane < 8 ? ksb : vsb;
    RQA_DMA4(slot + SLOT_S, src + (pos < lst ? pos : lst));
  }
}

// LDS byte offset of part g of row r16 in a slot's key or value block
__device__ __forceinline__ int ring_part(int r16, int g) {
  return 16 * (4 * r16 + ((g - (r16 >> 1)) & 3));
}

// The normalised output row o~ (lane: dims 2 lane, 2 lane + 1) rotated back,
// o = (o~ H / sqrt(128)) then the signs, stored as fp16 (and fp32) at
// out[base ..].
template <bool HAS_SIGNS>
__device__ __forceinline__ void finish_row(float o0, float o1, int lane,
                                           const int8_t* __restrict__ signs, int64_t base,
                                           uint16_t* __restrict__ out, float* __restrict__ out_f32) {
  // FWHT over the 128 dims
  float a = o0 + o1, c = o0 - o1;
#pragma unroll
  for (int bit = 0; bit < 6; ++bit) {
    const float pa = __shfl_xor(a, 1 << bit, 64), pc = __shfl_xor(c, 1 << bit, 64);
    const bool upper = (lane >> bit) & 1;
    a = upper ? pa - a : a + pa;
    c = upper ? pc - c : c + pc;
  }
  const float sc = 0.08838834764831845f;  // fp32(1 / sqrt(128))
  float r0 = a * sc, r1 = c * sc;
  if (HAS_SIGNS) {
    if (signs[2 * lane] < 0) r0 = -r0;
    if (signs[2 * lane + 1] < 0) r1 = -r1;
  }
  const int64_t at = base + 2 * lane;
  out[at] = f2h_rn(r0);
  out[at + 1] = f2h_rn(r1);
  if (out_f32 != nullptr) {
    out_f32[at] = r0;
    out_f32[at + 1] = r1;
  }
}

// NW wavefronts per workgroup.  FUSED: the workgroup covers the whole
// sequence of its KV head (one split) and finishes the job itself: after the
// merge of its wavefronts it normalises, rotates back and stores the output,
// so no records and no combine kernel are needed.
template <int GM, bool HAS_SIGNS, int NW = AW, bool FUSED = false, int NS = NSLOT>
__global__ __launch_bounds__(64 * NW) void decode_attn_split_kernel(
    const __half* __restrict__ q, const uint8_t* __restrict__ kc, const uint16_t* __restrict__ ks,
    const uint8_t* __restrict__ vc, const uint16_t* __restrict__ vs,
    const int32_t* __restrict__ lengths, int H, int G, int64_t S, int64_t chunk, float qscale,
    const int8_t* __restrict__ signs, float* __restrict__ part, uint16_t* __restrict__ out,
    float* __restrict__ out_f32) {
  // ring[NW][NS] tile slots (the tile in use and NS - 1 in flight), then the
  // f16 value tiles; the queries rotate
  // in the value-tile space before the first tile, and after the tile loop
  // the per-wavefront records reuse the ring (FUSED: the merged records go to
  // the value-tile space)
  constexpr int RING = NW * NS * SLOT;
  constexpr int VT = NW * AT * VPITCH * 2;
  static_assert(NW * GM * PREC * 4 <= RING, "records fit in the ring");
  static_assert(GM * AD * 4 <= VT && GM * PREC * 4 <= VT, "queries fit in the value tiles");
  __shared__ __align__(16) unsigned char smem[RING + VT];
  float(*red)[GM][PREC] = reinterpret_cast<float(*)[GM][PREC]>(smem);
  _Float16(*vt)[AT][VPITCH] = reinterpret_cast<_Float16(*)[AT][VPITCH]>(smem + RING);
  float(*qs)[AD] = reinterpret_cast<float(*)[AD]>(smem + RING);
  float(*fin)[PREC] = reinterpret_cast<float(*)[PREC]>(smem + RING);

  const int tid = threadIdx.x;
  // wave is uniform per wavefront; readfirstlane lets the compiler see that
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int64_t bh = blockIdx.y;
  const int64_t b = bh / H, h = bh % H;
  int64_t len = S;
  if (lengths != nullptr) {
    const int64_t l0 = lengths[b];
    len = l0 < 0 ? 0 : (l0 > S ? S : l0);
  }
  const int64_t p0 = (int64_t)blockIdx.x * chunk;
  const int64_t p1 = p0 + chunk < len ? p0 + chunk : len;
  const int64_t last = p1 > 0 ? p1 - 1 : 0;

  // ---- the G queries of this KV head to LDS, (q * s) (their loads complete
  // before the tile loads go out: waits count loads in issue order)
  for (int i = tid; i < GM * AD; i += 64 * NW) {
    const int qi = i / AD, d = i % AD;
    float v = 0.0f;
    if (qi < G) {
      v = h2f(__half_as_ushort(q[((b * H + h) * G + qi) * AD + d]));
      if (HAS_SIGNS && signs[d] < 0) v = -v;
    }
    qs[qi][d] = v;
  }

  // the wavefront's first three tiles go in flight while the queries rotate
  const uint8_t* kb = kc + bh * S * (AD / 2);
  const uint8_t* vb = vc + bh * S * (AD / 2);
  const uint16_t* ksb = ks + bh * S;
  const uint16_t* vsb = vs + bh * S;
  const uint32_t ring = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem +
                        (uint32_t)(wave * NS * SLOT);
  const unsigned char* ringp = smem + wave * NS * SLOT;
  constexpr int64_t kStep = AT * NW;
  const int64_t Pw = p0 + AT * wave;
#pragma unroll
  for (int i = 0; i < NS - 1; ++i) issue_tile(ring + i * SLOT, kb, vb, ksb, vsb, Pw + i * kStep, last, lane);

  // ---- rotate the queries: (q * s) H_128 in LDS
  __syncthreads();
#pragma unroll
  for (int hs = 1; hs < AD; hs <<= 1) {
    for (int i = tid; i < GM * AD / 2; i += 64 * NW) {
      const int qi = i / (AD / 2), j = i % (AD / 2);
      const int i0 = (j / hs) * 2 * hs + (j % hs);
      const float a = qs[qi][i0], c = qs[qi][i0 + hs];
      qs[qi][i0] = a + c;
      qs[qi][i0 + hs] = a - c;
    }
    __syncthreads();
  }

  // ---- MFMA B operand of the scores (Q~^T): lane (query r16, group g),
  // k-step t holds the dims qk_dim(g, t, .) of q~ * qscale as f16 hi + lo
  v8h qh[4], ql[4];
  const int qrow = r16 < G ? r16 : 0;
  const float qmask = r16 < G ? qscale : 0.0f;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = qs[qrow][qk_dim(g, t, e)] * qmask;
      const _Float16 hv = (_Float16)v;
      qh[t][e] = hv;
      ql[t][e] = (_Float16)(v - (float)hv);
    }

  // 8 sum_d q~'_d over the f16 parts the MFMA sees: the score offset of the
  // keys' +8 (query r16, every lane group)
  float q8 = 0.0f;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) q8 += (float)qh[t][e] + (float)ql[t][e];
  q8 = 8.0f * pair32_add(pair16_add(q8));
  __syncthreads();  // every wavefront has its query operands: qs becomes value tiles

  // ---- per-wavefront running state, all in the layout of query r16
  float m_run = kNegInf, l_run = 0.0f;
  v4f_a acc[AD / 16];  // o~^T: m-tile mt, element e = value column 16 mt + 4 g + e
#pragma unroll
  for (int mt = 0; mt < AD / 16; ++mt) acc[mt] = v4f_a{0.0f, 0.0f, 0.0f, 0.0f};
  _Float16* vrow = &vt[wave][r16][32 * g];
  // transposing read of the value tile: lane (j, g) points at row 4 g + j / 4,
  // column 4 (j % 4) of each 16-column block
  const _Float16* vtr = &vt[wave][4 * g + (r16 >> 2)][4 * (r16 & 3)];

  const int rpart = ring_part(r16, g);
  int slot = 0;
  for (int64_t P = Pw; P < p1; P += kStep) {
    // the tile NS - 1 steps ahead goes in flight, then this tile's loads (three
    // DMA instructions per tile) are in
    issue_tile(ring + ((slot + NS - 1) % NS) * SLOT, kb, vb, ksb, vsb, P + (NS - 1) * kStep, last,
               lane);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * (NS - 1)) : "memory");
    const unsigned char* sl = ringp + slot * SLOT;
    slot = (slot + 1) % NS;
    const int lim = (int)(p1 - P < AT ? p1 - P : AT);  // valid positions in the tile

    // keys and values: lane (position r16, group g) takes bytes 16g .. 16g + 15
    const uint4 kw = *reinterpret_cast<const uint4*>(sl + SLOT_K + rpart);
    const uint4 vw = *reinterpret_cast<const uint4*>(sl + SLOT_V + rpart);
    const uint2 k2 = *reinterpret_cast<const uint2*>(sl + SLOT_S + 8 * g);
    const uint2 v2 = *reinterpret_cast<const uint2*>(sl + SLOT_S + 32 + 8 * g);
    float ksc[4], vsc[4];
    ksc[0] = h2f((uint16_t)k2.x); ksc[1] = h2f((uint16_t)(k2.x >> 16));
    ksc[2] = h2f((uint16_t)k2.y); ksc[3] = h2f((uint16_t)(k2.y >> 16));
    vsc[0] = h2f((uint16_t)v2.x); vsc[1] = h2f((uint16_t)(v2.x >> 16));
    vsc[2] = h2f((uint16_t)v2.y); vsc[3] = h2f((uint16_t)(v2.y >> 16));

    // the value tile to LDS as f16 codes (row r16, columns 32g .. 32g + 31)
    const uint32_t vwa[4] = {vw.x, vw.y, vw.z, vw.w};
#pragma unroll
    for (int w = 0; w < 4; ++w) *reinterpret_cast<v8h*>(vrow + 8 * w) = nibbles_f16(vwa[w]);

    // S^T = K Q~^T: C lane (query r16, group g), element e = position 4g + e
    // two independent accumulation chains (hi and lo parts) halve the
    // dependent MFMA latency of the tile
    v4f_a ch = {0.0f, 0.0f, 0.0f, 0.0f}, cl = {0.0f, 0.0f, 0.0f, 0.0f};
    const uint32_t kwa[4] = {kw.x, kw.y, kw.z, kw.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const v8h a = nibbles_f16_offset(kwa[t]);
      ch = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qh[t], ch, 0, 0, 0);
      cl = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, ql[t], cl, 0, 0, 0);
    }
    const v4f_a c = ch + cl;
    float sv[4];
    float tmax = kNegInf;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sv[e] = 4 * g + e < lim ? __builtin_fmaf(c[e], kTwo24, -q8) * ksc[e] : kNegInf;
      tmax = fmaxf(tmax, sv[e]);
    }
    tmax = pair32_max(pair16_max(tmax));
    const float m_new = fmaxf(m_run, tmax);  // finite: position P is valid
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float psum = 0.0f;
    v4h ph, pl;  // B operand of the output product: p * vscale, f16 hi + lo
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p = __builtin_amdgcn_exp2f(sv[e] - m_new);
      psum += p;
      const float pv = p * vsc[e];
      const _Float16 hv = (_Float16)pv;
      ph[e] = hv;
      pl[e] = (_Float16)(pv - (float)hv);
    }
    psum = pair32_add(pair16_add(psum));
    l_run = __builtin_fmaf(l_run, alpha, psum);
    m_run = m_new;
    // rescale only when some query's running max moved (rare after the first tiles)
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
      for (int mt = 0; mt < AD / 16; ++mt) acc[mt] *= alpha;
    }

    // the tile's values are in LDS (one wavefront: its LDS operations are in order)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // o~^T += V^T (p vscale)^T: A = transposing read (dims x positions)
#pragma unroll
    for (int mt = 0; mt < AD / 16; ++mt) {
      const v4h a = __builtin_bit_cast(
          v4h, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                   (__attribute__((address_space(3))) v4s*)(vtr + 16 * mt)));
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, ph, acc[mt], 0, 0, 0);
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, pl, acc[mt], 0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  // the loads of tiles past the end are still in flight: drain them before
  // the ring is reused for the records
  RQA_WAIT_VM(0);
  __syncthreads();

  // ---- the wavefront's record: o~ = 2^24 acc
  if (r16 < GM) {
#pragma unroll
    for (int mt = 0; mt < AD / 16; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[wave][r16][4 + 16 * mt + 4 * g + e] = acc[mt][e] * kTwo24;
    if (g == 0) {
      red[wave][r16][0] = m_run;
      red[wave][r16][1] = l_run;
    }
  }
  __syncthreads();

  // ---- merge the wavefronts: the split's record (FUSED: into LDS)
  for (int i = tid; i < GM * PREC; i += 64 * NW) {
    const int qi = i / PREC, c0 = i % PREC;
    if (qi >= G || c0 == 2 || c0 == 3) continue;
    float mx = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, red[w][qi][0]);
    float accv = 0.0f;
    if (c0 == 0) {
      accv = mx;
    } else if (mx != kNegInf) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = __builtin_amdgcn_exp2f(red[w][qi][0] - mx);
        accv = __builtin_fmaf(f, red[w][qi][c0], accv);
      }
    }
    if constexpr (FUSED)
      fin[qi][c0] = accv;
    else
      part[((bh * gridDim.x + blockIdx.x) * G + qi) * PREC + c0] = accv;
  }
  if constexpr (FUSED) {
    __syncthreads();
    // wavefront qi finishes query qi: lane holds dims 2 lane, 2 lane + 1
    if (wave < G) {
      const float den = fin[wave][1];
      const float inv = den > 0.0f ? 1.0f / den : 0.0f;
      const float o0 = fin[wave][4 + 2 * lane] * inv, o1 = fin[wave][5 + 2 * lane] * inv;
      finish_row<HAS_SIGNS>(o0, o1, lane, signs, (bh * G + wave) * AD, out, out_f32);
    }
  }
}
#undef RQA_DMA16
#undef RQA_DMA4
#undef RQA_WAIT_VM

// One wavefront per (b * H + h, query): merge the splits, normalise, rotate
// back (o~ H / sqrt(128), then the signs) and store fp16 (and fp32).  Lane sp
// reads split sp's (max, sum); the output columns of 4 splits at a time
// load together before they are summed.
template <bool HAS_SIGNS>
__global__ __launch_bounds__(256) void decode_attn_combine_kernel(
    const float* __restrict__ part, int64_t rows, int G, int nsplit,
    const int8_t* __restrict__ signs, uint16_t* __restrict__ out, float* __restrict__ out_f32) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // uniform per wavefront
  const int64_t bh = row / G, qi = row % G;
  const float* rec0 = part + (bh * nsplit * G + qi) * PREC;  // split sp at rec0 + sp G PREC
  const int64_t rstep = (int64_t)G * PREC;
  // nsplit <= 64 (plan_splits): lane sp holds split sp's (max, sum).  The
  // output columns of the first 4 splits load together with them, so that a
  // row costs one round trip to memory when nsplit <= 4.
  const float2 ml = lane < nsplit ? *reinterpret_cast<const float2*>(rec0 + lane * rstep)
                                  : make_float2(kNegInf, 0.0f);
  float2 v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int jj = u < nsplit ? u : nsplit - 1;
    v[u] = *reinterpret_cast<const float2*>(rec0 + jj * rstep + 4 + 2 * lane);
  }
  float mx = ml.x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  const float f = lane < nsplit && mx != kNegInf ? __builtin_amdgcn_exp2f(ml.x - mx) : 0.0f;
  float den = f * ml.y;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) den += __shfl_xor(den, off, 64);
  float o0 = 0.0f, o1 = 0.0f;
  for (int j = 0; j < nsplit; j += 4) {
    if (j > 0) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int jj = j + u < nsplit ? j + u : nsplit - 1;
        v[u] = *reinterpret_cast<const float2*>(rec0 + jj * rstep + 4 + 2 * lane);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float fj = j + u < nsplit ? __shfl(f, j + u < nsplit ? j + u : 0, 64) : 0.0f;
      o0 = __builtin_fmaf(fj, v[u].x, o0);
      o1 = __builtin_fmaf(fj, v[u].y, o1);
    }
  }
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  finish_row<HAS_SIGNS>(o0 * inv, o1 * inv, lane, signs, row * AD, out, out_f32);
}

// Positions per split: about one full round of resident workgroups (3 per CU
// at the split kernel's register use), so that every workgroup streams a long
// chunk (the query rotation and the final merge are paid once per chunk) and
// the combine kernel merges few records; each chunk a multiple of 64
// positions (4 wavefronts x 16).
void plan_splits(int64_t bh, int64_t S, int64_t* chunk, int* nsplit) {
  const int64_t want = (int64_t)cu_count() * 3;
  int64_t splits = (want + bh - 1) / bh;
  int64_t max_splits = (S + 63) / 64;
  if (max_splits > 64) max_splits = 64;  // the combine kernel merges up to 64 splits
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  int64_t c = (S + splits - 1) / splits;
  c = (c + 63) / 64 * 64;
  *chunk = c;
  *nsplit = (int)((S + c - 1) / c);
}

// The fused workgroup: four wavefronts per SIMD, each with a two-slot ring
// (the tile in use and one in flight); 16 rings and value tiles take 138 KB.
// Twelve wavefronts with four-slot rings (153 KB) ran 43.8-44.4 us on the
// 32 x 8 x 4096 cache against 41.3-42.1 us for this, and twelve with
// two-slot rings 42.6-42.8 us.
constexpr int AW_FUSED = 16, NS_FUSED = 2;

template <int GM, bool HAS_SIGNS>
void launch_split(const uint16_t* q, const uint8_t* kc, const uint16_t* ks, const uint8_t* vc,
                  const uint16_t* vs, const int32_t* lengths, int64_t B, int64_t H, int G,
                  int64_t S, int64_t chunk, int nsplit, float qscale, const int8_t* signs,
                  float* part, bool fused, uint16_t* out, float* out_f32, hipStream_t stream) {
  if (fused)
    hipLaunchKernelGGL((decode_attn_split_kernel<GM, HAS_SIGNS, AW_FUSED, true, NS_FUSED>),
                       dim3(1u, (unsigned)(B * H)), dim3(64 * AW_FUSED), 0, stream,
                       reinterpret_cast<const __half*>(q), kc, ks, vc, vs, lengths, (int)H, G, S, S,
                       qscale, signs, part, out, out_f32);
  else
    hipLaunchKernelGGL((decode_attn_split_kernel<GM, HAS_SIGNS>), dim3((unsigned)nsplit, (unsigned)(B * H)),
                       dim3(64 * AW), 0, stream, reinterpret_cast<const __half*>(q), kc, ks, vc, vs,
                       lengths, (int)H, G, S, chunk, qscale, signs, part, out, out_f32);
}

}  // namespace

size_t decode_attention_workspace_bytes(int64_t batch, int64_t kv_heads, int64_t group,
                                        int64_t seq) {
  int64_t chunk;
  int nsplit;
  plan_splits(batch * kv_heads, seq, &chunk, &nsplit);
  return (size_t)(batch * kv_heads * nsplit * group) * PREC * sizeof(float);
}

hipError_t launch_decode_attention(const uint16_t* q, const uint8_t* kc, const uint16_t* ks,
                                   const uint8_t* vc, const uint16_t* vs, const int32_t* lengths,
                                   int64_t B, int64_t H, int64_t G, int64_t S,
                                   const int8_t* signs, float sm_scale, uint16_t* out,
                                   float* out_f32, void* workspace, hipStream_t stream) {
  int64_t chunk;
  int nsplit;
  plan_splits(B * H, S, &chunk, &nsplit);
  float* part = static_cast<float*>(workspace);
  // scores come out in log2 units: q~ carries 1/sqrt(128), the softmax scale and log2(e)
  const float qscale = 0.08838834764831845f * sm_scale * 1.4426950408889634f;
  const bool sg = signs != nullptr;
  // One workgroup per KV head over the whole sequence, finishing in place,
  // when the KV heads fill the CUs in whole rounds (the split kernel then
  // gains nothing from splitting and needs a combine launch).
  const bool fused = (B * H) % cu_count() == 0;
  if (G <= 4)
    sg ? launch_split<4, true>(q, kc, ks, vc, vs, lengths, B, H, (int)G, S, chunk, nsplit, qscale, signs, part, fused, out, out_f32, stream)
       : launch_split<4, false>(q, kc, ks, vc, vs, lengths, B, H, (int)G, S, chunk, nsplit, qscale, signs, part, fused, out, out_f32, stream);
  else
    sg ? launch_split<8, true>(q, kc, ks, vc, vs, lengths, B, H, (int)G, S, chunk, nsplit, qscale, signs, part, fused, out, out_f32, stream)
       : launch_split<8, false>(q, kc, ks, vc, vs, lengths, B, H, (int)G, S, chunk, nsplit, qscale, signs, part, fused, out, out_f32, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || fused) return e;
  const int64_t rows = B * H * G;
  const unsigned blocks = (unsigned)((rows + 3) / 4);
  if (sg)
    hipLaunchKernelGGL(decode_attn_combine_kernel<true>, dim3(blocks), dim3(256), 0, stream, part,
                       rows, (int)G, nsplit, signs, out, out_f32);
  else
    hipLaunchKernelGGL(decode_attn_combine_kernel<false>, dim3(blocks), dim3(256), 0, stream, part,
                       rows, (int)G, nsplit, signs, out, out_f32);
  return hipGetLastError();
}

}  // namespace rq
