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
// position tiles in turn and keep their own running max / sum / output.
//   * Scores: S^T = K Q~^T on the f16 MFMA 16x16x32.  A key row (64 bytes of
//     codes) is contiguous, so a lane loads 16 bytes and converts 8 nibbles
//     per k-step to f16 exactly (1024 + code' - 1032).  The query is split
//     into f16 hi + lo (about 22 significant bits) and both products
//     accumulate in fp32, so the scores keep fp32-level accuracy.
//   * The output: v^ is position-major, so the weighted sum runs on the VALU
//     with lanes owning head dimensions (lane L: 8 dimensions, one of 4
//     position slots), nibbles converted with v_cvt_f32_ubyte.
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
typedef float v4f_a __attribute__((ext_vector_type(4)));

constexpr int AD = 128;          // head dimension
constexpr int AW = 4;            // wavefronts per workgroup
constexpr int AT = 16;           // positions per wavefront step
constexpr int PREC = AD + 4;     // floats per split record: m, l, 2 pad, o~[128]
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

// 8 two's-complement nibbles (dims 0..7 of a word) as f16 in the order
// 0, 4, 1, 5, 2, 6, 3, 7: (w' >> 4k) & 0x000F000F puts nibbles k and k + 4
// in the two halves, 0x6400 makes them 1024 + code', and 1032 is subtracted.
__device__ __forceinline__ v8h nibbles_f16(uint32_t w) {
  const uint32_t x = w ^ 0x88888888u;
  v8h r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t pair = ((x >> (4 * k)) & 0x000F000Fu) | 0x64006400u;
    v2h h = __builtin_bit_cast(v2h, pair) - v2h{(_Float16)1032.0f, (_Float16)1032.0f};
    r[2 * k] = h[0];
    r[2 * k + 1] = h[1];
  }
  return r;
}

// Head dimension of element e of a k-step-t operand in lane group g.
__device__ __forceinline__ int qk_dim(int g, int t, int e) {
  return 32 * g + 8 * t + ((e & 1) << 2) + (e >> 1);
}

template <int GM, bool HAS_SIGNS>
__global__ __launch_bounds__(64 * AW) void decode_attn_split_kernel(
    const __half* __restrict__ q, const uint8_t* __restrict__ kc, const uint16_t* __restrict__ ks,
    const uint8_t* __restrict__ vc, const uint16_t* __restrict__ vs,
    const int32_t* __restrict__ lengths, int H, int G, int64_t S, int64_t chunk, float qscale,
    const int8_t* __restrict__ signs, float* __restrict__ part) {
  __shared__ float qs[GM][AD];            // rotated queries
  __shared__ float pt[AW][AT][GM];        // p * vscale of the wavefront's tile, [position][query]
  __shared__ float ar[AW][GM];            // rescale factor of the tile, per query
  __shared__ float red[AW][GM][PREC];     // per-wavefront (m, l, o~) records

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
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

  // ---- the G queries of this KV head, rotated: (q * s) H_128 in LDS
  for (int i = tid; i < GM * AD; i += 64 * AW) {
    const int qi = i / AD, d = i % AD;
    float v = 0.0f;
    if (qi < G) {
      v = h2f(__half_as_ushort(q[((b * H + h) * G + qi) * AD + d]));
      if (HAS_SIGNS && signs[d] < 0) v = -v;
    }
    qs[qi][d] = v;
  }
  __syncthreads();
#pragma unroll
  for (int hs = 1; hs < AD; hs <<= 1) {
    for (int i = tid; i < GM * AD / 2; i += 64 * AW) {
      const int qi = i / (AD / 2), j = i % (AD / 2);
      const int i0 = (j / hs) * 2 * hs + (j % hs);
      const float a = qs[qi][i0], c = qs[qi][i0 + hs];
      qs[qi][i0] = a + c;
      qs[qi][i0 + hs] = a - c;
    }
    __syncthreads();
  }

  // ---- MFMA B operand (Q~^T): lane (query r16, group g), k-step t holds the
  // dims qk_dim(g, t, .) of q~ * qscale as f16 hi + lo
  v8h qh[4], ql[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = r16 < G ? qs[r16][qk_dim(g, t, e)] * qscale : 0.0f;
      const _Float16 hv = (_Float16)v;
      qh[t][e] = hv;
      ql[t][e] = (_Float16)(v - (float)hv);
    }

  // ---- per-wavefront running state
  float m_run = kNegInf, l_run = 0.0f;  // of query r16 (score layout)
  float o[GM][8], corr[GM];             // output dims 8 (lane & 15) .., slot lane >> 4
#pragma unroll
  for (int qi = 0; qi < GM; ++qi) {
    corr[qi] = 0.0f;
#pragma unroll
    for (int d = 0; d < 8; ++d) o[qi][d] = 0.0f;
  }
  const int slot = lane >> 4, dblk = lane & 15;
  const uint8_t* kbase = kc + bh * S * (AD / 2);
  const uint8_t* vbase = vc + bh * S * (AD / 2);
  const uint16_t* ksb = ks + bh * S;
  const uint16_t* vsb = vs + bh * S;

  for (int64_t P = p0 + AT * wave; P < p1; P += AT * AW) {
    // keys: lane (position r16, group g) takes bytes 16g .. 16g + 15
    const int64_t kpos = P + r16;
    uint4 kw = make_uint4(0, 0, 0, 0);
    if (kpos < p1) kw = *reinterpret_cast<const uint4*>(kbase + kpos * (AD / 2) + 16 * g);
    // values: lane (dims 8 dblk .., slot) takes 4 bytes of positions P + 4i + slot
    uint32_t vw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t vpos = P + 4 * i + slot;
      vw[i] = 0;
      if (vpos < p1) vw[i] = *reinterpret_cast<const uint32_t*>(vbase + vpos * (AD / 2) + 4 * dblk);
    }
    // scales of positions P + 4g + e (score layout)
    float ksc[4], vsc[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t sp = P + 4 * g + e;
      ksc[e] = sp < p1 ? h2f(ksb[sp]) : 0.0f;
      vsc[e] = sp < p1 ? h2f(vsb[sp]) : 0.0f;
    }

    // S^T = K Q~^T: C lane (query r16, group g), element e = position 4g + e
    v4f_a c = {0.0f, 0.0f, 0.0f, 0.0f};
    const uint32_t kwa[4] = {kw.x, kw.y, kw.z, kw.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const v8h a = nibbles_f16(kwa[t]);
      c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qh[t], c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, ql[t], c, 0, 0, 0);
    }
    float s[4];
    float tmax = kNegInf;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s[e] = P + 4 * g + e < p1 ? c[e] * ksc[e] : kNegInf;
      tmax = fmaxf(tmax, s[e]);
    }
    tmax = pair32_max(pair16_max(tmax));
    const float m_new = fmaxf(m_run, tmax);
    const bool none = m_new == kNegInf;  // nothing seen yet (uniform per query)
    const float alpha = none ? 1.0f : exp2f(m_run - m_new);
    float psum = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p = none ? 0.0f : exp2f(s[e] - m_new);
      psum += p;
      if (r16 < GM) pt[wave][4 * g + e][r16] = r16 < G ? p * vsc[e] : 0.0f;
    }
    psum = pair32_add(pair16_add(psum));
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (g == 0 && r16 < GM) ar[wave][r16] = alpha;
    // LDS operations of one wavefront execute in order: fence the compiler only
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // o~ += p v^ on the VALU (codes as code' = code + 8; corr keeps sum p for the -8)
#pragma unroll
    for (int qi = 0; qi < GM; ++qi) {
      const float al = ar[wave][qi];
      corr[qi] *= al;
#pragma unroll
      for (int d = 0; d < 8; ++d) o[qi][d] *= al;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t x = vw[i] ^ 0x88888888u;
      const uint32_t lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;
      float f[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {  // (float) of a byte field: v_cvt_f32_ubyte<k>
        f[2 * k] = (float)((lo >> (8 * k)) & 0xFFu);
        f[2 * k + 1] = (float)((hi >> (8 * k)) & 0xFFu);
      }
#pragma unroll
      for (int qi = 0; qi < GM; ++qi) {
        const float pv = pt[wave][4 * i + slot][qi];
        corr[qi] += pv;
#pragma unroll
        for (int d = 0; d < 8; ++d) o[qi][d] = __builtin_fmaf(pv, f[d], o[qi][d]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- the wavefront's record: o~ = sum over the 4 slots of (o - 8 corr)
#pragma unroll
  for (int qi = 0; qi < GM; ++qi)
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const float v = __builtin_fmaf(-8.0f, corr[qi], o[qi][d]);
      o[qi][d] = pair32_add(pair16_add(v));
    }
  if (slot == 0) {
#pragma unroll
    for (int qi = 0; qi < GM; ++qi)
#pragma unroll
      for (int d = 0; d < 8; ++d) red[wave][qi][4 + 8 * dblk + d] = o[qi][d];
  }
  if (g == 0 && r16 < GM) {
    red[wave][r16][0] = m_run;
    red[wave][r16][1] = l_run;
  }
  __syncthreads();

  // ---- merge the 4 wavefronts and write the split's record
  for (int i = tid; i < GM * PREC; i += 64 * AW) {
    const int qi = i / PREC, c0 = i % PREC;
    if (qi >= G || c0 == 2 || c0 == 3) continue;
    float mx = kNegInf;
#pragma unroll
    for (int w = 0; w < AW; ++w) mx = fmaxf(mx, red[w][qi][0]);
    float acc = 0.0f;
    if (c0 == 0) {
      acc = mx;
    } else if (mx != kNegInf) {
#pragma unroll
      for (int w = 0; w < AW; ++w) {
        const float f = exp2f(red[w][qi][0] - mx);
        acc = __builtin_fmaf(f, red[w][qi][c0], acc);
      }
    }
    part[((bh * gridDim.x + blockIdx.x) * G + qi) * PREC + c0] = acc;
  }
}

// One wavefront per (b * H + h, query): merge the splits, normalise, rotate
// back (o~ H / sqrt(128), then the signs) and store fp16 (and fp32).
template <bool HAS_SIGNS>
__global__ __launch_bounds__(256) void decode_attn_combine_kernel(
    const float* __restrict__ part, int64_t rows, int G, int nsplit,
    const int8_t* __restrict__ signs, uint16_t* __restrict__ out, float* __restrict__ out_f32) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // uniform per wavefront
  const int64_t bh = row / G, qi = row % G;
  float mx = kNegInf;
  for (int sp = 0; sp < nsplit; ++sp) mx = fmaxf(mx, part[((bh * nsplit + sp) * G + qi) * PREC]);
  float den = 0.0f, o0 = 0.0f, o1 = 0.0f;
  if (mx != kNegInf) {
    for (int sp = 0; sp < nsplit; ++sp) {
      const float* r = part + ((bh * nsplit + sp) * G + qi) * PREC;
      const float f = exp2f(r[0] - mx);
      den = __builtin_fmaf(f, r[1], den);
      const float2 v = *reinterpret_cast<const float2*>(r + 4 + 2 * lane);
      o0 = __builtin_fmaf(f, v.x, o0);
      o1 = __builtin_fmaf(f, v.y, o1);
    }
  }
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  o0 *= inv;
  o1 *= inv;
  // FWHT over the 128 dims: lane holds dims 2 lane, 2 lane + 1
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
  const int64_t base = row * AD + 2 * lane;
  out[base] = f2h_rn(r0);
  out[base + 1] = f2h_rn(r1);
  if (out_f32 != nullptr) {
    out_f32[base] = r0;
    out_f32[base + 1] = r1;
  }
}

// Positions per split: enough splits for about 8 workgroups per CU, each a
// multiple of 64 positions (4 wavefronts x 16).
void plan_splits(int64_t bh, int64_t S, int64_t* chunk, int* nsplit) {
  const int64_t want = (int64_t)cu_count() * 8;
  int64_t splits = (want + bh - 1) / bh;
  const int64_t max_splits = (S + 63) / 64;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  int64_t c = (S + splits - 1) / splits;
  c = (c + 63) / 64 * 64;
  *chunk = c;
  *nsplit = (int)((S + c - 1) / c);
}

template <int GM, bool HAS_SIGNS>
void launch_split(const uint16_t* q, const uint8_t* kc, const uint16_t* ks, const uint8_t* vc,
                  const uint16_t* vs, const int32_t* lengths, int64_t B, int64_t H, int G,
                  int64_t S, int64_t chunk, int nsplit, float qscale, const int8_t* signs,
                  float* part, hipStream_t stream) {
  hipLaunchKernelGGL((decode_attn_split_kernel<GM, HAS_SIGNS>), dim3((unsigned)nsplit, (unsigned)(B * H)),
                     dim3(64 * AW), 0, stream, reinterpret_cast<const __half*>(q), kc, ks, vc, vs,
                     lengths, (int)H, G, S, chunk, qscale, signs, part);
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
  if (G <= 4)
    sg ? launch_split<4, true>(q, kc, ks, vc, vs, lengths, B, H, (int)G, S, chunk, nsplit, qscale, signs, part, stream)
       : launch_split<4, false>(q, kc, ks, vc, vs, lengths, B, H, (int)G, S, chunk, nsplit, qscale, signs, part, stream);
  else
    sg ? launch_split<8, true>(q, kc, ks, vc, vs, lengths, B, H, (int)G, S, chunk, nsplit, qscale, signs, part, stream)
       : launch_split<8, false>(q, kc, ks, vc, vs, lengths, B, H, (int)G, S, chunk, nsplit, qscale, signs, part, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
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
