/*
 * rq_ceiling.h -- ceiling probes exported by librq next to the hot path.
 *
 * They measure what one MI355X delivers at the sizes the hot path moves, so
 * the roofline fractions of the hot-path kernels can be read against a
 * practical ceiling as well as against the published peaks (HBM 8 TB/s;
 * dense int8 MFMA 5.0 POP/s).  [RQ] "Weight Absorption and Online Fast
 * Walsh-Hadamard Transforms", part 2 (the online rotation is bound by memory
 * bandwidth) and "Hardware Execution and Serving Economics", part 1 (integer
 * matrix throughput) name the two resources.  They compute nothing of the
 * method.
 *
 * Conventions: device pointers, asynchronous on `stream` (a hipStream_t as
 * void*, NULL = the null stream); nothing is allocated.  Return 0 on success,
 * 1 for a NULL pointer, 3 for a misaligned pointer or size, 5 for a failed
 * launch (rq_ceiling_mfma_i8: negative values).
 */
#ifndef RQ_CEILING_H_
#define RQ_CEILING_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Words of `sink` that rq_ceiling_read writes (one per workgroup). */
size_t rq_ceiling_read_sink_words(void);

/*
 * Read `bytes` (a multiple of 16) from src (16-byte aligned) with 16-byte
 * nontemporal loads, 1 KB per wavefront instruction, in a grid-stride loop
 * over up to 16 workgroups per CU; sink [rq_ceiling_read_sink_words()]
 * receives one xor word per workgroup.
 */
int rq_ceiling_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* Copy `bytes` (a multiple of 16) from src to dst (both 16-byte aligned,
 * not overlapping) with 16-byte nontemporal loads and stores. */
int rq_ceiling_copy(const void* src, void* dst, size_t bytes, void* stream);

/* int32 words of `out` that rq_ceiling_mfma_i8 writes for this occupancy. */
size_t rq_ceiling_mfma_out_words(int64_t waves_per_simd);

/*
 * waves_per_simd (1..8) wavefronts per SIMD on every CU each run `iters`
 * rounds of 8 independent v_mfma_i32_16x16x64_i8 on register operands and
 * store their accumulators to out [rq_ceiling_mfma_out_words(...)].
 * Returns the integer operations issued (2 * 16 * 16 * 64 per MFMA), or a
 * negative value on an error (-1 NULL, -2 bad size, -5 launch failure).
 */
int64_t rq_ceiling_mfma_i8(int32_t* out, int64_t waves_per_simd, int64_t iters, void* stream);

/*
 * The same loop on the 6-bit matrix unit: rounds of 8 independent
 * v_mfma_f32_16x16x128_f8f6f4 with E3M2 operands holding random INT4 codes
 * (the values rq_w4a4_gemm_f6 multiplies).  out takes
 * rq_ceiling_mfma_out_words(waves_per_simd) int32 words.  Returns the
 * operations issued (2 * 16 * 16 * 128 per MFMA), or a negative value on an
 * error (-1 NULL, -2 bad size, -5 launch failure).
 */
int64_t rq_ceiling_mfma_f6(int32_t* out, int64_t waves_per_simd, int64_t iters, void* stream);

/* Floats of `out` that rq_ceiling_issue writes for this occupancy. */
size_t rq_ceiling_issue_out_words(int64_t waves_per_simd);

/*
 * Issue-rate loop: waves_per_simd (1..8) wavefronts per SIMD on every CU
 * each run `iters` (1..2^24) rounds of one register-only instruction block
 * and store one float per lane to out [rq_ceiling_issue_out_words(...)]:
 *   kind 0: 8 independent v_mfma_i32_16x16x64_i8;
 *   kind 1: 32 independent (v_cvt_f32_i32, v_fmac_f32) pairs;
 *   kind 2: the blocks of kinds 0 and 1 in the same round;
 *   kind 3: 32 independent v_fmac_f32;
 *   kind 4: 32 independent v_fmac_f32_dpp (quad_perm lane exchange).
 * Kinds 0..2 show whether MFMA and VALU work of a SIMD overlap (the time
 * of kind 2 against the sum of kinds 0 and 1); kinds 3 and 4 the issue cost
 * of a lane-crossing DPP operation against a plain one.  Returns the
 * wavefront rounds run (blocks * 4 * iters), or -1 (NULL), -2 (bad kind or
 * size), -5 (launch failure).
 */
int64_t rq_ceiling_issue(float* out, int64_t kind, int64_t waves_per_simd, int64_t iters,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RQ_CEILING_H_ */
