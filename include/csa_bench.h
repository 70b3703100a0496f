/*
 * libcsa_bench -- standard causal softmax attention on the same tiling as
 * csa_forward, built only as an in-run comparison point for throughput.
 *
 * Computes eq. (12) of J. Su, "Continuous Softmax Attention" (Analysis of the
 * Result): o_t = sum_{i=1..t} e^{q_t . k_i} v_i / sum_{i=1..t} e^{q_t . k_i},
 * with query t = row t-1 and key i = row i-1; no k_0/v_0, no correction term,
 * no internal 1/sqrt(d) scale.
 *
 * Arguments, layouts, ownership, asynchrony and return codes are those of
 * csa_forward in csa.h, minus k0/v0; lse (if not NULL) receives the natural
 * log of sum_i e^{q_t . k_i}.
 */
#ifndef LIBCSA_CSA_BENCH_H
#define LIBCSA_CSA_BENCH_H

#include <stdint.h>

#include "csa.h"

#ifdef __cplusplus
extern "C" {
#endif

int std_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int64_t B,
            int64_t H, int64_t T, int64_t d, int dtype, void* stream);

/* The validation of std_fwd alone (no memory access, no HIP call). */
int std_fwd_check(const void* q, const void* k, const void* v, const void* out, const float* lse,
                  int64_t B, int64_t H, int64_t T, int64_t d, int dtype);

/*
 * csa_probe -- micro-benchmarks of the gfx950 SIMD, for measurement only: the MFMA-only
 * ceiling the forward kernels are compared with, the issue cost of the VALU instructions
 * the correction weights are made of, whether MFMA and VALU work of one SIMD overlap, and
 * the forward's weight arithmetic beside either MFMA shape (the choice of tiling).
 * One launch of `ceil(waves / 4)` work-groups of 256 threads (four waves) that run `iters`
 * iterations of a fixed instruction mix in every wave:
 *   kind 0  4 independent v_mfma_f32_16x16x32_bf16 chains (4 x 16384 FLOP per iteration)
 *   kind 1  8 independent fp32 FMA chains
 *   kind 2  8 independent v_exp_f32 chains
 *   kind 3  8 independent v_rcp_f32 chains
 *   kind 4  the MFMAs of kind 0 and 16 fp32 FMAs (two rounds of kind 1) per iteration
 *   kind 5  2 independent v_mfma_f32_32x32x16_bf16 chains (2 x 32768 FLOP per iteration)
 *   kind 6  the forward's correction-weight arithmetic for two keys per iteration (exp2,
 *           neighbour difference, reciprocal, both edge terms with the Taylor select)
 *   kind 7  kinds 6 and 0 together (two 16x16x32 MFMAs per key, the forward's ratio)
 *   kind 8  kinds 6 and 5 together (the same FLOP on 32x32x16 MFMAs)
 *   kind 9  the weights of kind 6 by the log-domain route (eq. (13): b as the log of the sum of
 *           the two phi_2 terms, each phi_2 in logs, log-sum-exp, then exp), two keys per iteration
 *   kind 10 kind 1 with 2 v_exp_f32 chains beside the 8 FMA chains
 *   kind 11 kind 1 with 2 v_rcp_f32 chains beside the 8 FMA chains
 *   kind 12 the weights of kind 6 with the reciprocal replaced by a 1024-entry LDS table
 *           lookup (one ds_read_b128 and two fmas per edge; placeholder table values)
 *   sink    device, >= ceil(waves / 4) floats: one result per work-group (keeps the work)
 *   cycles  device, 1 uint64, zeroed by the caller: raised (atomic max) to the shader-clock
 *           cycles (s_memtime) of the longest-running wave's loop
 *   stream  hipStream_t; the caller times the launch (events) and synchronises.
 * Returns CSA_OK, CSA_ERR_INVALID_ARG (unknown kind, waves < 1 or > 2^24, iters < 1 or > 2^30,
 * null sink or cycles; checked before any HIP call) or CSA_ERR_HIP.
 */
int csa_probe(int kind, int64_t waves, int64_t iters, float* sink, uint64_t* cycles, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBCSA_CSA_BENCH_H */
