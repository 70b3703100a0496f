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

#ifdef __cplusplus
}
#endif

#endif /* LIBCSA_CSA_BENCH_H */
