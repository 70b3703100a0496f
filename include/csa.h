/*
 * libcsa -- causal continuous softmax attention on AMD Instinct MI355X (gfx950):
 * the forward pass, its first-order and half-interval variants, few-query decoding
 * against a cache, and the backward pass.
 *
 * Method: J. Su, "Continuous Softmax Attention" (Scientific Spaces; English
 * translation on tylerromero.com).  Keys and values are linearly interpolated
 * between integer positions (Problem Statement, eq. (3)), with two extra
 * vectors k_0, v_0 at position 0, and the attention sum of standard softmax
 * attention becomes the ratio of two integrals over [0, t] (eq. (2)).  The
 * integrals reduce (Assembly and Simplification, eq. (10)-(11)) to
 *
 *     o_t = sum_{i=0..t} e^{a_{t,i} + b_{t,i}} v_i / sum_{i=0..t} e^{a_{t,i} + b_{t,i}},
 *     a_{t,i} = q_t . k_i,
 *     e^{b_{t,i}} = phi_2(a_{t,i-1} - a_{t,i}) + phi_2(a_{t,i+1} - a_{t,i}),
 *
 * where only the existing neighbour enters at i = 0 and i = t, and
 * phi_2(x) = (e^x - 1 - x)/x^2, phi_2(0) = 1/2 (Preliminaries, eq. (6)).
 *
 * Conventions shared by every entry point:
 *   - Query t = 1..T is row t-1 of q; key/value position i >= 1 is row i-1
 *     of k/v; position 0 is k0/v0.  No 1/sqrt(d) scale is applied inside:
 *     the logit is the bare dot product q_t . k_i, as in eq. (1)-(2).
 *   - All device buffers are owned by the caller; the library allocates no
 *     memory and keeps no state between calls (thread-safe, re-entrant).
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream) and do not synchronise.  Device-side faults surface through
 *     the HIP runtime of the caller, not through the return value.
 *   - Every argument is validated before any HIP API call; on failure the
 *     call returns an error code and launches nothing.
 */
#ifndef LIBCSA_CSA_H
#define LIBCSA_CSA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of q, k, v, k0, v0 and out. */
typedef enum {
  CSA_F32 = 0,  /* IEEE float32 */
  CSA_BF16 = 1  /* bfloat16 (round-to-nearest-even on output) */
} csa_dtype;

/* Return codes. */
enum {
  CSA_OK = 0,
  CSA_ERR_INVALID_ARG = 1, /* NULL pointer, non-positive size, misaligned or overlapping buffer, size overflow */
  CSA_ERR_UNSUPPORTED = 2, /* head dimension d not in {16, 64, 128}, or a dtype the entry point does not take */
  CSA_ERR_HIP = 3,         /* the kernel launch was rejected by the HIP runtime */
  CSA_ERR_SCRATCH_TOO_SMALL = 4 /* csa_decode_noalloc: the sizes need more than its static scratch */
};

/*
 * csa_forward -- o_t and lse_t for every query t = 1..T of every (batch, head)
 * by eq. (10)-(11) of "Continuous Softmax Attention" (the causal interval
 * [0, t] chosen under Problem Statement).
 *
 *   q, k, v  device, [B, H, T, d] contiguous, element type `dtype`, 16-byte aligned.
 *   k0, v0   device, [B, H, d] contiguous, `dtype`, 16-byte aligned; NULL means
 *            a zero vector (the "all zeros" choice under Analysis of the
 *            Result).  For the "copy the first key" choice pass a copy of
 *            k[:, :, 0, :] (resp. v).
 *   out      device, [B, H, T, d] contiguous, `dtype`, 16-byte aligned; must not
 *            overlap any input or lse.  Accumulation is float32; bf16 output is
 *            rounded to nearest even.
 *   lse      device, [B, H, T] float32, 4-byte aligned, or NULL (not written):
 *            natural log of sum_i e^{a_{t,i} + b_{t,i}}, i.e. of the
 *            denominator integral of eq. (2).
 *   B, H, T  >= 1.  d in {16, 64, 128}.
 *   dtype    CSA_F32 or CSA_BF16.
 *   stream   hipStream_t or NULL.
 *
 * Returns CSA_OK, or an error code from the enum above (nothing launched).
 */
int csa_forward(const void* q, const void* k, const void* v, const void* k0, const void* v0,
                void* out, float* lse, int64_t B, int64_t H, int64_t T, int64_t d, int dtype,
                void* stream);

/*
 * csa_forward_check -- the argument validation of csa_forward alone, with
 * the same arguments and the same return codes; touches no memory and makes
 * no HIP call (usable on a machine without a GPU).
 */
int csa_forward_check(const void* q, const void* k, const void* v, const void* k0, const void* v0,
                      const void* out, const float* lse, int64_t B, int64_t H, int64_t T, int64_t d,
                      int dtype);

/*
 * csa_forward_first_order -- the same forward with b replaced by its first-order
 * expansion (Analysis of the Result, eq. (13)): for 1 <= i <= t-1
 *
 *     b_{t,i} = (a_{t,i-1} + a_{t,i+1} - 2 a_{t,i}) / 6,
 *
 * the second difference of the logits (the "short convolution" reading of the
 * method), and at the two end positions, which keep a single phi_2 term in
 * eq. (10), b = -ln 2 + x/3 with x = a_{t,1} - a_{t,0} at i = 0 and
 * x = a_{t,t-1} - a_{t,t} at i = t (phi_2(x) = 1/2 + x/6 + ... expanded the same
 * way).  o_t is eq. (11) with these b; lse_t = ln sum_i e^{a_{t,i} + b_{t,i}}.
 *
 * Arguments, layouts, ownership and return codes as csa_forward, except that
 * dtype must be CSA_BF16 (CSA_F32 returns CSA_ERR_UNSUPPORTED).
 */
int csa_forward_first_order(const void* q, const void* k, const void* v, const void* k0,
                            const void* v0, void* out, float* lse, int64_t B, int64_t H, int64_t T,
                            int64_t d, int dtype, void* stream);

/* The argument validation of csa_forward_first_order alone (no HIP call). */
int csa_forward_first_order_check(const void* q, const void* k, const void* v, const void* k0,
                                  const void* v0, const void* out, const float* lse, int64_t B,
                                  int64_t H, int64_t T, int64_t d, int dtype);

/*
 * csa_forward_half_interval -- the interval variant of "Continuous Softmax
 * Attention" (Problem Statement: the original paper integrates eq. (2) over
 * [1/2, t + 1/2] rather than [0, t]).  With the interpolation of eq. (3)
 * unchanged, query t covers the upper half of segment [0, 1] (between k_0 and
 * k_1), the whole segments [1, 2] .. [t-1, t], and the lower half of segment
 * [t, t+1]: it reaches half a step toward position t+1.  For the last query
 * (t = T) position T+1 is taken equal to position T, so that half segment is
 * flat.  o_t is the ratio of the two integrals of eq. (2) over this interval and
 * lse_t the natural log of the denominator integral.
 *
 * Arguments, layouts, ownership and return codes as csa_forward, except that
 * dtype must be CSA_BF16 (CSA_F32 returns CSA_ERR_UNSUPPORTED).
 */
int csa_forward_half_interval(const void* q, const void* k, const void* v, const void* k0,
                              const void* v0, void* out, float* lse, int64_t B, int64_t H,
                              int64_t T, int64_t d, int dtype, void* stream);

/* The argument validation of csa_forward_half_interval alone (no HIP call). */
int csa_forward_half_interval_check(const void* q, const void* k, const void* v, const void* k0,
                                    const void* v0, const void* out, const float* lse, int64_t B,
                                    int64_t H, int64_t T, int64_t d, int dtype);

/*
 * csa_decode -- the forward for a few new queries against a key/value cache (decoding
 * or speculative verification): the Tq queries are the last positions T-Tq+1..T of a
 * sequence whose keys/values at positions 1..T (and k_0, v_0 at position 0) are in the
 * cache.  Query j (0-based) is position t_j = T - Tq + 1 + j and sees positions 0..t_j;
 * o and lse are exactly those rows of csa_forward (eq. (10)-(11)).
 *
 *   q          device, [B, H, Tq, d] contiguous, `dtype`, 16-byte aligned; 1 <= Tq <= 8, Tq <= T.
 *   k, v       device, [B, H, T, d] contiguous cache, `dtype`, 16-byte aligned.
 *   k0, v0     as in csa_forward (NULL = zeros).
 *   out        device, [B, H, Tq, d], `dtype`, 16-byte aligned.
 *   lse        device, [B, H, Tq] float32, 4-byte aligned, or NULL.
 *   workspace  device, 16-byte aligned, at least csa_decode_workspace_bytes(B, H, Tq, T, d)
 *              bytes, owned by the caller and used for per-split partial results; its
 *              contents need no initialisation and are scratch after the call.  Calls that
 *              share a workspace must be ordered on one stream.
 *   Other arguments and return codes as csa_forward (CSA_ERR_INVALID_ARG also for Tq out
 *   of range, a short or missing workspace, or any overlap among out, lse, workspace and
 *   the inputs).
 *
 * Two kernel launches on `stream`: per-split partials, then their merge.
 */
int csa_decode(const void* q, const void* k, const void* v, const void* k0, const void* v0,
               void* out, float* lse, void* workspace, int64_t workspace_bytes, int64_t B, int64_t H,
               int64_t Tq, int64_t T, int64_t d, int dtype, void* stream);

/* The argument validation of csa_decode alone (no HIP call). */
int csa_decode_check(const void* q, const void* k, const void* v, const void* k0, const void* v0,
                     const void* out, const float* lse, const void* workspace, int64_t workspace_bytes,
                     int64_t B, int64_t H, int64_t Tq, int64_t T, int64_t d, int dtype);

/* Workspace bytes csa_decode needs for these sizes, or -1 if the sizes are invalid. */
int64_t csa_decode_workspace_bytes(int64_t B, int64_t H, int64_t Tq, int64_t T, int64_t d);

/*
 * Bytes of the static device scratch that csa_decode_noalloc uses as its workspace: 64 MiB,
 * held on every GPU the library runs on until the process ends.
 */
#define CSA_DECODE_NOALLOC_SCRATCH_BYTES (64ll << 20)

/*
 * csa_decode_noalloc -- csa_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation, kernels and split plan, with the per-split partial results kept in a static
 * device array of CSA_DECODE_NOALLOC_SCRATCH_BYTES that the library holds on each GPU instead
 * of a caller-provided workspace.  The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine); its first call on a device looks up that device's copy of the
 * array once.
 *
 *   Arguments as csa_decode without workspace / workspace_bytes; the kernels run on the
 *   current device, so `stream` (NULL = the null stream) must belong to it.
 *
 * Returns CSA_OK; CSA_ERR_SCRATCH_TOO_SMALL (nothing launched) when
 * csa_decode_workspace_bytes(B, H, Tq, T, d) > CSA_DECODE_NOALLOC_SCRATCH_BYTES; CSA_ERR_HIP
 * when the scratch cannot be looked up, the stream belongs to another device, or a launch
 * fails; otherwise the codes of csa_decode.  Every call on one GPU shares that GPU's scratch:
 * calls that can overlap (different streams, or several host threads) race and must be
 * ordered by the caller.  The scratch needs no initialisation and keeps the last call's
 * partial results.
 */
int csa_decode_noalloc(const void* q, const void* k, const void* v, const void* k0, const void* v0,
                       void* out, float* lse, int64_t B, int64_t H, int64_t Tq, int64_t T, int64_t d,
                       int dtype, void* stream);

/* The argument validation of csa_decode_noalloc alone (no HIP call). */
int csa_decode_noalloc_check(const void* q, const void* k, const void* v, const void* k0, const void* v0,
                             const void* out, const float* lse, int64_t B, int64_t H, int64_t Tq, int64_t T,
                             int64_t d, int dtype);

/*
 * csa_backward -- gradients of the causal forward (eq. (10)-(11)) for training, the use the
 * pages' experiments make of the method (Experiments; trainable k_0, v_0 under Analysis of
 * the Result).  The pages print no backward; this is the plain derivative of eq. (10)-(11)
 * for the loss sum_t dO_t . o_t:
 *
 *     dS_{t,i} = P_{t,i} (dO_t . v_i - dO_t . o_t) + G_{(i-1,i)} - G_{(i,i+1)},
 *     G_{(i,i+1)} = (dO_t . v_i - dO_t . v_{i+1}) / Z_t * integral_0^1 s (1-s) e^{(1-s) a_i + s a_{i+1}} ds,
 *
 * with P_{t,i} = e^{a_{t,i} + b_{t,i}} / Z_t, edges only between consecutive positions 0..t,
 * and dq_t = sum_i dS_{t,i} k_i, dk_i = sum_t dS_{t,i} q_t, dv_i = sum_t P_{t,i} dO_t.
 *
 *   q, k, v    device, [B, H, T, d] `dtype`, 16-byte aligned (the forward's inputs).
 *   k0, v0     device, [B, H, d] `dtype`, 16-byte aligned, or NULL (zeros), as in csa_forward.
 *   o, lse     device: the forward's out [B, H, T, d] `dtype` and lse [B, H, T] float32 (4-byte
 *              aligned) for these inputs; P is recomputed from lse.
 *   dout       device, [B, H, T, d] `dtype`: dLoss/do.
 *   dq, dk, dv device, [B, H, T, d] `dtype` outputs (fully written).
 *   dk0, dv0   device, [B, H, d] `dtype` outputs (16-byte aligned), or NULL to skip; written even
 *              when k0 / v0 is NULL (the gradient at the zero vector).
 *   workspace  device, 16-byte aligned, at least csa_backward_workspace_bytes(B, H, T, d)
 *              bytes (row statistics and transposed copies of q and dout: about 4*B*H*T*d
 *              bytes), caller-owned scratch (no initialisation needed); calls sharing it must be
 *              ordered on one stream.  With at least csa_backward_workspace_bytes_kept(B, H, T,
 *              d, 1) bytes the call also keeps dS (bf16, about T*T bytes per head) so that it is
 *              computed once instead of twice: for as many heads at a time as the workspace
 *              holds (all B*H with csa_backward_workspace_bytes_fast bytes), the dk/dv and dq
 *              kernels running on one group of heads after another.  The results are bitwise
 *              identical whichever path and group size the workspace selects.
 *   d          16, 64 or 128.  dtype CSA_BF16 or CSA_F32.
 *   stream     hipStream_t or NULL.
 *
 * bf16 at d = 64, 128: the matrix-core kernels; gradients are accumulated in float32 and
 * rounded once to bf16, and the bf16 operands of the matrix products (P, dS) are rounded like
 * the forward's P.  float32 (any d) and bf16 at d = 16: VALU kernels in float32 throughout
 * (no rounding of P or dS; outputs rounded once to the dtype); the kept-dS workspace does not
 * apply to them.  Returns CSA_OK, or
 * CSA_ERR_INVALID_ARG (null required pointer, sizes, alignment, a short workspace, or any
 * output overlapping another output or an input), CSA_ERR_UNSUPPORTED, CSA_ERR_HIP; nothing is
 * launched on an error.  Up to five kernel launches on `stream`.
 */
int csa_backward(const void* q, const void* k, const void* v, const void* k0, const void* v0,
                 const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                 void* dk0, void* dv0, void* workspace, int64_t workspace_bytes, int64_t B, int64_t H,
                 int64_t T, int64_t d, int dtype, void* stream);

/* The argument validation of csa_backward alone (no HIP call). */
int csa_backward_check(const void* q, const void* k, const void* v, const void* k0, const void* v0,
                       const void* o, const float* lse, const void* dout, const void* dq,
                       const void* dk, const void* dv, const void* dk0, const void* dv0,
                       const void* workspace, int64_t workspace_bytes, int64_t B, int64_t H, int64_t T,
                       int64_t d, int dtype);

/* Workspace bytes csa_backward needs for these sizes, or -1 if the sizes are invalid. */
int64_t csa_backward_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t d);

/*
 * Workspace bytes with which csa_backward keeps dS between its kernels (the faster path;
 * grows as T^2: about B*H*T*T bytes), or -1 if the sizes are invalid or that size does not
 * fit in an int64.
 */
int64_t csa_backward_workspace_bytes_fast(int64_t B, int64_t H, int64_t T, int64_t d);

/*
 * Workspace bytes with which csa_backward keeps dS for `heads_per_group` heads at a time
 * (1 <= heads_per_group <= B*H; B*H gives csa_backward_workspace_bytes_fast): the bounded
 * form of the faster path for long sequences.  -1 if the sizes are invalid.
 */
int64_t csa_backward_workspace_bytes_kept(int64_t B, int64_t H, int64_t T, int64_t d, int64_t heads_per_group);

/* Static, NUL-terminated description of a return code. */
const char* csa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* LIBCSA_CSA_H */
