// Micro-benchmarks of the gfx950 SIMD, for measurement only (libcsa_bench): the MFMA-only
// ceiling against which the forward kernels are compared, the issue cost of the VALU
// instructions their correction weights are made of, whether MFMA and VALU work of the
// same SIMD overlap, and the forward's per-key weight arithmetic beside 16x16x32 or 32x32x16
// MFMAs at the forward's ratio (the choice of tiling).  Each kernel runs a fixed instruction
// mix for `iters` iterations in every wave; every wave reads the shader clock (s_memtime)
// around its loop and the largest count is kept (the waves of a SIMD do not all run to the
// end together: the oldest may finish well before the launch does), so that the host can turn
// event-timed durations into cycles.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "attn16.hpp"

namespace csa {

enum : int {
  kProbeMfma = 0,
  kProbeFma = 1,
  kProbeExp = 2,
  kProbeRcp = 3,
  kProbeMix = 4,
  kProbeMfma32 = 5,
  kProbeWeights = 6,
  kProbeWeightsMfma = 7,
  kProbeWeightsMfma32 = 8,
  kProbeLogWeights = 9,
  kProbeFmaExp = 10,
  kProbeFmaRcp = 11,
  kProbeTableWeights = 12,
  kProbeKinds = 13
};
constexpr int kProbeThreads = 256;  // four waves per work-group

namespace probe {
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// c += a b on a 16x16x32 bf16 MFMA with the accumulator in the same registers before and
// after: the builtin in a loop got a different destination than its source for some chains
// and a dozen accumulator moves per iteration, which would spoil an MFMA-only measurement.
// The chains are interleaved four deep, so each reads an accumulator written three MFMAs ago.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void mfma_acc(f32x4& c, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma32_acc(f32x16& c, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
#pragma clang diagnostic pop
}  // namespace probe

// Log-domain evaluation of the correction of eq. (10), as eq. (13) writes it (b = log of the
// sum of the two phi_2 terms): for one edge with logit difference x = a_r - a_l (natural units)
// the logs of both of its phi_2 terms, lR = log phi_2(x) (to the left position) and
// lL = log phi_2(-x) (to the right one), without overflow: with t = |x| and e = exp(-t),
//   the side whose difference is negative:  log(e - 1 + t) - 2 log t,
//   the other side:                         t + log(1 - e (1 + t)) - 2 log t,
// and below t < 0.25 the series -ln 2 +- x/3 + x^2/36.  Four transcendentals per edge; the
// weight of a position then takes log-sum-exp of its two logs (two more) and one exp.
__device__ __forceinline__ void log_phi2_edge(float x, float& lR, float& lL) {
  const float t = __builtin_fabsf(x);
  const float e = __builtin_amdgcn_exp2f(-t * kLog2e);
  const float lt2 = 2.0f * kLn2 * __builtin_amdgcn_logf(t);
  const float neg_side = __builtin_fmaf(kLn2, __builtin_amdgcn_logf(e - 1.0f + t), -lt2);
  const float pos_side = t + __builtin_fmaf(kLn2, __builtin_amdgcn_logf(__builtin_fmaf(-e, 1.0f + t, 1.0f)), -lt2);
  const float x3 = x * (1.0f / 3.0f), q = __builtin_fmaf(x, x * (1.0f / 36.0f), -kLn2);
  const bool small = t < 0.25f, pos = x >= 0.0f;
  lR = small ? q + x3 : (pos ? pos_side : neg_side);
  lL = small ? q - x3 : (pos ? neg_side : pos_side);
}

// kProbeMfma: 4 independent// kProbeMfma: 4 independent v_mfma_f32_16x16x32_bf16 chains (16384 FLOP each per iteration).
// kProbeFma: 8 independent fp32 FMA chains.  kProbeExp / kProbeRcp: 8 independent v_exp_f32 /
// v_rcp_f32 chains (exp2 of the negated value and the reciprocal keep every chain bounded).
// kProbeMix: the MFMAs of kProbeMfma and two rounds of the FMAs of kProbeFma per iteration.
// kProbeMfma32: 2 independent v_mfma_f32_32x32x16_bf16 chains (32768 FLOP each), the FLOP of
// kProbeMfma.  kProbeWeights: the forward's arithmetic for two keys per iteration (logit to
// alpha, exp2, neighbour difference, reciprocal, edge_yu with its Taylor select) on two
// interleaved chains of logits that wander in [-3, 3).  kProbeWeightsMfma / kProbeWeightsMfma32:
// kProbeWeights with the MFMAs of kProbeMfma / kProbeMfma32 -- two 16x16x32 MFMAs per key and
// lane, the forward's ratio (32 per 16 x 64 wave-tile).
// kProbeLogWeights: the weights of kProbeWeights by the log-domain route of eq. (13)
// (log_phi2_edge, log-sum-exp of a position's two logs, exp of logit + b), two keys per
// iteration on the same chains.  kProbeFmaExp / kProbeFmaRcp: the 8 FMA chains of kProbeFma
// with 2 v_exp_f32 / v_rcp_f32 chains beside them (does a transcendental cost issue slots of
// the plain VALU?).  kProbeTableWeights: an edge without the reciprocal -- its two terms
// interpolated in a 1024-entry LDS table indexed by the difference (index, clamp, fraction,
// one ds_read_b128, two fmas) and scaled by the larger end value -- two keys per iteration,
// to price that alternative against kProbeWeights (the table holds placeholder values).
template <int KIND>
__global__ void __launch_bounds__(kProbeThreads) probe_kernel(int iters, float* sink, unsigned long long* cycles) {
  using probe::bf16x8;
  using probe::f32x4;
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {  // small exact values that depend on the lane (not foldable)
    a[e] = (__bf16)(float)((lane + e) & 3);
    b[e] = (__bf16)(float)((lane * 3 + e) & 3);
  }
  bf16x8 b1 = b, b2 = b, b3 = b;  // one operand per chain, so no two chains look alike
  b1[0] = (__bf16)1.0f;
  b2[1] = (__bf16)1.0f;
  b3[2] = (__bf16)1.0f;
  f32x4 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  f32x16 e0 = {}, e1 = {};
  constexpr bool M16 = KIND == kProbeMfma || KIND == kProbeMix || KIND == kProbeWeightsMfma;
  constexpr bool M32 = KIND == kProbeMfma32 || KIND == kProbeWeightsMfma32;
  constexpr bool WGT = KIND == kProbeWeights || KIND == kProbeWeightsMfma || KIND == kProbeWeightsMfma32;
  float sv[2], ap[2], pc[2], lp[2], wsum[2];  // weight chains: logit, alpha, p, left term, sum
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    sv[k] = 0.3f * (float)((lane + k) & 7);
    ap[k] = -1.0f;
    pc[k] = 0.5f;
    lp[k] = 0.0f;
    wsum[k] = 0.0f;
  }
  float x[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) x[k] = 0.5f + 0.01f * (float)((lane + k) & 15);
  const float m = 0.999f + 1e-6f * (float)lane, s = 1e-3f * (float)(lane & 7);
  constexpr bool TAB = KIND == kProbeTableWeights;
  __shared__ f32x4 table[TAB ? 1024 : 1];
  if constexpr (TAB) {
    for (int r = threadIdx.x; r < 1024; r += kProbeThreads)
      table[r] = f32x4{0.24f + 1e-4f * (float)r, 1e-3f, 0.12f + 1e-4f * (float)r, -1e-3f};
    __syncthreads();
  }
  float lLp[2] = {-kLn2, -kLn2};  // log-domain chains: left log of the current position
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int i = 0; i < iters; ++i) {
    if constexpr (M16) {
      probe::mfma_acc(c0, a, b);
      probe::mfma_acc(c1, a, b1);
      probe::mfma_acc(c2, a, b2);
      probe::mfma_acc(c3, a, b3);
    }
    if constexpr (M32) {
      probe::mfma32_acc(e0, a, b);
      probe::mfma32_acc(e1, a, b1);
    }
    if constexpr (WGT) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        float v = __builtin_fmaf(sv[k], m, 0.37f);
        sv[k] = v >= 3.0f ? v - 6.0f : v;
        const float al = __builtin_fmaf(sv[k], kLog2e, -2.0f);
        const float pn = __builtin_amdgcn_exp2f(al);
        const float y = al - ap[k];
        float w;
        edge_yu(pc[k], pn, y, __builtin_amdgcn_rcpf(y), lp[k], w, lp[k]);
        wsum[k] += w;
        pc[k] = pn;
        ap[k] = al;
      }
    }
    if constexpr (KIND == kProbeLogWeights) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        float v = __builtin_fmaf(sv[k], m, 0.37f);
        const float a_prev = ap[k];  // logit of the previous position (natural units here)
        sv[k] = v >= 3.0f ? v - 6.0f : v;
        float lR, lL;
        log_phi2_edge(sv[k] - a_prev, lR, lL);
        // the previous position is finished: b = log(e^{lL_prev} + e^{lR})
        const float hi = fmaxf(lLp[k], lR), lo = fminf(lLp[k], lR);
        const float b = __builtin_fmaf(kLn2, __builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f((lo - hi) * kLog2e)), hi);
        wsum[k] += __builtin_amdgcn_exp2f(__builtin_fmaf(a_prev + b, kLog2e, -2.0f));
        lLp[k] = lL;
        ap[k] = sv[k];
      }
    }
    if constexpr (TAB) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        float v = __builtin_fmaf(sv[k], m, 0.37f);
        sv[k] = v >= 3.0f ? v - 6.0f : v;
        const float al = __builtin_fmaf(sv[k], kLog2e, -2.0f);
        const float pn = __builtin_amdgcn_exp2f(al);
        const float y = al - ap[k];
        const float tt = __builtin_amdgcn_fmed3f(__builtin_fmaf(y, 4.0f, 512.0f), 0.0f, 1022.0f);
        const int ix = (int)tt;
        const float fr = __builtin_amdgcn_fractf(tt);
        const f32x4 e = table[ix];
        const float pmax = fmaxf(pc[k], pn);
        wsum[k] += __builtin_fmaf(pmax, __builtin_fmaf(fr, e[1], e[0]), lp[k]);
        lp[k] = pmax * __builtin_fmaf(fr, e[3], e[2]);
        pc[k] = pn;
        ap[k] = al;
      }
    }
    if constexpr (KIND == kProbeFmaExp || KIND == kProbeFmaRcp) {
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = __builtin_fmaf(x[k], m, s);
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        if constexpr (KIND == kProbeFmaExp) lp[k] = __builtin_amdgcn_exp2f(-lp[k] - 0.5f);
        else lp[k] = __builtin_amdgcn_rcpf(lp[k] + 1.5f);
      }
    }
    if constexpr (KIND == kProbeFma || KIND == kProbeMix) {
#pragma unroll
      for (int r = 0; r < (KIND == kProbeMix ? 2 : 1); ++r)
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = __builtin_fmaf(x[k], m, s);
    }
    if constexpr (KIND == kProbeExp) {
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = __builtin_amdgcn_exp2f(-x[k]);
    }
    if constexpr (KIND == kProbeRcp) {
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = __builtin_amdgcn_rcpf(x[k]);
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  float acc = 0.0f;
  const f32x4 csum = c0 + c1 + c2 + c3;
  acc += csum[0] + csum[1] + csum[2] + csum[3];
  const f32x16 esum = e0 + e1;
#pragma unroll
  for (int k = 0; k < 16; ++k) acc += esum[k];
  acc += wsum[0] + wsum[1] + lp[0] + lp[1];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc += x[k];
  // one value per work-group (thread 0), so that the loop's results are used
  if (threadIdx.x == 0) sink[blockIdx.x] = acc;
  if ((threadIdx.x & 63) == 0) atomicMax(cycles, t1 - t0);  // vector atomic; the host zeroes it
}

inline hipError_t launch_probe(int kind, int64_t waves, int iters, float* sink, unsigned long long* cycles,
                               hipStream_t stream) {
  const dim3 grid((unsigned)((waves * 64 + kProbeThreads - 1) / kProbeThreads)), block(kProbeThreads);
  switch (kind) {
    case kProbeMfma: hipLaunchKernelGGL((probe_kernel<kProbeMfma>), grid, block, 0, stream, iters, sink, cycles); break;
    case kProbeFma: hipLaunchKernelGGL((probe_kernel<kProbeFma>), grid, block, 0, stream, iters, sink, cycles); break;
    case kProbeExp: hipLaunchKernelGGL((probe_kernel<kProbeExp>), grid, block, 0, stream, iters, sink, cycles); break;
    case kProbeRcp: hipLaunchKernelGGL((probe_kernel<kProbeRcp>), grid, block, 0, stream, iters, sink, cycles); break;
    case kProbeMix: hipLaunchKernelGGL((probe_kernel<kProbeMix>), grid, block, 0, stream, iters, sink, cycles); break;
    case kProbeMfma32: hipLaunchKernelGGL((probe_kernel<kProbeMfma32>), grid, block, 0, stream, iters, sink, cycles); break;
    case kProbeWeights: hipLaunchKernelGGL((probe_kernel<kProbeWeights>), grid, block, 0, stream, iters, sink, cycles); break;
    case kProbeWeightsMfma:
      hipLaunchKernelGGL((probe_kernel<kProbeWeightsMfma>), grid, block, 0, stream, iters, sink, cycles);
      break;
    case kProbeWeightsMfma32:
      hipLaunchKernelGGL((probe_kernel<kProbeWeightsMfma32>), grid, block, 0, stream, iters, sink, cycles);
      break;
    case kProbeLogWeights:
      hipLaunchKernelGGL((probe_kernel<kProbeLogWeights>), grid, block, 0, stream, iters, sink, cycles);
      break;
    case kProbeFmaExp: hipLaunchKernelGGL((probe_kernel<kProbeFmaExp>), grid, block, 0, stream, iters, sink, cycles); break;
    case kProbeFmaRcp: hipLaunchKernelGGL((probe_kernel<kProbeFmaRcp>), grid, block, 0, stream, iters, sink, cycles); break;
    default:
      hipLaunchKernelGGL((probe_kernel<kProbeTableWeights>), grid, block, 0, stream, iters, sink, cycles);
      break;
  }
  return hipGetLastError();
}

}  // namespace csa
