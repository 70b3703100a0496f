// Micro-benchmarks of the gfx950 SIMD, for measurement only (libcsa_bench): the MFMA-only
// ceiling against which the forward kernels are compared, the issue cost of the VALU
// instructions their correction weights are made of, and whether MFMA and VALU work of the
// same SIMD overlap.  Each kernel runs a fixed instruction mix for `iters` iterations in
// every wave; every wave reads the shader clock (s_memtime) around its loop and the largest
// count is kept (the waves of a SIMD do not all run to the end together: the oldest may finish
// well before the launch does), so that the host can turn event-timed durations into cycles.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace csa {

enum : int { kProbeMfma = 0, kProbeFma = 1, kProbeExp = 2, kProbeRcp = 3, kProbeMix = 4, kProbeKinds = 5 };
constexpr int kProbeThreads = 256;  // four waves per work-group

namespace probe {
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// c += a b on a 16x16x32 bf16 MFMA with the accumulator in the same registers before and
// after: the builtin in a loop got a different destination than its source for some chains
// and a dozen accumulator moves per iteration, which would spoil an MFMA-only measurement.
// The chains are interleaved four deep, so each reads an accumulator written three MFMAs ago.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void mfma_acc(f32x4& c, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
#pragma clang diagnostic pop
}  // namespace probe

// kProbeMfma: 4 independent v_mfma_f32_16x16x32_bf16 chains (16384 FLOP each per iteration).
// kProbeFma: 8 independent fp32 FMA chains.  kProbeExp / kProbeRcp: 8 independent v_exp_f32 /
// v_rcp_f32 chains (exp2 of the negated value and the reciprocal keep every chain bounded).
// kProbeMix: the MFMAs of kProbeMfma and two rounds of the FMAs of kProbeFma per iteration.
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
  float x[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) x[k] = 0.5f + 0.01f * (float)((lane + k) & 15);
  const float m = 0.999f + 1e-6f * (float)lane, s = 1e-3f * (float)(lane & 7);
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int i = 0; i < iters; ++i) {
    if constexpr (KIND == kProbeMfma || KIND == kProbeMix) {
      probe::mfma_acc(c0, a, b);
      probe::mfma_acc(c1, a, b1);
      probe::mfma_acc(c2, a, b2);
      probe::mfma_acc(c3, a, b3);
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
    default: hipLaunchKernelGGL((probe_kernel<kProbeMix>), grid, block, 0, stream, iters, sink, cycles); break;
  }
  return hipGetLastError();
}

}  // namespace csa
