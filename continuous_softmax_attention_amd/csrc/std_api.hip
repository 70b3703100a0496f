// C-ABI entry points of libcsa_bench: standard causal attention on the CSA tiling, and the
// SIMD micro-benchmarks the measurements are compared with.
#include <hip/hip_runtime.h>

#include "attn16.hpp"
#include "attn_fwd.hpp"
#include "csa_bench.h"
#include "probes.hpp"
#include "validate.hpp"

extern "C" int std_fwd_check(const void* q, const void* k, const void* v, const void* out,
                             const float* lse, int64_t B, int64_t H, int64_t T, int64_t d,
                             int dtype) {
  return csa::validate(q, k, v, nullptr, nullptr, out, lse, B, H, T, d, dtype, false);
}

extern "C" int std_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                       int64_t B, int64_t H, int64_t T, int64_t d, int dtype, void* stream) {
  const int st = csa::validate(q, k, v, nullptr, nullptr, out, lse, B, H, T, d, dtype, false);
  if (st != CSA_OK) return st;
  csa::FwdParams p{q, k, v, nullptr, nullptr, out, lse, (int)B, (int)H, (int)T, 0};
  hipError_t e = hipErrorInvalidValue;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == CSA_F32) {
    if (d == 16) e = csa::launch_attn<float, 16, false>(p, s);
    else if (d == 64) e = csa::launch_attn<float, 64, false>(p, s);
    else e = csa::launch_attn<float, 128, false>(p, s);
  } else {
    if (d == 16) e = csa::launch_attn16<16, csa::kSoftmax>(p, s);
    else if (d == 64) e = csa::launch_attn16<64, csa::kSoftmax>(p, s);
    else e = csa::launch_attn16<128, csa::kSoftmax>(p, s);
  }
  return e == hipSuccess ? CSA_OK : CSA_ERR_HIP;
}

extern "C" int csa_probe(int kind, int64_t waves, int64_t iters, float* sink, uint64_t* cycles, void* stream) {
  if (kind < 0 || kind >= csa::kProbeKinds || waves < 1 || iters < 1 || !sink || !cycles) return CSA_ERR_INVALID_ARG;
  if (waves > ((int64_t)1 << 24) || iters > ((int64_t)1 << 30)) return CSA_ERR_INVALID_ARG;
  const hipError_t e = csa::launch_probe(kind, waves, (int)iters, sink, (unsigned long long*)cycles, (hipStream_t)stream);
  return e == hipSuccess ? CSA_OK : CSA_ERR_HIP;
}
