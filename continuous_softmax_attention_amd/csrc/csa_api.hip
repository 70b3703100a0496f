// C-ABI entry points of libcsa: csa_forward and its validation.
#include <hip/hip_runtime.h>

#include "attn16.hpp"
#include "attn_fwd.hpp"
#include "csa.h"
#include "validate.hpp"

namespace {

template <bool CSA>
int dispatch(const csa::FwdParams& p, int64_t d, int dtype, hipStream_t s) {
  hipError_t e = hipErrorInvalidValue;
  if (dtype == CSA_F32) {
    if (d == 16) e = csa::launch_attn<float, 16, CSA>(p, s);
    else if (d == 64) e = csa::launch_attn<float, 64, CSA>(p, s);
    else e = csa::launch_attn<float, 128, CSA>(p, s);
  } else {
    if (d == 16) e = csa::launch_attn16<16, CSA>(p, s);
    else if (d == 64) e = csa::launch_attn16<64, CSA>(p, s);
    else e = csa::launch_attn16<128, CSA>(p, s);
  }
  return e == hipSuccess ? CSA_OK : CSA_ERR_HIP;
}

}  // namespace

extern "C" int csa_forward_check(const void* q, const void* k, const void* v, const void* k0,
                                 const void* v0, const void* out, const float* lse, int64_t B,
                                 int64_t H, int64_t T, int64_t d, int dtype) {
  return csa::validate(q, k, v, k0, v0, out, lse, B, H, T, d, dtype, true);
}

extern "C" int csa_forward(const void* q, const void* k, const void* v, const void* k0,
                           const void* v0, void* out, float* lse, int64_t B, int64_t H, int64_t T,
                           int64_t d, int dtype, void* stream) {
  const int st = csa::validate(q, k, v, k0, v0, out, lse, B, H, T, d, dtype, true);
  if (st != CSA_OK) return st;
  csa::FwdParams p{q, k, v, k0, v0, out, lse, (int)B, (int)H, (int)T, 0};
  return dispatch<true>(p, d, dtype, (hipStream_t)stream);
}

extern "C" const char* csa_status_string(int status) { return csa::status_string(status); }
