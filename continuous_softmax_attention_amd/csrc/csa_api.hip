// C-ABI entry points of libcsa: csa_forward, csa_forward_first_order,
// csa_forward_half_interval, csa_decode, csa_decode_noalloc and csa_backward, each with its
// argument validation.
#include <hip/hip_runtime.h>

#include <mutex>

#include "attn16.hpp"
#include "bwd16.hpp"
#include "bwdv.hpp"
#include "dec16.hpp"
#include "decode.hpp"
#include "attn_fwd.hpp"
#include "csa.h"
#include "validate.hpp"

namespace {

int dispatch_exact(const csa::FwdParams& p, int64_t d, int dtype, hipStream_t s) {
  hipError_t e = hipErrorInvalidValue;
  if (dtype == CSA_F32) {
    if (d == 16) e = csa::launch_attn<float, 16, true>(p, s);
    else if (d == 64) e = csa::launch_attn<float, 64, true>(p, s);
    else e = csa::launch_attn<float, 128, true>(p, s);
  } else {
    if (d == 16) e = csa::launch_attn16<16, csa::kExact>(p, s);
    else if (d == 64) e = csa::launch_attn16<64, csa::kExact>(p, s);
    else e = csa::launch_attn16<128, csa::kExact>(p, s);
  }
  return e == hipSuccess ? CSA_OK : CSA_ERR_HIP;
}

int dispatch_first_order(const csa::FwdParams& p, int64_t d, hipStream_t s) {
  hipError_t e = hipErrorInvalidValue;
  if (d == 16) e = csa::launch_attn16<16, csa::kFirstOrder>(p, s);
  else if (d == 64) e = csa::launch_attn16<64, csa::kFirstOrder>(p, s);
  else e = csa::launch_attn16<128, csa::kFirstOrder>(p, s);
  return e == hipSuccess ? CSA_OK : CSA_ERR_HIP;
}

int validate_first_order(const void* q, const void* k, const void* v, const void* k0,
                         const void* v0, const void* out, const float* lse, int64_t B,
                         int64_t H, int64_t T, int64_t d, int dtype) {
  const int st = csa::validate(q, k, v, k0, v0, out, lse, B, H, T, d, dtype, true);
  if (st != CSA_OK) return st;
  return dtype == CSA_BF16 ? CSA_OK : CSA_ERR_UNSUPPORTED;  // bf16 kernel only
}

int validate_half(const void* q, const void* k, const void* v, const void* k0, const void* v0,
                  const void* out, const float* lse, int64_t B, int64_t H, int64_t T, int64_t d,
                  int dtype) {
  const int st = csa::validate(q, k, v, k0, v0, out, lse, B, H, T, d, dtype, true);
  if (st != CSA_OK) return st;
  return dtype == CSA_BF16 ? CSA_OK : CSA_ERR_UNSUPPORTED;  // bf16 kernel only
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
  return dispatch_exact(p, d, dtype, (hipStream_t)stream);
}

extern "C" int csa_forward_first_order_check(const void* q, const void* k, const void* v,
                                             const void* k0, const void* v0, const void* out,
                                             const float* lse, int64_t B, int64_t H, int64_t T,
                                             int64_t d, int dtype) {
  return validate_first_order(q, k, v, k0, v0, out, lse, B, H, T, d, dtype);
}

extern "C" int csa_forward_first_order(const void* q, const void* k, const void* v,
                                       const void* k0, const void* v0, void* out, float* lse,
                                       int64_t B, int64_t H, int64_t T, int64_t d, int dtype,
                                       void* stream) {
  const int st = validate_first_order(q, k, v, k0, v0, out, lse, B, H, T, d, dtype);
  if (st != CSA_OK) return st;
  csa::FwdParams p{q, k, v, k0, v0, out, lse, (int)B, (int)H, (int)T, 0};
  return dispatch_first_order(p, d, (hipStream_t)stream);
}

extern "C" int csa_forward_half_interval_check(const void* q, const void* k, const void* v,
                                               const void* k0, const void* v0, const void* out,
                                               const float* lse, int64_t B, int64_t H, int64_t T,
                                               int64_t d, int dtype) {
  return validate_half(q, k, v, k0, v0, out, lse, B, H, T, d, dtype);
}

extern "C" int csa_forward_half_interval(const void* q, const void* k, const void* v,
                                         const void* k0, const void* v0, void* out, float* lse,
                                         int64_t B, int64_t H, int64_t T, int64_t d, int dtype,
                                         void* stream) {
  const int st = validate_half(q, k, v, k0, v0, out, lse, B, H, T, d, dtype);
  if (st != CSA_OK) return st;
  csa::FwdParams p{q, k, v, k0, v0, out, lse, (int)B, (int)H, (int)T, 0};
  hipError_t e;
  if (d == 16) e = csa::launch_attn16<16, csa::kHalf>(p, (hipStream_t)stream);
  else if (d == 64) e = csa::launch_attn16<64, csa::kHalf>(p, (hipStream_t)stream);
  else e = csa::launch_attn16<128, csa::kHalf>(p, (hipStream_t)stream);
  return e == hipSuccess ? CSA_OK : CSA_ERR_HIP;
}

extern "C" const char* csa_status_string(int status) { return csa::status_string(status); }

extern "C" int64_t csa_decode_workspace_bytes(int64_t B, int64_t H, int64_t Tq, int64_t T, int64_t d) {
  return csa::decode_workspace_bytes(B, H, Tq, T, d);
}

extern "C" int csa_decode_check(const void* q, const void* k, const void* v, const void* k0, const void* v0,
                                const void* out, const float* lse, const void* workspace,
                                int64_t workspace_bytes, int64_t B, int64_t H, int64_t Tq, int64_t T,
                                int64_t d, int dtype) {
  return csa::validate_decode(q, k, v, k0, v0, out, lse, workspace, workspace_bytes, B, H, Tq, T, d, dtype);
}

namespace {

int launch_decode_any(csa::DecParams& p, int64_t d, int dtype, hipStream_t s) {
  hipError_t e = hipErrorInvalidValue;
  if (dtype == CSA_F32) {
    if (d == 16) e = csa::launch_decode<float, 16>(p, s);
    else if (d == 64) e = csa::launch_decode<float, 64>(p, s);
    else e = csa::launch_decode<float, 128>(p, s);
  } else {
    // d = 64, 128: both contractions on the matrix cores (dec16.hpp)
    if (d == 16) e = csa::launch_decode<csa::bf16, 16>(p, s);
    else if (d == 64) e = csa::launch_decode16<64>(p, s);
    else e = csa::launch_decode16<128>(p, s);
  }
  return e == hipSuccess ? CSA_OK : CSA_ERR_HIP;
}

}  // namespace

extern "C" int csa_decode(const void* q, const void* k, const void* v, const void* k0, const void* v0,
                          void* out, float* lse, void* workspace, int64_t workspace_bytes, int64_t B,
                          int64_t H, int64_t Tq, int64_t T, int64_t d, int dtype, void* stream) {
  const int st =
      csa::validate_decode(q, k, v, k0, v0, out, lse, workspace, workspace_bytes, B, H, Tq, T, d, dtype);
  if (st != CSA_OK) return st;
  csa::DecParams p{q, k, v, k0, v0, out, lse, (float*)workspace,
                   (int)(B * H), (int)Tq, (int)T, 0, 0};  // split plan chosen at launch
  return launch_decode_any(p, d, dtype, (hipStream_t)stream);
}

// ---- csa_decode_noalloc: the decode workspace in a static device array.  In host code the
// array's name stands for a host-side shadow, not for device memory: its device address (one
// per GPU) is looked up once per device with hipGetSymbolAddress and only that address is
// handed to kernels.
static __device__ __align__(256) char scratch[CSA_DECODE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};  // device address of `scratch` on each device, once looked up

// Device address of the scratch on the current device (looked up on the first call there).
int scratch_on_current_device(void** out, hipStream_t stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CSA_ERR_HIP;
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess || sdev != dev) return CSA_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();  // the failure is reported by the return code
      return CSA_ERR_HIP;
    }
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return CSA_OK;
}

}  // namespace

extern "C" int csa_decode_noalloc_check(const void* q, const void* k, const void* v, const void* k0,
                                        const void* v0, const void* out, const float* lse, int64_t B, int64_t H,
                                        int64_t Tq, int64_t T, int64_t d, int dtype) {
  return csa::validate_decode_noalloc(q, k, v, k0, v0, out, lse, CSA_DECODE_NOALLOC_SCRATCH_BYTES, B, H, Tq, T, d,
                                      dtype);
}

extern "C" int csa_decode_noalloc(const void* q, const void* k, const void* v, const void* k0, const void* v0,
                                  void* out, float* lse, int64_t B, int64_t H, int64_t Tq, int64_t T, int64_t d,
                                  int dtype, void* stream) {
  int st = csa::validate_decode_noalloc(q, k, v, k0, v0, out, lse, CSA_DECODE_NOALLOC_SCRATCH_BYTES, B, H, Tq, T,
                                        d, dtype);
  if (st != CSA_OK) return st;
  void* ws = nullptr;
  st = scratch_on_current_device(&ws, (hipStream_t)stream);
  if (st != CSA_OK) return st;
  csa::DecParams p{q, k, v, k0, v0, out, lse, (float*)ws, (int)(B * H), (int)Tq, (int)T, 0, 0};
  return launch_decode_any(p, d, dtype, (hipStream_t)stream);
}

extern "C" int64_t csa_backward_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t d) {
  return csa::backward_workspace_bytes(B, H, T, d);
}

extern "C" int64_t csa_backward_workspace_bytes_fast(int64_t B, int64_t H, int64_t T, int64_t d) {
  return csa::backward_workspace_bytes_fast(B, H, T, d);
}

extern "C" int64_t csa_backward_workspace_bytes_kept(int64_t B, int64_t H, int64_t T, int64_t d,
                                                     int64_t heads_per_group) {
  return csa::backward_workspace_bytes_kept(B, H, T, d, heads_per_group);
}

extern "C" int csa_backward_check(const void* q, const void* k, const void* v, const void* k0, const void* v0,
                                  const void* o, const float* lse, const void* dout, const void* dq,
                                  const void* dk, const void* dv, const void* dk0, const void* dv0,
                                  const void* workspace, int64_t workspace_bytes, int64_t B, int64_t H,
                                  int64_t T, int64_t d, int dtype) {
  return csa::validate_backward(q, k, v, k0, v0, o, lse, dout, dq, dk, dv, dk0, dv0, workspace,
                                workspace_bytes, B, H, T, d, dtype);
}

extern "C" int csa_backward(const void* q, const void* k, const void* v, const void* k0, const void* v0,
                            const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                            void* dk0, void* dv0, void* workspace, int64_t workspace_bytes, int64_t B,
                            int64_t H, int64_t T, int64_t d, int dtype, void* stream) {
  const int st = csa::validate_backward(q, k, v, k0, v0, o, lse, dout, dq, dk, dv, dk0, dv0, workspace,
                                        workspace_bytes, B, H, T, d, dtype);
  if (st != CSA_OK) return st;
  // dS kept for as many heads at a time as the workspace holds (the kernels run on groups of
  // that many heads), else recomputed
  const int64_t kept = csa::backward_kept_heads_for(B, H, T, d, dtype, workspace_bytes);
  char* ds = kept > 0 ? (char*)workspace + csa::backward_ds_offset(B, H, T, d) : nullptr;
  csa::BwdParams p{q, k, v, k0, v0, o, lse, dout, dq, dk, dv, dk0, dv0, (char*)workspace,
                   (int)B, (int)H, (int)T, ds, csa::backward_ds_tiles_per_head(T), 0, (int)kept};
  const hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (dtype == CSA_F32) {  // float32: the VALU kernels (bwdv.hpp)
    e = d == 16 ? csa::launch_backward_valu<float, 16>(p, s)
        : d == 64 ? csa::launch_backward_valu<float, 64>(p, s)
                  : csa::launch_backward_valu<float, 128>(p, s);
  } else if (d == 16) {
    e = csa::launch_backward_valu<csa::bf16, 16>(p, s);
  } else {
    e = d == 64 ? csa::launch_backward<64>(p, s) : csa::launch_backward<128>(p, s);
  }
  return e == hipSuccess ? CSA_OK : CSA_ERR_HIP;
}
