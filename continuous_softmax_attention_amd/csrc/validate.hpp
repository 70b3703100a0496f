// Host-side argument validation shared by csa_forward and std_fwd.
// Pure C++: no HIP call, no memory access.
#pragma once

#include <cstdint>

#include "csa.h"

namespace csa {

struct Span {
  uintptr_t lo = 0, hi = 0;  // [lo, hi)
  bool valid() const { return hi > lo; }
};

inline bool overlaps(Span a, Span b) { return a.valid() && b.valid() && a.lo < b.hi && b.lo < a.hi; }

inline Span span_of(const void* p, int64_t bytes) {
  Span s;
  if (p) {
    s.lo = reinterpret_cast<uintptr_t>(p);
    s.hi = s.lo + static_cast<uintptr_t>(bytes);
  }
  return s;
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Checks shared by both entry points.  `with_sink` adds the k0/v0 buffers.
inline int validate(const void* q, const void* k, const void* v, const void* k0, const void* v0,
                    const void* out, const float* lse, int64_t B, int64_t H, int64_t T, int64_t d,
                    int dtype, bool with_sink) {
  if (dtype != CSA_F32 && dtype != CSA_BF16) return CSA_ERR_UNSUPPORTED;
  if (d != 16 && d != 64 && d != 128) return CSA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !out) return CSA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || T < 1) return CSA_ERR_INVALID_ARG;
  // size limits: grid of ceil(T/128) * B * H work-groups; 32-bit row indices
  const int64_t kMax32 = (int64_t(1) << 31) - 1;
  if (T > kMax32 / 2 || B > kMax32 || H > kMax32) return CSA_ERR_INVALID_ARG;
  if (B * H > kMax32 / ((T + 127) / 128)) return CSA_ERR_INVALID_ARG;
  const int64_t esize = dtype == CSA_F32 ? 4 : 2;
  if (B * H > INT64_MAX / (T * d * esize)) return CSA_ERR_INVALID_ARG;
  for (const void* p : {q, k, v, out})
    if (!aligned(p, 16)) return CSA_ERR_INVALID_ARG;
  if (with_sink) {
    if (k0 && !aligned(k0, 16)) return CSA_ERR_INVALID_ARG;
    if (v0 && !aligned(v0, 16)) return CSA_ERR_INVALID_ARG;
  }
  if (lse && !aligned(lse, 4)) return CSA_ERR_INVALID_ARG;
  const int64_t big = B * H * T * d * esize;
  const Span so = span_of(out, big), sl = span_of(lse, B * H * T * 4);
  Span ins[5] = {span_of(q, big), span_of(k, big), span_of(v, big), {}, {}};
  if (with_sink) {
    ins[3] = span_of(k0, B * H * d * esize);
    ins[4] = span_of(v0, B * H * d * esize);
  }
  for (const Span& s : ins)
    if (overlaps(so, s) || overlaps(sl, s)) return CSA_ERR_INVALID_ARG;
  if (overlaps(so, sl)) return CSA_ERR_INVALID_ARG;
  return CSA_OK;
}

// Checks of the decode entry points (csa_forward's rules for the shared arguments, plus
// 1 <= Tq <= 8, Tq <= T, and a workspace large enough and disjoint from everything).
inline int64_t decode_workspace_bytes(int64_t B, int64_t H, int64_t Tq, int64_t T, int64_t d) {
  if (B < 1 || H < 1 || T < 1 || Tq < 1 || Tq > 8 || Tq > T) return -1;
  if (d != 16 && d != 64 && d != 128) return -1;
  const int64_t kMax32 = (int64_t(1) << 31) - 1;
  if (T > kMax32 / 2 || B > kMax32 || H > kMax32 || B * H > kMax32) return -1;
  const int64_t nsplit = (T + 1 + 63) / 64;  // at most one split per 64 positions
  if (B * H > kMax32 / nsplit) return -1;
  return B * H * nsplit * Tq * (d + 2) * 4;
}

// Everything validate_decode checks except the workspace; with ws == nullptr the workspace
// is one the library holds (csa_decode_noalloc), which no caller buffer can overlap.
inline int validate_decode_core(const void* q, const void* k, const void* v, const void* k0, const void* v0,
                                const void* out, const float* lse, const void* ws, int64_t ws_need, int64_t B,
                                int64_t H, int64_t Tq, int64_t T, int64_t d, int dtype) {
  const int64_t esize = dtype == CSA_F32 ? 4 : 2;
  if (B * H > INT64_MAX / (T * d * esize)) return CSA_ERR_INVALID_ARG;
  for (const void* p : {q, k, v, out})
    if (!aligned(p, 16)) return CSA_ERR_INVALID_ARG;
  if (ws && !aligned(ws, 16)) return CSA_ERR_INVALID_ARG;
  if (k0 && !aligned(k0, 16)) return CSA_ERR_INVALID_ARG;
  if (v0 && !aligned(v0, 16)) return CSA_ERR_INVALID_ARG;
  if (lse && !aligned(lse, 4)) return CSA_ERR_INVALID_ARG;
  const int64_t cache = B * H * T * d * esize, qbytes = B * H * Tq * d * esize;
  const Span so = span_of(out, qbytes), sl = span_of(lse, B * H * Tq * 4), sw = span_of(ws, ws_need);
  const Span ins[5] = {span_of(q, qbytes), span_of(k, cache), span_of(v, cache),
                       span_of(k0, B * H * d * esize), span_of(v0, B * H * d * esize)};
  for (const Span& s : ins)
    if (overlaps(so, s) || overlaps(sl, s) || overlaps(sw, s)) return CSA_ERR_INVALID_ARG;
  if (overlaps(so, sl) || overlaps(so, sw) || overlaps(sl, sw)) return CSA_ERR_INVALID_ARG;
  return CSA_OK;
}

inline int validate_decode(const void* q, const void* k, const void* v, const void* k0, const void* v0,
                           const void* out, const float* lse, const void* ws, int64_t ws_bytes, int64_t B,
                           int64_t H, int64_t Tq, int64_t T, int64_t d, int dtype) {
  if (dtype != CSA_F32 && dtype != CSA_BF16) return CSA_ERR_UNSUPPORTED;
  if (d != 16 && d != 64 && d != 128) return CSA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !out || !ws) return CSA_ERR_INVALID_ARG;
  const int64_t need = decode_workspace_bytes(B, H, Tq, T, d);
  if (need < 0 || ws_bytes < need) return CSA_ERR_INVALID_ARG;
  return validate_decode_core(q, k, v, k0, v0, out, lse, ws, need, B, H, Tq, T, d, dtype);
}

// csa_decode_noalloc: csa_decode's checks with the library's static scratch of `scratch_bytes`
// as the workspace; sizes whose workspace exceeds it return CSA_ERR_SCRATCH_TOO_SMALL.
inline int validate_decode_noalloc(const void* q, const void* k, const void* v, const void* k0, const void* v0,
                                   const void* out, const float* lse, int64_t scratch_bytes, int64_t B, int64_t H,
                                   int64_t Tq, int64_t T, int64_t d, int dtype) {
  if (dtype != CSA_F32 && dtype != CSA_BF16) return CSA_ERR_UNSUPPORTED;
  if (d != 16 && d != 64 && d != 128) return CSA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !out) return CSA_ERR_INVALID_ARG;
  const int64_t need = decode_workspace_bytes(B, H, Tq, T, d);
  if (need < 0) return CSA_ERR_INVALID_ARG;
  if (need > scratch_bytes) return CSA_ERR_SCRATCH_TOO_SMALL;
  return validate_decode_core(q, k, v, k0, v0, out, lse, nullptr, 0, B, H, Tq, T, d, dtype);
}

// Checks of the backward entry points: bf16 only, d in {64, 128}; q, k, v, o, dO, dq, dk,
// dv [B, H, T, d] and the workspace required; k0, v0, dk0, dv0 optional; no output may
// overlap another output or any input.
inline int64_t backward_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t d) {
  if (B < 1 || H < 1 || T < 1) return -1;
  if (d != 16 && d != 64 && d != 128) return -1;
  const int64_t kMax32 = (int64_t(1) << 31) - 1;
  if (T > kMax32 / 2 || B > kMax32 || H > kMax32 || B * H > kMax32 / T) return -1;  // B*H*T rows < 2^31
  const int64_t tp = (T + 127) / 128 * 128;
  const int64_t head = (512 + 16 * B * H * T + B * H * 16 * 2 * 128 * 4 + 255) / 256 * 256;
  return head + 2 * B * H * d * tp * 2;  // see bwd16.hpp for the layout
}

// Optional last region of the backward workspace: the bf16 dS tiles that let dq be a plain
// product (bwd16.hpp).  Per (b, h): one 16 KiB tile per query block qb of 128 rows and key
// tile kb <= min(2 qb + 1, nkt - 1) of 64 keys, i.e. qb (qb + 1) tiles before block qb.
constexpr int64_t kBwdDsTileBytes = 8 * 64 * 32;  // 8 waves x 64 lanes x 16 bf16
inline int64_t backward_ds_tiles_per_head(int64_t T) {
  const int64_t nqb = (T + 127) / 128, nkt = (T + 63) / 64, last = nqb - 1;
  const int64_t kmax = 2 * last + 1 < nkt - 1 ? 2 * last + 1 : nkt - 1;
  return last * (last + 1) + kmax + 1;
}
inline int64_t backward_ds_offset(int64_t B, int64_t H, int64_t T, int64_t d) {
  const int64_t base = backward_workspace_bytes(B, H, T, d);
  return base < 0 ? -1 : (base + 255) / 256 * 256;
}
// Workspace with which the dS tiles of `heads` heads at a time are kept (1 <= heads <= B*H;
// the kernels then run on groups of that many heads), or -1.
inline int64_t backward_workspace_bytes_kept(int64_t B, int64_t H, int64_t T, int64_t d, int64_t heads) {
  if (d != 64 && d != 128) return -1;  // the kept-dS path: bf16 at d = 64, 128
  const int64_t off = backward_ds_offset(B, H, T, d);
  if (off < 0 || heads < 1 || heads > B * H) return -1;
  const int64_t tiles = backward_ds_tiles_per_head(T);
  if (tiles > (int64_t(1) << 62) / kBwdDsTileBytes / heads) return -1;
  return off + heads * tiles * kBwdDsTileBytes;
}
inline int64_t backward_workspace_bytes_fast(int64_t B, int64_t H, int64_t T, int64_t d) {
  if (B < 1 || H < 1) return -1;
  return backward_workspace_bytes_kept(B, H, T, d, B * H);
}
// Heads whose dS tiles fit a workspace of ws_bytes (0: the recompute path), at most B*H.
// (backward_kept_heads_for: 0 also for the float32 and d = 16 kernels, which keep no dS.)
inline int64_t backward_kept_heads(int64_t B, int64_t H, int64_t T, int64_t d, int64_t ws_bytes) {
  const int64_t one = backward_workspace_bytes_kept(B, H, T, d, 1);
  if (one < 0 || ws_bytes < one) return 0;
  const int64_t per_head = backward_ds_tiles_per_head(T) * kBwdDsTileBytes;
  const int64_t g = 1 + (ws_bytes - one) / per_head;
  return g < B * H ? g : B * H;
}

inline int64_t backward_kept_heads_for(int64_t B, int64_t H, int64_t T, int64_t d, int dtype, int64_t ws_bytes) {
  return dtype == CSA_BF16 && d != 16 ? backward_kept_heads(B, H, T, d, ws_bytes) : 0;
}

inline int validate_backward(const void* q, const void* k, const void* v, const void* k0, const void* v0,
                             const void* o, const float* lse, const void* dout, const void* dq, const void* dk,
                             const void* dv, const void* dk0, const void* dv0, const void* ws, int64_t ws_bytes,
                             int64_t B, int64_t H, int64_t T, int64_t d, int dtype) {
  if (dtype != CSA_BF16 && dtype != CSA_F32) return CSA_ERR_UNSUPPORTED;
  if (d != 16 && d != 64 && d != 128) return CSA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !ws) return CSA_ERR_INVALID_ARG;
  const int64_t need_min = backward_workspace_bytes(B, H, T, d);
  if (need_min < 0 || ws_bytes < need_min) return CSA_ERR_INVALID_ARG;
  const int64_t kept = backward_kept_heads_for(B, H, T, d, dtype, ws_bytes);
  const int64_t need = kept > 0 ? backward_workspace_bytes_kept(B, H, T, d, kept) : need_min;  // the part used
  for (const void* p : {q, k, v, o, dout, dq, dk, dv, ws})
    if (!aligned(p, 16)) return CSA_ERR_INVALID_ARG;
  for (const void* p : {k0, v0, dk0, dv0})
    if (p && !aligned(p, 16)) return CSA_ERR_INVALID_ARG;
  if (!aligned(lse, 4)) return CSA_ERR_INVALID_ARG;
  const int64_t esize = dtype == CSA_F32 ? 4 : 2;
  const int64_t big = B * H * T * d * esize, small = B * H * d * esize;
  const Span ins[8] = {span_of(q, big),  span_of(k, big),  span_of(v, big),  span_of(k0, small),
                       span_of(v0, small), span_of(o, big), span_of(lse, B * H * T * 4), span_of(dout, big)};
  const Span outs[6] = {span_of(dq, big),    span_of(dk, big),    span_of(dv, big),
                        span_of(dk0, small), span_of(dv0, small), span_of(ws, need)};
  for (int i = 0; i < 6; ++i) {
    for (const Span& s : ins)
      if (overlaps(outs[i], s)) return CSA_ERR_INVALID_ARG;
    for (int j = i + 1; j < 6; ++j)
      if (overlaps(outs[i], outs[j])) return CSA_ERR_INVALID_ARG;
  }
  return CSA_OK;
}

inline const char* status_string(int s) {
  switch (s) {
    case CSA_OK: return "ok";
    case CSA_ERR_INVALID_ARG: return "invalid argument (null pointer, size, alignment or overlap)";
    case CSA_ERR_UNSUPPORTED: return "unsupported head dimension or dtype";
    case CSA_ERR_HIP: return "HIP launch failure";
    case CSA_ERR_SCRATCH_TOO_SMALL:
      return "sizes need more workspace than the static scratch of csa_decode_noalloc holds "
             "(csa_decode_workspace_bytes > CSA_DECODE_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

}  // namespace csa
