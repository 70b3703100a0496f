// Backward pass for float32 inputs (any d) and for bf16 at d = 16: the same gradients as
// bwd16.hpp (the plain derivative of eq. (10)-(11) of "Continuous Softmax Attention"; see the
// header of bwd16.hpp for the edge form of dS), computed on the VALU in float32 throughout --
// no bf16 rounding of P or dS.  These shapes are small (the float32 workloads are at most
// 4 heads of 1024 rows), so the kernels are written for clarity and exactness first:
//
//   bwdv_pre   D_t = dO_t . o_t and mu_t = log2(c^2 Z_t) from the forward's lse (as bwd_transpose does for bf16).
//   bwdv_dq    one wave per query t: the positions 0..t in chunks of 62, lane j holding
//              position base - 1 + j (neighbours in lanes j -+ 1); its logit a_{t,i} and
//              dO_t . v_i by dot products, P and dS from the edge terms; dq_t = sum_i dS_{t,i} k_i
//              with the lanes over d (dS_i broadcast from its lane).
//   bwdv_dkdv  one wave per position i = 0..T (0 = k_0 / v_0): the queries t >= max(i, 1) in
//              chunks of 64, one per lane, each forming the logits and dO . v of positions
//              i-1, i, i+1 itself; dk_i = sum_t dS_{t,i} q_t and dv_i = sum_t P_{t,i} dO_t with
//              the lanes over d (for position 0: dk_0, dv_0).
//
// Edge terms in float32 ("p-form", units of 1/Z as bwd16.hpp): for consecutive positions
// (l, r) with y = (a_r - a_l) log2 e, u = 1/y, p = 2^{a log2 e - mu}:
//   R/Z = (u (p_r - p_l) - c p_l) u,  L/Z = (c p_r - u (p_r - p_l)) u,
//   C/Z = u^2 ((p_l + p_r) - (2/c) u (p_r - p_l)),
// below |y| < 1 their Taylor series of degree 8 (float32 accuracy):
//   R/Z = p_l sum_n c^{n+2} y^n / (n+2)!,  L/Z = p_r sum_n c^{n+2} (-y)^n / (n+2)!,
//   C/Z = p_l sum_n c^{n+2} y^n (n+1) / (n+3)!.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "attn_fwd.hpp"
#include "bwd16.hpp"

namespace csa {

namespace bwdv {

template <typename TT>
__device__ __forceinline__ float ld(const TT* p) {
  return (float)*p;
}

// R/Z, L/Z, C/Z of one existing edge (float32, see the header)
__device__ __forceinline__ void edge_f32(float al, float pl, float ar, float pr, float& R, float& L, float& C) {
  const float y = ar - al;
  const bool small = __builtin_fabsf(y) < Taylor<true>::Y0;
  const float u = __builtin_amdgcn_rcpf(small ? 1.0f : y);  // the closed forms only where |y| >= 1
  const float du = (pr - pl) * u;
  const float rc = __builtin_fmaf(-kLn2, pl, du) * u;
  const float lc = __builtin_fmaf(kLn2, pr, -du) * u;
  const float cc = __builtin_fmaf(-2.0f / kLn2, du, pl + pr) * (u * u);
  float gp, gm;
  Taylor<true>::eval(y, gp, gm);  // sum_n c^{n+2} (+-y)^n / (n+2)!, n <= 8
  // sum_n c^{n+2} (n+1) y^n / (n+3)!, n <= 8
  constexpr float m[9] = {0.0800755023f, 0.0277520543f, 0.00577087746f, 0.000888903876f, 0.000110025217f,
                          1.14395504e-05f, 1.02787119e-06f, 8.14246881e-08f, 5.77220042e-09f};
  float gc = m[8];
#pragma unroll
  for (int n = 7; n >= 0; --n) gc = __builtin_fmaf(gc, y, m[n]);
  R = small ? pl * gp : rc;
  L = small ? pr * gm : lc;
  C = small ? pl * gc : cc;
}

}  // namespace bwdv

template <typename TT, int D>
__global__ void __launch_bounds__(256) bwdv_pre_kernel(BwdParams p) {
  const int BH = p.B * p.H, T = p.T;
  const BwdWs w = bwd_ws(p.ws, BH, T, D);
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // one wave per row
  if (row >= (int64_t)BH * T) return;
  const TT* a = (const TT*)p.dout + row * D;
  const TT* b = (const TT*)p.o + row * D;
  float acc = 0.0f;
  for (int d = lane; d < D; d += 64) acc = __builtin_fmaf(bwdv::ld(a + d), bwdv::ld(b + d), acc);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (lane == 0) {
    w.delta[row] = acc;
    w.mu[row] = __builtin_fmaf(p.lse[row], kLog2e, kMuShift);
  }
}

// dot product of a D-element row held as float in LDS with a TT row in global memory
template <typename TT, int D>
__device__ __forceinline__ float dot_row(const float* a, const TT* b) {
  float acc = 0.0f;
#pragma unroll 8
  for (int d = 0; d < D; ++d) acc = __builtin_fmaf(a[d], bwdv::ld(b + d), acc);
  return acc;
}

// one wave per query row t (4 waves per work-group)
template <typename TT, int D>
__global__ void __launch_bounds__(256) bwdv_dq_kernel(BwdParams p) {
  constexpr int DPL = (D + 63) / 64;  // d-columns per lane in the dq accumulation
  __shared__ float qs[4][D], os[4][D];
  const int BH = p.B * p.H, Tn = p.T;
  const BwdWs ws = bwd_ws(p.ws, BH, Tn, D);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * 4 + wv;
  const bool active = row < (int64_t)BH * Tn;
  const int bh = active ? (int)(row / Tn) : 0;
  const int r = active ? (int)(row % Tn) : 0;
  const int t = r + 1;  // query position
  const size_t head = (size_t)bh * Tn * D;
  const TT* K = (const TT*)p.k + head;
  const TT* V = (const TT*)p.v + head;
  const TT* K0 = p.k0 ? (const TT*)p.k0 + (size_t)bh * D : nullptr;
  const TT* V0 = p.v0 ? (const TT*)p.v0 + (size_t)bh * D : nullptr;
  for (int d = lane; d < D; d += 64) {
    qs[wv][d] = bwdv::ld((const TT*)p.q + head + (size_t)r * D + d);
    os[wv][d] = bwdv::ld((const TT*)p.dout + head + (size_t)r * D + d);
  }
  __syncthreads();
  if (!active) return;
  const float mu = ws.mu[row], delta = ws.delta[row];
  float acc[DPL];
#pragma unroll
  for (int c = 0; c < DPL; ++c) acc[c] = 0.0f;
  for (int base = 0; base <= t; base += 62) {
    // lane j: position i = base - 1 + j (exists for 0 <= i <= t)
    const int i = base - 1 + lane;
    const bool ex = i >= 0 && i <= t;
    float a = 0.0f, dp = 0.0f;
    if (ex) {
      if (i == 0) {
        float sa = 0.0f, sd = 0.0f;
        for (int d = 0; d < D; ++d) {
          sa = __builtin_fmaf(qs[wv][d], K0 ? bwdv::ld(K0 + d) : 0.0f, sa);
          sd = __builtin_fmaf(os[wv][d], V0 ? bwdv::ld(V0 + d) : 0.0f, sd);
        }
        a = sa;
        dp = sd;
      } else {
        a = dot_row<TT, D>(qs[wv], K + (size_t)(i - 1) * D);
        dp = dot_row<TT, D>(os[wv], V + (size_t)(i - 1) * D);
      }
    }
    const float al = __builtin_fmaf(a, kLog2e, -mu);
    const float pv = ex ? __builtin_amdgcn_exp2f(al) : 0.0f;
    // edge (i, i+1): terms from the next lane's values
    const float ar = __shfl_down(al, 1), pr = __shfl_down(pv, 1), dpr = __shfl_down(dp, 1);
    const bool edge = ex && i + 1 <= t && lane < 63;
    float R = 0.0f, L = 0.0f, C = 0.0f;
    if (edge) bwdv::edge_f32(al, pv, ar, pr, R, L, C);
    const float G = C * (dp - dpr);
    const float Lleft = __shfl_up(L, 1), Gleft = __shfl_up(G, 1);
    // positions of lanes 1..62 are this chunk's (lane 0 and 63 only supply neighbours)
    const bool own = ex && lane >= 1 && lane <= 62;
    const float P = own ? (i > 0 ? Lleft : 0.0f) + R : 0.0f;
    const float dS = own ? __builtin_fmaf(P, dp - delta, (i > 0 ? Gleft : 0.0f) - G) : 0.0f;
    // dq += sum over the chunk's positions of dS_i k_i, lanes over d (dS_i read from lane j)
    for (int j = 1; j <= 62; ++j) {
      const int ij = base - 1 + j;
      if (ij > t) break;
      const float s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dS), j));
#pragma unroll
      for (int c = 0; c < DPL; ++c) {
        const int d = lane + 64 * c;
        if (d < D) {
          const float kv = ij == 0 ? (K0 ? bwdv::ld(K0 + d) : 0.0f) : bwdv::ld(K + (size_t)(ij - 1) * D + d);
          acc[c] = __builtin_fmaf(s, kv, acc[c]);
        }
      }
    }
  }
#pragma unroll
  for (int c = 0; c < DPL; ++c) {
    const int d = lane + 64 * c;
    if (d < D) ((TT*)p.dq)[head + (size_t)r * D + d] = (TT)acc[c];
  }
}

// one wave per position i = 0 .. T of one (b, h) (4 waves per work-group)
template <typename TT, int D>
__global__ void __launch_bounds__(256) bwdv_dkdv_kernel(BwdParams p) {
  constexpr int DPL = (D + 63) / 64;
  __shared__ float kr[4][3][D], vr[4][3][D];
  const int BH = p.B * p.H, Tn = p.T;
  const BwdWs ws = bwd_ws(p.ws, BH, Tn, D);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t item = (int64_t)blockIdx.x * 4 + wv;
  const bool active = item < (int64_t)BH * (Tn + 1);
  const int bh = active ? (int)(item / (Tn + 1)) : 0;
  const int i = active ? (int)(item % (Tn + 1)) : 0;  // position
  const size_t head = (size_t)bh * Tn * D;
  const TT* Q = (const TT*)p.q + head;
  const TT* O = (const TT*)p.dout + head;
  const TT* K0 = p.k0 ? (const TT*)p.k0 + (size_t)bh * D : nullptr;
  const TT* V0 = p.v0 ? (const TT*)p.v0 + (size_t)bh * D : nullptr;
  // rows of positions i-1, i, i+1 (k_0 / v_0 at position 0; zeros where the position is
  // outside 0..T -- those edges are never used)
  for (int e = 0; e < 3; ++e) {
    const int pos = i - 1 + e;
    for (int d = lane; d < D; d += 64) {
      float kv = 0.0f, vv = 0.0f;
      if (pos == 0) {
        kv = K0 ? bwdv::ld(K0 + d) : 0.0f;
        vv = V0 ? bwdv::ld(V0 + d) : 0.0f;
      } else if (pos >= 1 && pos <= Tn) {
        kv = bwdv::ld((const TT*)p.k + head + (size_t)(pos - 1) * D + d);
        vv = bwdv::ld((const TT*)p.v + head + (size_t)(pos - 1) * D + d);
      }
      kr[wv][e][d] = kv;
      vr[wv][e][d] = vv;
    }
  }
  __syncthreads();
  if (!active) return;
  float ak[DPL], av[DPL];
#pragma unroll
  for (int c = 0; c < DPL; ++c) ak[c] = av[c] = 0.0f;
  const int t0 = i > 1 ? i : 1;
  for (int tb = t0; tb <= Tn; tb += 64) {
    const int t = tb + lane;  // query position of this lane
    const bool ex = t <= Tn;
    float P = 0.0f, dS = 0.0f;
    if (ex) {
      const int r = t - 1;
      const float mu = ws.mu[(size_t)bh * Tn + r], delta = ws.delta[(size_t)bh * Tn + r];
      float a[3] = {0.0f, 0.0f, 0.0f}, dp[3] = {0.0f, 0.0f, 0.0f};
      for (int d = 0; d < D; ++d) {
        const float qd = bwdv::ld(Q + (size_t)r * D + d), od = bwdv::ld(O + (size_t)r * D + d);
#pragma unroll
        for (int e = 0; e < 3; ++e) {
          a[e] = __builtin_fmaf(qd, kr[wv][e][d], a[e]);
          dp[e] = __builtin_fmaf(od, vr[wv][e][d], dp[e]);
        }
      }
      float al[3], pv[3];
#pragma unroll
      for (int e = 0; e < 3; ++e) {
        al[e] = __builtin_fmaf(a[e], kLog2e, -mu);
        pv[e] = __builtin_amdgcn_exp2f(al[e]);
      }
      // left edge (i-1, i) exists iff i >= 1; right edge (i, i+1) iff i + 1 <= t
      float Rl = 0.0f, Ll = 0.0f, Cl = 0.0f, Rr = 0.0f, Lr = 0.0f, Cr = 0.0f;
      if (i >= 1) bwdv::edge_f32(al[0], pv[0], al[1], pv[1], Rl, Ll, Cl);
      if (i + 1 <= t) bwdv::edge_f32(al[1], pv[1], al[2], pv[2], Rr, Lr, Cr);
      const float Gl = Cl * (dp[0] - dp[1]), Gr = Cr * (dp[1] - dp[2]);
      P = Ll + Rr;
      dS = __builtin_fmaf(P, dp[1] - delta, Gl - Gr);
    }
    // dk_i += sum_t dS_{t,i} q_t, dv_i += sum_t P_{t,i} dO_t over the chunk, lanes over d
    // (P and dS of query tb + j read from lane j)
    const int nq = Tn - tb + 1 < 64 ? Tn - tb + 1 : 64;
    for (int j = 0; j < nq; ++j) {
      const int r = tb + j - 1;
      const float sj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dS), j));
      const float pj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(P), j));
#pragma unroll
      for (int c = 0; c < DPL; ++c) {
        const int d = lane + 64 * c;
        if (d < D) {
          ak[c] = __builtin_fmaf(sj, bwdv::ld(Q + (size_t)r * D + d), ak[c]);
          av[c] = __builtin_fmaf(pj, bwdv::ld(O + (size_t)r * D + d), av[c]);
        }
      }
    }
  }
#pragma unroll
  for (int c = 0; c < DPL; ++c) {
    const int d = lane + 64 * c;
    if (d >= D) continue;
    if (i == 0) {
      if (p.dk0) ((TT*)p.dk0)[(size_t)bh * D + d] = (TT)ak[c];
      if (p.dv0) ((TT*)p.dv0)[(size_t)bh * D + d] = (TT)av[c];
    } else {
      ((TT*)p.dk)[head + (size_t)(i - 1) * D + d] = (TT)ak[c];
      ((TT*)p.dv)[head + (size_t)(i - 1) * D + d] = (TT)av[c];
    }
  }
}

template <typename TT, int D>
inline hipError_t launch_backward_valu(const BwdParams& prm, hipStream_t stream) {
  const int64_t BH = (int64_t)prm.B * prm.H;
  const int64_t rows = BH * prm.T;
  hipLaunchKernelGGL((bwdv_pre_kernel<TT, D>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, prm);
  hipLaunchKernelGGL((bwdv_dq_kernel<TT, D>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, prm);
  const int64_t items = BH * (prm.T + 1);
  hipLaunchKernelGGL((bwdv_dkdv_kernel<TT, D>), dim3((unsigned)((items + 3) / 4)), dim3(256), 0, stream, prm);
  return hipGetLastError();
}

}  // namespace csa
