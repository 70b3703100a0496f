// Forward of the interval variant [1/2, t + 1/2] (bf16, 16x16x32 MFMAs, gfx950).
//
// Method: J. Su, "Continuous Softmax Attention", Problem Statement: the original paper
// integrates eq. (2) over [1/2, t + 1/2] instead of [0, t].  With the interpolation of
// eq. (3) unchanged, query t covers half of segment [0, 1] (sigma in [1/2, 1]), the whole
// segments [1, 2] .. [t-1, t], and half of segment [t, t+1] (sigma in [0, 1/2]); position
// T+1, needed by the last query only, repeats position T (its half segment is flat).
//
// Weights (in the forward's units: c^2 e^{a} x integral, scaled by 2^{-m}; p = 2^{alpha},
// alpha = a log2 e - m, c = ln 2).  A whole segment (i, i+1) gives the forward's R, L
// (attn_fwd.hpp).  For a segment with endpoint values p_l, p_r, midpoint value
// p_m = 2^{(alpha_l + alpha_r)/2}, y = alpha_r - alpha_l and u = 1/y:
//   right half (sigma in [0, 1/2]):  HL = ((c/2) p_m - (p_m - p_l) u) u  (to the right end),
//                                    HR = c (p_m - p_l) u - HL           (to the left end);
//   left half (sigma in [1/2, 1]):   HL' = (c (p_r - p_m/2) - (p_r - p_m) u) u,
//                                    HR' = c (p_r - p_m) u - HL';
// below |y| < 0.1 their second-order Taylor forms in x = c y:
//   HL = c^2 p_l (1/8 + x/24 + x^2/128),   HR = c^2 p_l (3/8 + x/12 + 5 x^2/384),
//   HL' = c^2 p_l (3/8 + 7x/24 + 15 x^2/128), HR' = c^2 p_l (1/8 + x/12 + 11 x^2/384).
// Position 0 receives HR' of segment (0, 1) and position 1 its HL'; position t receives
// HR of segment (t, t+1) and position t+1 its HL (for the last query both go to position T,
// c^2 p_T / 2 in total).  lse = ln of the integral, as the forward's.
//
// Decomposition: the forward's (128 query rows per work-group, 8 waves x 16 queries) with
// the backward's self-contained 64-key tiles (bwd16.hpp): S^T from a row-layout K tile plus
// one halo block (keys J-1 and J+64), P per lane over 16 consecutive keys, O^T += V^T P^T
// from a transposed-layout V tile; online softmax over tiles.  A wave's tiles run to the
// one holding key row qw + 16 (the last query of the wave reaches position t+1).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "bwd16.hpp"

namespace csa {

namespace half {

constexpr float kC = 0.6931471805599453f;  // ln 2
constexpr float kC2 = 0.4804530139182014f;  // c^2
constexpr float kY0 = 0.1f;                 // Taylor below |y| < 0.1 for the half segments

// right half (sigma in [0, 1/2]) of segment (l, r): HR to l, HL to r
__device__ __forceinline__ void right_half(float al, float pl, float ar, float& HR, float& HL) {
  const float y = ar - al;
  const float pm = exp2_fast(0.5f * (al + ar));
  const float u = __builtin_amdgcn_rcpf(y);
  const float dm = pm - pl;
  const float hl = __builtin_fmaf(0.5f * kC, pm, -dm * u) * u;
  const float hr = __builtin_fmaf(kC * dm, u, -hl);
  const float x = kC * y;
  const float cp = kC2 * pl;
  const float hlt = cp * __builtin_fmaf(x, __builtin_fmaf(x, 1.0f / 128.0f, 1.0f / 24.0f), 0.125f);
  const float hrt = cp * __builtin_fmaf(x, __builtin_fmaf(x, 5.0f / 384.0f, 1.0f / 12.0f), 0.375f);
  const bool small = __builtin_fabsf(y) < kY0;
  HR = small ? hrt : hr;
  HL = small ? hlt : hl;
}

// left half (sigma in [1/2, 1]) of segment (l, r): HR' to l, HL' to r
__device__ __forceinline__ void left_half(float al, float pl, float ar, float pr, float& HR, float& HL) {
  const float y = ar - al;
  const float pm = exp2_fast(0.5f * (al + ar));
  const float u = __builtin_amdgcn_rcpf(y);
  const float dm = pr - pm;
  const float hl = __builtin_fmaf(kC, pr - 0.5f * pm, -dm * u) * u;
  const float hr = __builtin_fmaf(kC * dm, u, -hl);
  const float x = kC * y;
  const float cp = kC2 * pl;
  const float hlt = cp * __builtin_fmaf(x, __builtin_fmaf(x, 15.0f / 128.0f, 7.0f / 24.0f), 0.375f);
  const float hrt = cp * __builtin_fmaf(x, __builtin_fmaf(x, 11.0f / 384.0f, 1.0f / 12.0f), 0.125f);
  const bool small = __builtin_fabsf(y) < kY0;
  HR = small ? hrt : hr;
  HL = small ? hlt : hl;
}

}  // namespace half

template <int D>
__global__ void __launch_bounds__(512, 2) half_fwd_kernel(FwdParams p) {
  using WT = WaveTile<D>;
  constexpr int CH = WT::CH, ROWB = WT::ROWB, NSTEP = WT::NSTEP, NMB = WT::NMB;
  constexpr int TILE = WT::TILE, HALO = WT::HALO;
  constexpr int BUF = 2 * TILE + HALO;  // Krow | Vtr | Khalo
  static_assert(D == 64 || D == 128, "head dimension");

  __shared__ __attribute__((aligned(1024))) char smem[2 * BUF];
  CSA_LDS char* lds = (CSA_LDS char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int Tn = p.T, BH = p.B * p.H;
  const int bh = blockIdx.x % BH;
  const int qb = p.nqb - 1 - blockIdx.x / BH;  // longest query blocks first
  const int q0 = qb * kBlockRows;
  const int qw = q0 + 16 * wave;
  const int qr = qw + n;
  const bool wave_rows = qw < Tn;
  // last tile: the one holding key row qw + 16 (position t+1 of the wave's last query)
  const int jw = wave_rows ? min(qw + 16, Tn - 1) / kTile : -1;
  const int jmax = min(q0 + kBlockRows, Tn - 1) / kTile;

  const size_t head = (size_t)bh * (size_t)Tn * D;
  const char* Kg = (const char*)((const bf16*)p.k + head);
  const char* Vg = (const char*)((const bf16*)p.v + head);

  for (int i = tid; i < 2 * 14 * CH; i += 512) {  // zero rows 2..15 of both halo buffers
    const int buf = i / (14 * CH), chunk = i % (14 * CH);
    *(CSA_LDS f32x4*)(lds + buf * BUF + 2 * TILE + halo_zero_off<D>(chunk)) = f32x4{};
  }
  const int roff = row_layout_src<ROWB>(tid), toff = tr_layout_src<ROWB>(tid);
  auto stage = [&](int buf, int tile) {
    CSA_LDS char* b = lds + buf * BUF;
    stage_tile<D>(b, Kg, tile * kTile, roff, Tn, wave);
    stage_tile<D>(b + TILE, Vg, tile * kTile, toff, Tn, wave);
    if (wave == 0 && lane <= 2 * CH) {  // halo rows J-1 (row 0 for the first tile) and J+64
      const int J = tile * kTile;
      bool right;
      const int c = halo_src_chunk<D>(lane, right);
      const int row = right ? min(J + kTile, Tn - 1) : max(J - 1, 0);
      lds_copy16_ptr(Kg + (size_t)row * ROWB + 16 * c,
                     __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(b + 2 * TILE)));
    }
  };

  bf16x8 qreg[NSTEP];
  {
    const bf16* Qg = (const bf16*)p.q + head + (size_t)min(qr, Tn - 1) * D;
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) qreg[s] = *(const bf16x8*)(Qg + (4 * s + g) * 8);
  }
  // query-wide reductions over the four lane groups (lanes n, n+16, n+32, n+48)
  auto qsum = [&](float x) {
    const unsigned u = __float_as_uint(x);
    const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
    const Half h32 = pair_values(x);
    return h32.lo + h32.hi;
  };
  auto qmax = [&](float x) {
    const unsigned u = __float_as_uint(x);
    const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
    const Half h32 = pair_values(x);
    return fmaxf(h32.lo, h32.hi);
  };
  // logit of position 0 (zero when k0 is null)
  float a0 = 0.0f;
  if (p.k0 != nullptr) {
    const bf16* K0 = (const bf16*)p.k0 + (size_t)bh * D;
    float part = 0.0f;
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      const bf16x8 kc = *(const bf16x8*)(K0 + (4 * s + g) * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) part = __builtin_fmaf((float)qreg[s][e], (float)kc[e], part);
    }
    a0 = qsum(part);
  }

  const int kbase = row_kbase(n, g);
  int vbase[2];
  tr_vbase(n, g, vbase);
  const int hoff = n * WT::HROW + 16 * g;
  const bool last_q = qr == Tn - 1;

  f32x4 O[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) O[mb] = f32x4{};
  float lsum = 0.0f, w0 = 0.0f;
  float m_run = -__builtin_inff();

  stage(0, 0);
  wait_vmem();
  __syncthreads();
  // one key tile: MASKED when some key or edge of it is cut for some query of the wave
  auto iter = [&](int j, auto masked_c) {
    constexpr bool masked = decltype(masked_c)::value;
    if (j + 1 <= jmax) stage((j + 1) & 1, j + 1);
    if (j <= jw) {
      CSA_LDS const char* b = lds + (j & 1) * BUF;
      const int J = j * kTile;
      float s[16];
      f32x4 H;
      logits_tile<D>(b, b + 2 * TILE, kbase, hoff, qreg, s, H);
      float sl, sr;
      neighbours(s, H, n, g, sl, sr);
      const bool start = J + 16 * g == 0;  // left neighbour is position 0
      if (start) sl = a0;
      const int lim = qr < Tn ? qr - (J + 16 * g) : -3;   // key t is position <= t_query iff t <= lim
      const int vis = last_q ? lim : lim + 1;              // last visible key of this lane

      // running maximum over visible keys, the right halo when visible, and position 0
      float mx = -__builtin_inff();
#pragma unroll
      for (int t = 0; t < 16; ++t) mx = fmaxf(mx, (!masked || t <= vis) ? s[t] : -__builtin_inff());
      if (g == 3 && (!masked || 16 <= vis)) mx = fmaxf(mx, sr);
      if (j == 0) mx = fmaxf(mx, a0);
      mx = qmax(mx);
      // lazy shift: moves only when the maximum grows by more than 2^8 (weights stay <= 2^8)
      const float m_new = fmaxf(m_run, mx * kLog2e);
      if (__builtin_amdgcn_ballot_w64(m_new > m_run + 8.0f) != 0) {
        const float sc = exp2_fast(m_run - m_new);
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) O[mb] *= sc;
        lsum *= sc;
        w0 *= sc;
        m_run = m_new;
      }
      const float mr = m_run;
      auto alpha = [&](float x) { return __builtin_fmaf(x, kLog2e, -mr); };

      float w[16];
      float aP = alpha(sl), pP = exp2_fast(aP);
      float aC = alpha(s[0]), pC = exp2_fast(aC);
      float Lprev;
      {  // edge (key -1, key 0)
        float R, L;
        edge_terms<false>(aP, pP, aC, pC, R, L);
        if (start) {
          float HRl, HLl;
          half::left_half(aP, pP, aC, pC, HRl, HLl);
          if (j == 0) w0 = HRl;
          L = HLl;
        } else if constexpr (masked) {
          float HR, HL;
          half::right_half(aP, pP, aC, HR, HL);
          L = lim >= 0 ? L : (lim == -1 && !last_q ? HL : 0.0f);
        }
        Lprev = L;
      }
      // on masked tiles the edge (lim, lim+1) is this query's lower half segment: its
      // endpoint values are kept while the loop passes and its terms added after it
      float hA = 0.0f, hP = 0.0f, hB = 0.0f;
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const float aN = alpha(t < 15 ? s[t + 1] : sr);
        const float pN = exp2_fast(aN);
        float R, L;
        edge_terms<false>(aC, pC, aN, pN, R, L);
        if constexpr (masked) {  // edge (t, t+1): whole if t+1 <= lim, else left out here
          const bool whole = t + 1 <= lim;
          hA = t == lim ? aC : hA;
          hP = t == lim ? pC : hP;
          hB = t == lim ? aN : hB;
          w[t] = t <= vis ? Lprev + (whole ? R : 0.0f) : 0.0f;
          L = whole ? L : 0.0f;
        } else {
          w[t] = Lprev + R;
        }
        Lprev = L;
        aC = aN;
        pC = pN;
      }
      if constexpr (masked) {
        // lower half of segment (lim, lim+1): HR to key lim, HL to key lim+1; for the last
        // query the segment is flat (position T+1 repeats T) and all of it, c^2 p/2, goes to
        // key lim.  For lim = 15 the HL term belongs to the next lane group's key 0, which
        // takes it from its own first edge.
        float HR, HL;
        half::right_half(hA, hP, hB, HR, HL);
        const float Rh = last_q ? 0.5f * half::kC2 * hP : HR;
        const float Lh = last_q ? 0.0f : HL;
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          w[t] = t == lim ? w[t] + Rh : w[t];
          if (t > 0) w[t] = t == lim + 1 ? Lh : w[t];  // lim = -1: key 0 has its HL already
        }
      }
      // O^T += V^T P^T and the row sums of the same rounded P
      const bf16x2 one2 = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        bf16x8 P;
#pragma unroll
        for (int e = 0; e < 8; ++e) P[e] = (bf16)w[8 * c + e];
#pragma unroll
        for (int e = 0; e < 8; e += 2)
          lsum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{P[e], P[e + 1]}, one2, lsum, false);
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
          O[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tr_read(b + TILE, vbase, c, mb), P, O[mb], 0, 0, 0);
      }
    }
    wait_vmem();
    __syncthreads();
  };
  // tiles entirely below the wave's diagonal (no masks), then the others
  const int jm = wave_rows ? qw / kTile : 0;
  int j = 0;
  for (; j < jm; ++j) iter(j, std::false_type{});
  for (; j <= jmax; ++j) iter(j, std::true_type{});
  if (!wave_rows) return;

  float l = qsum(lsum);
  const float w0q = __int_as_float(__builtin_amdgcn_ds_bpermute(n << 2, __float_as_int(w0)));
  l += w0q;
  const float inv = 1.0f / l;
  if (qr < Tn) {
    const bf16* V0 = p.v0 != nullptr ? (const bf16*)p.v0 + (size_t)bh * D : nullptr;
    bf16* Og = (bf16*)p.out + head + (size_t)qr * D;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      const int d0 = 16 * mb + 4 * g;
      float o4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float acc = O[mb][r];
        if (V0) acc = __builtin_fmaf(w0q, (float)V0[d0 + r], acc);
        o4[r] = acc * inv;
      }
      *(bf16x4*)(Og + d0) = bf16x4{(bf16)o4[0], (bf16)o4[1], (bf16)o4[2], (bf16)o4[3]};
    }
    if (p.lse != nullptr && g == 0)
      p.lse[(size_t)bh * Tn + qr] = (m_run + __builtin_amdgcn_logf(l)) * kLn2 + 0.7330258411633287f;  // -2 ln c
  }
}

template <int D>
inline hipError_t launch_half(const FwdParams& prm, hipStream_t stream) {
  FwdParams p = prm;
  p.nqb = (prm.T + kBlockRows - 1) / kBlockRows;
  hipLaunchKernelGGL((half_fwd_kernel<D>), dim3((unsigned)(p.nqb * prm.B * prm.H)), dim3(512), 0, stream, p);
  return hipGetLastError();
}

}  // namespace csa
