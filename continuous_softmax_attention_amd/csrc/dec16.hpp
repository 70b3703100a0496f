// Few-query decode of continuous softmax attention on the matrix cores (bf16, d in
// {64, 128}, 1 .. 8 queries): the same split-K structure and partial-result layout as
// decode_partial_kernel (decode.hpp, which keeps float32 and d = 16), with both
// contractions on 16x16x32 bf16 MFMAs.
//
// Method: J. Su, "Continuous Softmax Attention", eq. (10)-(11): the weight of a position
// is the sum of its two edge terms, each a phi_2 of a neighbour difference; the p-form and
// the Taylor branch are those of the bf16 forward kernel (edge_yu, attn16.hpp).
//
// Why: with lanes over d (decode_partial_kernel) every key costs each query a weight
// broadcast and d/64 FMAs per lane, so eight queries make that kernel VALU-issue bound at
// about a third of HBM bandwidth.  Here a wave holds 16 query slots (Tq used, the rest
// zero) in the layout of the forward kernel -- S^T = K Q^T with lane (n, g) holding query
// slot n and keys 16g .. 16g+15 of a 64-key tile -- so the logits and P V take 32 MFMAs
// per tile, and the VALU computes the weights only (16 per lane per tile).  The unused
// slots cost nothing that matters in a kernel bound by HBM: one query streams faster
// here than with lanes over d, whose K and V loads are narrower.
//
// One wave per (batch*head, split); a split is a run of `chunk` (a multiple of 64) key
// rows, row r being position r + 1; split 0 also owns position 0 (k_0, v_0).  Per tile:
//   * K rows go straight from HBM into the MFMA operand registers, one tile ahead;
//   * V rows are copied HBM -> LDS (global_load_lds) in the forward kernel's V layout and
//     read back transposed (ds_read_b64_tr_b16);
//   * the next tile's S^T comes first: its first key is the right neighbour of this
//     tile's last key; at the split's two edges the neighbours come from the adjacent
//     splits (a lane-parallel dot product on the left, an extra one-block MFMA product
//     on the right);
//   * the weights are rounded to bf16 once, and the weight sum uses the rounded values.
// The partial results (O [d], running maximum, weight sum) go to the workspace in the
// layout decode_merge_kernel reads.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "decode.hpp"

namespace csa {

constexpr int kDec16Waves = 4;  // splits per work-group (one per wave)

template <int D>
__global__ void __launch_bounds__(64 * kDec16Waves, 2) decode16_kernel(DecParams p) {
  static_assert(D == 64 || D == 128, "head dimension");
  constexpr int ROWB = 2 * D;                     // bytes per row
  constexpr int NSTEP = D / 32;                   // QK^T contraction steps
  constexpr int NMB = D / 16;                     // 16-row blocks of O^T
  constexpr int RW = 4;                           // 16-byte chunks per row segment of a V region
  constexpr int REGION = 64 * RW * 16;            // 32 d-columns of a 64-row tile
  constexpr int TILE_BYTES = kTile * ROWB;
  constexpr int NCOPY = TILE_BYTES / 1024;        // 16-byte copies per lane per V tile
  __shared__ __attribute__((aligned(1024))) char vst[kDec16Waves][TILE_BYTES];

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;  // query slot
  const int g = lane >> 4;  // lane group: keys 16g .. 16g+15 of a tile
  const int item = blockIdx.x * kDec16Waves + wv;
  if (item >= p.BH * p.nsplit) return;  // whole wave; this kernel has no barrier
  const int bh = item / p.nsplit;
  const int sp = item % p.nsplit;
  const int Tn = p.T;
  const int Tq = p.Tq;
  const int rs = sp * p.chunk;            // first key row of the split
  const int re = min(rs + p.chunk, Tn);   // one past its last
  const int nt = (re - rs + kTile - 1) / kTile;
  const bool right_halo = re < Tn;        // row re (next split) is the last row's right neighbour
  // query slot n sits at position T - Tq + 1 + n, i.e. its own key is row rq; slots past Tq
  // hold zero queries and see every row (finite, never stored)
  const int rq = n < Tq ? Tn - Tq + n : Tn - 1;
  const int vend = min(rq, re - 1);       // last row weighted for slot n in this split
  const bool diag = vend == rq;           // ... and it is the diagonal (left term only)
  const int used_end = diag ? vend : vend + 1;  // last row whose logit slot n uses
  // tiles [0, nt_full) have every row visible to every slot and a right neighbour
  const int clear_end = min(re, Tn - Tq);  // rows < clear_end: both terms for all slots
  const int nt_full = clear_end > rs ? min(nt, (clear_end - rs) / kTile) : 0;

  const bf16* Kh = (const bf16*)p.k + (size_t)bh * Tn * D;
  const bf16* Vh = (const bf16*)p.v + (size_t)bh * Tn * D;

  // ---- query operand: qreg[s] = chunk 4s + g of slot n (zero past Tq)
  bf16x8 qreg[NSTEP];
  {
    const bf16* Qg = (const bf16*)p.q + ((size_t)bh * Tq + min(n, Tq - 1)) * D;
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      qreg[s] = *(const bf16x8*)(Qg + (4 * s + g) * 8);
      if (n >= Tq) {
#pragma unroll
        for (int e = 0; e < 8; ++e) qreg[s][e] = (bf16)0.0f;
      }
    }
  }

  // reductions over the four lane groups of a slot (lanes n, n+16, n+32, n+48)
  auto qmax = [&](float x) {
    const unsigned u = __float_as_uint(x);
    const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
    const Half h32 = pair_values(x);
    return fmaxf(h32.lo, h32.hi);
  };
  auto qsum = [&](float x) {
    const unsigned u = __float_as_uint(x);
    const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
    const Half h32 = pair_values(x);
    return h32.lo + h32.hi;
  };
  auto from_lane = [&](int src, float x) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(x)));
  };
  const int lane_dn = (lane + 16) & 63;  // same slot, next lane group
  const int lane_up = (lane - 16) & 63;  // same slot, previous lane group

  // q . k for one key row (all slots at once; every lane gets its slot's value)
  auto row_logit = [&](const bf16* row) {
    float part = 0.0f;
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      const bf16x8 kc = *(const bf16x8*)(row + (4 * s + g) * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) part = __builtin_fmaf((float)qreg[s][e], (float)kc[e], part);
    }
    return qsum(part);
  };

  // ---- K operand registers: block b, step s = row r0 + 16(n >> 2) + 4b + (n & 3) (clamped
  // to the last row), chunk 4s + g; S^T block b then holds keys 16g + 4b + r in element r.
  // Every K row is read once per call: the loads carry the non-temporal hint (measured on the
  // B16 H8 T8192 cache: 5.6 -> 6.3 TB/s; the same hint on the V copies into LDS lost 9%).
  bf16x8 kreg[4][NSTEP];
  auto load_k = [&](int r0, int nb) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if (b < nb) {  // wave-uniform
        const int row = min(r0 + 16 * (n >> 2) + 4 * b + (n & 3), Tn - 1);
#pragma unroll
        for (int s = 0; s < NSTEP; ++s)
          kreg[b][s] = __builtin_nontemporal_load((const bf16x8*)(Kh + (size_t)row * D + (4 * s + g) * 8));
      }
    }
    asm volatile("" ::: "memory");  // issued here, not sunk towards their use
  };
  auto qk = [&](f32x4 (&S)[4], int nb) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if (b < nb) {
        S[b] = f32x4{};
#pragma unroll
        for (int s = 0; s < NSTEP; ++s) S[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kreg[b][s], qreg[s], S[b], 0, 0, 0);
      }
    }
  };

  // ---- V tile in LDS, the forward kernel's layout: slot sigma (16 bytes at 16 sigma) holds
  // row (sigma mod 256) / 4, chunk 4 (sigma / 256) + ((sigma mod 4) ^ 2 ((row >> 4) & 1))
  CSA_LDS char* vb = (CSA_LDS char*)&vst[wv][0];
  const unsigned vb_addr = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)vb);
  auto stage_v = [&](int r0) {
    const char* base = (const char*)(Vh + (size_t)r0 * D);
    const int rows_left = Tn - r0;  // >= 1
#pragma unroll
    for (int c = 0; c < NCOPY; ++c) {
      const int sigma = 64 * c + lane;
      const int region = sigma / (64 * RW);
      const int within = sigma % (64 * RW);
      const int row = within / RW;
      const int cc = (within % RW) ^ ((2 * ((row >> 4) & 1)) & (RW - 1));
      lds_copy16(base, min(row, rows_left - 1) * ROWB + (region * RW + cc) * 16, vb_addr + 1024 * c);
    }
  };
  // V^T operand (d-block mb, key chunk c): lane (n, g) gets d = 16mb + n, keys 16g + 8c + e
  int vbase[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int cc = ((2 * par) & (RW - 1)) + ((n >> 1) & 1);
    vbase[par] = (16 * g + (n >> 2)) * RW * 16 + 16 * (cc ^ ((2 * (g & 1)) & (RW - 1))) + 8 * (n & 1);
  }
  auto vread = [&](int c, int mb) -> bf16x8 {
    CSA_LDS const char* a = vb + vbase[mb & 1] + (2 * mb / RW) * REGION + 8 * c * RW * 16;
    const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CSA_LDS s16x4*)a);
    const s16x4 r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CSA_LDS s16x4*)(a + 4 * RW * 16));
    const bf16x4 b1 = __builtin_bit_cast(bf16x4, r1);
    const bf16x4 b2 = __builtin_bit_cast(bf16x4, r2);
    return bf16x8{b1[0], b1[1], b1[2], b1[3], b2[0], b2[1], b2[2], b2[3]};
  };

  f32x4 O[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) O[mb] = f32x4{};
  float lsum = 0.0f;
  float m_run = -__builtin_inff();
  float carry = 0.0f;  // lanes g = 3: left term of the next tile's first key
  float w0 = 0.0f;     // split 0: weight of position 0

  // logit of the split's left neighbour: row rs - 1, or position 0 (k_0, zero when absent)
  float a_left = 0.0f;
  if (rs > 0) {
    a_left = row_logit(Kh + (size_t)(rs - 1) * D);
  } else if (p.k0 != nullptr) {
    a_left = row_logit((const bf16*)p.k0 + (size_t)bh * D);
  }
  const bool left_used = rs == 0 || rs <= vend;

  // ---------------------------------------------------------------- one tile
  // Sc: S^T of this tile (first row r0); Sn: S^T of the next tile (block 0 at least) when
  // has_next.  MASKED: rows past vend get 0, the diagonal row its left term only.
  auto tile = [&](auto masked_c, int j, const f32x4 (&Sc)[4], const f32x4 (&Sn)[4], bool has_next) {
    constexpr bool MASKED = decltype(masked_c)::value;
    const int r0 = rs + j * kTile;
    float s[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) s[t] = Sc[t >> 2][t & 3];
    int lim = vend - (r0 + 16 * g);  // s[t] is weighted iff t <= lim
    asm volatile("" : "+v"(lim));

    float mx = -__builtin_inff();
    if constexpr (MASKED) {
      const int ulim = used_end - (r0 + 16 * g);
#pragma unroll
      for (int t = 0; t < 16; ++t) mx = fmaxf(mx, t <= ulim ? s[t] : -__builtin_inff());
    } else {
#pragma unroll
      for (int t = 0; t < 16; ++t) mx = fmaxf(mx, s[t]);
    }
    float halo = 0.0f;  // logit of row r0 + 64 (lane n, g = 0 of the next tile's block 0)
    if (has_next) {
      halo = from_lane(n, Sn[0][0]);
      if (!MASKED || r0 + kTile <= used_end) mx = fmaxf(mx, halo);
    }
    if (j == 0 && left_used) mx = fmaxf(mx, a_left);
    mx = qmax(mx);
    {
      const float m_new = fmaxf(m_run, mx * kLog2e);
      if (__builtin_amdgcn_ballot_w64(m_new > m_run + 8.0f) != 0) {
        // a slot with nothing visible yet keeps -inf and factor 1
        const float sc = m_new > m_run ? exp2_fast(m_run - m_new) : 1.0f;
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) O[mb] *= sc;
        lsum *= sc;
        carry *= sc;
        w0 *= sc;
        m_run = m_new;
      }
    }
    const float mr = m_run;
    auto alpha = [&](int t) { return __builtin_fmaf(s[t], kLog2e, -mr); };
    float w[16];

    const float al0 = alpha(0);
    const float pv0 = exp2_fast(al0);
    const float al15 = alpha(15);
    const float pv15 = exp2_fast(al15);
    // right neighbour of key 15: the next group's key 0, or (g = 3) the next tile's first row
    float ar = from_lane(lane_dn, al0);
    float pr = from_lane(lane_dn, pv0);
    if (g == 3) {
      ar = has_next ? __builtin_fmaf(halo, kLog2e, -mr) : al15;
      pr = exp2_fast(ar);
    }
    float R15, Lnext;
    edge_terms<false>(al15, pv15, ar, pr, R15, Lnext);
    const float Lsend = g == 3 ? carry : Lnext;
    float Lprev = from_lane(lane_up, Lsend);
    carry = Lnext;
    if (j == 0) {  // left edge of the split: row rs - 1 or position 0
      const float all = __builtin_fmaf(a_left, kLog2e, -mr);
      float Rl, Ll;
      edge_terms<false>(all, exp2_fast(all), al0, pv0, Rl, Ll);
      if (g == 0) Lprev = Ll;
      if (rs == 0) w0 = Rl;  // position 0 has its right term only
    }
    float pc = pv0;
    float an = alpha(1), pn = exp2_fast(an);
    float yc = an - al0, uc = __builtin_amdgcn_rcpf(yc);
#pragma unroll
    for (int t = 0; t < 15; ++t) {
      float ann = 0.0f, pnn = 0.0f, yn = 0.0f, un = 0.0f;
      if (t + 2 < 15) {
        ann = alpha(t + 2);
        pnn = exp2_fast(ann);
      } else if (t + 2 == 15) {
        ann = al15;
        pnn = pv15;
      }
      if (t + 2 <= 15) {
        yn = ann - an;
        un = __builtin_amdgcn_rcpf(yn);
      }
      if constexpr (!MASKED) {
        edge_yu(pc, pn, yc, uc, Lprev, w[t], Lprev);
      } else {
        float R, L;
        edge_yu(pc, pn, yc, uc, 0.0f, R, L);
        w[t] = t < lim ? Lprev + R : (t == lim ? (diag ? Lprev : Lprev + R) : 0.0f);
        Lprev = L;
      }
      pc = pn;
      yc = yn;
      uc = un;
      an = ann;
      pn = pnn;
    }
    if constexpr (!MASKED) {
      w[15] = Lprev + R15;
    } else {
      w[15] = 15 < lim ? Lprev + R15 : (15 == lim ? (diag ? Lprev : Lprev + R15) : 0.0f);
    }

    // P V: key chunk c holds keys 16g + 8c .. 16g + 8c + 7 of every lane group
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      bf16x8 P;
#pragma unroll
      for (int e = 0; e < 8; ++e) P[e] = (bf16)w[8 * c + e];
      const bf16x2 one2 = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
      for (int e = 0; e < 8; e += 2) lsum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{P[e], P[e + 1]}, one2, lsum, false);
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) O[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vread(c, mb), P, O[mb], 0, 0, 0);
    }
  };

  // ---- pipeline: K of tile j+1 is in registers while tile j's weights are formed; V of
  // tile j is in LDS; the copies of tile j+1's V start once tile j's P V has read its rows.
  // Tile nt (after the split) is only the right neighbour's row block, when there is one.
  auto next_blocks = [&](int jn) { return jn < nt ? 4 : (jn == nt && right_halo ? 1 : 0); };
  f32x4 Sc[4], Sn[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) Sn[b] = f32x4{};
  load_k(rs, 4);
  stage_v(rs);
  qk(Sc, 4);
  if (next_blocks(1) > 0) load_k(rs + kTile, next_blocks(1));
  using BF = std::integral_constant<bool, false>;
  using BT = std::integral_constant<bool, true>;
  auto step = [&](auto masked_c, int j) {
    const int nbn = next_blocks(j + 1);
    if (nbn > 0) qk(Sn, nbn);  // waits for K of tile j+1 and (earlier) V of tile j
    if (next_blocks(j + 2) > 0) load_k(rs + (j + 2) * kTile, next_blocks(j + 2));
    if (nbn == 0) wait_vmem();  // V of tile j (otherwise awaited with K of tile j+1)
    tile(masked_c, j, Sc, Sn, nbn > 0);
    if (j + 1 < nt) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this tile's V reads are done
      stage_v(rs + (j + 1) * kTile);
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) Sc[b] = Sn[b];
  };
  int j = 0;
  for (; j < nt_full; ++j) step(BF{}, j);
  for (; j < nt; ++j) step(BT{}, j);

  // ---- partial results of this split
  float l = qsum(lsum);
  if (rs == 0) {
    const float w0q = from_lane(n, w0);
    l += w0q;
    if (p.v0 != nullptr) {
      const bf16* V0 = (const bf16*)p.v0 + (size_t)bh * D;
      bf16x4 v0r[NMB];  // every load issued before the first is used
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) v0r[mb] = *(const bf16x4*)(V0 + 16 * mb + 4 * g);
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) O[mb][r] = __builtin_fmaf(w0q, (float)v0r[mb][r], O[mb][r]);
    }
  }
  if (n < Tq) {
    float* dst = p.ws + (((size_t)bh * p.nsplit + sp) * Tq + n) * (D + 2);
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[16 * mb + 4 * g + r] = O[mb][r];
    if (g == 0) {
      dst[D] = m_run;
      dst[D + 1] = l;
    }
  }
}

// prm.BH, Tq (1 .. 8), T set; chooses chunk and nsplit for this device and launches the
// partial kernel and the merge.
template <int D>
inline hipError_t launch_decode16(const DecParams& prm_in, hipStream_t stream) {
  static const int bpc = [] {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, decode16_kernel<D>, 64 * kDec16Waves, 0) != hipSuccess) b = 0;
    return b;
  }();
  DecParams prm = prm_in;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int64_t cap = (int64_t)(bpc > 0 ? bpc : 1) * kDec16Waves * (cus > 0 ? cus : 1);
  prm.chunk = decode_chunk(prm.BH, prm.T, cap);  // splits of key rows (position 0 rides with split 0)
  prm.nsplit = (prm.T + prm.chunk - 1) / prm.chunk;
  const int items = prm.BH * prm.nsplit;
  hipLaunchKernelGGL((decode16_kernel<D>), dim3((items + kDec16Waves - 1) / kDec16Waves), dim3(64 * kDec16Waves), 0,
                     stream, prm);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<bf16, D>), dim3(prm.BH * prm.Tq), dim3(64), 0, stream, prm);
  return hipGetLastError();
}

}  // namespace csa
