// Decode / few-query forward of continuous softmax attention on gfx950: Tq <= 8 new
// queries (the last positions T-Tq+1..T of a sequence) against a key/value cache of T
// positions plus k_0, v_0.  This file's partial kernel serves float32 and d = 16; bf16
// at d = 64, 128 runs on the matrix cores (dec16.hpp) and shares the merge kernel and
// the split plan (decode_chunk).
//
// Method: J. Su, "Continuous Softmax Attention", eq. (10)-(11); the correction weights
// use the p-form of attn_fwd.hpp (edge_terms, float32 Taylor branch).  The result of a
// query is exactly the corresponding row of the full forward.
//
// This path reads every cached key and value once per call and does ~2 d FLOP per
// key and query, so it is bound by HBM bandwidth, not by the matrix cores: it is
// written for streaming, not for MFMA.
//
//   Pass 1 (decode_partial_kernel): one wave per (batch*head, split) where a split is a run
//   of 64 .. 1024 consecutive positions, its length chosen per call so that the waves fill
//   the device in whole rounds (decode_chunk; the kernel is instantiated for at most 1, 2, 4
//   or 8 queries, so that small Tq keep few registers and many waves in flight).  Blocks of
//   64 positions, one position per lane:
//     * logits q_j . k_p for the Tq queries (lane = position; q broadcast from LDS;
//       v_dot2_f32_bf16 for bf16);
//     * neighbours through ds_bpermute inside the block; across blocks from the
//       previous / next block, and at the split's two edges from a halo logit
//       (one lane-parallel dot product per edge);
//     * both edges of each position in the p-form, with the running maximum of the
//       split (lazy rescale as in the forward kernels), masks for the query's
//       diagonal (left term only), position 0 (right term only) and positions past
//       the query;
//     * P V on the VALU with lanes over d (the weight of each key is read from its
//       lane with v_readlane).
//   It writes (O partial [d], running maximum m, weight sum l) per (head, split, query)
//   to the caller's workspace.
//   Pass 2 (decode_merge_kernel): one wave per (head, query) combines the splits with
//   the usual max-rescaled sums, writes o and lse.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "attn16.hpp"

namespace csa {

constexpr int kDecMaxQ = 8;     // queries per call
constexpr int kDecWaves = 4;    // splits per work-group (one per wave)

struct DecParams {
  const void* q;   // [B, H, Tq, d]
  const void* k;   // [B, H, T, d]
  const void* v;   // [B, H, T, d]
  const void* k0;  // [B, H, d] or null
  const void* v0;  // [B, H, d] or null
  void* out;       // [B, H, Tq, d]
  float* lse;      // [B, H, Tq] or null
  float* ws;       // [B*H, nsplit, Tq, d + 2] float32
  int BH, Tq, T, nsplit;
  int chunk;       // positions per split (a multiple of 64)
};

// Positions (or key rows) per split for B*H heads of `units` of them when `cap` waves of the partial
// kernel fit on the device at once: every split is one wave, and a wave's time grows with its
// number of 64-position blocks, so the partial pass takes about rounds x (blocks per split + a
// fixed cost); the merge walks a head's splits 16 at a time, one memory round trip each, about a
// quarter of a block's time (B16 H8 T8192 d128: ~10 us per block round, ~2.5 us per merge
// batch).  Choose the split length (1 .. 16 blocks) that minimises the sum.  A fixed length of
// 256 positions put 128 heads x 8193 positions into 33 splits per head: 4224 waves for 4096
// slots, a second round for the last 3% and half the bandwidth; without the merge term a single
// head of 131072 positions took 2048 one-block splits and 128 merge batches.
inline int decode_chunk(int64_t BH, int64_t units, int64_t cap) {
  const int64_t blocks = (units + 63) / 64;
  int best = 4;
  double best_t = 1e300;
  for (int cb = 1; cb <= 16; ++cb) {
    const int64_t ns = (blocks + cb - 1) / cb;
    const int64_t rounds = (BH * ns + cap - 1) / cap;
    const double t = (double)rounds * (cb + 0.5) + 0.25 * (double)((ns + 15) / 16);
    if (t <= best_t) {  // ties: the longer splits (fewer partial results to merge)
      best_t = t;
      best = cb;
    }
  }
  return 64 * best;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
    const int src = ((int)(threadIdx.x & 63) ^ s) << 2;
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(x))));
  }
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
    const int src = ((int)(threadIdx.x & 63) ^ s) << 2;
    x += __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(x)));
  }
  return x;
}
__device__ __forceinline__ float lane_value(int src_lane, float x) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src_lane << 2, __float_as_int(x)));
}

// Elements lane*DPL .. lane*DPL + DPL-1 of a row as float (DPL = d/64, or 1 for d = 16,
// where lanes >= 16 read a clamped address and get 0): one unconditional load per lane.
template <typename TT, int D>
__device__ __forceinline__ void load_lane_values(const TT* row, int lane, float (&x)[D >= 64 ? D / 64 : 1]) {
  if constexpr (D == 128 && sizeof(TT) == 2) {
    const unsigned u = *(const unsigned*)(row + 2 * lane);  // two bf16
    x[0] = __uint_as_float(u << 16);
    x[1] = __uint_as_float(u & 0xffff0000u);
  } else if constexpr (D == 128) {
    typedef float f32x2v __attribute__((ext_vector_type(2)));
    const f32x2v f = *(const f32x2v*)(row + 2 * lane);
    x[0] = f[0];
    x[1] = f[1];
  } else {
    const int dd = lane < D ? lane : D - 1;
    const float f = (float)row[dd];
    x[0] = lane < D ? f : 0.0f;
  }
}

template <typename TT, int D, int QMAX>
__global__ void __launch_bounds__(64 * kDecWaves) decode_partial_kernel(DecParams p) {
  static_assert(D == 16 || D == 64 || D == 128, "head dimension");
  constexpr bool F32 = sizeof(TT) == 4;
  constexpr int EPC = 16 / (int)sizeof(TT);  // elements per 16-byte chunk of a row
  constexpr int NCH = D / EPC;               // chunks per row
  constexpr int DPL = D >= 64 ? D / 64 : 1;  // d elements per lane in P V (lanes >= D idle)
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

  constexpr int ROWB = NCH * 16;             // bytes per row
  constexpr int NST = 32 * ROWB / 1024;      // 1 KiB copy instructions per 32-row stage
  static_assert(NST >= 1 && 32 * ROWB % 1024 == 0, "stage size");
  __shared__ __attribute__((aligned(16))) TT qs[kDecWaves][QMAX][D];
  // K rows of 32 positions at a time, per wave: row r at r * ROWB, its 16-byte chunk cc at
  // position cc ^ (r & (NCH - 1)) -- filled by whole-KiB (coalesced) global_load_lds copies,
  // read back one row per lane without bank conflicts
  __shared__ __attribute__((aligned(1024))) char kst[kDecWaves][32 * ROWB];
  static_assert(QMAX >= 1 && QMAX <= kDecMaxQ, "query bound");

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int item = blockIdx.x * kDecWaves + wv;
  if (item >= p.BH * p.nsplit) return;  // whole wave; this kernel has no barrier
  const int bh = item / p.nsplit;
  const int sp = item % p.nsplit;
  const int Tn = p.T;
  const int Tq = p.Tq;
  const int p0 = sp * p.chunk;
  const int pend = min(p0 + p.chunk, Tn + 1);  // this split owns positions [p0, pend)
  const int nb = (pend - p0 + 63) / 64;

  // queries of this head into the wave's LDS slice (read back as broadcasts); slots past Tq
  // hold zeros, so their logits and P V sums run unconditionally and stay finite and unused
  {
    const TT* Qg = (const TT*)p.q + (size_t)bh * Tq * D;
    for (int i = lane; i < QMAX * D; i += 64) qs[wv][i / D][i % D] = i < Tq * D ? Qg[i] : (TT)0.0f;
  }
  const TT* Kh = (const TT*)p.k + (size_t)bh * Tn * D;
  const TT* Vh = (const TT*)p.v + (size_t)bh * Tn * D;
  const TT* K0 = p.k0 ? (const TT*)p.k0 + (size_t)bh * D : nullptr;
  const TT* V0 = p.v0 ? (const TT*)p.v0 + (size_t)bh * D : nullptr;

  // row of position pos (0: k_0 / v_0, which may be absent = zeros), or null
  auto krow = [&](int pos) -> const TT* { return pos == 0 ? K0 : Kh + (size_t)(pos - 1) * D; };
  auto vrow = [&](int pos) -> const TT* { return pos == 0 ? V0 : Vh + (size_t)(pos - 1) * D; };

  // logits of one (wave-uniform) position, lane-parallel over d; 0 if it does not exist
  auto halo = [&](int pos, float (&a)[QMAX]) {
#pragma unroll
    for (int j = 0; j < QMAX; ++j) a[j] = 0.0f;
    if (pos < 0 || pos > Tn) return;
    const TT* row = krow(pos);
    if (row == nullptr) return;
    float kv[DPL];
    load_lane_values<TT, D>(row, lane, kv);  // this lane's d elements (0 past d)
#pragma unroll
    for (int j = 0; j < QMAX; ++j) {
      if (j < Tq) {
        float part = 0.0f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) {
          const int dd = min(lane * DPL + e, D - 1);
          part = __builtin_fmaf(kv[e], (float)qs[wv][j][dd], part);
        }
        a[j] = wave_sum(part);
      }
    }
  };

  // logits of positions base + lane for every query; 0 where the row does not exist.  Two
  // stages of 32 rows: each row's K is staged in LDS by coalesced copies, lanes r and r + 32
  // each take half of row r (lane-per-row loads straight from HBM reached ~4.2 TB/s on this
  // chip against ~5.6 TB/s for whole-KiB reads); position 0 (k_0) comes from halo().
  CSA_LDS char* kw = (CSA_LDS char*)&kst[wv][0];
  const unsigned kw_addr = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)kw);
  auto stage_logits = [&](int first, float (&part)[QMAX]) {  // positions first .. first + 31
    // k rows of positions first + r (position p is row p - 1), clamped to existing rows; the
    // offsets are taken from the stage's first row so that they stay small for any T
    const int sb = min(max(first - 1, 0), Tn - 1);
    const char* sbase = (const char*)(Kh + (size_t)sb * D);
#pragma unroll
    for (int c = 0; c < NST; ++c) {
      const int byte = 1024 * c + 16 * lane;
      const int r = byte / ROWB, slot = (byte % ROWB) / 16;
      const int cc = slot ^ (r & (NCH - 1));
      const int krow_i = min(max(first + r - 1, 0), Tn - 1);  // >= sb
      lds_copy16(sbase, (krow_i - sb) * ROWB + 16 * cc, kw_addr + 1024 * c);
    }
    wait_vmem();
    asm volatile("" ::: "memory");
    const int r = lane & 31, h = lane >> 5;
    float acc[QMAX];
#pragma unroll
    for (int j = 0; j < QMAX; ++j) acc[j] = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH / 2; ++c) {
      const int cc = h * (NCH / 2) + c;
      const f32x4v kc = *(CSA_LDS const f32x4v*)(kw + r * ROWB + 16 * (cc ^ (r & (NCH - 1))));
#pragma unroll
      for (int j = 0; j < QMAX; ++j) {
        const f32x4v qc = *(const f32x4v*)&qs[wv][j][cc * EPC];  // broadcast read
        if constexpr (F32) {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[j] = __builtin_fmaf(kc[e], qc[e], acc[j]);
        } else {
          // whole-chunk bit casts, then element pairs (a bit cast of a single vector
          // element would read element 0)
          const bf16x8 kb = __builtin_bit_cast(bf16x8, kc);
          const bf16x8 qb = __builtin_bit_cast(bf16x8, qc);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[j] = __builtin_amdgcn_fdot2_f32_bf16(bf16x2v{kb[2 * e], kb[2 * e + 1]},
                                                     bf16x2v{qb[2 * e], qb[2 * e + 1]}, acc[j], false);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < QMAX; ++j) {  // the two halves of row r: lanes r and r + 32
      const Half hv = pair_values(acc[j]);
      part[j] = hv.lo + hv.hi;
    }
  };
  auto logits = [&](int base, float (&a)[QMAX]) {  // positions base + lane
    float lo[QMAX], hi[QMAX];
    stage_logits(base, lo);
    stage_logits(base + 32, hi);
    const int pos = base + lane;
#pragma unroll
    for (int j = 0; j < QMAX; ++j) {
      const float v = lane < 32 ? lo[j] : hi[j];
      a[j] = pos >= 1 && pos <= Tn ? v : 0.0f;
    }
    if (base == 0) {  // position 0: k_0 (zeros when absent)
      float a0[QMAX];
      halo(0, a0);
#pragma unroll
      for (int j = 0; j < QMAX; ++j) a[j] = lane == 0 ? a0[j] : a[j];
    }
  };
  float m_run[QMAX], l_run[QMAX], O[QMAX][DPL];
#pragma unroll
  for (int j = 0; j < QMAX; ++j) {
    m_run[j] = -__builtin_inff();
    l_run[j] = 0.0f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) O[j][e] = 0.0f;
  }

  float acur[QMAX], anxt[QMAX], aleft0[QMAX];
  logits(p0, acur);
  halo(p0 - 1, aleft0);  // left neighbour of the split's first position (none at p0 = 0)

  for (int b = 0; b < nb; ++b) {
    const int base = p0 + 64 * b;
    const int pos = base + lane;
    float aright63[QMAX];  // right neighbour of lane 63
    if (b + 1 < nb) {
      logits(base + 64, anxt);
#pragma unroll
      for (int j = 0; j < QMAX; ++j)
        aright63[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(anxt[j]), 0));
    } else {
      halo(pend, aright63);  // position pend belongs to the next split (none past T)
    }

    float wq[QMAX];
#pragma unroll
    for (int j = 0; j < QMAX; ++j) {
      wq[j] = 0.0f;
      if (j >= Tq) continue;  // wave-uniform
      const int tj = Tn - Tq + 1 + j;                 // position of query j
      const bool vis = pos <= tj && pos < pend;       // visible and owned by this split
      const bool hasL = pos >= 1;                     // left neighbour exists
      const bool hasR = pos < tj;                     // right term applies (not the diagonal)
      const float a = acur[j];
      const float from_left = lane_value((lane + 63) & 63, a);   // every lane takes part
      const float from_right = lane_value((lane + 1) & 63, a);
      const float aL = lane == 0 ? aleft0[j] : from_left;
      const float aR = lane == 63 ? aright63[j] : from_right;
      float x = -__builtin_inff();
      if (vis) x = fmaxf(a, fmaxf(hasL ? aL : -__builtin_inff(), hasR ? aR : -__builtin_inff()));
      const float mx = wave_max(x);
      const float m_new = fmaxf(m_run[j], mx * kLog2e);
      if (m_new > m_run[j] + 8.0f) {  // wave-uniform (m_run and mx are)
        const float sc = exp2_fast(m_run[j] - m_new);
        l_run[j] *= sc;
#pragma unroll
        for (int e = 0; e < DPL; ++e) O[j][e] *= sc;
        m_run[j] = m_new;
      }
      const float mr = m_run[j];
      const float al = __builtin_fmaf(a, kLog2e, -mr);
      const float pc = exp2_fast(al);
      const float alL = __builtin_fmaf(aL, kLog2e, -mr);
      const float alR = __builtin_fmaf(aR, kLog2e, -mr);
      float R, Lx, Rx, Lt;
      edge_terms<true>(al, pc, alR, exp2_fast(alR), R, Lx);   // edge (pos, pos+1): right term of pos
      edge_terms<true>(alL, exp2_fast(alL), al, pc, Rx, Lt);  // edge (pos-1, pos): left term of pos
      float w = (hasL ? Lt : 0.0f) + (hasR ? R : 0.0f);
      w = vis ? w : 0.0f;
      wq[j] = w;
      l_run[j] += w;
    }

    // P V: lanes over d; 16 keys per batch of loads
    const int nkeys = min(64, min(pend, Tn + 1) - base);
    for (int kb = 0; kb < nkeys; kb += 16) {
      // all 16 loads unconditional (clamped to an existing row) and zeroed by a factor,
      // not a select: a select lets the compiler sink each load into a branch, one
      // memory round trip per key
      float vv[16][DPL];
      const TT* vrow0 = V0 != nullptr ? V0 : Vh;  // stand-in row for an absent v_0
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) {
        const int kp = min(base + kb + kk, Tn);
        const TT* row = kp == 0 ? vrow0 : Vh + (size_t)(kp - 1) * D;
        const float live = (kb + kk < nkeys && !(kp == 0 && V0 == nullptr)) ? 1.0f : 0.0f;
        load_lane_values<TT, D>(row, lane, vv[kk]);
#pragma unroll
        for (int e = 0; e < DPL; ++e) vv[kk][e] *= live;
      }
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) {
#pragma unroll
        for (int j = 0; j < QMAX; ++j) {  // weights of query slots past Tq are 0
          const float s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wq[j]), kb + kk));
#pragma unroll
          for (int e = 0; e < DPL; ++e) O[j][e] = __builtin_fmaf(s, vv[kk][e], O[j][e]);
        }
      }
    }

    // the next block's left neighbour of lane 0 is this block's lane 63
#pragma unroll
    for (int j = 0; j < QMAX; ++j) {
      aleft0[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acur[j]), 63));
      acur[j] = anxt[j];
    }
  }

  // partial results of this split
#pragma unroll
  for (int j = 0; j < QMAX; ++j) {
    if (j < Tq) {
      const float lsum = wave_sum(l_run[j]);
      float* dst = p.ws + (((size_t)bh * p.nsplit + sp) * Tq + j) * (D + 2);
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        const int dd = lane * DPL + e;
        if (dd < D) dst[dd] = O[j][e];
      }
      if (lane == 0) {
        dst[D] = m_run[j];
        dst[D + 1] = lsum;
      }
    }
  }
}

// One wave per (head, query): the splits' partial results combined with max-rescaled sums,
// 16 splits per batch with all of a batch's loads issued together (lanes over d for O, every
// lane reading the splits' m and l), so that a call of up to 16 splits costs one memory round
// trip; further batches fold into the running (M, L, acc) like an online softmax.
template <typename TT, int D>
__global__ void __launch_bounds__(64) decode_merge_kernel(DecParams p) {
  constexpr int DPL = D >= 64 ? D / 64 : 1;
  constexpr int NB = 16;
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x;  // (bh, j)
  const int bh = item / p.Tq;
  const int j = item % p.Tq;
  const int ns = p.nsplit;
  const float* src = p.ws + ((size_t)bh * ns * p.Tq + j) * (D + 2);
  const size_t stride = (size_t)p.Tq * (D + 2);  // between splits
  const int dl = min(lane * DPL, D - DPL);        // d elements of this lane (d = 16: lanes >= 16 repeat)
  float M = -__builtin_inff(), L = 0.0f, acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.0f;
  for (int s0 = 0; s0 < ns; s0 += NB) {
    float ms[NB], ls[NB], x[NB][DPL];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const float* part = src + (size_t)min(s0 + u, ns - 1) * stride;
      ms[u] = s0 + u < ns ? part[D] : -__builtin_inff();
      ls[u] = part[D + 1];
#pragma unroll
      for (int e = 0; e < DPL; ++e) x[u][e] = part[dl + e];
    }
    float Mn = M;
#pragma unroll
    for (int u = 0; u < NB; ++u) Mn = fmaxf(Mn, ms[u]);
    if (Mn == -__builtin_inff()) continue;  // nothing weighted yet (uniform)
    const float sc = M == -__builtin_inff() ? 0.0f : exp2_fast(M - Mn);
    L *= sc;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] *= sc;
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const float f = ms[u] == -__builtin_inff() ? 0.0f : exp2_fast(ms[u] - Mn);
      L = __builtin_fmaf(ls[u], f, L);
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] = __builtin_fmaf(x[u][e], f, acc[e]);
    }
    M = Mn;
  }
  const float inv = 1.0f / L;
  TT* o = (TT*)p.out + ((size_t)bh * p.Tq + j) * D;
#pragma unroll
  for (int e = 0; e < DPL; ++e) {
    const int dd = lane * DPL + e;
    if (dd < D) o[dd] = (TT)(acc[e] * inv);
  }
  if (p.lse != nullptr && lane == 0)
    p.lse[(size_t)bh * p.Tq + j] = (M + __builtin_amdgcn_logf(L)) * kLn2 + 0.7330258411633287f;  // -2 ln(ln 2)
}

// Work-groups of the partial kernel resident per CU (the same on every gfx950 device: a
// property of the compiled kernel), queried once.
template <typename TT, int D, int QMAX>
inline int decode_blocks_per_cu() {
  static const int n = [] {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, decode_partial_kernel<TT, D, QMAX>, 64 * kDecWaves, 0) !=
        hipSuccess)
      b = 0;
    return b;
  }();
  return n;
}

// prm.BH, Tq, T set; fills in chunk and nsplit for this device and launches both passes.
template <typename TT, int D>
inline hipError_t launch_decode(const DecParams& prm_in, hipStream_t stream) {
  DecParams prm = prm_in;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int bpc = prm.Tq <= 1   ? decode_blocks_per_cu<TT, D, 1>()
                  : prm.Tq <= 2 ? decode_blocks_per_cu<TT, D, 2>()
                  : prm.Tq <= 4 ? decode_blocks_per_cu<TT, D, 4>()
                                : decode_blocks_per_cu<TT, D, 8>();
  const int64_t cap = (int64_t)(bpc > 0 ? bpc : 1) * kDecWaves * (cus > 0 ? cus : 1);
  prm.chunk = decode_chunk(prm.BH, prm.T + 1, cap);
  prm.nsplit = (prm.T + 1 + prm.chunk - 1) / prm.chunk;
  const int items = prm.BH * prm.nsplit;
  const dim3 grid((items + kDecWaves - 1) / kDecWaves), block(64 * kDecWaves);
  if (prm.Tq <= 1) hipLaunchKernelGGL((decode_partial_kernel<TT, D, 1>), grid, block, 0, stream, prm);
  else if (prm.Tq <= 2) hipLaunchKernelGGL((decode_partial_kernel<TT, D, 2>), grid, block, 0, stream, prm);
  else if (prm.Tq <= 4) hipLaunchKernelGGL((decode_partial_kernel<TT, D, 4>), grid, block, 0, stream, prm);
  else hipLaunchKernelGGL((decode_partial_kernel<TT, D, 8>), grid, block, 0, stream, prm);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<TT, D>), dim3(prm.BH * prm.Tq), dim3(64), 0, stream, prm);
  return hipGetLastError();
}

}  // namespace csa
