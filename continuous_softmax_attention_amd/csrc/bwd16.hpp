// Backward pass of the bf16 causal CSA forward for gfx950 on 16x16x32 MFMAs.
//
// Method: J. Su, "Continuous Softmax Attention", eq. (10)-(11): o_t = sum_i P_{t,i} v_i with
// P_{t,i} = e^{a_{t,i} + b_{t,i}} / Z_t, where every edge (i, i+1) (consecutive positions
// 0..t) contributes a right term R_e = e^{a_i} phi_2(a_{i+1} - a_i) to position i and a
// left term L_e = e^{a_{i+1}} phi_2(a_i - a_{i+1}) to position i+1.  The pages print no
// backward; differentiating eq. (10) gives, for the loss sum_t dO_t . o_t:
//
//   * dR_e/da_{i+1} = dL_e/da_i = C_e = integral_0^1 s (1-s) e^{(1-s) a_i + s a_{i+1}} ds,
//     and dR_e/da_i = R_e - C_e, dL_e/da_{i+1} = L_e - C_e;
//   * with dP_{t,i} = dO_t . v_i, D_t = dO_t . o_t, c_e = C_e / Z_t and
//     G_e = c_e (dP_i - dP_{i+1}), the logit gradient is a two-point stencil of edge terms
//     on top of the softmax one:
//         dS_{t,i} = P_{t,i} (dP_{t,i} - D_t) + G_{(i-1,i)} - G_{(i,i+1)};
//   * dq_t = sum_i dS_{t,i} k_i,  dk_i = sum_t dS_{t,i} q_t,  dv_i = sum_t P_{t,i} dO_t,
//     position 0 entering through k_0, v_0 (dk_0, dv_0 are the sums over t at i = 0).
//
// Arithmetic ("p-form", as the forward).  mu_t = log2(c^2 Z_t) = lse_t log2 e + 2 log2 c
// (c = ln 2) comes from the forward's lse; p_i = 2^{a_i log2 e - mu_t} = e^{a_i} / (c^2 Z_t).
// For an edge with y = (a_{i+1} - a_i) log2 e, u = 1/y and dp = p_{i+1} - p_i:
//     R/Z = (u dp - c p_i) u,   L/Z = (c p_{i+1} - u dp) u,
//     c_e = u^2 ((p_i + p_{i+1}) - (2/c) u dp),
// with Taylor forms below |y| < 0.07 (R, L) and |y| < 0.25 (c_e), where the differences
// cancel: R/Z = p_i (c^2/2 + c^3 y/6), L/Z = p_{i+1} (c^2/2 - c^3 y/6),
// c_e = p_i (c^2/6 + c^3 y/12 + c^4 y^2/40).
//
// Kernels (one launch each, in this order on the caller's stream):
//   bwd_transpose  Q^T and dO^T ([B*H][D][T rounded up to 128], zeros past T) into the
//             workspace: the A operands of bwd_dkdv's dK / dV products; its dO work-groups
//             also write D_t = dO_t . o_t and mu_t, and work-group 0 the zero rows standing in
//             for a null k_0 / v_0.
//   bwd_dq    one work-group per 128 query rows (the forward's decomposition: 8 waves x
//             16 queries, 64-key tiles double-buffered in LDS).  Per tile S^T = K Q^T and
//             dP^T = V dO^T on MFMAs, plus one 16-row "halo" block whose rows 0 and 1 are
//             keys J-1 and J+64, so that every tile is self-contained; P and dS per lane
//             (16 consecutive keys of one query, neighbours across lane groups by
//             ds_bpermute); dQ^T += K^T dS^T with K^T through transposed LDS reads.  Also
//             writes dS and P of position 0 per query.
//   bwd_sink  dk_0 = sum_t dS_{t,0} q_t, dv_0 = sum_t P_{t,0} dO_t: partial sums over 16
//             row ranges per (b, h), then their fixed-order sum (skipped when both are null).
//   bwd_dkdv  one work-group per 64 key rows, looping over 128-row query tiles: the same
//             S^T, dP^T, P and dS per wave; P and dS (bf16) go through LDS so that
//             dV^T += dO^T P and dK^T += Q^T dS contract over queries on MFMAs, with Q^T and
//             dO^T read from the transposed copies (two work-groups per CU).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "attn16.hpp"

namespace csa {

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* k0;    // may be null (zeros)
  const void* v0;    // may be null (zeros)
  const void* o;     // forward output
  const float* lse;  // forward lse (natural log)
  const void* dout;  // dO
  void* dq;
  void* dk;
  void* dv;
  void* dk0;  // may be null (not written)
  void* dv0;  // may be null (not written)
  char* ws;   // workspace of csa_backward_workspace_bytes() bytes
  int B, H, T;
  char* ds;          // dS tiles (optional last workspace region), or null: dq recomputes dS
  int64_t ds_tiles;  // dS tiles per (b, h)
  int h0, nh;        // heads h0 .. h0 + nh - 1 (of the B*H) in this launch; the dS region holds
                     // the tiles of these nh heads (the launch's head index 0 .. nh - 1)
};

// dS tiles for the dq product: for every (b, h), query block qb (128 rows) and key tile
// kb <= min(2 qb + 1, nkt - 1), 8 waves x 2 halves x 64 lanes x 8 bf16 -- each lane's 16
// consecutive keys of its query in the order of the dq product's B operand, the 8 keys of
// half h of every lane of a wave in one contiguous KiB (byte 2048 wave + 1024 h + 16 lane), so
// that each 16-byte load or store of a wave covers one KiB; qb (qb + 1) tiles precede block qb.
// (With each lane's 32 bytes together every 16-byte store of bwd_dkdv touched a 2 KiB span at
// half density; this layout made bwd_dkdv about 2% faster.)  Both sides use non-temporal
// accesses: every byte is written once and read once, and as streamed data it does not evict
// the K / V / Q^T / dO^T rows the two kernels re-read from L2 (the backward ran ~3% faster).
constexpr int kDsTileBytes = 8 * 64 * 32;
__device__ __forceinline__ int64_t ds_tile_index(int qb, int kb) { return (int64_t)qb * (qb + 1) + kb; }

// Workspace: 512 zero bytes (two rows of up to 128 bf16), then four float arrays of
// B*H*T: D_t, mu_t, dS_{t,0}, P_{t,0}; then the float partial sums of dk_0 and dv_0,
// B*H x 16 chunks x 2 x 128 (sized for d = 128 whatever d is).
constexpr int kBwdZeroBytes = 512;

// Then, 256-byte aligned, Q^T and dO^T of every head: [B*H][D][Tp] bf16 with Tp = T rounded up
// to a multiple of 128 and zeros past T (written by bwd_transpose, read by bwd_dkdv as the
// operands of its dK / dV products).
constexpr int kSinkChunks = 16;
__host__ __device__ constexpr int64_t bwd_tp(int64_t T) { return (T + 127) / 128 * 128; }
__host__ __device__ constexpr int64_t bwd_qt_offset(int64_t BH, int64_t T) {
  return (kBwdZeroBytes + 16 * BH * T + BH * kSinkChunks * 2 * 128 * 4 + 255) / 256 * 256;
}

struct BwdWs {
  const char* zero;
  float* delta;
  float* mu;
  float* ds0;
  float* p0;
  float* sink;
  bf16* qt;   // Q^T [B*H][D][Tp]
  bf16* dot;  // dO^T [B*H][D][Tp]
};
__device__ __forceinline__ BwdWs bwd_ws(char* ws, int BH, int T, int D) {
  const size_t n = (size_t)BH * (size_t)T;
  float* f = (float*)(ws + kBwdZeroBytes);
  bf16* qt = (bf16*)(ws + bwd_qt_offset(BH, T));
  return {ws, f, f + n, f + 2 * n, f + 3 * n, f + 4 * n, qt, qt + (size_t)BH * D * bwd_tp(T)};
}

constexpr float kMuShift = -1.0575327458897954f;  // 2 log2(ln 2)

// ---------------------------------------------------------------- LDS tile layouts
// The two 64-row layouts of attn16.hpp, as free functions of the row width.  A tile of
// 64 rows x D columns is D/32 regions of 4 KiB (32 columns each).
//   row layout ("K"): row r in 64-byte slot 4 (r & 3) + (r >> 4) + 16 ((r >> 2) & 3),
//     chunk cc at position cc ^ (r & 3); read as the A operand of S^T = K Q^T.
//   transposed layout ("V"): row r at slot r, chunk cc at position cc ^ 2 bit4(r); read
//     with ds_read_b64_tr_b16 as 16 columns x 32 rows.
constexpr int kRegion = 4096;

// HBM byte offset, relative to the tile's first row, of LDS slot sigma (16 bytes at 16 sigma)
template <int ROWB>
__device__ __forceinline__ int row_layout_src(int sigma) {
  const int region = sigma >> 8, within = sigma & 255;
  const int gi = within >> 2;
  const int row = 16 * (gi & 3) + 4 * (gi >> 4) + ((gi >> 2) & 3);
  const int cc = (within & 3) ^ (row & 3);
  return row * ROWB + (region * 4 + cc) * 16;
}
template <int ROWB>
__device__ __forceinline__ int tr_layout_src(int sigma) {
  const int region = sigma >> 8, within = sigma & 255;
  const int row = within >> 2;
  const int cc = (within & 3) ^ (2 * ((row >> 4) & 1));
  return row * ROWB + (region * 4 + cc) * 16;
}
// LDS byte offset of chunk cc (of 16-byte chunks along the row) of row r, transposed layout
__device__ __forceinline__ int tr_layout_at(int r, int cc) {
  return (cc >> 2) * kRegion + r * 64 + 16 * ((cc & 3) ^ (2 * ((r >> 4) & 1)));
}

// The P / dS buffers of bwd_dkdv: the transposed layout with the chunk position further
// XORed with bits 2..3 of the row, so that the 16 rows one lane group writes (one 16-byte
// chunk each) fall on 16 different bank slots (in the plain layout four rows share one).
__device__ __forceinline__ int ptr_layout_at(int r, int cc) {
  return (cc >> 2) * kRegion + r * 64 + 16 * ((cc & 3) ^ (2 * ((r >> 4) & 1)) ^ ((r >> 2) & 3));
}
// tr_read of such a buffer: row 16g + 8c + 4rd + (n >> 2) has bits 2..3 equal to (2c + rd) & 3,
// the same in every lane, so each of the four (c, rd) reads takes its own XORed base:
// pbase[par][k] = vbase[par] ^ 16 k (the added offsets are multiples of 64 bytes).
__device__ __forceinline__ void ptr_bases(const int (&vbase)[2], int (&pbase)[2][4]) {
#pragma unroll
  for (int par = 0; par < 2; ++par)
#pragma unroll
    for (int k = 0; k < 4; ++k) pbase[par][k] = vbase[par] ^ (16 * k);
}
__device__ __forceinline__ bf16x8 ptr_read(CSA_LDS const char* tile, const int (&pbase)[2][4], int c, int mb) {
  CSA_LDS const char* a1 = tile + pbase[mb & 1][(2 * c) & 3] + (mb >> 1) * kRegion + 8 * c * 64;
  CSA_LDS const char* a2 = tile + pbase[mb & 1][(2 * c + 1) & 3] + (mb >> 1) * kRegion + 8 * c * 64 + 4 * 64;
  const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CSA_LDS s16x4*)a1);
  const s16x4 r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CSA_LDS s16x4*)a2);
  const bf16x4 b1 = __builtin_bit_cast(bf16x4, r1);
  const bf16x4 b2 = __builtin_bit_cast(bf16x4, r2);
  return bf16x8{b1[0], b1[1], b1[2], b1[3], b2[0], b2[1], b2[2], b2[3]};
}

// A operand of S^T for 16-key block b, contraction step s (row layout)
__device__ __forceinline__ bf16x8 row_read(CSA_LDS const char* tile, int kbase, int s, int b) {
  return *(CSA_LDS const bf16x8*)(tile + kbase + s * kRegion + b * 1024);
}
// 16 columns (block mb) x 32 rows (16g + 8c + e, e = 0..7 for lane group g) of a transposed tile
__device__ __forceinline__ bf16x8 tr_read(CSA_LDS const char* tile, const int (&vbase)[2], int c, int mb) {
  CSA_LDS const char* a = tile + vbase[mb & 1] + (mb >> 1) * kRegion + 8 * c * 64;
  const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CSA_LDS s16x4*)a);
  const s16x4 r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CSA_LDS s16x4*)(a + 4 * 64));
  const bf16x4 b1 = __builtin_bit_cast(bf16x4, r1);
  const bf16x4 b2 = __builtin_bit_cast(bf16x4, r2);
  return bf16x8{b1[0], b1[1], b1[2], b1[3], b2[0], b2[1], b2[2], b2[3]};
}

// One 16-byte HBM -> LDS copy per lane from a per-lane 64-bit address (lane i writes
// lds_addr + 16 i); completion is awaited like lds_copy16's.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_copy16_ptr(const char* src, unsigned lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds_addr)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// ---------------------------------------------------------------- per-element arithmetic
// Edge (i, i+1) of one query from alpha_i, p_i, alpha_{i+1}, p_{i+1}: W = Lprev + R/Z (the
// finished P of position i when Lprev is its left term), L/Z and c_e as in the header.  When
// the edge does not exist, W = Lprev and L = c_e = 0 (selects, so that values of positions
// that do not exist for this query never reach the result).  MASKED = false: the caller knows
// that every edge exists and the selects are left out.  Every operation is written out
// (contraction off): an existing edge gets the same bits in both forms, so the kernels that
// compute dS (bwd_dq, bwd_dkdv) agree bit for bit whichever form each takes for a tile.
template <bool MASKED>
__device__ __forceinline__ void edge_grad(float al, float pl, float ar, float pr, bool exists, float Lprev,
                                          float& W, float& L, float& C) {
#pragma clang fp contract(off)
  constexpr float k0 = 0.2402265069591007f;     // c^2/2
  constexpr float k1 = 0.055504108664821576f;   // c^3/6
  constexpr float m0 = 0.08007550231970023f;    // c^2/6
  constexpr float m1 = 0.027752054332410788f;   // c^3/12
  constexpr float m2 = 0.005770877464577086f;   // c^4/40
  constexpr float two_over_c = 2.8853900817779268f;
  const float y = ar - al;
  const float ay = __builtin_fabsf(y);
  const bool small = ay < 0.07f;
  const float u = __builtin_amdgcn_rcpf(y);
  const float du = (pr - pl) * u;
  const float w = __builtin_fmaf(__builtin_fmaf(-kLn2, pl, du), u, Lprev);
  const float l = __builtin_fmaf(kLn2, pr, -du) * u;
  const float c = __builtin_fmaf(-two_over_c, du, pl + pr) * (u * u);
  const float wt = __builtin_fmaf(pl, __builtin_fmaf(y, k1, k0), Lprev);
  const float lt = pr * __builtin_fmaf(y, -k1, k0);
  const float ct = pl * __builtin_fmaf(y, __builtin_fmaf(y, m2, m1), m0);
  const float wv = small ? wt : w;
  const float lv = small ? lt : l;
  const float cv = ay < 0.25f ? ct : c;
  if constexpr (MASKED) {
    W = exists ? wv : Lprev;
    L = exists ? lv : 0.0f;
    C = exists ? cv : 0.0f;
  } else {
    W = wv;
    L = lv;
    C = cv;
  }
}

// P and dS of one lane's 16 consecutive keys base+t of its query, rounded to bf16 (to nearest
// even) as they are formed: P8[h][e], dS8[h][e] for key base + 8h + e.  s/dp: logits and
// dO.v - D_t of those keys (the dP products start from -D_t: the softmax term of dS is then
// P dp, and the differences of dp in the edge terms do not change); sl, dpl and sr, dpr: the
// same for keys base-1 and base+16.  Key base+t is
// visible iff t <= lim.  Also returns P and dS of key base-1 (float) as they follow from its
// right edge alone: exact when key base-1 is position 0 (which has no left edge).
// MASKED = false when every key of the tile and its right neighbour are visible (lim >= 16 in
// every lane).
template <bool MASKED, typename Emit>
__device__ __forceinline__ void tile_grad(const float (&s)[16], const float (&dp)[16], float sl, float dpl,
                                          float sr, float dpr, float mu, int lim, Emit&& emit,
                                          float& p_left, float& ds_left) {
#pragma clang fp contract(off)
  bf16x8 P8, dS8;
  // Opaque copies of the inputs: callers inline the masked and the unmasked form behind one
  // branch, and without them the compiler computed everything the two forms share (every
  // exponential and difference of the tile) above the branch, all live at once (spills).
  float mu_o = mu, dpl_o = dpl, dpr_o = dpr;
  asm volatile("" : "+v"(mu_o), "+v"(dpl_o), "+v"(dpr_o));
  float dpo[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    dpo[t] = dp[t];
    asm volatile("" : "+v"(dpo[t]));
  }
  auto alpha = [&](float x) { return __builtin_fmaf(x, kLog2e, -mu_o); };
  float aC = alpha(sl), pC = exp2_fast(aC), dC = dpl_o;
  float aN = alpha(s[0]), pN = exp2_fast(aN), dN = dpo[0];
  float W, L, C;
  edge_grad<MASKED>(aC, pC, aN, pN, 0 <= lim, 0.0f, W, L, C);
  float G = C * (dC - dN);
  p_left = W;
  ds_left = __builtin_fmaf(W, dC, -G);
  float Lprev = L, Gprev = G;
  aC = aN;
  pC = pN;
  dC = dN;
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    if (t < 15) {
      aN = alpha(s[t + 1]);
      dN = dpo[t + 1];
    } else {
      aN = alpha(sr);
      dN = dpr_o;
    }
    pN = exp2_fast(aN);
    edge_grad<MASKED>(aC, pC, aN, pN, t + 1 <= lim, Lprev, W, L, C);
    G = C * (dC - dN);
    P8[t & 7] = (bf16)W;
    dS8[t & 7] = (bf16)__builtin_fmaf(W, dC, Gprev - G);
    if ((t & 7) == 7) emit(t >> 3, P8, dS8);  // keys 8h .. 8h + 7 done
    if ((t & 3) == 3) __builtin_amdgcn_sched_barrier(0);  // bounds how far work is hoisted (registers)
    Lprev = L;
    Gprev = G;
    aC = aN;
    pC = pN;
    dC = dN;
  }
}

// ---------------------------------------------------------------- shared per-wave pieces
template <int D>
struct WaveTile {
  static constexpr int CH = D / 8;
  static constexpr int ROWB = 2 * D;
  static constexpr int NSTEP = D / 32;
  static constexpr int NMB = D / 16;
  static constexpr int TILE = kTile * ROWB;  // 64 rows
  // Halo block: 16 rows (keys J-1, J+64, then 14 zero rows) at a pitch of one row plus 16
  // bytes, so that the 16 rows one lane group reads for an MFMA operand start on 16 different
  // 16-byte bank slots (an unpadded pitch put all of them on the same banks).
  static constexpr int HROW = ROWB + 16;
  static constexpr int HALO = 16 * HROW;
};

// Byte offset of chunk `chunk` (0 .. 14 CH - 1) of the zero rows 2..15 of a halo block.
template <int D>
__device__ __forceinline__ int halo_zero_off(int chunk) {
  return (2 + chunk / (D / 8)) * WaveTile<D>::HROW + 16 * (chunk % (D / 8));
}

// LDS read bases of a lane (the attn16 forms)
__device__ __forceinline__ int row_kbase(int n, int g) { return (4 * (n & 3) + (n >> 2)) * 64 + 16 * (g ^ (n & 3)); }
__device__ __forceinline__ void tr_vbase(int n, int g, int (&vb)[2]) {
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int cc = 2 * par + ((n >> 1) & 1);
    vb[par] = (16 * g + (n >> 2)) * 64 + 16 * (cc ^ (2 * (g & 1))) + 8 * (n & 1);
  }
}

// S^T (or dP^T) of 16 queries x 64 keys from a row-layout tile, plus the halo block
// (rows 0, 1 = keys J-1, J+64) -> lanes g = 0 get them in elements 0 and 1.
template <int D>
__device__ __forceinline__ void logits_tile(CSA_LDS const char* tile, CSA_LDS const char* halo, int kbase,
                                            int hoff, const bf16x8 (&b)[D / 32], float c0, float (&s)[16],
                                            f32x4& H) {
  constexpr int NSTEP = D / 32;
  const f32x4 init = {c0, c0, c0, c0};  // every accumulator element belongs to the lane's query
  f32x4 S[4];
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    S[blk] = init;
#pragma unroll
    for (int st = 0; st < NSTEP; ++st)
      S[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(row_read(tile, kbase, st, blk), b[st], S[blk], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);  // one block's operands in flight at a time (register pressure)
  }
  H = init;
#pragma unroll
  for (int st = 0; st < NSTEP; ++st) {
    const bf16x8 a = *(CSA_LDS const bf16x8*)(halo + hoff + st * 64);
    H = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[st], H, 0, 0, 0);
  }
#pragma unroll
  for (int t = 0; t < 16; ++t) s[t] = S[t >> 2][t & 3];
}

// Neighbour values of a lane's 16 keys: key base-1 from the previous lane group (or, for
// g = 0, the halo's key J-1), key base+16 from the next (or, for g = 3, key J+64).
__device__ __forceinline__ void neighbours(const float (&x)[16], const f32x4& H, int n, int g, float& left,
                                           float& right) {
  const int lane = (g << 4) | n;
  const int lane_up = (lane - 16) & 63, lane_dn = (lane + 16) & 63;
  const float l = __int_as_float(__builtin_amdgcn_ds_bpermute(lane_up << 2, __float_as_int(x[15])));
  const float r = __int_as_float(__builtin_amdgcn_ds_bpermute(lane_dn << 2, __float_as_int(x[0])));
  const float h1 = __int_as_float(__builtin_amdgcn_ds_bpermute(n << 2, __float_as_int(H[1])));
  left = g == 0 ? H[0] : l;
  right = g == 3 ? h1 : r;
}

// Source chunk and row (0 = left, 1 = right) of the 16-byte halo slot that lane `lane` fills
// (lane i writes LDS bytes 16 i .. 16 i + 15 of the block): lanes 0 .. CH-1 fill row 0, lane CH
// the pad after it (with a copy of row 1's chunk 0), lanes CH+1 .. 2 CH row 1.
template <int D>
__device__ __forceinline__ int halo_src_chunk(int lane, bool& right) {
  constexpr int CH = D / 8;
  right = lane >= CH;
  return right ? max(lane - CH - 1, 0) : lane;
}

// Stage the halo rows: K rows (J-1, J+64) into halo rows 0, 1 and the same V rows into the
// V halo, from per-lane addresses (row J-1 of position 0 is k0 / v0).  Wave-uniform caller.
template <int D>
__device__ __forceinline__ void stage_halo(CSA_LDS char* khalo, CSA_LDS char* vhalo, const char* kleft,
                                           const char* kright, const char* vleft, const char* vright, int lane) {
  constexpr int CH = D / 8;
  if (lane <= 2 * CH) {
    bool right;
    const int c = halo_src_chunk<D>(lane, right);
    lds_copy16_ptr((right ? kright : kleft) + 16 * c,
                   __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)khalo));
    lds_copy16_ptr((right ? vright : vleft) + 16 * c,
                   __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)vhalo));
  }
}

// Stage 64 rows starting at row0 (rows past T repeat row T-1, so every address stays inside
// the tensor) into dst; off = the calling thread's source offset for round 0 of the layout.
template <int D>
__device__ __forceinline__ void stage_tile(CSA_LDS char* dst, const char* src, int row0, int off, int Tn,
                                           int wave) {
  constexpr int ROWB = 2 * D, CH = D / 8, ROUNDS = (kTile * CH + 511) / 512;
  const int base_row = min(row0, Tn - 1);
  const int row = off / ROWB;
  off += (min(row0 + row, Tn - 1) - base_row - row) * ROWB;
  const char* base = src + (size_t)base_row * ROWB;
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    if (r * 512 + wave * 64 < kTile * CH) {  // wave-uniform
      const unsigned d = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(dst + (r * 512 + wave * 64) * 16));
      lds_copy16(base + 128 * r, off, d);
    }
  }
}

// ---------------------------------------------------------------- kernels
template <int D>
__global__ void __launch_bounds__(512, 2) bwd_dq_kernel(BwdParams p) {
  using WT = WaveTile<D>;
  constexpr int CH = WT::CH, ROWB = WT::ROWB, NSTEP = WT::NSTEP, NMB = WT::NMB;
  constexpr int TILE = WT::TILE, HALO = WT::HALO;
  constexpr int BUF = 3 * TILE + 2 * HALO;  // Krow | Ktr | Vrow | Khalo | Vhalo
  static_assert(D == 64 || D == 128, "head dimension");

  __shared__ __attribute__((aligned(1024))) char smem[2 * BUF];
  CSA_LDS char* lds = (CSA_LDS char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int Tn = p.T, BH = p.B * p.H;
  const int nqb = (Tn + kBlockRows - 1) / kBlockRows;
  int bhl, qrank;
  xcd_head_order<4>(blockIdx.x, p.nh, nqb, bhl, qrank);  // as the forward, over the launch's heads
  const int bh = p.h0 + bhl;
  const int qb = nqb - 1 - qrank;                        // longest query blocks first
  const int q0 = qb * kBlockRows;
  const int qw = q0 + 16 * wave;
  const int qr = qw + n;
  const bool wave_rows = qw < Tn;
  const int jw = wave_rows ? min(qw + 15, Tn - 1) / kTile : -1;
  const int jmax = min(q0 + kBlockRows - 1, Tn - 1) / kTile;
  const BwdWs ws = bwd_ws(p.ws, BH, Tn, D);

  const size_t head = (size_t)bh * (size_t)Tn * D;
  const char* Kg = (const char*)((const bf16*)p.k + head);
  const char* Vg = (const char*)((const bf16*)p.v + head);
  const char* K0 = p.k0 ? (const char*)((const bf16*)p.k0 + (size_t)bh * D) : ws.zero;
  const char* V0 = p.v0 ? (const char*)((const bf16*)p.v0 + (size_t)bh * D) : ws.zero;

  // zero rows 2..15 of both halo buffers (never written again)
  for (int i = tid; i < 2 * 2 * 14 * CH; i += 512) {
    const int buf = i / (2 * 14 * CH), rest = i % (2 * 14 * CH);
    const int which = rest / (14 * CH), chunk = rest % (14 * CH);
    *(CSA_LDS f32x4*)(lds + buf * BUF + 3 * TILE + which * HALO + halo_zero_off<D>(chunk)) = f32x4{};
  }

  const int roff = row_layout_src<ROWB>(tid), toff = tr_layout_src<ROWB>(tid);
  auto stage = [&](int buf, int tile) {
    CSA_LDS char* b = lds + buf * BUF;
    stage_tile<D>(b, Kg, tile * kTile, roff, Tn, wave);
    stage_tile<D>(b + TILE, Kg, tile * kTile, toff, Tn, wave);
    stage_tile<D>(b + 2 * TILE, Vg, tile * kTile, roff, Tn, wave);
    if (wave == 0) {
      const int J = tile * kTile;
      const int rr = min(J + kTile, Tn - 1);
      stage_halo<D>(b + 3 * TILE, b + 3 * TILE + HALO, J > 0 ? Kg + (size_t)(J - 1) * ROWB : K0,
                    Kg + (size_t)rr * ROWB, J > 0 ? Vg + (size_t)(J - 1) * ROWB : V0, Vg + (size_t)rr * ROWB, lane);
    }
  };

  // per-query operands: Q and dO rows (chunk 4s + g), mu_t and D_t
  bf16x8 qreg[NSTEP], dreg[NSTEP];
  const int rowc = min(qr, Tn - 1);
  {
    const bf16* Qg = (const bf16*)p.q + head + (size_t)rowc * D;
    const bf16* Dg = (const bf16*)p.dout + head + (size_t)rowc * D;
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      qreg[s] = *(const bf16x8*)(Qg + (4 * s + g) * 8);
      dreg[s] = *(const bf16x8*)(Dg + (4 * s + g) * 8);
    }
  }
  const float mu = ws.mu[(size_t)bh * Tn + rowc];
  const float delta = ws.delta[(size_t)bh * Tn + rowc];

  const int kbase = row_kbase(n, g);
  int vbase[2];
  tr_vbase(n, g, vbase);
  const int hoff = n * WT::HROW + 16 * g;

  f32x4 acc[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) acc[mb] = f32x4{};
  float ds0 = 0.0f, p0 = 0.0f;  // position 0 (lanes g = 0)

  stage(0, 0);
  wait_vmem();
  __syncthreads();
  for (int j = 0; j <= jmax; ++j) {
    if (j + 1 <= jmax) stage((j + 1) & 1, j + 1);
    if (j <= jw) {
      CSA_LDS const char* b = lds + (j & 1) * BUF;
      float s[16], dp[16];
      f32x4 Hs, Hd;
      logits_tile<D>(b, b + 3 * TILE, kbase, hoff, qreg, 0.0f, s, Hs);
      logits_tile<D>(b + 2 * TILE, b + 3 * TILE + HALO, kbase, hoff, dreg, -delta, dp, Hd);
      float sl, sr, dl, dr;
      neighbours(s, Hs, n, g, sl, sr);
      neighbours(dp, Hd, n, g, dl, dr);
      int lim = qr < Tn ? qr - (j * kTile + 16 * g) : -2;
      bf16x8 dS8[2];
      float pl, dsl;
      auto keep = [&](int h, const bf16x8&, const bf16x8& ds) { dS8[h] = ds; };
      // every edge of the tile exists for every query of the wave (rows past T only feed
      // their own, unstored, dq rows)
      if ((j + 1) * kTile <= qw) tile_grad<false>(s, dp, sl, dl, sr, dr, mu, lim, keep, pl, dsl);
      else tile_grad<true>(s, dp, sl, dl, sr, dr, mu, lim, keep, pl, dsl);
      if (j == 0) {
        p0 = pl;
        ds0 = dsl;
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
          acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tr_read(b + TILE, vbase, c, mb), dS8[c], acc[mb], 0, 0, 0);
      }
    }
    wait_vmem();
    __syncthreads();
  }
  if (!wave_rows) return;

  // dq = (K^T dS^T)^T + dS_{t,0} k_0;  position 0's P and dS for the k_0 / v_0 gradients
  const float ds0q = __int_as_float(__builtin_amdgcn_ds_bpermute(n << 2, __float_as_int(ds0)));
  if (qr < Tn) {
    const bf16* k0v = p.k0 ? (const bf16*)p.k0 + (size_t)bh * D : nullptr;
    bf16* out = (bf16*)p.dq + head + (size_t)qr * D;
    bf16x4 k0r[NMB];  // this lane's elements of k_0, every load issued before the first is used
    if (k0v) {
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) k0r[mb] = *(const bf16x4*)(k0v + 16 * mb + 4 * g);
    }
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      const int d0 = 16 * mb + 4 * g;
      float o4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        o4[r] = acc[mb][r];
        if (k0v) o4[r] = __builtin_fmaf(ds0q, (float)k0r[mb][r], o4[r]);
      }
      *(bf16x4*)(out + d0) = bf16x4{(bf16)o4[0], (bf16)o4[1], (bf16)o4[2], (bf16)o4[3]};
    }
    if (g == 0) {
      ws.ds0[(size_t)bh * Tn + qr] = ds0;
      ws.p0[(size_t)bh * Tn + qr] = p0;
    }
  }
}

// dq from the dS tiles bwd_dkdv<D, true> stored: the forward's decomposition (128 query rows
// per work-group, wave w owns rows 16 w .. 16 w + 15), K tiles in the transposed LDS layout,
// dQ^T += K^T dS^T on MFMAs with dS (bf16) read straight into the B operand; the same
// products in the same order as bwd_dq, so the two paths give identical results.
template <int D>
__global__ void __launch_bounds__(512, 2) bwd_dq_from_ds_kernel(BwdParams p) {
  using WT = WaveTile<D>;
  constexpr int ROWB = WT::ROWB, NMB = WT::NMB, TILE = WT::TILE;
  static_assert(D == 64 || D == 128, "head dimension");

  __shared__ __attribute__((aligned(1024))) char smem[2 * TILE];  // K (transposed), two buffers
  CSA_LDS char* lds = (CSA_LDS char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int Tn = p.T, BH = p.B * p.H;
  const int nqb = (Tn + kBlockRows - 1) / kBlockRows;
  int bhl, qrank;
  xcd_head_order<4>(blockIdx.x, p.nh, nqb, bhl, qrank);  // as the forward, over the launch's heads
  const int bh = p.h0 + bhl;
  const int qb = nqb - 1 - qrank;                        // longest query blocks first
  const int q0 = qb * kBlockRows;
  const int qw = q0 + 16 * wave;
  const int qr = qw + n;
  const bool wave_rows = qw < Tn;
  const int jw = wave_rows ? min(qw + 15, Tn - 1) / kTile : -1;
  const int jmax = min(q0 + kBlockRows - 1, Tn - 1) / kTile;
  const BwdWs ws = bwd_ws(p.ws, BH, Tn, D);

  const size_t head = (size_t)bh * (size_t)Tn * D;
  const char* Kg = (const char*)((const bf16*)p.k + head);
  const char* dsl = p.ds + ((size_t)bhl * (size_t)p.ds_tiles + (size_t)ds_tile_index(qb, 0)) * kDsTileBytes +
                    (size_t)(wave * 2048 + lane * 16);
  const int toff = tr_layout_src<ROWB>(tid);
  int vbase[2];
  tr_vbase(n, g, vbase);

  f32x4 acc[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) acc[mb] = f32x4{};
  bf16x8 bc[2], bn[2];
  auto load_ds = [&](int j, bf16x8 (&b)[2]) {
    const char* src = dsl + (size_t)j * kDsTileBytes;
    b[0] = __builtin_nontemporal_load((const bf16x8*)src);
    b[1] = __builtin_nontemporal_load((const bf16x8*)(src + 1024));
  };
  if (jw >= 0) load_ds(0, bc);
  stage_tile<D>(lds, Kg, 0, toff, Tn, wave);
  wait_vmem();
  __syncthreads();
  for (int j = 0; j <= jmax; ++j) {
    if (j + 1 <= jmax) stage_tile<D>(lds + ((j + 1) & 1) * TILE, Kg, (j + 1) * kTile, toff, Tn, wave);
    if (j + 1 <= jw) load_ds(j + 1, bn);
    if (j <= jw) {
      CSA_LDS const char* b = lds + (j & 1) * TILE;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
          acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tr_read(b, vbase, c, mb), bc[c], acc[mb], 0, 0, 0);
      }
    }
    bc[0] = bn[0];
    bc[1] = bn[1];
    wait_vmem();
    __syncthreads();
  }
  if (!wave_rows || qr >= Tn) return;

  // dq = (K^T dS^T)^T + dS_{t,0} k_0
  const float ds0 = ws.ds0[(size_t)bh * Tn + qr];
  const bf16* k0v = p.k0 ? (const bf16*)p.k0 + (size_t)bh * D : nullptr;
  bf16* out = (bf16*)p.dq + head + (size_t)qr * D;
  bf16x4 k0r[NMB];  // this lane's elements of k_0, every load issued before the first is used
  if (k0v) {
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) k0r[mb] = *(const bf16x4*)(k0v + 16 * mb + 4 * g);
  }
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
    const int d0 = 16 * mb + 4 * g;
    float o4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      o4[r] = acc[mb][r];
      if (k0v) o4[r] = __builtin_fmaf(ds0, (float)k0r[mb][r], o4[r]);
    }
    *(bf16x4*)(out + d0) = bf16x4{(bf16)o4[0], (bf16)o4[1], (bf16)o4[2], (bf16)o4[3]};
  }
}

// dk_0 = sum_t dS_{t,0} q_t and dv_0 = sum_t P_{t,0} dO_t in two passes: kSinkChunks
// work-groups per (b, h) each sum a contiguous range of query rows into float32 partials
// in the workspace; one work-group per (b, h) adds the partials (fixed order: the result
// does not depend on scheduling) and rounds once.

template <int D>
__global__ void __launch_bounds__(256) bwd_sink_partial_kernel(BwdParams p) {
  constexpr int CH = D / 8;
  constexpr int NPH = 256 / CH;  // row phases
  __shared__ float red[2][NPH][D];
  const int BH = p.B * p.H, Tn = p.T;
  const BwdWs ws = bwd_ws(p.ws, BH, Tn, D);
  const int bh = blockIdx.x / kSinkChunks, chunk = blockIdx.x % kSinkChunks;
  const int rows = (Tn + kSinkChunks - 1) / kSinkChunks;
  const int t0 = chunk * rows, t1 = min(Tn, t0 + rows);
  const int c = threadIdx.x % CH, ph = threadIdx.x / CH;
  const size_t head = (size_t)bh * (size_t)Tn * D;
  float ak[8] = {}, av[8] = {};
  for (int t = t0 + ph; t < t1; t += NPH) {
    const float a = ws.ds0[(size_t)bh * Tn + t];
    const float b = ws.p0[(size_t)bh * Tn + t];
    const bf16x8 qv = *(const bf16x8*)((const bf16*)p.q + head + (size_t)t * D + 8 * c);
    const bf16x8 dv = *(const bf16x8*)((const bf16*)p.dout + head + (size_t)t * D + 8 * c);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ak[e] = __builtin_fmaf(a, (float)qv[e], ak[e]);
      av[e] = __builtin_fmaf(b, (float)dv[e], av[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    red[0][ph][8 * c + e] = ak[e];
    red[1][ph][8 * c + e] = av[e];
  }
  __syncthreads();
  if (threadIdx.x < 2 * D) {
    const int which = threadIdx.x / D, d = threadIdx.x % D;
    float sum = 0.0f;
    for (int i = 0; i < NPH; ++i) sum += red[which][i][d];
    ws.sink[((size_t)bh * kSinkChunks + chunk) * 2 * D + which * D + d] = sum;
  }
}

template <int D>
__global__ void __launch_bounds__(256) bwd_sink_final_kernel(BwdParams p) {
  const int BH = p.B * p.H;
  const BwdWs ws = bwd_ws(p.ws, BH, p.T, D);
  const int bh = blockIdx.x;
  if (threadIdx.x < 2 * D) {
    const int which = threadIdx.x / D, d = threadIdx.x % D;
    float sum = 0.0f;
    for (int i = 0; i < kSinkChunks; ++i) sum += ws.sink[((size_t)bh * kSinkChunks + i) * 2 * D + which * D + d];
    bf16* dst = (bf16*)(which == 0 ? p.dk0 : p.dv0);
    if (dst) dst[(size_t)bh * D + d] = (bf16)sum;
  }
}

// Q^T and dO^T of every head into the workspace ([B*H][D][Tp] bf16, zeros past T): one
// work-group per (head, 64-row tile, tensor) stages the rows in LDS at a pitch of D/2 + 1 words
// (the 8 rows one lane reads for a column fall on distinct banks across the wave) and writes 8
// consecutive rows of one column per lane, 8 lanes covering one column's 128 bytes.
template <int D>
__global__ void __launch_bounds__(256) bwd_transpose_kernel(BwdParams p) {
  constexpr int PW = D / 2 + 1;  // words per staged row
  __shared__ unsigned buf[64 * PW];
  const int BH = p.B * p.H, Tn = p.T;
  const int Tp = (int)bwd_tp(Tn), ntile = Tp / 64;
  const int which = blockIdx.x & 1, tile = (blockIdx.x >> 1) % ntile, bh = (blockIdx.x >> 1) / ntile;
  const BwdWs ws = bwd_ws(p.ws, BH, Tn, D);
  const bf16* src = (const bf16*)(which ? p.dout : p.q) + (size_t)bh * Tn * D;
  if (blockIdx.x == 0 && threadIdx.x < kBwdZeroBytes / 4) ((float*)p.ws)[threadIdx.x] = 0.0f;
  for (int i = threadIdx.x; i < 64 * D / 8; i += 256) {
    const int r = i / (D / 8), c = i % (D / 8), t = tile * 64 + r;
    uint4 v = {0u, 0u, 0u, 0u};
    if (t < Tn) v = *(const uint4*)(src + (size_t)t * D + 8 * c);
    unsigned* w = buf + r * PW + 4 * c;
    w[0] = v.x;
    w[1] = v.y;
    w[2] = v.z;
    w[3] = v.w;
    if (which) {  // the dO work-groups also form D_t = dO_t . o_t and mu_t of their rows
      float acc = 0.0f;
      if (t < Tn) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, v);
        const bf16x8 b = *(const bf16x8*)((const bf16*)p.o + (size_t)bh * Tn * D + (size_t)t * D + 8 * c);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)a[e], (float)b[e], acc);
      }
#pragma unroll
      for (int m = 1; m < D / 8; m <<= 1) acc += __shfl_xor(acc, m);  // the D/8 lanes of row r
      if (t < Tn && c == 0) {
        const size_t row = (size_t)bh * Tn + t;
        ws.delta[row] = acc;
        ws.mu[row] = __builtin_fmaf(p.lse[row], kLog2e, kMuShift);
      }
    }
  }
  __syncthreads();
  bf16* dst = (which ? ws.dot : ws.qt) + (size_t)bh * D * Tp + tile * 64;
  const bf16* sb = (const bf16*)buf;
  for (int i = threadIdx.x; i < D * 8; i += 256) {
    const int tc = i & 7, dcol = i >> 3;
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = sb[(8 * tc + e) * (2 * PW) + dcol];
    *(bf16x8*)(dst + (size_t)dcol * Tp + 8 * tc) = o;
  }
}

// dK and dV: one work-group (8 waves) per 64 key rows, looping over the 128-row query blocks
// from the key block on.  Per block each wave forms S^T and dP^T of its 16 queries on the
// MFMAs (K, V and the halo rows staged once in LDS), then P and dS (tile_grad), which go to
// LDS in the transposed layout; after a barrier dK^T += Q^T dS and dV^T += dO^T P contract
// over the block's 128 queries on the MFMAs, wave w owning d-block w % (D/16) of dK and dV
// for KPW 16-key blocks.  The A operands Q^T, dO^T come from the transposed copies in the
// workspace (16 contiguous bytes per lane), so the work-group holds only K, V, halo, P and dS
// in LDS (73 KiB at d = 128) and two work-groups share a CU: four waves per SIMD.
// WRITE_DS: also store this wave's dS into its dS tile (for bwd_dq_from_ds) and, for the
// first key block, P and dS of position 0 (for the k_0 / v_0 gradients and dq's k_0 term).
template <int D, bool WRITE_DS>
__global__ void __launch_bounds__(512, 4) bwd_dkdv_kernel(BwdParams p) {
  using WT = WaveTile<D>;
  constexpr int ROWB = WT::ROWB, NSTEP = WT::NSTEP, NMB = WT::NMB;
  constexpr int TILE = WT::TILE, HALO = WT::HALO;
  constexpr int CH = WT::CH;
  constexpr int PT = 2 * 64 * 128;  // P or dS: 128 queries x 64 keys bf16 (two 64-row tiles)
  // Krow | Vrow | Khalo | Vhalo | P | dS
  constexpr int OFF_V = TILE, OFF_KH = 2 * TILE, OFF_VH = 2 * TILE + HALO, OFF_P = 2 * TILE + 2 * HALO;
  constexpr int OFF_DS = OFF_P + PT;
  constexpr int LDS_BYTES = OFF_DS + PT;
  constexpr int KPW = 4 * NMB / 8;  // 16-key blocks per wave: 4 at d = 128, 2 at d = 64
  static_assert(D == 64 || D == 128, "head dimension");

  __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];
  CSA_LDS char* lds = (CSA_LDS char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int Tn = p.T, BH = p.B * p.H;
  const int Tp = (int)bwd_tp(Tn);
  // heads four at a time per XCD, key block 0 (the most queries) first
  int bhl, kb;
  xcd_head_order<4>(blockIdx.x, p.nh, (Tn + kTile - 1) / kTile, bhl, kb);
  const int bh = p.h0 + bhl;
  const int J = kb * kTile;
  const BwdWs ws = bwd_ws(p.ws, BH, Tn, D);

  const size_t head = (size_t)bh * (size_t)Tn * D;
  const char* Kg = (const char*)((const bf16*)p.k + head);
  const char* Vg = (const char*)((const bf16*)p.v + head);
  const char* Qg = (const char*)((const bf16*)p.q + head);
  const char* Og = (const char*)((const bf16*)p.dout + head);
  const char* K0 = p.k0 ? (const char*)((const bf16*)p.k0 + (size_t)bh * D) : ws.zero;
  const char* V0 = p.v0 ? (const char*)((const bf16*)p.v0 + (size_t)bh * D) : ws.zero;

  for (int i = tid; i < 2 * 14 * CH; i += 512) {
    const int which = i / (14 * CH), chunk = i % (14 * CH);
    *(CSA_LDS f32x4*)(lds + OFF_KH + which * HALO + halo_zero_off<D>(chunk)) = f32x4{};
  }
  const int roff = row_layout_src<ROWB>(tid);
  // the key block and its halo rows, once
  stage_tile<D>(lds, Kg, J, roff, Tn, wave);
  stage_tile<D>(lds + OFF_V, Vg, J, roff, Tn, wave);
  if (wave == 0) {
    const int rr = min(J + kTile, Tn - 1);
    stage_halo<D>(lds + OFF_KH, lds + OFF_VH, J > 0 ? Kg + (size_t)(J - 1) * ROWB : K0, Kg + (size_t)rr * ROWB,
                  J > 0 ? Vg + (size_t)(J - 1) * ROWB : V0, Vg + (size_t)rr * ROWB, lane);
  }

  const int kbase = row_kbase(n, g);
  int vbase[2];
  tr_vbase(n, g, vbase);
  const int hoff = n * WT::HROW + 16 * g;
  // this wave's output blocks: d-block mb, 16-key blocks kc0 .. kc0 + KPW - 1
  const int mb = wave % NMB;
  const int kc0 = KPW * (wave / NMB);
  f32x4 dK[KPW], dV[KPW];
#pragma unroll
  for (int i = 0; i < KPW; ++i) dK[i] = dV[i] = f32x4{};
  // A operands of the dK / dV products: row 16 mb + n of Q^T / dO^T, 8 queries per lane group
  // (uniform bases and 32-bit per-lane offsets: one VGPR per address)
  const bf16* qt_head = ws.qt + (size_t)bh * D * Tp;
  const bf16* dot_head = ws.dot + (size_t)bh * D * Tp;
  const int row_off = (16 * mb + n) * Tp;

  // P / dS rows of this wave in LDS: query tile row 16 wave + n = tile (wave >> 2), row 16 (wave & 3) + n
  const int prow = 16 * (wave & 3) + n;
  const int pt_off = (wave >> 2) * (PT / 2);

  const int i0 = J / kBlockRows;
  const int i1 = (Tn - 1) / kBlockRows;
  wait_vmem();  // the key block and its halo
  __syncthreads();
  for (int it = i0; it <= i1; ++it) {
    const int Q0 = it * kBlockRows;
    const int qr = Q0 + 16 * wave + n;
    // this wave's query rows (the logits' B operands), one tensor at a time (registers)
    const int rowc = min(qr, Tn - 1);
    float s[16], dp[16];
    f32x4 Hs, Hd;
    // The logits products run at the lowest wave priority and the rest of the block at the
    // next one, so that a SIMD issues its other waves' gradient (VALU) work ahead of a wave's
    // logits (A/B on lm: about 1% faster than equal priorities; prioritising the products
    // instead was 1% slower).
    __builtin_amdgcn_s_setprio(0);
    bf16x8 dreg[NSTEP];
    float delta, mu;
    {
      bf16x8 qreg[NSTEP];
#pragma unroll
      for (int st = 0; st < NSTEP; ++st) qreg[st] = *(const bf16x8*)(Qg + (rowc * ROWB + (4 * st + g) * 16));
      // the dO rows are issued with the Q rows, so that their latency passes under the S product
#pragma unroll
      for (int st = 0; st < NSTEP; ++st) dreg[st] = *(const bf16x8*)(Og + (rowc * ROWB + (4 * st + g) * 16));
      delta = (ws.delta + (size_t)bh * Tn)[rowc];
      mu = (ws.mu + (size_t)bh * Tn)[rowc];
      logits_tile<D>(lds, lds + OFF_KH, kbase, hoff, qreg, 0.0f, s, Hs);
    }
    __builtin_amdgcn_sched_barrier(0);
    logits_tile<D>(lds + OFF_V, lds + OFF_VH, kbase, hoff, dreg, -delta, dp, Hd);
    __builtin_amdgcn_s_setprio(1);
    float sl, sr, dl, dr;
    neighbours(s, Hs, n, g, sl, sr);
    neighbours(dp, Hd, n, g, dl, dr);
    const int lim = qr < Tn ? qr - (J + 16 * g) : -2;
    float pl, dsl;
    // keys 16g + 8h + e = chunks 2g + h of the P / dS row: to LDS (and dS to its tile) as soon
    // as the 8 keys of a half are done
    auto emit = [&](int h, const bf16x8& pv, const bf16x8& dv) {
      const int at = pt_off + ptr_layout_at(prow, 2 * g + h);
      *(CSA_LDS bf16x8*)(lds + OFF_P + at) = pv;
      *(CSA_LDS bf16x8*)(lds + OFF_DS + at) = dv;
      if constexpr (WRITE_DS)  // uniform tile base, 32-bit lane offset
        __builtin_nontemporal_store(dv, (bf16x8*)(p.ds + ((size_t)bhl * (size_t)p.ds_tiles +
                                                          (size_t)ds_tile_index(it, kb)) * kDsTileBytes +
                                                 (wave * 2048 + h * 1024 + lane * 16)));
    };
    // every edge exists for every query of the wave, and no row of the wave lies past T
    // (those rows must contribute zeros to dK and dV)
    const int qw = Q0 + 16 * wave;
    if (qw >= J + kTile && qw + 15 < Tn) tile_grad<false>(s, dp, sl, dl, sr, dr, mu, lim, emit, pl, dsl);
    else tile_grad<true>(s, dp, sl, dl, sr, dr, mu, lim, emit, pl, dsl);
    if constexpr (WRITE_DS) {
      if (J == 0 && g == 0 && qr < Tn) {
        (ws.p0 + (size_t)bh * Tn)[qr] = pl;
        (ws.ds0 + (size_t)bh * Tn)[qr] = dsl;
      }
    }
    // the block's Q^T / dO^T operands: 4 steps of 32 queries, step (st, c) = queries
    // Q0 + 64 st + 16 g + 8 c .. + 7 for lane group g (the rows the P / dS reads below take)
    bf16x8 aq[4], ad[4];
    __builtin_amdgcn_sched_barrier(0);  // not hoisted above the gradients (registers)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int off = Q0 + 64 * (u >> 1) + 16 * g + 8 * (u & 1);
      aq[u] = *(const bf16x8*)(qt_head + (row_off + off));
      ad[u] = *(const bf16x8*)(dot_head + (row_off + off));
    }
    __syncthreads();
    // dV^T += dO^T P and dK^T += Q^T dS over the block's 128 queries (4 steps of 32)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int st = u >> 1, c = u & 1;
      // the read bases formed here, from opaque copies (hoisted out of the loop they stayed live
      // across the gradients: 16 registers, spilled)
      int vb[2] = {vbase[0], vbase[1]};
      asm volatile("" : "+v"(vb[0]), "+v"(vb[1]));
      int pbase[2][4];
      ptr_bases(vb, pbase);
#pragma unroll
      for (int i = 0; i < KPW; ++i) {
        const bf16x8 bs = ptr_read(lds + OFF_DS + st * (PT / 2), pbase, c, kc0 + i);
        const bf16x8 bp = ptr_read(lds + OFF_P + st * (PT / 2), pbase, c, kc0 + i);
        dK[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[u], bs, dK[i], 0, 0, 0);
        dV[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ad[u], bp, dV[i], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // lane (n, g) holds dK^T[16 mb + 4g + r][key 16 kc + n]
#pragma unroll
  for (int i = 0; i < KPW; ++i) {
    const int row = J + 16 * (kc0 + i) + n;
    if (row < Tn) {
      const int d0 = 16 * mb + 4 * g;
      bf16* ok = (bf16*)p.dk + head + (size_t)row * D + d0;
      bf16* ov = (bf16*)p.dv + head + (size_t)row * D + d0;
      const f32x4 k4 = dK[i], v4 = dV[i];
      *(bf16x4*)ok = bf16x4{(bf16)k4[0], (bf16)k4[1], (bf16)k4[2], (bf16)k4[3]};
      *(bf16x4*)ov = bf16x4{(bf16)v4[0], (bf16)v4[1], (bf16)v4[2], (bf16)v4[3]};
    }
  }
}

// prm.h0 = 0 and prm.nh = B*H on entry.  With dS kept (prm.ds set), prm.nh is the number of
// heads whose dS tiles fit the workspace: bwd_dkdv and bwd_dq_from_ds run on groups of that
// many heads in turn (the second reads the tiles the first wrote for the same group).
template <int D>
inline hipError_t launch_backward(const BwdParams& prm_in, hipStream_t stream) {
  BwdParams prm = prm_in;
  const int BH = prm.B * prm.H;
  const int group = prm.nh;
  prm.h0 = 0;
  prm.nh = BH;
  hipLaunchKernelGGL((bwd_transpose_kernel<D>), dim3((unsigned)(BH * (bwd_tp(prm.T) / 64) * 2)), dim3(256), 0, stream,
                     prm);
  const int nqb = (prm.T + kBlockRows - 1) / kBlockRows;
  const int nkb = (prm.T + kTile - 1) / kTile;
  auto sink = [&]() {
    if (prm.dk0 != nullptr || prm.dv0 != nullptr) {
      hipLaunchKernelGGL((bwd_sink_partial_kernel<D>), dim3((unsigned)(BH * kSinkChunks)), dim3(256), 0, stream, prm);
      hipLaunchKernelGGL((bwd_sink_final_kernel<D>), dim3((unsigned)BH), dim3(256), 0, stream, prm);
    }
  };
  if (prm.ds != nullptr) {  // dS computed once (in bwd_dkdv) and stored; dq is then a plain product
    for (int h0 = 0; h0 < BH; h0 += group) {
      BwdParams g = prm;
      g.h0 = h0;
      g.nh = BH - h0 < group ? BH - h0 : group;
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, true>), dim3((unsigned)(nkb * g.nh)), dim3(512), 0, stream, g);
      hipLaunchKernelGGL((bwd_dq_from_ds_kernel<D>), dim3((unsigned)(nqb * g.nh)), dim3(512), 0, stream, g);
    }
    sink();  // reads P and dS of position 0, written by bwd_dkdv for every head
  } else {  // dS recomputed by bwd_dq (workspace without the dS tiles)
    hipLaunchKernelGGL((bwd_dq_kernel<D>), dim3((unsigned)(nqb * BH)), dim3(512), 0, stream, prm);
    sink();
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, false>), dim3((unsigned)(nkb * BH)), dim3(512), 0, stream, prm);
  }
  return hipGetLastError();
}

}  // namespace csa
