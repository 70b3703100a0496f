// bf16 causal attention forward for gfx950 on 16x16x32 MFMAs, with four weight rules
// on the identical tiling: continuous softmax attention (kExact), its first-order form
// (kFirstOrder), its interval variant [1/2, t + 1/2] (kHalf) and standard softmax
// attention (kSoftmax).
//
// Method: J. Su, "Continuous Softmax Attention", eq. (10)-(11) -- see attn_fwd.hpp
// for the correction-weight arithmetic ("p-form"), which is shared; the first-order
// form replaces b by the second difference of the logits (Analysis of the Result,
// eq. (13)).
//
// Why a second tiling.  With 32 queries per wave (32x32 MFMAs) the accumulator of
// O^T alone takes 64 VGPRs and the kernel needs ~244, which caps the SIMD at two
// waves; the correction weights are VALU work whose latency (exp/rcp, LDS, MFMA
// results, barriers) and VALU dual issue need other waves.  Here a wave owns 16
// queries: O^T is 32 VGPRs, Q 16, S 16, and four waves fit per SIMD.  Measured with
// the per-key weight arithmetic beside the MFMAs of this ratio (csa_probe kinds 7 and
// 8): the 32x32x16 shape is 2% faster than 16x16x32 at equal occupancy, but two
// waves per SIMD on it take 7% longer than four on 16x16x32 for the same work.
//
// Work decomposition
//   * One work-group = 8 waves = 128 query rows of one (b, h); wave w owns rows
//     q0 + 16w .. +15.  Key tiles are 64 rows of k, double-buffered in LDS.
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16, four 16-key blocks per tile.
//     Lane (n, g) -- n = lane % 16 (query), g = lane / 16 -- receives rows 4g..4g+3
//     of each block; the K operand rows are permuted so that these are keys
//     16g + 4b + r: every lane holds 16 CONSECUTIVE keys of its query, and the
//     four lanes of a query hold the tile in order.  The neighbour stencil of
//     eq. (10) is in-register except at the three group boundaries (exchanged with
//     ds_bpermute) and at the tile's right edge, whose neighbour -- the next tile's
//     first key -- comes from computing block 0 of the next tile's S^T early.
//   * O^T += V^T P^T on 16x16x32 MFMAs with P (bf16) straight from registers
//     (lane (n, g) holds keys 16g + 8c + e of query n for key chunk c), V^T via
//     ds_read_b64_tr_b16.  Row sums take the same bf16-rounded P (v_dot2_f32_bf16
//     against (1, 1)), so numerator and denominator see identical weights.
//
// LDS layouts (16-byte chunks, both filled by global_load_lds_dwordx4; every
// copy instruction of a wave reads whole 64-byte row segments from HBM):
//   K tile: one region per contraction step (4 chunks x 64 rows = 4 KiB); inside
//           it, row r sits in 64-byte slot 4 (r & 3) + (r >> 4) + 16 ((r >> 2) & 3)
//           with its chunk cc at position cc ^ (r & 3).  This is the placement
//           that measured free of LDS bank conflicts for the 16 rows one lane group
//           reads for an MFMA A operand (a plain XOR by r >> 4 was not), and every
//           K address is one per-lane base plus an immediate.
//   V tile: one region per 32 d-columns (4 chunks x 64 rows); chunk cc of row r at
//           position cc ^ 2 bit4(r), so the two half-waves of a transposed read use
//           disjoint banks; one per-lane base per parity of the 16-column block.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "attn_fwd.hpp"

namespace csa {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves16 = 8;  // 8 waves x 16 queries = 128 rows, as kBlockRows

// Weight rule of a launch: standard softmax attention (eq. (12)), continuous softmax
// attention (eq. (10)-(11)), or its first-order form with b expanded as in eq. (13).
enum : int { kSoftmax = 0, kExact = 1, kFirstOrder = 2, kHalf = 3 };

// One 16-byte HBM -> LDS copy per lane (global_load_lds_dwordx4): lane i reads
// base + voff and writes LDS address lds_addr + 16 i (no instruction offset: it would
// move the LDS destination as well).  Issued as inline asm so that the compiler does
// not track it: it would otherwise make every later transposed LDS read wait for all
// copies in flight (it cannot tell the buffers apart).  Completion is awaited
// explicitly (s_waitcnt vmcnt(0) and a barrier) before any wave reads the destination.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_copy16(const char* base, int voff, unsigned lds_addr) {
  // base is wave-uniform by construction; the read-first-lane makes that explicit where the
  // compiler's divergence analysis cannot see it (free when it can)
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)b);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(b >> 32));
  const char* ub = (const char*)(uintptr_t)(((uint64_t)hi << 32) | lo);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(ub), "s"(lds_addr)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(0) as an instruction the compiler sees (so it also knows that its
// own loads, e.g. of Q, have completed and adds no later waits for them).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Edge (t, t+1) of eq. (10) from p_t, p_{t+1}, y = alpha_{t+1} - alpha_t and u = 1/y,
// in the p-form of attn_fwd.hpp (bf16 outputs: Taylor branch below |y| < 0.07).
// Returns w_left = Lprev + (right term of t) and the left term of t+1.
__device__ __forceinline__ void edge_yu(float pl, float pr, float y, float u, float Lprev,
                                        float& w_left, float& L_right) {
  const float du = (pr - pl) * u;
  const float wr = __builtin_fmaf(__builtin_fmaf(-kLn2, pl, du), u, Lprev);
  const float lr = __builtin_fmaf(kLn2, pr, -du) * u;
  float gp, gm;
  Taylor<false>::eval(y, gp, gm);
  const float wt = __builtin_fmaf(pl, gp, Lprev);
  const float lt = pr * gm;
  const bool small = __builtin_fabsf(y) < Taylor<false>::Y0;
  w_left = small ? wt : wr;
  L_right = small ? lt : lr;
}

// The same edge for the off-diagonal tiles, with the series formed only when some lane of the
// wave has |y| < kY0Ballot (a wave-uniform branch on the compare's lane mask).  Between
// kY0Ballot and Taylor<false>::Y0 the closed form is kept: its cancellation turns the two exp2
// roundings (up to 1 ulp each) into a relative error of about 1e-6 / y^2 on R and L, at most
// 3.3e-3 at |y| = 0.02 in a float32 emulation, which is under the bf16 rounding (up to 2^-8
// relative) that every weight takes before the P V product.  Such small neighbour differences
// are rare at the logit scales of attention (about 1% of elements), so a wave skips the series
// on about half of its key steps (64 lanes decide together).
constexpr float kY0Ballot = 0.02f;
__device__ __forceinline__ void edge_yu_ballot(float pl, float pr, float y, float u, float Lprev,
                                               float& w_left, float& L_right) {
  const float du = (pr - pl) * u;
  w_left = __builtin_fmaf(__builtin_fmaf(-kLn2, pl, du), u, Lprev);
  L_right = __builtin_fmaf(kLn2, pr, -du) * u;
  const bool small = __builtin_fabsf(y) < kY0Ballot;
  if (__builtin_amdgcn_ballot_w64(small) != 0) {
    // the lanes that need the series overwrite the closed form under the execution mask (no
    // selects); the wave-uniform test in front skips the block, with no change of the mask,
    // when no lane needs it (a plain divergent branch changed the mask on every key: slower
    // where the series is rare); the empty asm keeps the compiler from folding the two tests
    // into one divergent branch
    asm volatile("");
    if (small) {
      float gp, gm;
      Taylor<false>::eval(y, gp, gm);
      // written into the registers of the closed form (tied operands): as plain code the
      // compiler formed the first in Lprev's register and copied it over
      asm("v_fma_f32 %0, %2, %3, %4\n\tv_mul_f32 %1, %5, %6"
          : "+v"(w_left), "+v"(L_right)
          : "v"(pl), "v"(gp), "v"(Lprev), "v"(pr), "v"(gm));
    }
  }
}

// Work-group i -> (head bh, rank of its block among the head's nblk blocks, 0 = the most work).
// Work-groups go to the 8 XCDs round robin (i -> XCD i mod 8), each XCD with its own 4 MB L2.
// With B*H a multiple of 8 * G, XCD x takes its heads x, x+8, x+16, ... G at a time, each group's
// blocks in rank order with the group's heads interleaved: the blocks resident on an XCD then
// share the key/value (or query/gradient) rows of G heads rather than of every head the XCD
// holds.  G is set by how long one block is against an XCD's share of the launch: the last
// group's biggest blocks must still start early enough not to be left for the end.  Otherwise
// heads fastest, ranks in order.
template <int G>
__device__ __forceinline__ void xcd_head_order(int i, int BH, int nblk, int& bh, int& rank) {
  if (BH % (8 * G) == 0) {
    const int k = i >> 3, grp = k / (G * nblk), r = k % (G * nblk);
    bh = (i & 7) + 8 * (G * grp + r % G);
    rank = r / G;
  } else {
    bh = i % BH;
    rank = i / BH;
  }
}

// Half segments of the interval variant [1/2, t + 1/2] (Problem Statement: the original
// paper integrates eq. (2) over that interval).  In the forward's units (c^2 e^{a} x the
// integral, scaled by 2^{-m}; p = 2^{alpha}, alpha = a log2 e - m, c = ln 2), for a segment
// with endpoint values p_l, p_r, midpoint value p_m = 2^{(alpha_l + alpha_r)/2},
// y = alpha_r - alpha_l and u = 1/y:
//   lower half (sigma in [0, 1/2]):  HL = ((c/2) p_m - (p_m - p_l) u) u  (to the right end),
//                                    HR = c (p_m - p_l) u - HL           (to the left end);
//   upper half (sigma in [1/2, 1]):  HL' = (c (p_r - p_m/2) - (p_r - p_m) u) u,
//                                    HR' = c (p_r - p_m) u - HL';
// below |y| < 0.1 their second-order Taylor forms in x = c y:
//   HL = c^2 p_l (1/8 + x/24 + x^2/128),   HR = c^2 p_l (3/8 + x/12 + 5 x^2/384),
//   HL' = c^2 p_l (3/8 + 7x/24 + 15 x^2/128), HR' = c^2 p_l (1/8 + x/12 + 11 x^2/384).
namespace half {

constexpr float kC = 0.6931471805599453f;   // ln 2
constexpr float kC2 = 0.4804530139182014f;  // c^2
constexpr float kY0 = 0.1f;                 // Taylor below |y| < 0.1

// lower half (sigma in [0, 1/2]) of segment (l, r): HR to l, HL to r
__device__ __forceinline__ void lower_half(float al, float pl, float ar, float& HR, float& HL) {
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

// upper half (sigma in [1/2, 1]) of segment (l, r): HR' to l, HL' to r
__device__ __forceinline__ void upper_half(float al, float pl, float ar, float pr, float& HR, float& HL) {
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

// The lane index, produced where it is used: an instruction pair the compiler can neither
// hoist nor merge, so that values derived from the lane index are formed anew at each use
// instead of being kept in registers across the tile loop.
__device__ inline int lane_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// kHalf differs from kExact in two places only: position 0 and position 1 share the upper
// half of segment (0, 1) (first tile), and the query's own position t and position t+1 share
// the lower half of segment (t, t+1) -- all of it, c^2 p_t / 2, to position t for the last
// query, whose position T+1 repeats T.  The second is added in the epilogue from two
// lane-parallel dot products (keys t and t+1) and two value rows, so the key tiles and the
// diagonal masks are the forward's.
template <int D, int W>
__global__ void __launch_bounds__(512, 4) attn16_kernel(FwdParams p) {
  static_assert(D == 16 || D == 64 || D == 128, "head dimension");
  static_assert(W == kSoftmax || W == kExact || W == kFirstOrder || W == kHalf, "weight rule");
  constexpr bool CSA = W != kSoftmax;  // position 0, halo and neighbour terms
  constexpr int CH = D / 8;                      // 16-byte chunks per row
  constexpr int ROWB = D * 2;                    // bytes per row in HBM
  constexpr int NSTEP = D >= 32 ? D / 32 : 1;    // QK^T contraction steps (32 d each)
  constexpr int NMB = D / 16;                    // 16-row blocks of O^T
  constexpr int TILE_BYTES = kTile * ROWB;
  constexpr int SLOTS = kTile * CH;              // 16-byte slots per tile
  constexpr int ROUNDS = (SLOTS + 511) / 512;
  constexpr int RW = CH < 4 ? CH : 4;            // chunks per row segment of a region
  constexpr int REGION = 64 * RW * 16;           // bytes per region

  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE_BYTES];  // K0 K1 V0 V1
  // Per query of the block, values used only outside the steady tile loop, kept here instead
  // of in registers across it (with them in registers the d = 128 kernels spilled 6 to 25
  // VGPRs to scratch at 128 VGPRs): slot 0 a0, 1 a_t, 2 a_t1 (interval variant), 3 the HL
  // of position t + 1 when it opens the next tile (interval variant), 4 the weight of
  // position 0 (rescaled in place when the shift moves).  Each wave owns its 16 queries'
  // slots, so no barrier is involved; a wave's LDS accesses complete in order.
  __shared__ float parked[kWaves16 * 16 * 8];
  // interval variant: the value row of position t + 1 of a wave's last query when it opens
  // the next tile (its weight is added in the epilogue), loaded in the prologue
  __shared__ bf16 vnext[W == kHalf ? kWaves16 * D : 1];
  CSA_LDS char* lds = (CSA_LDS char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;   // query of this lane within the wave
  const int g = lane >> 4;   // lane group: keys 16g .. 16g+15 of every tile
  const int Tn = p.T;
  const int BH = p.B * p.H;
  // heads four at a time per XCD, longest query blocks first (lm: fetched bytes 820 -> 420 MB per
  // launch, time unchanged; two at a time fetched 262 MB but left the last group's 32-tile blocks
  // to the end: 17% slower)
  int bh, qrank;
  xcd_head_order<4>(blockIdx.x, BH, p.nqb, bh, qrank);
  const int qb = p.nqb - 1 - qrank;
  const int q0 = qb * kBlockRows;
  const int qw = q0 + 16 * wave;
  const int qr = qw + n;
  const bool wave_rows = qw < Tn;
  const int jw = wave_rows ? min(qw + 15, Tn - 1) / kTile : -1;  // last tile of this wave
  const int jmax = min(q0 + kBlockRows - 1, Tn - 1) / kTile;      // last tile of the block

  const size_t head = (size_t)bh * (size_t)Tn * D;
  const char* __restrict__ Kg = (const char*)((const bf16*)p.k + head);
  const char* __restrict__ Vg = (const char*)((const bf16*)p.v + head);

  // ---- HBM -> LDS: slot sigma = round*512 + tid of a tile; its source (row, chunk)
  // under the K or V layout above, as a byte offset inside the tile's rows.
  auto ksrc = [&](int sigma) {
    const int region = sigma / (64 * RW);  // contraction step
    const int within = sigma % (64 * RW);
    const int gi = within / RW;            // row segment slot: 4 (r & 3) + (r >> 4) + 16 ((r >> 2) & 3)
    const int row = 16 * (gi & 3) + 4 * (gi >> 4) + ((gi >> 2) & 3);
    const int cc = (within % RW) ^ (row & (RW - 1));
    return row * ROWB + (region * RW + cc) * 16;
  };
  auto vsrc = [&](int sigma) {
    const int region = sigma / (64 * RW);  // 32 d-columns
    const int within = sigma % (64 * RW);
    const int row = within / RW;
    const int cc = (within % RW) ^ ((2 * ((row >> 4) & 1)) & (RW - 1));
    return row * ROWB + (region * RW + cc) * 16;
  };
  // round r of a copy reads the same rows as round 0, 8 chunks (128 bytes) further
  const int koffg = ksrc(tid), voffg = vsrc(tid);
  auto stage = [&](int buf, const char* __restrict__ src, int tile, bool is_v) {
    const char* base = src + (size_t)tile * TILE_BYTES;
    const int rows_left = Tn - tile * kTile;  // >= 1
    int off = is_v ? voffg : koffg;
    if (rows_left < kTile) {  // last tile of the sequence: clamp rows past T
      const int row = off / ROWB;
      off -= (row - min(row, rows_left - 1)) * ROWB;
    }
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
      if (r * 512 + wave * 64 < SLOTS) {  // wave-uniform
        const unsigned dst = __builtin_amdgcn_readfirstlane(
            (unsigned)(uintptr_t)(lds + buf * TILE_BYTES + (r * 512 + wave * 64) * 16));
        lds_copy16(base + 128 * r, off, dst);
      }
    }
  };

  // ---- prologue copies first, K_0, V_0, K_1 into LDS: the loads of Q, k0 and (interval
  // variant) of the key and value rows below are then in flight together with them, and
  // the whole prologue waits for one round trip to memory instead of two or three
  stage(0, Kg, 0, false);
  stage(2, Vg, 0, true);
  if (jmax >= 1) stage(1, Kg, 1, false);

  // ---- Q operand in registers: qreg[s] = chunk 4s + g of row qr (zero past d)
  bf16x8 qreg[NSTEP];
  {
    const bf16* Qg = (const bf16*)p.q + head;
    const int row = min(qr, Tn - 1);
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      if (4 * s + g < CH) {
        qreg[s] = *(const bf16x8*)(Qg + (size_t)row * D + (4 * s + g) * 8);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qreg[s][e] = (bf16)0.0f;
      }
    }
  }

  // query-wide reductions over the four lane groups (lanes n, n+16, n+32, n+48)
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
  auto from_lane = [&](int src, float x) {  // value of x in lane src
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(x)));
  };
  auto from_addr = [&](int addr, float x) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(addr, __float_as_int(x)));
  };
  // lanes of the same query in the next / previous lane group, formed where used from the
  // lane index (kept live across the tile loop they were spilled to scratch)
  auto lane_dn = [&]() {
    const int l = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    int r = (l + 16) & 63;
    asm volatile("" : "+v"(r));
    return r;
  };
  auto lane_up = [&]() {
    const int l = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    int r = (l + 48) & 63;
    asm volatile("" : "+v"(r));
    return r;
  };

  // ds_bpermute byte addresses of the lane of the same query in the next / previous lane group
  // and of lane n (group 0): formed once and kept across the tile loop (10 VALU per tile fewer
  // than forming them at each use), except for the interval variant, whose registers they would
  // push into scratch
  const int addr_dn_k = ((lane + 16) & 63) << 2, addr_up_k = ((lane + 48) & 63) << 2, addr_n_k = n << 2;
  auto addr_dn = [&]() { return W == kHalf ? lane_dn() << 2 : addr_dn_k; };
  auto addr_up = [&]() { return W == kHalf ? lane_up() << 2 : addr_up_k; };
  auto addr_n = [&]() { return W == kHalf ? (lane_here() & 15) << 2 : addr_n_k; };

  // this lane's query slot k of `parked`, addressed from the lane index where used
  auto park = [&](int k) -> CSA_LDS float* {
    const int off = (16 * wave + (lane_here() & 15)) * 32 + 4 * k;
    return (CSA_LDS float*)((CSA_LDS char*)parked + off);
  };

  // this lane's query row, formed from the lane index where used (not kept across the loop)
  auto qrow = [&]() { return qw + (lane_here() & 15); };

  // ---- the prologue's own loads, all issued before any of them is waited for: the key of
  // position 0 and, for the interval variant, the key rows qr (position t) and qr + 1
  // (position t + 1), whose logits the lower half of segment (t, t+1) on the diagonal tile
  // needs, and -- when the wave's last query's position t + 1 opens the next tile (wave-
  // uniform) -- the value row of that position, one 4-byte piece per lane, for `vnext`
  const bool have_k0 = CSA && p.k0 != nullptr;
  // without k0 any readable row serves (the product is discarded): the loads stay unconditional
  const bf16* K0 = have_k0 ? (const bf16*)p.k0 + (size_t)bh * D : (const bf16*)p.q + head;
  bf16x8 kc[NSTEP], kt[W == kHalf ? NSTEP : 1], kn[W == kHalf ? NSTEP : 1];
#pragma unroll
  for (int s = 0; s < NSTEP; ++s) {
    if (CSA && 4 * s + g < CH) kc[s] = *(const bf16x8*)(K0 + (4 * s + g) * 8);
  }
  if constexpr (W == kHalf) {
    const bf16* Kh = (const bf16*)p.k + head;
    const int rt = min(qr, Tn - 1), rn = min(qr + 1, Tn - 1);
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      if (4 * s + g < CH) {
        kt[s] = *(const bf16x8*)(Kh + (size_t)rt * D + (4 * s + g) * 8);
        kn[s] = *(const bf16x8*)(Kh + (size_t)rn * D + (4 * s + g) * 8);
      }
    }
  }
  const bool vrow_wave = W == kHalf && ((qw + 15) & 63) == 63;
  unsigned vpiece = 0;
  if (vrow_wave && lane_here() < D / 2)
    vpiece = *(const unsigned*)((const bf16*)p.v + head + (size_t)min(qw + 16, Tn - 1) * D +
                                2 * lane_here());

  // ---- logit of position 0: a0 = q . k0 (zero when k0 is null)
  float a0 = 0.0f;
  if constexpr (CSA) {
    float part = 0.0f;
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      if (4 * s + g < CH) {
#pragma unroll
        for (int e = 0; e < 8; ++e) part = __builtin_fmaf((float)qreg[s][e], (float)kc[s][e], part);
      }
    }
    a0 = have_k0 ? qsum(part) : 0.0f;
  }
  if (CSA) *park(0) = a0;
  float a_t = 0.0f, a_t1 = 0.0f;
  if constexpr (W == kHalf) {
    float pt = 0.0f, pn = 0.0f;
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      if (4 * s + g < CH) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pt = __builtin_fmaf((float)qreg[s][e], (float)kt[s][e], pt);
          pn = __builtin_fmaf((float)qreg[s][e], (float)kn[s][e], pn);
        }
      }
    }
    a_t = qsum(pt);
    a_t1 = qsum(pn);
    *park(1) = a_t;
    *park(2) = a_t1;
    if (vrow_wave && lane_here() < D / 2)
      *(CSA_LDS unsigned*)((CSA_LDS char*)vnext + 2 * D * wave + 4 * lane_here()) = vpiece;
  }

  // ---- LDS read bases
  // K operand (block b, step s): row 16(n >> 2) + 4b + (n & 3), chunk 4s + g (for d = 16,
  // lanes g >= 2 re-read chunk g - 2 against zero Q)  ->  kbase + s*REGION + b*16*RW*16
  const int kbase = (4 * (n & 3) + (n >> 2)) * RW * 16 + 16 * ((g & (RW - 1)) ^ (n & (RW - 1)));
  // V^T operand (d-block mb, key chunk c, read rd): row 16g + 8c + 4rd + (n >> 2), column
  // 16mb + 4(n & 3)  ->  vbase[mb & 1] + (mb*2 / RW)*REGION + (8c + 4rd)*RW*16
  int vbase[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int cc = ((2 * par) & (RW - 1)) + ((n >> 1) & 1);
    vbase[par] = (16 * g + (n >> 2)) * RW * 16 + 16 * (cc ^ ((2 * (g & 1)) & (RW - 1))) + 8 * (n & 1);
  }

  auto kread = [&](int buf, int s, int b) -> bf16x8 {
    return *(CSA_LDS const bf16x8*)(lds + buf * TILE_BYTES + kbase + s * REGION + b * 16 * RW * 16);
  };
  auto vread = [&](int vbuf, int c, int mb) -> bf16x8 {
    CSA_LDS const char* a = lds + vbuf * TILE_BYTES + vbase[mb & 1] + (2 * mb / RW) * REGION + 8 * c * RW * 16;
    const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CSA_LDS s16x4*)a);
    const s16x4 r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CSA_LDS s16x4*)(a + 4 * RW * 16));
    const bf16x4 b1 = __builtin_bit_cast(bf16x4, r1);
    const bf16x4 b2 = __builtin_bit_cast(bf16x4, r2);
    return bf16x8{b1[0], b1[1], b1[2], b1[3], b2[0], b2[1], b2[2], b2[3]};
  };
  // S^T blocks [b0, b1) of a tile, contraction steps pipelined one operand ahead
  auto qk = [&](int buf, f32x4 (&S)[4], int b0, int b1) {
#pragma unroll
    for (int b = b0; b < b1; ++b) S[b] = f32x4{};
    bf16x8 a = kread(buf, 0, b0);
#pragma unroll
    for (int b = b0; b < b1; ++b) {
#pragma unroll
      for (int s = 0; s < NSTEP; ++s) {
        const bf16x8 cur = a;
        if (s + 1 < NSTEP) a = kread(buf, s + 1, b);
        else if (b + 1 < b1) a = kread(buf, 0, b + 1);
        S[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur, qreg[s], S[b], 0, 0, 0);
      }
    }
  };

  f32x4 O[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) O[mb] = f32x4{};
  float lsum = 0.0f;     // this lane's share of the row sum of the rounded P
  float m_run = -__builtin_inff();
  float carry = 0.0f;   // lanes g = 3: left term of the next tile's first key (exact rule)
  float carry_s = 0.0f; // logit of this lane's key 15 in the previous tile (first-order rule)
  if (CSA) *park(4) = 0.0f;  // weight of position 0 (lanes g = 0 write it)

  auto rescale_all = [&](float sc) {
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) O[mb] *= sc;
    lsum *= sc;
    carry *= sc;
    if (CSA && g == 0) *park(4) *= sc;
  };

  // ---------------------------------------------------------------- one tile
  // PAR = j & 1: K_{j+1} sits in K buffer 1 - PAR, V_j in V buffer PAR (LDS buffer 2 + PAR).
  // Scur holds S^T of tile j; a tile before the diagonal computes S^T of tile j+1 into Snext.
  //
  // The weights are produced in 16 steps, one key per step (its exponential and, for
  // CSA, the reciprocal of the next neighbour difference one step ahead).  The tile's
  // MFMAs are pinned between the steps: the next tile's S^T (blocks 1..3) during steps
  // 0..7, P V of keys 0..7 during steps 8..15, the rest after; so every wave keeps the
  // matrix cores busy while its VALU works, instead of alternating the two.
  auto tile = [&](auto par_c, auto last_c, auto first_c, int j, f32x4 (&Scur)[4], f32x4 (&Snext)[4]) {
    constexpr int PAR = decltype(par_c)::value;
    constexpr int KNEXT = 1 - PAR;
    constexpr int VBUF = 2 + PAR;
    constexpr bool last = decltype(last_c)::value;  // the tile holding this wave's diagonal
    const bool first = decltype(first_c)::value || (last && j == 0);
    // Wave priority 1 while the wave forms the weights of keys 0..7 and issues the next tile's
    // S^T products, 0 for keys 8..15 and the first key chunk's P V products (2 for the second
    // chunk's, after the weight steps; see there): a SIMD serves waves that have just
    // entered a tile, whose S^T products start the next tile's dependency chain, ahead of waves
    // finishing one.  Interleaved A/B against equal priorities: +2% lm, +3% long, +12% stress
    // (logit std 8); lowering after key 3 or 11, or a priority falling with every four keys
    // (or rising), were all weaker.
    __builtin_amdgcn_s_setprio(1);
    constexpr int NQ = 3 * NSTEP;  // MFMAs of S^T blocks 1..3 of the next tile
    constexpr int NP = NMB + 1;    // units of one key chunk of P V: NMB MFMAs, then the row sums

    // block 0 of the next tile first: its key 0 is the right halo of this tile
    if constexpr (!last) qk(KNEXT, Snext, 0, 1);
    float s[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) s[t] = Scur[t >> 2][t & 3];
    // key row of s[t] is j*64 + 16g + t; visible to this lane's query iff t <= lim
    int lim = 0;
    if constexpr (last) {
      const int l = lane_here();
      lim = qw + (l & 15) - (j * kTile + 16 * (l >> 4));
      asm volatile("" : "+v"(lim));  // opaque: keeps "t <= lim" from becoming 16 constants
    }

    // -- running maximum (lazy: the shift moves only when the maximum grows by > 2^8)
    float mx = -__builtin_inff();
    if constexpr (last) {
#pragma unroll
      for (int t = 0; t < 16; ++t) mx = fmaxf(mx, (t <= lim) ? s[t] : -__builtin_inff());
    } else {
#pragma unroll
      for (int t = 0; t < 16; ++t) mx = fmaxf(mx, s[t]);
    }
    float halo = 0.0f;
    if constexpr (CSA && !last) {
      halo = from_addr(addr_n(), Snext[0][0]);  // key 0 of tile j+1 (lane n, g = 0)
      mx = fmaxf(mx, halo);
    }
    // a0: in a register for the peeled first tile, from `parked` for a diagonal tile 0
    float a0v = 0.0f;
    if constexpr (CSA) {
      if constexpr (decltype(first_c)::value) a0v = a0;
      else if (first) a0v = *park(0);
    }
    float a_tv = 0.0f, a_t1v = 0.0f;
    if constexpr (W == kHalf && last) {
      a_tv = *park(1);
      a_t1v = *park(2);
    }
    if (CSA && first) mx = fmaxf(mx, a0v);
    if (W == kHalf && last && qrow() != Tn - 1) mx = fmaxf(mx, a_t1v);  // position t + 1 takes a weight
    // the shift moves only if some lane's own maximum passes m_run + 8 (the same test as on
    // the query-wide maximum, which is the largest of its lanes'); only then the maximum over
    // the query's four lanes, and every query of the wave takes its new shift (unchanged
    // where it did not grow: factor exactly 1)
    if (__builtin_amdgcn_ballot_w64(mx * kLog2e > m_run + 8.0f) != 0) {
      const float m_new = fmaxf(m_run, qmax(mx) * kLog2e);
      rescale_all(exp2_fast(m_run - m_new));
      m_run = m_new;
    }
    float mr = m_run;
    asm volatile("" : "+v"(mr));  // each path keeps its own exponentials
    float* w = s;                 // finished weights overwrite the logits in place
    auto alpha = [&](int t) { return __builtin_fmaf(s[t], kLog2e, -mr); };

    // -- MFMA work placed between the weight steps
    bf16x8 ak, av, P0;
    if constexpr (!last) ak = kread(KNEXT, 0, 1);
    auto qk_unit = [&](int u) {
      const int b = 1 + u / NSTEP, st = u % NSTEP;
      const bf16x8 cur = ak;
      if (u + 1 < NQ) ak = kread(KNEXT, (u + 1) % NSTEP, 1 + (u + 1) / NSTEP);
      Snext[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur, qreg[st], st == 0 ? f32x4{} : Snext[b], 0, 0, 0);
    };
    auto pv_unit = [&](int c, int u, const bf16x8& P) {
      if (u < NMB) {
        const bf16x8 cur = av;
        if (u + 1 < NMB) av = vread(VBUF, c, u + 1);
        else if (c == 0) av = vread(VBUF, 1, 0);  // first operand of the second chunk
        O[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur, P, O[u], 0, 0, 0);
      } else {  // row sums of the same rounded P as the numerator
        const bf16x2 one2 = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
        for (int e = 0; e < 8; e += 2)
          lsum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{P[e], P[e + 1]}, one2, lsum, false);
      }
    };
    auto pack = [&](int c) {
      bf16x8 P;
#pragma unroll
      for (int e = 0; e < 8; ++e) P[e] = (bf16)w[8 * c + e];
      return P;
    };
    auto slot = [&](int t) {  // after weight step t
      if (!last && t < 8) {
#pragma unroll
        for (int u = t * NQ / 8; u < (t + 1) * NQ / 8; ++u) qk_unit(u);
      }
      if (t == 6) av = vread(VBUF, 0, 0);
      if (t == 7) P0 = pack(0);
      if (t >= 8) {
#pragma unroll
        for (int u = (t - 8) * NP / 8; u < (t - 7) * NP / 8; ++u) pv_unit(0, u, P0);
      }
      if (t == 7) __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
    };

    if constexpr (!CSA) {
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const float e = exp2_fast(alpha(t));
        w[t] = (!last || t <= lim) ? e : 0.0f;
        slot(t);
      }
    } else if constexpr (W == kFirstOrder) {
      // b to first order (eq. (13)); ends -ln 2 + x/3.  In base 2 with beta = alpha/6 an
      // interior weight is 2^(4 beta_t + beta_{t-1} + beta_{t+1}) and an end weight
      // 2^(4 beta_t + 2 beta_nb - 1); both exponents are averages of alphas covered by the
      // running maximum, so the weights stay below 2^8.
      const float c6 = kLog2e * (1.0f / 6.0f);
      const float m6 = mr * (1.0f / 6.0f);
      auto beta = [&](float logit) { return __builtin_fmaf(logit, c6, -m6); };
      // neighbours as raw logits: left of key 0 is the previous group's key 15, or (g = 0)
      // the previous tile's key 63 carried by lanes g = 3, or (first tile) position 0;
      // right of key 15 is the next group's key 0, or (g = 3) the halo
      const float lsend = g == 3 ? carry_s : s[15];
      float left = from_addr(addr_up(), lsend);
      float right = from_addr(addr_dn(), s[0]);
      carry_s = s[15];
      if (first && g == 0) left = a0v;
      if (!last && g == 3) right = halo;
      if (first && g == 0)  // position 0 has only its right neighbour, the first key
        *park(4) = exp2_fast(__builtin_fmaf(4.0f, beta(a0v), __builtin_fmaf(2.0f, beta(s[0]), -1.0f)));
      float bl = beta(left);
      float bc = beta(s[0]);
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const float bn = t < 15 ? beta(s[t + 1]) : beta(right);
        float wv;
        if constexpr (!last) {
          wv = exp2_fast(__builtin_fmaf(4.0f, bc, bl + bn));
        } else {  // diagonal tile: column t takes the end rule, columns > t get 0
          const float x = t < lim ? bl + bn : __builtin_fmaf(2.0f, bl, -1.0f);
          const float we = exp2_fast(__builtin_fmaf(4.0f, bc, x));
          wv = t <= lim ? we : 0.0f;
        }
        w[t] = wv;
        bl = bc;
        bc = bn;
        slot(t);
      }
    } else {
      const float al0 = alpha(0);
      const float pv0 = exp2_fast(al0);
      const float al15 = alpha(15);
      const float pv15 = exp2_fast(al15);
      // right neighbour of key 15: the next group's key 0, or (g = 3) the halo; its logit is
      // fetched and its exponential formed here in every lane (the halo's is needed anyway, and
      // an exponential costs no more issue than a second lane exchange and two selects; the
      // bits are those the neighbouring lane forms for its key 0)
      float sr = from_addr(addr_dn(), s[0]);
      if (!last && g == 3) sr = halo;
      const float ar = __builtin_fmaf(sr, kLog2e, -mr);
      const float pr = exp2_fast(ar);
      float R15, Lnext;
      if constexpr (last) {
        edge_terms<false>(al15, pv15, ar, pr, R15, Lnext);
      } else {
        const float y15 = ar - al15;
        edge_yu_ballot(pv15, pr, y15, __builtin_amdgcn_rcpf(y15), 0.0f, R15, Lnext);
      }
      // left term of key 0: from the previous group, or (g = 0) carried from the
      // previous tile's group 3, or (first tile) from the edge with position 0
      const float Lsend = g == 3 ? carry : Lnext;
      float Lprev = from_addr(addr_up(), Lsend);
      carry = Lnext;  // lanes g = 3: left term of key 64(j+1)
      if (first) {    // position 0: only its right neighbour (eq. (10), i = 0)
        const float a0l = __builtin_fmaf(a0v, kLog2e, -mr);
        float R0, L1;
        if constexpr (W == kHalf) half::upper_half(a0l, exp2_fast(a0l), al0, pv0, R0, L1);
        else edge_terms<false>(a0l, exp2_fast(a0l), al0, pv0, R0, L1);
        if (g == 0) {
          *park(4) = R0;
          Lprev = L1;
        }
      }
      // interval variant, diagonal tile: the lower half of segment (t, t+1) -- HR to the
      // query's own key (column lim), HL to the next (column lim + 1, or the next tile's
      // first key when lim = 15 in lane group 3: added in the epilogue)
      float hR = 0.0f, hL = 0.0f;
      if constexpr (W == kHalf && last) {
        const float alt = __builtin_fmaf(a_tv, kLog2e, -mr);
        const float ptv = exp2_fast(alt);
        half::lower_half(alt, ptv, __builtin_fmaf(a_t1v, kLog2e, -mr), hR, hL);
        if (qrow() == Tn - 1) {  // position T+1 repeats T: the whole half segment goes to T
          hR = 0.5f * half::kC2 * ptv;
          hL = 0.0f;
        }
        if (g == 3) *park(3) = lim == 15 ? hL : 0.0f;  // HL of the next tile's first key
      }
      // edge (t, t+1) needs p_t, p_{t+1}, y_t = alpha_{t+1} - alpha_t and 1/y_t; the
      // values of key t+2 are formed one step ahead
      float pc = pv0;
      float an = alpha(1), pn = exp2_fast(an);
      float yc = an - al0, uc = __builtin_amdgcn_rcpf(yc);
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        if (t < 15) {
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
          if constexpr (!last) {
            edge_yu_ballot(pc, pn, yc, uc, Lprev, w[t], Lprev);
          } else {  // diagonal tile: column t keeps only its left term, columns > t get 0
            float R, L;
            edge_yu(pc, pn, yc, uc, 0.0f, R, L);
            if constexpr (W == kHalf)  // plus the lower half of segment (t, t+1)
              w[t] = t < lim ? Lprev + R : (t == lim ? Lprev + hR : (t == lim + 1 ? hL : 0.0f));
            else
              w[t] = t < lim ? Lprev + R : (t == lim ? Lprev : 0.0f);
            Lprev = L;
          }
          pc = pn;
          yc = yn;
          uc = un;
          an = ann;
          pn = pnn;
        } else {
          if constexpr (last && W == kHalf)
            w[15] = 15 < lim ? Lprev + R15 : (15 == lim ? Lprev + hR : (15 == lim + 1 ? hL : 0.0f));
          else
            w[15] = last ? (15 < lim ? Lprev + R15 : (15 == lim ? Lprev : 0.0f)) : Lprev + R15;
        }
        slot(t);
      }
    }
    // P V of keys 8..15 of every lane group, at the highest of the tile's priorities: a wave
    // that has formed its last weights issues the tile's last products ahead of the other waves'
    // weight work and reaches the barrier sooner (lm +1.3% to +2.4% in three interleaved A/Bs,
    // level on long and stress)
    __builtin_amdgcn_s_setprio(2);
    const bf16x8 P1 = pack(1);
#pragma unroll
    for (int u = 0; u < NP; ++u) pv_unit(1, u, P1);
  };

  // ---- prologue: S^T of tile 0 (its copies were issued first)
  wait_vmem();
  __syncthreads();
  f32x4 SA[4], SB[4];
  if (jw >= 0) qk(0, SA, 0, 4);
  __syncthreads();  // K_0's buffer is refilled in iteration 0

  // ---- main loop: one iteration (one barrier) per key tile of the block for every
  // wave; computation only on the wave's own tiles, the diagonal one last.
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using BF = std::integral_constant<bool, false>;
  using BT = std::integral_constant<bool, true>;
  auto refill = [&](int j) {
    if (j + 2 <= jmax) stage(j & 1, Kg, j + 2, false);
    if (j + 1 <= jmax) stage(2 + ((j + 1) & 1), Vg, j + 1, true);
  };
  auto sync = [&]() {
    wait_vmem();
    __syncthreads();
  };
  int j = 0;
  if (jw > 0) {  // tile 0 also takes the edge with position 0
    refill(0);
    tile(I0{}, BF{}, BT{}, 0, SA, SB);
    sync();
    j = 1;
  }
  for (; j + 1 < jw; j += 2) {  // j odd
    refill(j);
    tile(I1{}, BF{}, BF{}, j, SB, SA);
    sync();
    refill(j + 1);
    tile(I0{}, BF{}, BF{}, j + 1, SA, SB);
    sync();
  }
  if (j < jw) {  // j odd
    refill(j);
    tile(I1{}, BF{}, BF{}, j, SB, SA);
    sync();
    ++j;
  }
  if (j == jw) {
    refill(j);
    if ((j & 1) == 0) tile(I0{}, BT{}, BF{}, j, SA, SB);
    else tile(I1{}, BT{}, BF{}, j, SB, SA);
    sync();
    ++j;
  }
  for (; j <= jmax; ++j) {
    refill(j);
    sync();
  }

  if (!wave_rows) return;

  // ---- epilogue: position-0 term, normalisation, stores
  float l = qsum(lsum);
  float w0q = 0.0f;
  if (CSA) {
    w0q = *park(4);
    l += w0q;
  }
  if constexpr (W == kHalf) {
    if (vrow_wave) {  // its last query's t + 1 opens the next tile
      const float wn = *park(3);
      l += wn;
      // the row of the wave's query 15, the only one whose wn is not zero
      CSA_LDS const bf16* Vn = (CSA_LDS const bf16*)vnext + D * wave;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        const bf16x4 vn = *(CSA_LDS const bf16x4*)(Vn + 16 * mb + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) O[mb][r] = __builtin_fmaf(wn, (float)vn[r], O[mb][r]);
      }
    }
  }
  const float inv = 1.0f / l;
  const int qe = qrow();
  if (qe < Tn) {
    const bf16* V0 = (CSA && p.v0 != nullptr) ? (const bf16*)p.v0 + (size_t)bh * D : nullptr;
    bf16* Og = (bf16*)p.out + head + (size_t)qe * D;
    // this lane's elements of v_0 (4 per block), every load issued before the first is used
    bf16x4 v0r[NMB];
    if (V0) {
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) v0r[mb] = *(const bf16x4*)(V0 + 16 * mb + 4 * g);
    }
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      const int d0 = 16 * mb + 4 * g;
      float o4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float acc = O[mb][r];
        if (V0) acc = __builtin_fmaf(w0q, (float)v0r[mb][r], acc);
        o4[r] = acc * inv;
      }
      *(bf16x4*)(Og + d0) = bf16x4{(bf16)o4[0], (bf16)o4[1], (bf16)o4[2], (bf16)o4[3]};
    }
    if (p.lse != nullptr && g == 0) {
      const float corr = (W == kExact || W == kHalf) ? 0.7330258411633287f : 0.0f;  // -2 ln(ln 2)
      p.lse[(size_t)bh * Tn + qe] = (m_run + __builtin_amdgcn_logf(l)) * kLn2 + corr;
    }
  }
}

template <int D, int W>
inline hipError_t launch_attn16(const FwdParams& prm, hipStream_t stream) {
  const int nqb = (prm.T + kBlockRows - 1) / kBlockRows;
  FwdParams p = prm;
  p.nqb = nqb;
  const dim3 grid((unsigned)(nqb * prm.B * prm.H));
  hipLaunchKernelGGL((attn16_kernel<D, W>), grid, dim3(64 * kWaves16), 0, stream, p);
  return hipGetLastError();
}

}  // namespace csa
