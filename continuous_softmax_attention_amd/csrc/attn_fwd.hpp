// Flash-style causal attention forward for gfx950 (MI355X): continuous softmax
// attention (CSA = true) and, on the identical tiling, standard softmax
// attention (CSA = false).
//
// Method: J. Su, "Continuous Softmax Attention".  The kernel evaluates the
// simplified form eq. (10)-(11) (Assembly and Simplification): standard
// attention logits a_{t,i} = q_t . k_i, a correction e^{b_{t,i}} built from the
// two neighbour differences through phi_2 (eq. (6)), one extra position 0
// holding k_0, v_0, and a normalised weighted sum of the values.  The pages
// note that the FlashAttention principle carries over (Simple Experiments);
// here it is re-derived for CDNA4.
//
// Work decomposition
//   * One work-group = 4 waves = 128 consecutive query rows of one (b, h).
//     Each wave owns 32 query rows.  Key tiles are 64 rows of k (positions
//     64j+1 .. 64j+64); position 0 (k_0) is handled per query block.
//   * Logits are computed TRANSPOSED, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16
//     (v_mfma_f32_32x32x2f32 for float32).  The 32x32 accumulator gives lane
//     (n, h) -- n = lane % 32, h = lane / 32 -- query n and 16 key rows per
//     block; the K operand rows are permuted (kappa below) so that lane (n, h)
//     holds the 32 CONSECUTIVE keys 32h .. 32h+31 of the tile for query n.
//     The neighbour stencil of eq. (10) is then in-register except at one
//     cross-half edge (keys 31|32, exchanged with v_permlane32_swap) and at
//     the tile's right edge, whose neighbour is the next tile's first key.
//   * The next tile's logits are computed one iteration early; they supply
//     that right halo and let the MFMAs of tile j+1 overlap the VALU work of
//     tile j.
//   * The weights of tile j feed O^T += V^T P^T directly from registers as the
//     MFMA B operand (lane (n, h) holds P for query n, keys 32h + 8c + e); V^T
//     rows come from row-major V in LDS through ds_read_b64_tr_b16.  Row sums
//     of the bf16-rounded P come from one extra MFMA block against a constant
//     "ones" operand, so numerator and denominator see the same rounded P.
//   * K and V tiles move HBM -> LDS with global_load_lds_dwordx4 (16 B per
//     lane, no VGPR staging), double-buffered, XOR-swizzled on 16-byte
//     chunks so that both the K-operand reads and the transposed V reads are
//     free of bank conflicts.
//
// Correction weights ("p-form").  With the running row maximum m (base-2
// units), alpha_i = a_i log2(e) - m and p_i = 2^{alpha_i}.  For each edge
// (i, i+1) with y = alpha_{i+1} - alpha_i, u = 1/y, D = p_{i+1} - p_i:
//     c^2 e^{a_i - m ln2} phi_2(a_{i+1} - a_i)     = (D u - c p_i) u
//     c^2 e^{a_{i+1} - m ln2} phi_2(a_i - a_{i+1}) = (c p_{i+1} - D u) u,   c = ln 2,
// which is eq. (6) rewritten with e^{x} = p_{i+1}/p_i.  The common factor c^2
// cancels in the ratio eq. (11) and is removed from lse.  For |y| < Y0 the
// differences cancel, so p_i phi_2(+-x) is taken from the Taylor series of
// phi_2 instead (branch-free select).  Position i = 0 uses only its right
// term, the diagonal column i = t only its left term (the end cases of
// eq. (10)); columns beyond t get weight 0.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

namespace csa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define CSA_LDS __attribute__((address_space(3)))
#define CSA_GLOBAL __attribute__((address_space(1)))

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* k0;  // may be null
  const void* v0;  // may be null
  void* out;
  float* lse;      // may be null
  int B, H, T;
  int nqb;         // query blocks of 128 rows per (b, h)
};

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int EPC = 4;  // elements per 16-byte chunk
  using Chunk = f32x4;
};
template <>
struct Elem<bf16> {
  static constexpr int EPC = 8;
  using Chunk = bf16x8;
};

constexpr int kWaves = 4;
constexpr int kBlockRows = 32 * kWaves;  // query rows per work-group
constexpr int kTile = 64;                // key rows per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 16-byte-chunk swizzles of tile rows; the same permutation is used by the
// HBM->LDS copies and by every LDS read of that tile.
//  K tiles: the 16 rows one quarter-wave reads together for the K operand
//           (rows 4g+jj and 32+4g+jj, g in {0,1} or {2,3}) land in 16 distinct
//           chunk slots.
//  V tiles: the 4 rows one transposed read takes (8c+e, e = 0..3) put the
//           same logical chunk quad into 4 distinct bank quads; rows r and
//           r + 4 share the swizzle, so both reads of a chunk share a base.
__device__ __forceinline__ int swz_k(int row) {
  return ((row & 3) << 2) | ((row >> 2) & 1) | (((row >> 5) & 1) << 1);
}
__device__ __forceinline__ int swz_v(int row) { return (row & 3) << 2; }

// K-operand row permutation: MFMA row m of block b reads key row kappa(b, m),
// so that accumulator register r of block b in lane half h is key 32h + 16b + r.
__device__ __forceinline__ int kappa(int b, int m) {
  return 32 * ((m >> 2) & 1) + 16 * b + 4 * (m >> 3) + (m & 3);
}

struct Half {
  float lo, hi;  // the value held by lane j and by lane j + 32 of this lane's pair
};

// Both lanes of a pair (j, j+32) receive both values of x (v_permlane32_swap).
__device__ __forceinline__ Half pair_values(float x) {
  const unsigned u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Correction-weight constants per precision.  Y0 is the |y| below which the
// Taylor series replaces the cancelling closed form; the series is that of
// c^2 phi_2(c y) = sum_n c^{n+2} y^n / (n+2)!  (eq. (6) expanded).
template <bool F32>
struct Taylor;

template <>
struct Taylor<false> {  // bf16 outputs: relative weight error ~2e-4 << bf16 rounding of P
  static constexpr float Y0 = 0.07f;
  __device__ __forceinline__ static void eval(float y, float& gp, float& gm) {
    constexpr float k0 = 0.24022650695910072f;  // c^2/2
    constexpr float k1 = 0.05550410866482158f;  // c^3/6
    gp = __builtin_fmaf(y, k1, k0);
    gm = __builtin_fmaf(y, -k1, k0);
  }
};

template <>
struct Taylor<true> {  // float32 outputs: relative weight error ~1e-6
  static constexpr float Y0 = 1.0f;
  __device__ __forceinline__ static void eval(float y, float& gp, float& gm) {
    constexpr float k0 = 0.24022650695910072f;     // c^2/2!
    constexpr float k1 = 0.05550410866482158f;     // c^3/3!
    constexpr float k2 = 0.009618129107628477f;    // c^4/4!
    constexpr float k3 = 0.0013333558146428443f;   // c^5/5!
    constexpr float k4 = 0.00015403530393381608f;  // c^6/6!
    constexpr float k5 = 1.525273380405984e-05f;   // c^7/7!
    constexpr float k6 = 1.3215486790144307e-06f;  // c^8/8!
    constexpr float k7 = 1.0178086009239699e-07f;  // c^9/9!
    constexpr float k8 = 7.054911620801123e-09f;   // c^10/10!
    const float y2 = y * y;
    const float ev = __builtin_fmaf(y2, __builtin_fmaf(y2, __builtin_fmaf(y2, __builtin_fmaf(y2, k8, k6), k4), k2), k0);
    const float od = __builtin_fmaf(y2, __builtin_fmaf(y2, __builtin_fmaf(y2, k7, k5), k3), k1);
    gp = __builtin_fmaf(y, od, ev);
    gm = __builtin_fmaf(-y, od, ev);
  }
};

// One edge (i, i+1) of eq. (10), scaled by c^2 2^{-m}:
//   R = c^2 e^{a_i} phi_2(a_{i+1} - a_i),  L = c^2 e^{a_{i+1}} phi_2(a_i - a_{i+1}).
// Returns w_left = Lprev + R (the finished weight of the left position when
// Lprev is its left term) and the left term of the right position.
template <bool F32>
__device__ __forceinline__ void edge(float al, float pl, float ar, float pr, float Lprev,
                                     float& w_left, float& L_right) {
  const float y = ar - al;
  const float u = __builtin_amdgcn_rcpf(y);
  const float dp = pr - pl;
  const float du = dp * u;
  const float t1 = __builtin_fmaf(-kLn2, pl, du);
  const float wr = __builtin_fmaf(t1, u, Lprev);
  const float t2 = __builtin_fmaf(kLn2, pr, -du);
  const float lr = t2 * u;
  float gp, gm;
  Taylor<F32>::eval(y, gp, gm);
  const float wt = __builtin_fmaf(pl, gp, Lprev);
  const float lt = pr * gm;
  const bool small = __builtin_fabsf(y) < Taylor<F32>::Y0;
  w_left = small ? wt : wr;
  L_right = small ? lt : lr;
}

// Same edge with the two terms returned separately (diagonal tiles).
template <bool F32>
__device__ __forceinline__ void edge_terms(float al, float pl, float ar, float pr, float& R, float& L) {
  edge<F32>(al, pl, ar, pr, 0.0f, R, L);
}

// Rescale the bf16 row sums: lanes 0..15 hold queries n' (element 0) and n' + 16
// (element 1) of the 16x16x32 accumulator; the second takes the factor of lane n' + 16.
__device__ __forceinline__ void rescale_lacc(f32x4& Lacc, float sc) {
  const unsigned su = __float_as_uint(sc);
  const auto sw = __builtin_amdgcn_permlane16_swap(su, su, false, false);
  Lacc[0] *= sc;
  Lacc[1] *= __uint_as_float(sw[1]);
}

template <typename T, int D, bool CSA>
__global__ void __launch_bounds__(256, (sizeof(T) == 2 ? 2 : 1)) attn_fwd_kernel(FwdParams p) {
  using Chunk = typename Elem<T>::Chunk;
  constexpr bool F32 = sizeof(T) == 4;
  constexpr int EPC = Elem<T>::EPC;
  constexpr int CH = D / EPC;                // 16-byte chunks per row
  constexpr int ROWB = CH * 16;              // bytes per row (global and LDS)
  constexpr int NSTEP = CH / 2;              // QK^T contraction steps
  constexpr int NQK = 2 * NSTEP;             // (step, 32-key block) pairs of one S^T tile
  constexpr int NMB = (D + 31) / 32;         // 32-row blocks of O^T
  constexpr int TILE_BYTES = kTile * ROWB;
  constexpr int SWZ_MASK = CH - 1;
  constexpr int ROUNDS = (kTile * CH + 255) / 256;
  static_assert(CH >= 2 && (CH & (CH - 1)) == 0, "chunk count must be a power of two");

  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE_BYTES];  // K0 K1 V0 V1
  CSA_LDS char* lds = (CSA_LDS char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int n = lane & 31;
  const int Tn = p.T;
  const int BH = p.B * p.H;
  const int bh = blockIdx.x % BH;              // heads fastest: every block of a head on one XCD
  const int qb = p.nqb - 1 - blockIdx.x / BH;  // longest (last) query blocks first
  const int q0 = qb * kBlockRows;
  const int qw = q0 + 32 * wave;               // first query row of this wave
  const int qr = qw + n;                       // this lane's query row
  const bool wave_rows = qw < Tn;
  const int jw = wave_rows ? min(qw + 31, Tn - 1) / kTile : -1;  // last tile of this wave
  const int jmax = min(q0 + kBlockRows - 1, Tn - 1) / kTile;      // last tile of the block

  const size_t head = (size_t)bh * (size_t)Tn * D;
  const char* __restrict__ Kg = (const char*)((const T*)p.k + head);
  const char* __restrict__ Vg = (const char*)((const T*)p.v + head);

  // ---- HBM -> LDS tile copy: 16 B per lane, swizzled rows, rows past T clamped.
  // Slot (r*256 + tid) of a tile holds logical chunk slot ^ swz(row): its source
  // byte offset inside the tile is (slot*16) ^ (swz(row) << 4) (no row padding).
  auto stage = [&](int buf, const char* __restrict__ src, int tile, bool is_v) {
    const char* base = src + (size_t)tile * TILE_BYTES;
    const bool full = (tile + 1) * kTile <= Tn;
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
      if (r * 256 + wave * 64 < kTile * CH) {  // wave-uniform
        const int slot = r * 256 + tid;
        const int row = slot / CH;
        const int sw = (is_v ? swz_v(row) : swz_k(row)) & SWZ_MASK;
        int off = (slot * 16) ^ (sw << 4);
        if (!full) off -= (row - min(row, Tn - 1 - tile * kTile)) * ROWB;
        CSA_LDS char* dst = lds + buf * TILE_BYTES + (r * 256 + wave * 64) * 16;
        __builtin_amdgcn_global_load_lds((const CSA_GLOBAL void*)(base + off), (CSA_LDS void*)dst, 16, 0, 0);
      }
    }
  };

  // ---- this lane's query row in registers: chunk 2i + h of row qr (the MFMA B operand)
  Chunk qreg[NSTEP];
  {
    const T* Qg = (const T*)p.q + head;
    const int row = min(qr, Tn - 1);
#pragma unroll
    for (int i = 0; i < NSTEP; ++i) qreg[i] = *(const Chunk*)(Qg + (size_t)row * D + (2 * i + h) * EPC);
  }

  // ---- logit of position 0: a0 = q . k0 (zero when k0 is null)
  float a0 = 0.0f;
  if (CSA && p.k0 != nullptr) {
    const T* K0 = (const T*)p.k0 + (size_t)bh * D;
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < NSTEP; ++i) {
      const Chunk kc = *(const Chunk*)(K0 + (2 * i + h) * EPC);
#pragma unroll
      for (int e = 0; e < EPC; ++e) part = __builtin_fmaf((float)qreg[i][e], (float)kc[e], part);
    }
    const Half hp = pair_values(part);
    a0 = hp.lo + hp.hi;
  }

  // ---- per-lane LDS read offsets (bytes inside a tile buffer)
  // K operand of step i, block 0 (block 1 is 16 rows further): row kappa(0, n),
  // physical chunk (2i + h) ^ swz_k(row) -- the same swizzle for both blocks.
  int koff[NSTEP];
  {
    const int row = kappa(0, n);
    const int z = swz_k(row) & SWZ_MASK;
#pragma unroll
    for (int i = 0; i < NSTEP; ++i) koff[i] = row * ROWB + (((2 * i + h) ^ z) << 4);
  }
  // V^T operand (bf16, ds_read_b64_tr_b16) of d-block mb, key chunk c, read r:
  // row 32h + 8c + 4r + e (e = (lane & 15) >> 2), column 32mb + 16 g2 + 4 (lane & 3);
  // rows 8c + 4r share the swizzle of row 32h + e, so c and r are immediate offsets.
  int voff[NMB];
  {
    const int g2 = (lane >> 4) & 1;
    const int jl = lane & 15;
    const int row = 32 * h + (jl >> 2);
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      const bool live = 32 * mb + 16 * g2 < D;  // a whole 16-lane group is in or out
      const int col = live ? 32 * mb + 16 * g2 + 4 * (jl & 3) : 4 * (jl & 3);
      voff[mb] = row * ROWB + (((col / EPC) ^ (swz_v(row) & SWZ_MASK)) << 4) + ((col % EPC) / 4) * 8;
    }
  }
  const bool vlive_g = F32 || (16 * ((lane >> 4) & 1) < D);  // d = 16: upper 16-lane group reads nothing

  // QK^T work unit q = (step i = q / 2, block b = q % 2) of the tile in buffer `buf`
  auto kread = [&](int buf, int q) -> Chunk {
    const int i = q >> 1, b = q & 1;
    return *(CSA_LDS const Chunk*)(lds + buf * TILE_BYTES + b * 16 * ROWB + koff[i]);
  };
  auto kmfma = [&](int q, const Chunk& a, f32x16 (&S)[2]) {
    const int i = q >> 1, b = q & 1;
    if constexpr (F32) {
#pragma unroll
      for (int u = 0; u < 4; ++u) S[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[u], qreg[i][u], S[b], 0, 0, 0);
    } else {
      S[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[i], S[b], 0, 0, 0);
    }
  };
  auto qk_burst = [&](int buf, f32x16 (&S)[2]) {
    S[0] = f32x16{};
    S[1] = f32x16{};
    Chunk a = kread(buf, 0);
#pragma unroll
    for (int q = 0; q < NQK; ++q) {
      const Chunk cur = a;
      if (q + 1 < NQK) a = kread(buf, q + 1);
      kmfma(q, cur, S);
    }
  };
  // V^T operand of (key chunk c, d-block mb) for the bf16 path
  auto vread = [&](int vbuf, int c, int mb) -> bf16x8 {
    CSA_LDS const char* a1 = lds + vbuf * TILE_BYTES + voff[mb] + 8 * c * ROWB;
    const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CSA_LDS s16x4*)a1);
    const s16x4 r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CSA_LDS s16x4*)(a1 + 4 * ROWB));
    const bf16x4 b1 = __builtin_bit_cast(bf16x4, r1);
    const bf16x4 b2 = __builtin_bit_cast(bf16x4, r2);
    bf16x8 A;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      A[e] = vlive_g ? b1[e] : (bf16)0.0f;
      A[4 + e] = vlive_g ? b2[e] : (bf16)0.0f;
    }
    return A;
  };

  f32x16 O[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) O[mb] = f32x16{};
  // bf16: row sums of the rounded P from v_mfma_f32_16x16x32_bf16 against a 0/1
  // operand.  Its 16-lane groups g = lane/16 hold queries n' = lane%16 (g = 0, 2)
  // and n' + 16 (g = 1, 3); A row 0 selects groups 0 and 2, row 1 groups 1 and 3:
  // C[0][n'] = l(query n'), C[1][n'] = l(query n'+16).
  f32x4 Lacc = f32x4{};
  bf16x8 ones;
  {
    const int m16 = lane & 15, g16 = lane >> 4;
    const bool sel = (m16 == 0 && (g16 & 1) == 0) || (m16 == 1 && (g16 & 1) == 1);
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = (bf16)(sel ? 1.0f : 0.0f);
  }
  float lsum = 0.0f;        // f32: per-lane partial row sum
  float m_run = -__builtin_inff();
  float carry = 0.0f;       // left term of the next tile's first key (lanes h = 0)
  float w0 = 0.0f;          // weight of position 0 (lanes h = 0)

  auto rescale_all = [&](float sc) {
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) O[mb] *= sc;
    rescale_lacc(Lacc, sc);
    lsum *= sc;
    carry *= sc;
    w0 *= sc;
  };

  // running maximum over this tile's visible logits (+ position 0 on tile 0);
  // lazy: the shift moves only when the maximum grows by more than 2^8
  auto update_max = [&](const float (&s)[32], int j, bool last, int lim) {
    float mx = -__builtin_inff();
    if (last) {
#pragma unroll
      for (int kk = 0; kk < 32; ++kk) mx = fmaxf(mx, (kk <= lim) ? s[kk] : -__builtin_inff());
    } else {
#pragma unroll
      for (int kk = 0; kk < 32; ++kk) mx = fmaxf(mx, s[kk]);
    }
    if (CSA && j == 0) mx = fmaxf(mx, a0);
    const Half hm = pair_values(mx);
    mx = fmaxf(hm.lo, hm.hi);
    const float m_new = fmaxf(m_run, mx * kLog2e);
    if (__builtin_amdgcn_ballot_w64(m_new > m_run + 8.0f) != 0) {
      rescale_all(exp2_fast(m_run - m_new));
      m_run = m_new;
    }
  };

  // fp32 path: O^T += V^T P^T with P in float32, one MFMA per key
  auto pv_f32 = [&](int vbuf, const float (&w)[32]) {
    CSA_LDS const char* vb = lds + vbuf * TILE_BYTES;
#pragma unroll
    for (int kk = 0; kk < 32; ++kk) lsum += w[kk];
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      const int row = 32 * h + c;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        const int col = 32 * mb + n;
        float a = 0.0f;
        if (col < D) {
          const int phys = (col / EPC) ^ (swz_v(row) & SWZ_MASK);
          a = *(CSA_LDS const float*)(vb + (row * CH + phys) * 16 + (col % EPC) * 4);
        }
        O[mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, w[c], O[mb], 0, 0, 0);
      }
    }
  };
  // bf16 path: one key chunk c (keys 32h + 8c + e) of O^T += V^T P^T, plus its row sums
  auto pack = [&](const float (&w)[32], int c) -> bf16x8 {
    bf16x8 P;
#pragma unroll
    for (int e = 0; e < 8; ++e) P[e] = (bf16)w[8 * c + e];
    return P;
  };
  auto pv_burst_bf16 = [&](int vbuf, const float (&w)[32]) {
    bf16x8 a = vread(vbuf, 0, 0);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bf16x8 P = pack(w, c);
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        const bf16x8 cur = a;
        if (mb + 1 < NMB) a = vread(vbuf, c, mb + 1);
        else if (c + 1 < 4) a = vread(vbuf, c + 1, 0);
        O[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, P, O[mb], 0, 0, 0);
      }
      Lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, P, Lacc, 0, 0, 0);
    }
  };

  // ---------------------------------------------------------------- one tile
  // PAR = j & 1: K_{j+1} sits in K buffer 1 - PAR, V_j in V buffer PAR (LDS buffer 2 + PAR).
  // Scur holds S^T of tile j; for a tile before the diagonal, Snext receives S^T of tile j+1.
  auto tile = [&](auto par_c, auto last_c, int j, f32x16 (&Scur)[2], f32x16 (&Snext)[2]) {
    constexpr int PAR = decltype(par_c)::value;
    constexpr int KNEXT = 1 - PAR;
    constexpr int VBUF = 2 + PAR;
    constexpr bool last = decltype(last_c)::value;  // the only tile crossing this wave's diagonal
    float s[32];
#pragma unroll
    for (int kk = 0; kk < 32; ++kk) s[kk] = Scur[kk >> 4][kk & 15];
    // key row of s[kk] is j*64 + 32h + kk; visible to this lane's query iff kk <= lim
    int lim = qr - (j * kTile + 32 * h);
    // opaque: otherwise "kk <= lim" becomes 32 loop-invariant per-key constants
    asm volatile("" : "+v"(lim));
    update_max(s, j, last, lim);
    float* w = s;  // finished weights overwrite the logits in place

    if constexpr (!CSA) {
      // ---------------- standard softmax attention: w = 2^(a log2 e - m), masked on the diagonal
      if (!last) {
        float mr = m_run;
        asm volatile("" : "+v"(mr));
#pragma unroll
        for (int kk = 0; kk < 32; ++kk) w[kk] = exp2_fast(__builtin_fmaf(s[kk], kLog2e, -mr));
        if constexpr (F32) pv_f32(VBUF, s);
        else pv_burst_bf16(VBUF, s);
        qk_burst(KNEXT, Snext);
      } else {
        float mr = m_run;
        asm volatile("" : "+v"(mr));
#pragma unroll
        for (int kk = 0; kk < 32; ++kk)
          w[kk] = (kk <= lim) ? exp2_fast(__builtin_fmaf(s[kk], kLog2e, -mr)) : 0.0f;
        if constexpr (F32) pv_f32(VBUF, s);
        else pv_burst_bf16(VBUF, s);
      }
      return;
    } else {
      // ---------------- continuous softmax attention
      const float al0 = __builtin_fmaf(s[0], kLog2e, -m_run);
      const float pv0 = exp2_fast(al0);
      float al31 = __builtin_fmaf(s[31], kLog2e, -m_run);
      float pv31 = exp2_fast(al31);
      // edge (key 31, key 32) across the lane halves, computed identically by both lanes:
      // R -> key 31 (h = 0), L -> key 32 (h = 1)
      const Half xa0 = pair_values(al0), xp0 = pair_values(pv0);
      const Half xa31 = pair_values(al31), xp31 = pair_values(pv31);
      float RE1, LE1;
      edge_terms<F32>(xa31.lo, xp31.lo, xa0.hi, xp0.hi, RE1, LE1);
      if (j == 0) {  // position 0: only its right neighbour (eq. (10), i = 0)
        const float a0l = __builtin_fmaf(a0, kLog2e, -m_run);
        float R0, L1;
        edge_terms<F32>(a0l, exp2_fast(a0l), al0, pv0, R0, L1);
        w0 = R0;
        carry = L1;
      }
      float Lprev = h == 0 ? carry : LE1;
      float ac = al0, pc = pv0;

      if (!last) {
        // private copy of the shift: the two branches must not share (and hoist) their exponentials
        float mr = m_run;
        asm volatile("" : "+v"(mr));
#pragma unroll
        for (int kk = 0; kk < 31; ++kk) {
          float an = al31, pn = pv31;
          if (kk + 1 < 31) {
            an = __builtin_fmaf(s[kk + 1], kLog2e, -mr);
            pn = exp2_fast(an);
          }
          edge<F32>(ac, pc, an, pn, Lprev, w[kk], Lprev);
          ac = an;
          pc = pn;
        }
        // key 31 of each lane half: h = 0 has both terms; for h = 1 (key 63) the right
        // term needs the next tile's first logit and is added after the next QK^T
        w[31] = Lprev + (h == 0 ? RE1 : 0.0f);
        if constexpr (F32) pv_f32(VBUF, s);
        else pv_burst_bf16(VBUF, s);
        qk_burst(KNEXT, Snext);
        // right halo: the next tile's first key (lanes h = 0 of Snext)
        float ah = pair_values(__builtin_fmaf(Snext[0][0], kLog2e, -m_run)).lo;
        if (__builtin_amdgcn_ballot_w64(ah > 8.0f) != 0) {
          // rare: the halo exceeds the shift by more than 2^8 -- move the shift now
          const float dm = fmaxf(ah, 0.0f);
          rescale_all(exp2_fast(-dm));
          al31 -= dm;
          pv31 *= exp2_fast(-dm);
          ah -= dm;
          m_run += dm;
        }
        // edge (key 63, halo) computed identically by both lanes: R -> key 63 (h = 1),
        // L -> the next tile's key 0 (kept by h = 0)
        const Half ya31 = pair_values(al31), yp31 = pair_values(pv31);
        float RE2, LE2;
        edge_terms<F32>(ya31.hi, yp31.hi, ah, exp2_fast(ah), RE2, LE2);
        carry = LE2;
        const float r63 = h == 1 ? RE2 : 0.0f;  // weight still missing from key 63
        if constexpr (F32) {
          lsum += r63;
          CSA_LDS const char* vb = lds + VBUF * TILE_BYTES;
          const int row = 32 * h + 31;
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb) {
            const int col = 32 * mb + n;
            float a = 0.0f;
            if (col < D) {
              const int phys = (col / EPC) ^ (swz_v(row) & SWZ_MASK);
              a = *(CSA_LDS const float*)(vb + (row * CH + phys) * 16 + (col % EPC) * 4);
            }
            O[mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, r63, O[mb], 0, 0, 0);
          }
        } else {
          // rank-1 update: key chunk 3 with only key 63 (element 7 of lanes h = 1) non-zero
          bf16x8 P3;
#pragma unroll
          for (int e = 0; e < 8; ++e) P3[e] = (bf16)0.0f;
          P3[7] = (bf16)r63;
          bf16x8 a = vread(VBUF, 3, 0);
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb) {
            const bf16x8 cur = a;
            if (mb + 1 < NMB) a = vread(VBUF, 3, mb + 1);
            O[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, P3, O[mb], 0, 0, 0);
          }
          Lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, P3, Lacc, 0, 0, 0);
        }
      } else {
        // diagonal tile: column t keeps only its left term, columns > t get 0
        float mr = m_run;
        asm volatile("" : "+v"(mr));
#pragma unroll
        for (int kk = 0; kk < 32; ++kk) {
          float R = 0.0f, Lnext = 0.0f;
          float an = 0.0f, pn = 0.0f;
          if (kk < 31) {
            an = al31;
            pn = pv31;
            if (kk + 1 < 31) {
              an = __builtin_fmaf(s[kk + 1], kLog2e, -mr);
              pn = exp2_fast(an);
            }
            edge_terms<F32>(ac, pc, an, pn, R, Lnext);
          } else {
            R = RE1;  // key 31 (h = 0); key 63 (h = 1) is never left of a visible key here
          }
          w[kk] = kk < lim ? Lprev + R : (kk == lim ? Lprev : 0.0f);
          Lprev = Lnext;
          ac = an;
          pc = pn;
        }
        if constexpr (F32) pv_f32(VBUF, s);
        else pv_burst_bf16(VBUF, s);
      }
    }
  };

  // ---- prologue: K_0, V_0, K_1 into LDS; S^T of tile 0
  stage(0, Kg, 0, false);
  stage(2, Vg, 0, true);
  if (jmax >= 1) stage(1, Kg, 1, false);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  f32x16 SA[2], SB[2];
  if (jw >= 0) qk_burst(0, SA);
  __syncthreads();  // K_0's buffer is refilled in iteration 0

  // ---- main loop.  Every wave runs one iteration (one barrier) per key tile of the
  // block, j = 0..jmax, but computes only on its own tiles: j < jw before its diagonal
  // (unrolled by two so that every LDS buffer offset is a constant), then j = jw.
  // Iteration j refills K buffer j&1 with K_{j+2} and V buffer (j+1)&1 with V_{j+1}.
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using BF = std::integral_constant<bool, false>;
  using BT = std::integral_constant<bool, true>;
  auto refill = [&](int j) {
    if (j + 2 <= jmax) stage(j & 1, Kg, j + 2, false);
    if (j + 1 <= jmax) stage(2 + ((j + 1) & 1), Vg, j + 1, true);
  };
  auto sync = [&]() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  int j = 0;
  for (; j + 1 < jw; j += 2) {
    refill(j);
    tile(I0{}, BF{}, j, SA, SB);
    sync();
    refill(j + 1);
    tile(I1{}, BF{}, j + 1, SB, SA);
    sync();
  }
  if (j < jw) {  // j even
    refill(j);
    tile(I0{}, BF{}, j, SA, SB);
    sync();
    ++j;
  }
  if (j == jw) {
    refill(j);
    if ((j & 1) == 0) tile(I0{}, BT{}, j, SA, SB);
    else tile(I1{}, BT{}, j, SB, SA);
    sync();
    ++j;
  }
  for (; j <= jmax; ++j) {
    refill(j);
    sync();
  }

  if (!wave_rows) return;

  // ---- epilogue: position-0 term, normalisation, stores
  const Half hw0 = pair_values(w0);
  const float w0q = hw0.lo;  // valid in lanes h = 0; both halves need it
  float l;
  if constexpr (F32) {
    const Half hl = pair_values(lsum);
    l = hl.lo + hl.hi;
  } else {
    // l(query n) sits in lane n % 16, element n / 16 of Lacc.  (Elements are copied
    // to scalars first: __builtin_bit_cast of an ext_vector element reads element 0.)
    const int src = n & 15;
    const float s0 = Lacc[0], s1 = Lacc[1];
    const float c0 = __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(s0)));
    const float c1 = __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(s1)));
    l = n < 16 ? c0 : c1;
  }
  if (CSA) l += w0q;
  const float inv = 1.0f / l;
  if (qr < Tn) {
    const T* V0 = (CSA && p.v0 != nullptr) ? (const T*)p.v0 + (size_t)bh * D : nullptr;
    T* Og = (T*)p.out + head + (size_t)qr * D;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * mb + 8 * g + 4 * h;
        if (d0 < D) {
          float o4[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            float acc = O[mb][4 * g + jj];
            if (V0) acc = __builtin_fmaf(w0q, (float)V0[d0 + jj], acc);
            o4[jj] = acc * inv;
          }
          if constexpr (F32) {
            *(f32x4*)(Og + d0) = f32x4{o4[0], o4[1], o4[2], o4[3]};
          } else {
            *(bf16x4*)(Og + d0) = bf16x4{(bf16)o4[0], (bf16)o4[1], (bf16)o4[2], (bf16)o4[3]};
          }
        }
      }
    }
    if (p.lse != nullptr && h == 0) {
      // lse = ln sum e^{a+b}: undo the base-2 shift and (for CSA) the c^2 scale
      const float corr = CSA ? 0.7330258411633287f : 0.0f;  // -2 ln(ln 2)
      p.lse[(size_t)bh * Tn + qr] = (m_run + __builtin_amdgcn_logf(l)) * kLn2 + corr;
    }
  }
}

template <typename T, int D, bool CSA>
inline hipError_t launch_attn(const FwdParams& prm, hipStream_t stream) {
  const int nqb = (prm.T + kBlockRows - 1) / kBlockRows;
  FwdParams p = prm;
  p.nqb = nqb;
  const dim3 grid((unsigned)(nqb * prm.B * prm.H));
  hipLaunchKernelGGL((attn_fwd_kernel<T, D, CSA>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace csa
