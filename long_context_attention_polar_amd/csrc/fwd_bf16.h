// Fused Polar Attention forward, bf16 inputs, fp32 accumulation, on gfx950 MFMA.
//
// [ATMA §2.2, fused kernel]: one streaming pass over the visible keys keeps, per query,
// the running maximum, sum p, sum p^2 and the value accumulator; a move of the maximum
// rescales sum p and acc by alpha and sum p^2 by alpha^2.  The T x T score matrix is
// never stored.
//
// Work decomposition
//   * A workgroup of NW waves owns BM = 32 * NW query rows of one (b, h); each wave
//     owns 32 rows.  Keys stream through LDS in tiles of BN, double-buffered: the next
//     tile's global loads are issued before the current tile is computed and written
//     to the other LDS buffer afterwards, one barrier per tile.
//   * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16
//     (A = K rows from LDS, B = the wave's Q^T fragment held in registers).  In the
//     32x32 accumulator layout lane l then holds query (l % 32) and 16 of every 32 keys,
//     so a row's maximum and sums are one cross-half exchange away, and its
//     correction factor is a per-lane scalar.
//   * The output is accumulated transposed, O^T += V^T P^T.  The probabilities are
//     already where the B operand needs them (the lane's own query, 8 keys per k-step)
//     once the keys of each 16-key step are taken in the order
//     0-3, 8-11, 4-7, 12-15; V^T is stored in LDS in that order, so the A operand is
//     one 16-byte LDS read per lane.
//   * sum p and sum p^2 are per-lane partial sums in fp32, taken from the fp32 p before
//     it is rounded to bf16 for the P V product; the two halves of the wave are added
//     once, in the epilogue.
#pragma once

#include "polar_common.h"

namespace polar {

// Position, inside a 16-key step of V^T in LDS, of key group g (4 keys each).
__device__ __forceinline__ int vt_group_pos(int g) { return (g == 1) ? 2 : (g == 2) ? 1 : g; }

template <int D, int BN, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void polar_fwd_bf16_kernel(const FwdParams p) {
  constexpr int NT = NW * 64;
  constexpr int BM = NW * 32;
  constexpr int KSTR = D + 8;          // K row stride in LDS (elements)
  constexpr int VSTR = BN + 8;         // V^T row stride in LDS (elements)
  constexpr int MB = BN / 32;          // 32-key blocks per tile
  constexpr int KS = D / 16;           // k-steps of Q K^T
  constexpr int DM = D / 32;           // 32-wide d blocks of P V
  constexpr int PS = BN / 16;          // k-steps of P V
  constexpr int KCHUNKS = BN * D / 8;  // 16-byte chunks per K tile
  constexpr int KPT = (KCHUNKS + NT - 1) / NT;
  constexpr int VUNITS = (BN / 4) * (D / 8);  // (4 keys x 8 dims) units per V tile
  constexpr int VPT = (VUNITS + NT - 1) / NT;
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");

  __shared__ __attribute__((aligned(16))) __bf16 k_lds[2][BN * KSTR];
  __shared__ __attribute__((aligned(16))) __bf16 vt_lds[2][D * VSTR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;
  const int half = lane >> 5;

  int qt, bh;
  tile_coords(blockIdx.x, p.n_qt, p.B * p.H, qt, bh);
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int hk = h / (p.H / p.Hkv);
  const int Tq = p.Tq, Tk = p.Tk;
  const int off = Tk - Tq;
  const int q0 = qt * BM;
  const int qrow = q0 + wave * 32 + col;

  const __bf16* qb = (const __bf16*)p.q + (size_t)bh * Tq * D;
  const __bf16* kb = (const __bf16*)p.k + (size_t)(b * p.Hkv + hk) * Tk * D;
  const __bf16* vb = (const __bf16*)p.v + (size_t)(b * p.Hkv + hk) * Tk * D;

  const int hpi = h * p.hp_stride;
  const int n_vis = visible_keys(qrow, Tq, Tk, CAUSAL);
  const float lam = length_temperature(p.hp.tau[hpi], n_vis);
  const float c = lam * p.scale * kLog2e;
  // Largest key index this lane's query may see.
  const int kmax = CAUSAL ? min(qrow + off, Tk - 1) : Tk - 1;

  // Q^T fragments: lane holds query qrow, dims ks*16 + 8*half + [0, 8).
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (qrow < Tq) {
      qf[ks] = *(const bf16x8*)(qb + (size_t)qrow * D + ks * 16 + 8 * half);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[ks][e] = (__bf16)0.0f;
    }
  }

  const int kv_end = CAUSAL ? min(Tk, q0 + BM + off) : Tk;
  const int ntiles = (kv_end + BN - 1) / BN;
  const int first_mask_tile = CAUSAL ? (q0 + off + 1) / BN : Tk / BN;
  const int wave_kmax = CAUSAL ? min(q0 + wave * 32 + 31 + off, Tk - 1) : Tk - 1;

  // ---- global -> registers -> LDS staging of one K/V tile
  u32x4 kreg[KPT];
  u32x4 vreg[VPT][4];
  auto load_tile = [&](int t) {
    const int kv0 = t * BN;
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      const int cidx = tid + r * NT;
      if (KCHUNKS % NT == 0 || cidx < KCHUNKS) {
        const int row = cidx / (D / 8), c8 = cidx % (D / 8);
        const int key = kv0 + row;
        kreg[r] = key < Tk ? *(const u32x4*)(kb + (size_t)key * D + c8 * 8) : u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int r = 0; r < VPT; ++r) {
      const int u = tid + r * NT;
      if (VUNITS % NT == 0 || u < VUNITS) {
        const int dch = u % (D / 8), kg = u / (D / 8);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = kv0 + 4 * kg + j;
          vreg[r][j] = key < Tk ? *(const u32x4*)(vb + (size_t)key * D + dch * 8) : u32x4{0, 0, 0, 0};
        }
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      const int cidx = tid + r * NT;
      if (KCHUNKS % NT == 0 || cidx < KCHUNKS) {
        const int row = cidx / (D / 8), c8 = cidx % (D / 8);
        *(u32x4*)(&k_lds[buf][row * KSTR + c8 * 8]) = kreg[r];
      }
    }
#pragma unroll
    for (int r = 0; r < VPT; ++r) {
      const int u = tid + r * NT;
      if (VUNITS % NT == 0 || u < VUNITS) {
        const int dch = u % (D / 8), kg = u / (D / 8);
        const int pos = (kg >> 2) * 16 + 4 * vt_group_pos(kg & 3);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t a0 = vreg[r][0][w], a1 = vreg[r][1][w], a2 = vreg[r][2][w], a3 = vreg[r][3][w];
          // dim 2w: low halves; dim 2w+1: high halves; keys 0..3 packed along the row
          const u32x2 lo = {(a0 & 0xffffu) | (a1 << 16), (a2 & 0xffffu) | (a3 << 16)};
          const u32x2 hi = {(a0 >> 16) | (a1 & 0xffff0000u), (a2 >> 16) | (a3 & 0xffff0000u)};
          *(u32x2*)(&vt_lds[buf][(dch * 8 + 2 * w) * VSTR + pos]) = lo;
          *(u32x2*)(&vt_lds[buf][(dch * 8 + 2 * w + 1) * VSTR + pos]) = hi;
        }
      }
    }
  };

  // ---- running statistics (base-2 units), per lane = per query, split over 2 lanes
  float m_ref = kMaxInit;   // reference maximum the sums are relative to
  float m_true = kMaxInit;  // true running maximum
  float s1 = 0.0f, s2 = 0.0f;
  f32x16 o[DM];
#pragma unroll
  for (int dm = 0; dm < DM; ++dm)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[dm][e] = 0.0f;

  auto compute_tile = [&](int buf, int kv0, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    f32x16 s[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[mb][e] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const bf16x8 a = *(const bf16x8*)(&k_lds[buf][(mb * 32 + col) * KSTR + ks * 16 + 8 * half]);
        s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[mb], 0, 0, 0);
      }
    }
    if constexpr (MASK) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int key = kv0 + mb * 32 + 8 * i + 4 * half + j;
            if (key > kmax) s[mb][4 * i + j] = -INFINITY;
          }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) tmax = fmaxf(tmax, s[mb][e]);
    tmax = fmaxf(tmax, xor32(tmax));
    const float cm = c * tmax;
    m_true = fmaxf(m_true, cm);
    if (__ballot(cm > m_ref + kRescaleSlack) != 0) {
      const float m_new = fmaxf(m_ref, cm);
      const float alpha = fast_exp2(m_ref - m_new);
      s1 *= alpha;
      s2 *= alpha * alpha;  // squared correction factor
#pragma unroll
      for (int dm = 0; dm < DM; ++dm)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[dm][e] *= alpha;
      m_ref = m_new;
    }
    const float neg_m = -m_ref;
    bf16x8 pf[PS];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float pv = fast_exp2(fmaf(c, s[mb][4 * i + j], neg_m));
          s1 += pv;
          s2 = fmaf(pv, pv, s2);
          pf[mb * 2 + (i >> 1)][(i & 1) * 4 + j] = (__bf16)pv;
        }
#pragma unroll
    for (int kst = 0; kst < PS; ++kst) {
#pragma unroll
      for (int dm = 0; dm < DM; ++dm) {
        const bf16x8 a = *(const bf16x8*)(&vt_lds[buf][(dm * 32 + col) * VSTR + kst * 16 + 8 * half]);
        o[dm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kst], o[dm], 0, 0, 0);
      }
    }
  };

  // ---- main loop
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);
    const int kv0 = t * BN;
    if (!CAUSAL || kv0 <= wave_kmax) {
      if (t >= first_mask_tile)
        compute_tile(buf, kv0, std::true_type{});
      else
        compute_tile(buf, kv0, std::false_type{});
    }
    if (t + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: combine the two halves, form the channels [ATMA §2.1]
  s1 += xor32(s1);
  s2 += xor32(s2);
  const float to_true = fast_exp2(m_ref - m_true);
  const float S1 = s1 * to_true;
  const float S2 = s2 * to_true * to_true;
  float nn = 0.0f;
#pragma unroll
  for (int dm = 0; dm < DM; ++dm)
#pragma unroll
    for (int e = 0; e < 16; ++e) nn = fmaf(o[dm][e], o[dm][e], nn);
  nn += xor32(nn);
  const float inv = nn > 0.0f ? 1.0f / sqrtf(nn) : 0.0f;
  if (qrow < Tq) {
    const size_t row = (size_t)bh * Tq + qrow;
    float* drow = p.dir + row * D;
#pragma unroll
    for (int dm = 0; dm < DM; ++dm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 val = {o[dm][4 * i] * inv, o[dm][4 * i + 1] * inv, o[dm][4 * i + 2] * inv,
                           o[dm][4 * i + 3] * inv};
        *(f32x4*)(drow + dm * 32 + 8 * i + 4 * half) = val;
      }
    if (half == 0) {
      const float m_nat = m_true * kLn2;
      float neff, conf, count;
      magnitude_channel(m_nat, S1, S2, n_vis, lam, p.floor_on != 0, p.hp.beta[hpi], p.hp.kinv[hpi], neff, conf,
                        count);
      p.neff[row] = neff;
      if (p.conf) p.conf[row] = conf;
      if (p.count) p.count[row] = count;
      if (p.stats) {
        p.stats[row * 3 + 0] = m_nat;
        p.stats[row * 3 + 1] = S1;
        p.stats[row * 3 + 2] = S2;
      }
    }
  }
}

}  // namespace polar
