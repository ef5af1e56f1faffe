// Fused Polar Attention forward, bf16 inputs, fp32 accumulation, on gfx950 MFMA.
//
// [ATMA §2.2, fused kernel]: one streaming pass over the visible keys keeps, per query,
// the running maximum, sum p, sum p^2 and the value accumulator; a move of the maximum
// rescales sum p and acc by alpha and sum p^2 by alpha^2.  The T x T score matrix is
// never stored.
//
// Work decomposition
//   * A workgroup of NW waves owns BM = 32 * NB * NW query rows of one (b, h); each wave
//     owns NB blocks of 32 rows (two at d = 64, so every K and V operand read from LDS
//     feeds two MFMAs).  Keys stream through LDS in tiles of BN = 64 rows,
//     double-buffered, with direct global->LDS buffer loads (no registers, no LDS store
//     instructions): the loads of tile t+1 are in flight while tile t is computed, and
//     one barrier per tile publishes them.  Rows past the end of the keys fall outside
//     the buffer range and read as zero.  K and V stay row-major in LDS; the 16-byte
//     chunks of a row are XOR-swizzled so both read patterns below are free of bank
//     conflicts.
//   * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16
//     (A = K rows from LDS, B = the wave's Q^T fragment held in registers).  In the
//     32x32 accumulator layout lane l holds query (l % 32) and 16 of every 32 keys, so a
//     row's statistics are per-lane scalars split over two lanes (l, l ^ 32).
//   * The output is accumulated transposed, O^T += V^T P^T.  The weights are used in
//     place as the B operand once the keys of each 16-key step are taken in the order
//     0-3, 8-11, 4-7, 12-15; the matching V^T operand comes straight from the row-major
//     V tile through two ds_read_b64_tr_b16 transpose reads, each delivering four
//     consecutive keys of one dimension to a lane.
//   * The weights of a tile are formed against the current reference maximum, with no
//     maximum taken first.  When some lane's weights of the tile sum to more than 2^16 (so
//     a weight may exceed 2^16; always on the wave's first tile), the wave moves the
//     reference of its rows to the tile maximum, rescales sum p and acc by alpha and
//     sum p^2 by alpha^2, and forms the tile's weights again from its scores, which are
//     still in registers.  Later moves happen only when a row's maximum grows by more
//     than 16 in base-2 units.  The variant that reports statistics tracks the true
//     maximum on the side.
//   * sum p and sum p^2 are summed in fp32 from the fp32 weights, before these are rounded
//     to bf16 for P V, as per-lane partial sums combined once in the epilogue.  Sums of
//     the bf16 weights would move n_eff = S1^2 / S2 by up to about 4 * 2^-8 on rows whose
//     weight mass and squared mass sit on keys rounded in opposite directions.
//   * Reading variants that change the inner loop are template flags: KF, a per-key
//     floor (1: weight max(e^s - e^f, 0); 2: e^s only when s > f), for which a row's
//     reference starts at its floor f so the floor's own weight e^{f - m_ref} never
//     exceeds 1; WIN, a sliding window, which skips the tiles before a workgroup's
//     window and masks the tiles it starts in.
#pragma once

#include <type_traits>

#include "polar_common.h"

namespace polar {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
#define POLAR_LDS(p) ((__attribute__((address_space(3))) void*)(p))
#define POLAR_GLOBAL(p) ((__attribute__((address_space(1))) void*)(p))

// XOR swizzle of the 16-byte chunks of an LDS row of K or V (row = key index in the
// tile).  D = 64: two rows share the 64 banks; the chunk index is permuted by a map of
// (row / 2) whose consecutive even/odd pairs land in different chunk pairs.  D = 128:
// a row spans all banks; the chunk index is XORed with a permutation of (row % 16)
// whose four consecutive rows fall into four different quarters.
template <int D>
__device__ __forceinline__ int chunk_swizzle(int row) {
  if constexpr (D == 64) {
    const int e = (row >> 1) & 7;
    return (e >> 1) | ((e & 1) << 2);
  } else {
    return ((row & 3) << 2) | ((row >> 2) & 3);
  }
}

// Byte offset, inside a K or V tile, of the 16-byte global chunk this lane loads with
// the wave's first tile-load instruction.  Every wave-wide load fills 1 KiB of LDS
// (lane i -> bytes [16 i, 16 i + 16)); the lane picks its global chunk so that the LDS
// image is the swizzled tile.  Instruction r of the wave (tile bytes
// [(wave + NW r) KiB, +1 KiB)) reads NW KiB further on in the head's rows, where the
// swizzle repeats, so the same offset serves every instruction and every tile.
template <int D, int NW>
__device__ __forceinline__ uint32_t tile_lane_offset(int wave, int lane) {
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  static_assert((NW * 64 / CPR) % 16 == 0, "the row advance per instruction must keep the swizzle");
  const int idx = wave * 64 + lane;
  const int row = idx / CPR;
  const int lc = (idx % CPR) ^ chunk_swizzle<D>(row);
  return (uint32_t)((row * D + lc * 8) * 2);
}

// Issue the buffer loads that bring the BN x D bf16 tile starting at key kv0 straight
// into LDS.  Rows at or past the end of the head's keys lie outside the buffer range
// and read as zero.
template <int D, int BN, int NW>
__device__ __forceinline__ void load_tile(__amdgpu_buffer_rsrc_t rsrc, int kv0, uint32_t voff, __bf16* dst,
                                          int wave) {
  constexpr int INSTR = BN * D * 2 / 1024;
  static_assert(INSTR % NW == 0, "tile must split evenly over the waves");
#pragma unroll
  for (int r = 0; r < INSTR / NW; ++r) {
    const int i = wave + r * NW;
    // the whole byte offset sits in the VGPR operand, which the range check covers
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, POLAR_LDS(dst + i * 512), 16,
                                             voff + (uint32_t)(kv0 * D * 2 + r * NW * 1024), 0, 0, 0);
  }
}

// Make the tile loads of every wave visible to the workgroup: wait for this wave's own
// global->LDS loads (vmcnt), then the barrier.  The explicit wait is needed because the
// compiler's workgroup barrier does not wait for these loads by itself: their LDS writes
// are not ordered by the barrier's memory fence, and without the wait a wave may read a
// tile that another wave's loads have not finished writing.
__device__ __forceinline__ void publish_tiles() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt and lgkmcnt unconstrained
  __syncthreads();
}

template <int D, int BN, int NW, int NB, int OCC, bool CAUSAL, bool STATS, int KF = POLAR_KEY_FLOOR_NULL,
          bool WIN = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(OCC, OCC))) void polar_fwd_bf16_kernel(
    const FwdParams p) {
  static_assert(BN == 32 || BN == 64, "key tile");
  static_assert(!WIN || CAUSAL, "a sliding window needs the causal alignment");
  static_assert(D == 64 || D == 128, "head_dim");
  static_assert(NB == 1 || NB == 2, "query blocks per wave");
  constexpr int QPW = 32 * NB;  // query rows per wave
  constexpr int BM = NW * QPW;  // query rows per workgroup
  constexpr int MB = BN / 32;   // 32-key blocks per tile
  constexpr int KS = D / 16;    // k-steps of Q K^T
  constexpr int DM = D / 32;    // 32-wide d blocks of P V
  constexpr int PS = BN / 16;   // k-steps of P V
  // workgroups resident at once: 256 CUs x 4 SIMDs x OCC waves per SIMD, NW waves each
  constexpr int kResidentBlocks = 256 * 4 * OCC / NW;

  __shared__ __attribute__((aligned(1024))) __bf16 k_buf0[BN * D];
  __shared__ __attribute__((aligned(1024))) __bf16 k_buf1[BN * D];
  __shared__ __attribute__((aligned(1024))) __bf16 v_buf0[BN * D];
  __shared__ __attribute__((aligned(1024))) __bf16 v_buf1[BN * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int col = lane & 31;
  const int half = lane >> 5;

  int qt, bh;
  tile_coords<kResidentBlocks>(blockIdx.x, p.n_qt, p.B * p.H, qt, bh);
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int hk = h / (p.H / p.Hkv);
  const int Tq = p.Tq, Tk = p.Tk;
  const int off = Tk - Tq;
  const int q0 = qt * BM;
  const int wq0 = q0 + wave * QPW;  // first query row of this wave

  const __bf16* qb = (const __bf16*)p.q + (size_t)bh * Tq * D;
  const size_t kv_head = (size_t)(b * p.Hkv + hk) * Tk * D;
  const uint32_t head_bytes = (uint32_t)((size_t)Tk * D * 2);
  const __amdgpu_buffer_rsrc_t kb =
      __builtin_amdgcn_make_buffer_rsrc((void*)((const __bf16*)p.k + kv_head), (short)0, head_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vb =
      __builtin_amdgcn_make_buffer_rsrc((void*)((const __bf16*)p.v + kv_head), (short)0, head_bytes, 0x00020000);
  const uint32_t voff = tile_lane_offset<D, NW>(wave, lane);

  const int kv_end = CAUSAL ? min(Tk, q0 + BM + off) : Tk;
  const int ntiles = (kv_end + BN - 1) / BN;
  // last key any row of the wave may see, and the smallest such limit over its rows
  const int wave_kmax = CAUSAL ? min(wq0 + QPW - 1 + off, Tk - 1) : Tk - 1;
  const int wave_kmin = CAUSAL ? min(wq0 + off, Tk - 1) : Tk - 1;
  // sliding window: row i sees keys from i + off - win + 1; the first tile of the
  // workgroup, and the smallest and largest first key over the wave's rows
  const int win = WIN ? p.hp.window : 0;
  const int t_begin = WIN ? max(0, q0 + off - win + 1) / BN : 0;
  const int wave_klo_min = wq0 + off - win + 1;
  const int wave_klo_max = wq0 + QPW - 1 + off - win + 1;

  // Start the first tile's loads before anything else.
  load_tile<D, BN, NW>(kb, t_begin * BN, voff, k_buf0, wave);
  load_tile<D, BN, NW>(vb, t_begin * BN, voff, v_buf0, wave);

  // a1: per query block: row, visible count, temperature, base-2 logit scale, mask limits
  const int hpi = h * p.hp_stride;
  int qrow[NB], n_vis[NB], kmax[NB], klo[NB];
  float lam[NB], c[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    qrow[nb] = wq0 + nb * 32 + col;
    n_vis[nb] = context_count(qrow[nb], Tq, Tk, CAUSAL, p.ctx_k);
    if (WIN) n_vis[nb] = min(n_vis[nb], win);
    lam[nb] = row_temperature(p.hp, hpi, n_vis[nb]);
    c[nb] = logit_scale(lam[nb], p.scale);
    kmax[nb] = CAUSAL ? min(qrow[nb] + off, Tk - 1) : Tk - 1;
    klo[nb] = WIN ? qrow[nb] + off - win + 1 : 0;
  }

  // Q^T fragments: lane holds query qrow[nb], dims ks*16 + 8*half + [0, 8).
  bf16x8 qf[NB][KS];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (qrow[nb] < Tq) {
        qf[nb][ks] = *(const bf16x8*)(qb + (size_t)qrow[nb] * D + ks * 16 + 8 * half);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[nb][ks][e] = (__bf16)0.0f;
      }
    }

  // LDS byte offsets of this lane's operand reads (same for both buffers).
  // K (A operand of S^T): row mb*32 + col, logical chunk 2*ks + half, stored at chunk
  // (2 ks + half) ^ sw = 2 (ks ^ (x >> 1)) + (x & 1) with x = half ^ sw, so the byte
  // offset is k_base + ((32 ks) ^ k_xor).
  const int k_x = half ^ chunk_swizzle<D>(col);
  const uint32_t k_base = (uint32_t)(col * D * 2 + 16 * (k_x & 1));
  const uint32_t k_xor = (uint32_t)(32 * (k_x >> 1));
  // V (A operand of O^T via transpose reads): in the 16-lane group g = lane / 16 the lane
  // points at key (4 * half + gi / 4) [+ 8 for the second read] and dims
  // dm*32 + 16*(g & 1) + 4*(gi & 3) .. + 3.
  const int gi = lane & 15;
  const int g = lane >> 4;
  int v_off[2][DM];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int row = 8 * r + 4 * half + (gi >> 2);
    const int sw = chunk_swizzle<D>(row);
#pragma unroll
    for (int dm = 0; dm < DM; ++dm) {
      const int lchunk = 4 * dm + 2 * (g & 1) + ((gi & 3) >> 1);
      v_off[r][dm] = row * D + ((lchunk ^ sw) << 3) + 4 * (gi & 1);
    }
  }

  // per-key floor: the row's floor f in base-2 units (the data-adaptive level needs the
  // norm of q, whose halves sit in lanes l and l ^ 32)
  float f2[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) f2[nb] = 0.0f;
  if constexpr (KF != POLAR_KEY_FLOOR_NULL) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float qq = 0.0f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) qq = fmaf((float)qf[nb][ks][e], (float)qf[nb][ks][e], qq);
      qq += xor32(qq);
      const float sigma = p.hp.level_form == POLAR_LEVEL_QNORM ? p.scale * sqrtf(qq) : 1.0f;
      f2[nb] = null_floor(p.hp, hpi, n_vis[nb], lam[nb], sigma) * kLog2e;
    }
  }

  // running statistics (base 2), per lane and query block; each row is split over the
  // two lanes l and l ^ 32
  float m_ref[NB], t_max[NB], s1[NB][2], s2[NB][2];
  f32x16 o[NB][DM];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    // the reference maximum the sums are relative to; with a per-key floor it starts at
    // the floor, so e^{f - m_ref} <= 1 throughout
    m_ref[nb] = KF != POLAR_KEY_FLOOR_NULL ? f2[nb] : kMaxInit;
    t_max[nb] = -INFINITY;  // true maximum of this lane's raw scores
    s1[nb][0] = s1[nb][1] = s2[nb][0] = s2[nb][1] = 0.0f;
#pragma unroll
    for (int dm = 0; dm < DM; ++dm)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[nb][dm][e] = 0.0f;
  }

  auto compute_tile = [&](const __bf16* kt, const __bf16* vt, int kv0) {
    // ---- a3: S^T = K Q^T; each K fragment feeds the NB query blocks
    f32x16 s[NB][MB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[nb][mb][e] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const bf16x8 a = *(const bf16x8*)((const char*)kt + (k_base + ((32u * ks) ^ k_xor)) + mb * 32 * D * 2);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          s[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[nb][ks], s[nb][mb], 0, 0, 0);
      }
    bf16x8 pf[NB][PS];
    // ---- mask on the diagonal / tail tiles (and the window's first tiles) only (in place)
    if (kv0 + BN - 1 > wave_kmin || (WIN && kv0 < wave_klo_max)) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int lim = kmax[nb] - kv0 - 4 * half;    // key offset limits for this lane
        const int lim_lo = klo[nb] - kv0 - 4 * half;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int r = mb * 32 + 8 * i + j;
              if (r > lim || (WIN && r < lim_lo)) s[nb][mb][4 * i + j] = -INFINITY;
            }
      }
    }
    // ---- a5: p = exp2(c s - m_ref), rounded to bf16 in the B-operand order; the tile's
    // sum p and sum p^2 are taken from the fp32 weights
    float t1[NB], t2[NB];
    auto weights = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const float neg_m = -m_ref[nb];
        // per-key floor: the floor's weight e^{f - m_ref} (soft), or its offset f - m_ref (gate)
        const float fl = KF == POLAR_KEY_FLOOR_SOFT ? fast_exp2(f2[nb] - m_ref[nb]) : f2[nb] - m_ref[nb];
        auto weight = [&](float sc) __attribute__((always_inline)) {
          const float t = fmaf(c[nb], sc, neg_m);
          if constexpr (KF == POLAR_KEY_FLOOR_SOFT) return fmaxf(fast_exp2(t) - fl, 0.0f);
          if constexpr (KF == POLAR_KEY_FLOOR_GATE) return t > fl ? fast_exp2(t) : 0.0f;
          return fast_exp2(t);
        };
        float a1 = 0.0f, a2 = 0.0f;  // one chain per sum, over the fp32 weights
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; j += 2) {
              const float w0 = weight(s[nb][mb][4 * i + j]);
              const float w1 = weight(s[nb][mb][4 * i + j + 1]);
              a1 += w0;
              a1 += w1;
              a2 = fmaf(w0, w0, a2);
              a2 = fmaf(w1, w1, a2);
              pf[nb][mb * 2 + (i >> 1)][(i & 1) * 4 + j] = (__bf16)w0;
              pf[nb][mb * 2 + (i >> 1)][(i & 1) * 4 + j + 1] = (__bf16)w1;
            }
        t1[nb] = a1;
        t2[nb] = a2;
      }
    };
    auto lane_max = [&](int nb) __attribute__((always_inline)) {
      float a = s[nb][0][0], b2 = s[nb][0][1];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = (mb == 0 ? 2 : 0); e < 16; e += 2) {
          a = fmaxf(a, s[nb][mb][e]);
          b2 = fmaxf(b2, s[nb][mb][e + 1]);
        }
      return fmaxf(a, b2);
    };
    weights();
    if constexpr (STATS) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) t_max[nb] = fmaxf(t_max[nb], lane_max(nb));
    }
    // ---- a4: some weight of the wave may exceed 2^16 (a lane's tile sum does; always on
    // the wave's first tile): move the reference of the rows to the tile maximum,
    // rescale sum p and acc by alpha and sum p^2 by alpha^2, and form the weights again
    bool big = false;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) big |= t1[nb] > kWeightLimit;
    if (__ballot(big) != 0) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const float mx = lane_max(nb);
        const float row_max = fmaxf(mx, xor32(mx));
        const float m_new = fmaxf(m_ref[nb], c[nb] * row_max);
        const float alpha = fast_exp2(m_ref[nb] - m_new);
        const float alpha2 = alpha * alpha;  // squared correction factor
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          s1[nb][u] *= alpha;
          s2[nb][u] *= alpha2;
        }
#pragma unroll
        for (int dm = 0; dm < DM; ++dm)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[nb][dm][e] *= alpha;
        m_ref[nb] = m_new;
      }
      weights();
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      s1[nb][0] += t1[nb];
      s2[nb][0] += t2[nb];
    }
    // ---- a6: O^T += V^T P^T; each V fragment feeds the NB query blocks
#pragma unroll
    for (int kst = 0; kst < PS; ++kst)
#pragma unroll
      for (int dm = 0; dm < DM; ++dm) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(vt + v_off[0][dm] + kst * 16 * D));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(vt + v_off[1][dm] + kst * 16 * D));
        const s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8 a = __builtin_bit_cast(bf16x8, both);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          o[nb][dm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[nb][kst], o[nb][dm], 0, 0, 0);
      }
  };

  // a tile the wave needs: not past its last visible key, not before its window
  auto wave_needs = [&](int kv0) __attribute__((always_inline)) {
    return kv0 <= wave_kmax && (!WIN || kv0 + BN - 1 >= wave_klo_min);
  };

  // ---- main loop: tile t is read from one buffer pair while tile t+1 loads into the other
  publish_tiles();
  for (int t = t_begin; t < ntiles; t += 2) {
    if (t + 1 < ntiles) {
      load_tile<D, BN, NW>(kb, (t + 1) * BN, voff, k_buf1, wave);
      load_tile<D, BN, NW>(vb, (t + 1) * BN, voff, v_buf1, wave);
    }
    if (wave_needs(t * BN)) compute_tile(k_buf0, v_buf0, t * BN);
    publish_tiles();
    if (t + 1 >= ntiles) break;
    if (t + 2 < ntiles) {
      load_tile<D, BN, NW>(kb, (t + 2) * BN, voff, k_buf0, wave);
      load_tile<D, BN, NW>(vb, (t + 2) * BN, voff, v_buf0, wave);
    }
    if (wave_needs((t + 1) * BN)) compute_tile(k_buf1, v_buf1, (t + 1) * BN);
    publish_tiles();
  }

  // ---- a7: combine the two halves of each row and form the channels [ATMA §2.1].
  // n_eff, the confidence and the direction do not depend on the reference, so they are
  // formed from the sums relative to it; the statistics, when requested, are brought to
  // the true maximum, which that variant tracks on the side.
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float S1 = s1[nb][0] + s1[nb][1];
    float S2 = s2[nb][0] + s2[nb][1];
    S1 += xor32(S1);
    S2 += xor32(S2);
    const float row_tmax = STATS ? fmaxf(t_max[nb], xor32(t_max[nb])) : 0.0f;  // all lanes take part
    float nn = 0.0f;
#pragma unroll
    for (int dm = 0; dm < DM; ++dm)
#pragma unroll
      for (int e = 0; e < 16; ++e) nn = fmaf(o[nb][dm][e], o[nb][dm][e], nn);
    nn += xor32(nn);
    const float inv = nn == 0.0f ? 0.0f : 1.0f / sqrtf(nn);  // a NaN norm stays NaN
    // the data-adaptive floor level needs the norm of the row's q (all lanes take part)
    float sigma = 1.0f;
    if (p.hp.level_form == POLAR_LEVEL_QNORM) {
      float qq = 0.0f;
      if (qrow[nb] < Tq) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 x = *(const bf16x8*)(qb + (size_t)qrow[nb] * D + ks * 16 + 8 * half);
#pragma unroll
          for (int e = 0; e < 8; ++e) qq = fmaf((float)x[e], (float)x[e], qq);
        }
      }
      qq += xor32(qq);
      sigma = p.scale * sqrtf(qq);
    }
    if (STATS && p.part) {
      // partial mode: the statistics of this call's keys relative to their true maximum
      if (qrow[nb] < Tq) {
        const float m_true = c[nb] * row_tmax;
        // with a per-key floor the reference may sit above the true maximum; the sums are
        // then 0 (no key above the floor) and must not meet an overflowing factor
        const float to_true = S1 > 0.0f ? fast_exp2(m_ref[nb] - m_true) : 0.0f;
        const size_t row = (size_t)bh * Tq + qrow[nb];
        float* out = p.part + (row * p.part_S + p.part_s) * (D + 3);
#pragma unroll
        for (int dm = 0; dm < DM; ++dm)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) out[3 + dm * 32 + 8 * i + 4 * half + j] = o[nb][dm][4 * i + j] * to_true;
        if (half == 0) {
          out[0] = m_true * kLn2;
          out[1] = S1 * to_true;
          out[2] = S2 * to_true * to_true;
        }
      }
      continue;
    }
    if (qrow[nb] < Tq) {
      const size_t row = (size_t)bh * Tq + qrow[nb];
      float* drow = p.dir + row * D;
#pragma unroll
      for (int dm = 0; dm < DM; ++dm)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 val = {o[nb][dm][4 * i] * inv, o[nb][dm][4 * i + 1] * inv, o[nb][dm][4 * i + 2] * inv,
                             o[nb][dm][4 * i + 3] * inv};
          *(f32x4*)(drow + dm * 32 + 8 * i + 4 * half) = val;
        }
      if (half == 0) {
        float neff, conf, count;
        const float f = null_floor(p.hp, hpi, n_vis[nb], lam[nb], sigma);
        magnitude_channel(p.hp, hpi, m_ref[nb] * kLn2, S1, S2, f, p.floor_on != 0, neff, conf, count);
        p.neff[row] = neff;
        if (p.conf) p.conf[row] = conf;
        if (p.count) p.count[row] = count;
        if (STATS && p.stats) {
          const float m_true = c[nb] * row_tmax;
          const float to_true = S1 > 0.0f ? fast_exp2(m_ref[nb] - m_true) : 0.0f;
          p.stats[row * 3 + 0] = m_true * kLn2;
          p.stats[row * 3 + 1] = S1 * to_true;
          p.stats[row * 3 + 2] = S2 * to_true * to_true;
        }
      }
    }
  }
}

}  // namespace polar
