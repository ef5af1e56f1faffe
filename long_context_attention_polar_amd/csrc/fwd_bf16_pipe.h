// Fused Polar Attention forward, bf16 inputs, fp32 accumulation: the software-pipelined
// form of the prefill kernel for the default reading (no per-key floor, no window).
//
// [ATMA §2.2, fused kernel]: one streaming pass over the visible keys keeps, per query,
// the running maximum, sum p, sum p^2 and the value accumulator; a move of the maximum
// rescales sum p and acc by alpha and sum p^2 by alpha^2.
//
// The operand layouts, the LDS image of K and V (64-key tiles, XOR-swizzled rows, direct
// buffer->LDS loads) and the arithmetic of a block of keys are those of
// polar_fwd_bf16_kernel (fwd_bf16.h).  What differs is the order of the work.  On this
// part the matrix cores and the vector ALU of a SIMD overlap only when one wave's
// instruction stream interleaves them, so a wave works on three 32-key blocks at once:
// while its vector ALU forms the weights of block b, the matrix cores compute the scores
// of block b+1 and the P V product of block b-1.  Each 64-key tile is taken in two such
// steps, one before and one after the workgroup's barrier:
//
//   step 1 of tile t:  scores (t, 1)   | weights (t, 0) | P V (t-1, 1)
//   barrier; loads of K of tile t+2 and V of tile t+1
//   step 2 of tile t:  scores (t+1, 0) | weights (t, 1) | P V (t, 0)
//
// Step 1 reads only K of tile t and V of tile t-1, step 2 only K of tile t+1 and V of
// tile t.  K therefore runs one tile ahead of V, and each of them is double-buffered: the
// buffers that step 1 was the last to read are refilled right after the barrier, and every
// load has the two steps of a whole tile to land before the barrier that publishes it.
//
// The tiles that every row of the workgroup sees in full go through these steps.  The
// others (from the tile where the workgroup's causal diagonal begins, and a ragged last
// tile) take the plain path, tile by tile: in step 1 the scores of both blocks, masked
// where a row does not see a key, and their weights against one reference; in step 2
// their P V products.
//
// The reference maximum moves lazily, as in the plain kernel: when some lane's weights of
// a block sum to more than 2^16 (always on the wave's first block), the wave moves the
// reference of its rows to the block maximum, rescales sum p, sum p^2 (by alpha^2) and acc,
// and forms the block's weights again.  acc then already holds the P V product of the
// previous block, whose weights were formed against the old reference, so the rescale
// applies to it too.  sum p and sum p^2 are summed in fp32 from the fp32 weights, before
// these are rounded to bf16 for P V.
#pragma once

#include "fwd_bf16.h"

namespace polar {

template <int D, int NW, int NB, int OCC, bool CAUSAL, bool STATS>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(OCC, OCC))) void polar_fwd_bf16_pipe_kernel(
    const FwdParams p) {
  static_assert(D == 64 || D == 128, "head_dim");
  static_assert(NB == 1 || NB == 2, "query blocks per wave");
  constexpr int BN = 64;        // keys per LDS tile: two 32-key blocks
  constexpr int QPW = 32 * NB;  // query rows per wave
  constexpr int BM = NW * QPW;  // query rows per workgroup
  constexpr int KS = D / 16;    // k-steps of Q K^T per block
  constexpr int DM = D / 32;    // 32-wide d blocks of P V
  constexpr int kResidentBlocks = 256 * 4 * OCC / NW;

  __shared__ __attribute__((aligned(1024))) __bf16 k_buf0[BN * D];
  __shared__ __attribute__((aligned(1024))) __bf16 k_buf1[BN * D];
  __shared__ __attribute__((aligned(1024))) __bf16 v_buf0[BN * D];
  __shared__ __attribute__((aligned(1024))) __bf16 v_buf1[BN * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const int wq0 = q0 + wave * QPW;

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
  const int wave_kmax = CAUSAL ? min(wq0 + QPW - 1 + off, Tk - 1) : Tk - 1;

  // K of tiles 0 and 1 and V of tile 0 before anything else
  load_tile<D, BN, NW>(kb, 0, voff, k_buf0, wave);
  load_tile<D, BN, NW>(vb, 0, voff, v_buf0, wave);
  if (ntiles > 1) load_tile<D, BN, NW>(kb, BN, voff, k_buf1, wave);

  // a1: per query block: row, visible count, temperature, base-2 logit scale, mask limit
  const int hpi = h * p.hp_stride;
  int qrow[NB], n_vis[NB], kmax[NB];
  float lam[NB], c[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    qrow[nb] = wq0 + nb * 32 + col;
    n_vis[nb] = context_count(qrow[nb], Tq, Tk, CAUSAL, p.ctx_k);
    lam[nb] = row_temperature(p.hp, hpi, n_vis[nb]);
    c[nb] = logit_scale(lam[nb], p.scale);
    kmax[nb] = CAUSAL ? min(qrow[nb] + off, Tk - 1) : Tk - 1;
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

  // LDS byte offsets of this lane's operand reads, as in polar_fwd_bf16_kernel
  const int k_x = half ^ chunk_swizzle<D>(col);
  const uint32_t k_base = (uint32_t)(col * D * 2 + 16 * (k_x & 1));
  const uint32_t k_xor = (uint32_t)(32 * (k_x >> 1));
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

  // running statistics (base 2) per query block; a row's sums are split over lanes l, l ^ 32
  float m_ref[NB], t_max[NB], s1[NB], s2[NB];
  f32x16 o[NB][DM];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m_ref[nb] = kMaxInit;
    t_max[nb] = -INFINITY;
    s1[nb] = s2[nb] = 0.0f;
#pragma unroll
    for (int dm = 0; dm < DM; ++dm)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[nb][dm][e] = 0.0f;
  }

  // ---- a3 for one 32-key block: S^T = K Q^T, each K fragment feeding the NB query blocks
  auto qk_block = [&](const __bf16* kt, int hb, f32x16(&s)[NB]) __attribute__((always_inline)) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[nb][e] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 a = *(const bf16x8*)((const char*)kt + (k_base + ((32u * ks) ^ k_xor)) + hb * 32 * D * 2);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) s[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[nb][ks], s[nb], 0, 0, 0);
    }
  };
  // ---- a6 for one 32-key block: O^T += V^T P^T, each V fragment feeding the NB query blocks
  auto pv_block = [&](const __bf16* vt, int hb, const bf16x8(&pf)[NB][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kst = 0; kst < 2; ++kst)
#pragma unroll
      for (int dm = 0; dm < DM; ++dm) {
        const int k16 = (hb * 2 + kst) * 16 * D;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(vt + v_off[0][dm] + k16));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(vt + v_off[1][dm] + k16));
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          o[nb][dm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[nb][kst], o[nb][dm], 0, 0, 0);
      }
  };
  // a3 of one block and a6 of another in one stream, their matrix instructions alternating
  // (a k-step of the scores, then a (k-step, d block) of P V), so that the dependent score
  // MFMAs, which accumulate into one register block, are spaced by independent ones
  constexpr int NPV = 2 * DM;                   // (k-step, d block) pairs of P V per block
  constexpr int NST = KS > NPV ? KS : NPV;      // alternation steps
  auto qk_pv_block = [&](const __bf16* kt, int hq, f32x16(&s)[NB], const __bf16* vt, int hv,
                         const bf16x8(&pf)[NB][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[nb][e] = 0.0f;
#pragma unroll
    for (int i = 0; i < NST; ++i) {
      if (i < KS) {
        const bf16x8 a = *(const bf16x8*)((const char*)kt + (k_base + ((32u * i) ^ k_xor)) + hq * 32 * D * 2);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) s[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[nb][i], s[nb], 0, 0, 0);
      }
      if (i < NPV) {
        const int kst = i / DM, dm = i % DM;
        const int k16 = (hv * 2 + kst) * 16 * D;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(vt + v_off[0][dm] + k16));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(vt + v_off[1][dm] + k16));
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          o[nb][dm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[nb][kst], o[nb][dm], 0, 0, 0);
      }
    }
  };
  // ---- a5 for one 32-key block: p = exp2(c s - m_ref), rounded to bf16 in the B-operand
  // order; the block's sum p and sum p^2 over the fp32 weights, one chain each
  auto weights_block = [&](const f32x16(&s)[NB], bf16x8(&pf)[NB][2], float(&t1)[NB], float(&t2)[NB])
                           __attribute__((always_inline)) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float neg_m = -m_ref[nb];
      float a1 = 0.0f, a2 = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; j += 2) {
          const float w0 = fast_exp2(fmaf(c[nb], s[nb][4 * i + j], neg_m));
          const float w1 = fast_exp2(fmaf(c[nb], s[nb][4 * i + j + 1], neg_m));
          a1 += w0;
          a1 += w1;
          a2 = fmaf(w0, w0, a2);
          a2 = fmaf(w1, w1, a2);
          pf[nb][i >> 1][(i & 1) * 4 + j] = (__bf16)w0;
          pf[nb][i >> 1][(i & 1) * 4 + j + 1] = (__bf16)w1;
        }
      t1[nb] = a1;
      t2[nb] = a2;
    }
  };
  auto lane_max = [&](const f32x16& s) __attribute__((always_inline)) {
    float a = s[0], b2 = s[1];
#pragma unroll
    for (int e = 2; e < 16; e += 2) {
      a = fmaxf(a, s[e]);
      b2 = fmaxf(b2, s[e + 1]);
    }
    return fmaxf(a, b2);
  };
  // a4: move the reference of the rows to `row_max` (base-2 tile units) and rescale
  auto move_reference = [&](int nb, float tile_max) __attribute__((always_inline)) {
    const float row_max = fmaxf(tile_max, xor32(tile_max));
    const float m_new = fmaxf(m_ref[nb], c[nb] * row_max);
    const float alpha = fast_exp2(m_ref[nb] - m_new);
    s1[nb] *= alpha;
    s2[nb] *= alpha * alpha;  // squared correction factor
#pragma unroll
    for (int dm = 0; dm < DM; ++dm)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[nb][dm][e] *= alpha;
    m_ref[nb] = m_new;
  };
  // weights, sums and the lazy reference of one fully visible block
  auto settle_block = [&](const f32x16(&s)[NB], bf16x8(&pf)[NB][2], bool interleave) __attribute__((always_inline)) {
    float t1[NB], t2[NB];
    weights_block(s, pf, t1, t2);
    if constexpr (STATS) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) t_max[nb] = fmaxf(t_max[nb], lane_max(s[nb]));
    }
    bool big = false;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) big |= t1[nb] > kWeightLimit;
    if (interleave) {
      // Keep the whole block's weights, sums and bf16 rounding ahead of the branch, where
      // they can fill the gaps between the step's matrix instructions: the empty asm takes
      // them as inputs, so they are formed here rather than sunk past the branch.
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) asm volatile("" ::"v"(pf[nb][0]), "v"(pf[nb][1]), "v"(t2[nb]));
      // the order the step's instructions are issued in: the LDS reads of the next
      // alternation step, the matrix instructions of this one, and an equal share of the
      // weights' vector work
      constexpr int kValu = (72 * NB + NST - 1) / NST;
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
      for (int i = 0; i < NST; ++i) {
        if (i + 1 < NST) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * NB, 0);               // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);                // VALU
      }
    }
    if (__ballot(big) != 0) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) move_reference(nb, lane_max(s[nb]));
      weights_block(s, pf, t1, t2);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      s1[nb] += t1[nb];
      s2[nb] += t2[nb];
    }
  };
  // the plain path's step 1 for a tile that crosses the wave's diagonal or the end of the
  // keys: scores of both blocks, masked, and their weights against one reference
  auto masked_tile = [&](const __bf16* kt, int kv0, f32x16(&sa)[NB], f32x16(&sb)[NB], bf16x8(&pa)[NB][2],
                         bf16x8(&pb)[NB][2]) __attribute__((always_inline)) {
    qk_block(kt, 0, sa);
    qk_block(kt, 1, sb);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int lim = kmax[nb] - kv0 - 4 * half;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (8 * i + j > lim) sa[nb][4 * i + j] = -INFINITY;
          if (32 + 8 * i + j > lim) sb[nb][4 * i + j] = -INFINITY;
        }
    }
    float ta1[NB], ta2[NB], tb1[NB], tb2[NB];
    weights_block(sa, pa, ta1, ta2);
    weights_block(sb, pb, tb1, tb2);
    if constexpr (STATS) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) t_max[nb] = fmaxf(t_max[nb], fmaxf(lane_max(sa[nb]), lane_max(sb[nb])));
    }
    bool big = false;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) big |= ta1[nb] + tb1[nb] > kWeightLimit;
    if (__ballot(big) != 0) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) move_reference(nb, fmaxf(lane_max(sa[nb]), lane_max(sb[nb])));
      weights_block(sa, pa, ta1, ta2);
      weights_block(sb, pb, tb1, tb2);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      s1[nb] += ta1[nb];
      s1[nb] += tb1[nb];
      s2[nb] += ta2[nb];
      s2[nb] += tb2[nb];
    }
  };

  // ---- main loop, in two parts.  Part 1: the tiles every row of the workgroup sees in
  // full (the same count for all its waves), in the pipelined steps.  Part 2: the rest,
  // tile by tile on the plain path (each wave masks what its rows do not see).
  const int n_pipe = CAUSAL ? min(ntiles, (min(q0 + off, Tk - 1) + 1) / BN) : Tk / BN;
  f32x16 sa[NB], sb[NB];        // scores of block 0 / block 1 of a tile
  bf16x8 pa[NB][2], pb[NB][2];  // their bf16 weights
  // Step 1 of the first tile runs the P V product of a "previous" block against V buffer 1
  // with zero weights; the buffer is zeroed first so that no stale LDS bits reach acc.
  {
    constexpr int kWords = BN * D * 2 / 16;  // 16-byte words of a V tile
    for (int i = tid; i < kWords; i += NW * 64) ((u32x4*)v_buf1)[i] = u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int kst = 0; kst < 2; ++kst)
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[nb][kst][e] = (__bf16)0.0f;
  publish_tiles();
  // One pipelined tile; kc, vc: the K and V buffers of tile t, kn, vp: the other two.  The
  // loop below is unrolled by two so that every buffer address is a constant.
  auto pipe_tile = [&](int t, const __bf16* kc, const __bf16* kn, const __bf16* vc, const __bf16* vp)
                       __attribute__((always_inline)) {
    // step 1: scores (t, 1) | weights (t, 0) | P V (t-1, 1); reads K of tile t, V of tile t-1
    qk_pv_block(kc, 1, sb, vp, 1, pb);
    settle_block(sa, pa, true);
    publish_tiles();
    // K of tile t+2 into the buffer of K of tile t, V of tile t+1 into that of V of tile t-1
    if (t + 2 < ntiles) load_tile<D, BN, NW>(kb, (t + 2) * BN, voff, (__bf16*)kc, wave);
    if (t + 1 < ntiles) load_tile<D, BN, NW>(vb, (t + 1) * BN, voff, (__bf16*)vp, wave);
    // step 2: scores (t+1, 0) | weights (t, 1) | P V (t, 0); reads K of tile t+1, V of tile t.
    // After the last pipelined tile the scores are of whatever the other K buffer holds and
    // are not used.
    qk_pv_block(kn, 0, sa, vc, 0, pa);
    settle_block(sb, pb, true);
  };
  if (n_pipe > 0) qk_block(k_buf0, 0, sa);
  int t = 0;
  for (; t + 1 < n_pipe; t += 2) {
    pipe_tile(t, k_buf0, k_buf1, v_buf0, v_buf1);
    pipe_tile(t + 1, k_buf1, k_buf0, v_buf1, v_buf0);
  }
  if (t < n_pipe) pipe_tile(t, k_buf0, k_buf1, v_buf0, v_buf1);
  // P V of block 1 of the last pipelined tile, before the barrier that frees its V buffer
  if (n_pipe > 0) pv_block(((n_pipe - 1) & 1) ? v_buf1 : v_buf0, 1, pb);
  for (int t = n_pipe; t < ntiles; ++t) {
    const bool odd = (t & 1) != 0;
    const int kv0 = t * BN;
    const bool needed = kv0 <= wave_kmax;
    // step 1: the tile's scores, masked, and weights (K of tile t)
    if (needed) masked_tile(odd ? k_buf1 : k_buf0, kv0, sa, sb, pa, pb);
    publish_tiles();
    if (t + 2 < ntiles) load_tile<D, BN, NW>(kb, (t + 2) * BN, voff, odd ? k_buf1 : k_buf0, wave);
    if (t + 1 < ntiles) load_tile<D, BN, NW>(vb, (t + 1) * BN, voff, odd ? v_buf0 : v_buf1, wave);
    // step 2: its P V products (V of tile t)
    if (needed) {
      pv_block(odd ? v_buf1 : v_buf0, 0, pa);
      pv_block(odd ? v_buf1 : v_buf0, 1, pb);
    }
  }

  // ---- a7: combine the two halves of each row and form the channels [ATMA §2.1]
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float S1 = s1[nb], S2 = s2[nb];
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
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) qq = fmaf((float)qf[nb][ks][e], (float)qf[nb][ks][e], qq);
      qq += xor32(qq);
      sigma = p.scale * sqrtf(qq);
    }
    if (STATS && p.part) {
      // partial mode: the statistics of this call's keys relative to their true maximum
      if (qrow[nb] < Tq) {
        const float m_true = c[nb] * row_tmax;
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
