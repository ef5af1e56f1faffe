// Backward pass on the matrix cores for bf16 inputs.
//
// The gradient is the one written out in bwd.h (chain rule through the forward
// definition [ATMA §2.1]); its products have the shape of five matrix products per
// (query tile, key tile), which run here as v_mfma_f32_32x32x16_bf16 with the operand
// layouts of the bf16 forward kernel:
//   rows   the forward kernel in partial mode gives every row's (m, S1, S2, acc); a small
//          kernel turns them and the upstream gradients into w (bf16) and the row
//          constants (m in base 2, c, cl c1, 2 cl c2) with cl = lam scale, the factor that
//          dq and dk carry, so both take cl dS = P (cl c1 + 2 cl c2 P + cl G);
//   dq     per query tile: S^T = K Q^T and G^T = V W^T (K, V rows from LDS, Q and W in
//          registers, lane = query); cl dS on the vector ALUs, rounded to bf16 in the
//          B-operand key order; dQ^T += K^T (cl dS)^T with K^T read from the row-major K
//          tile by transpose reads;
//   dk/dv  per key tile, over the query rows of every query head of its GQA group:
//          S = Q K^T and G = W V^T (Q, W rows from LDS, K in registers, lane = key);
//          P and cl dS with the per-row constants read from LDS; dK^T += Q^T (cl dS) and
//          dV^T += W^T P with Q^T and W^T from transpose reads.  The V operand of G sits
//          in registers at d = 64; at d = 128 the four accumulators and both K and V
//          fragments would not fit one wave's share of two waves per SIMD, so the
//          workgroup's 128 V rows are loaded once into LDS and G reads its V operand
//          from there, which keeps S computed once for both dk and dv.  Under a causal
//          mask the first key tiles see ~Tq/128 times the query rows of the last, so a
//          key tile's (head, query tile) pairs may be cut into runs of one workgroup
//          each, whose partial dk and dv a last kernel adds in run order.
// P, dS and w enter the products as bf16 (round to nearest even); every sum is fp32.
#pragma once

#include "bwd.h"
#include "fwd_bf16.h"

namespace polar {

struct BwdMfmaParams {
  const __bf16* q;       // [B, H, Tq, D]
  const __bf16* k;       // [B, Hkv, Tk, D]
  const __bf16* v;
  const float* part;     // [B, H, Tq, D + 3]: the forward's (m, S1, S2, acc) of every row
  const float* g_dir;    // upstream gradients (null = 0)
  const float* g_neff;
  const float* g_conf;
  const float* g_count;
  __bf16* W;             // [B, H, Tq, D]: w of every row, bf16
  f32x4* R;              // [B, H, Tq]: (m in base 2, c = lam scale log2 e, cl c1, 2 cl c2), cl = lam scale
  float* dq;             // [B, H, Tq, D]
  float* dk;             // [B, Hkv, Tk, D]
  float* dv;
  int B, H, Hkv, Tq, Tk;
  int n_qt;              // query tiles per (b, h) of the dq kernel
  int n_kt;              // key tiles per (b, kv head) of the dk/dv kernel
  int n_split;           // workgroups per key tile of the dk/dv kernel (1: no partial sums)
  float* dk_part;        // n_split > 1: [n_split, B, Hkv, Tk, D] partial dk, then dv alike
  float* dv_part;
  long long part_n4;     // B * Hkv * Tk * D / 4: f32x4 elements of dk (and of dv)
  int floor_on;
  int hp_stride;
  float scale;
  HeadParams hp;
};

// Sixteen lanes per query row (four rows per wave): w = (g_u - u (u . g_u)) / ||acc|| as
// bf16, and the row constants, which the row's first lane forms.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void polar_bwd_prep_kernel(const BwdMfmaParams p) {
  constexpr int DPL = D / 16;  // dims per lane: lane c of a row holds dims e * 16 + c
  const int c = threadIdx.x & 15;
  const size_t row = (size_t)blockIdx.x * 16 + (threadIdx.x >> 4);  // (b * H + h) * Tq + i
  const size_t rows = (size_t)p.B * p.H * p.Tq;
  const bool ok = row < rows;  // a row past the end still takes part in the lane sums
  const size_t rr = ok ? row : 0;
  const float* pr = p.part + rr * (D + 3);
  float acc[DPL], gu[DPL];
  float nn = 0.0f;
#pragma unroll
  for (int e = 0; e < DPL; ++e) {
    acc[e] = ok ? pr[3 + 16 * e + c] : 0.0f;
    gu[e] = ok && p.g_dir ? p.g_dir[rr * D + 16 * e + c] : 0.0f;
    nn = fmaf(acc[e], acc[e], nn);
  }
#pragma unroll
  for (int sh = 8; sh >= 1; sh >>= 1) nn += __shfl_xor(nn, sh, 16);
  const float a = sqrtf(nn);
  const float inv_a = a > 0.0f ? 1.0f / a : 0.0f;  // acc == 0: zero direction, w = 0
  float ug = 0.0f;
#pragma unroll
  for (int e = 0; e < DPL; ++e) ug = fmaf(acc[e] * inv_a, gu[e], ug);
#pragma unroll
  for (int sh = 8; sh >= 1; sh >>= 1) ug += __shfl_xor(ug, sh, 16);
  if (!ok) return;
#pragma unroll
  for (int e = 0; e < DPL; ++e) p.W[row * D + 16 * e + c] = (__bf16)((gu[e] - acc[e] * inv_a * ug) * inv_a);
  if (c == 0) {
    const int i = (int)(row % p.Tq);
    const int h = (int)((row / p.Tq) % p.H);
    const int hpi = h * p.hp_stride;
    const int n = visible_keys(i, p.Tq, p.Tk, CAUSAL);
    const float lam = row_temperature(p.hp, hpi, n);
    const float m_nat = pr[0];
    float c1, c2;
    row_constants(p.hp, hpi, p.floor_on != 0, n, lam, m_nat, pr[1], pr[2], p.g_neff ? p.g_neff[row] : 0.0f,
                  p.g_conf ? p.g_conf[row] : 0.0f, p.g_count ? p.g_count[row] : 0.0f, c1, c2);
    // the products take dS scaled by cl = lam scale, the factor dq and dk carry:
    // cl dS = p (cl c1 + 2 cl c2 p + cl <w, v>)
    const float cs = logit_scale(lam, p.scale);
    const float cl = cs * kLn2;
    p.R[row] = f32x4{m_nat * kLog2e, cs, cl * c1, 2.0f * cl * c2};
  }
}

// dq: a workgroup of NW waves owns 32 * NW query rows of one (b, h); keys stream through
// LDS in double-buffered tiles of BN rows exactly as in the forward kernel.
template <int D, int BN, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void polar_bwd_dq_mfma_kernel(
    const BwdMfmaParams p) {
  constexpr int BM = NW * 32;
  constexpr int MB = BN / 32;
  constexpr int KS = D / 16;
  constexpr int DM = D / 32;
  constexpr int PS = BN / 16;

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
  tile_coords(blockIdx.x, p.n_qt, p.B * p.H, qt, bh);
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int hk = h / (p.H / p.Hkv);
  const int Tq = p.Tq, Tk = p.Tk;
  const int off = Tk - Tq;
  const int q0 = qt * BM;
  const int wq0 = q0 + wave * 32;

  const size_t kv_head = (size_t)(b * p.Hkv + hk) * Tk * D;
  const uint32_t head_bytes = (uint32_t)((size_t)Tk * D * 2);
  const __amdgpu_buffer_rsrc_t kb =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + kv_head), (short)0, head_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vb =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + kv_head), (short)0, head_bytes, 0x00020000);
  const uint32_t voff = tile_lane_offset<D, NW>(wave, lane);

  const int kv_end = CAUSAL ? min(Tk, q0 + BM + off) : Tk;
  const int ntiles = (kv_end + BN - 1) / BN;
  const int wave_kmax = CAUSAL ? min(wq0 + 31 + off, Tk - 1) : Tk - 1;
  const int wave_kmin = CAUSAL ? min(wq0 + off, Tk - 1) : Tk - 1;

  load_tile<D, BN, NW>(kb, 0, voff, k_buf0, wave);
  load_tile<D, BN, NW>(vb, 0, voff, v_buf0, wave);

  const int qrow = wq0 + col;
  const bool live = qrow < Tq;
  const int kmax = CAUSAL ? min(qrow + off, Tk - 1) : Tk - 1;
  const size_t ri = (size_t)bh * Tq + qrow;
  // a row past the end gets weight 0 everywhere (m = +inf); its output is never written
  const f32x4 rv = live ? p.R[ri] : f32x4{INFINITY, 1.0e-30f, 0.0f, 0.0f};
  const float neg_m = -rv[0], c = rv[1], cc1 = rv[2], cc2 = rv[3], cl = c * kLn2;

  // Q^T and W^T fragments: lane holds row qrow, dims ks * 16 + 8 * half + [0, 8)
  bf16x8 qf[KS], wf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (live) {
      qf[ks] = *(const bf16x8*)(p.q + ri * D + ks * 16 + 8 * half);
      wf[ks] = *(const bf16x8*)(p.W + ri * D + ks * 16 + 8 * half);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[ks][e] = wf[ks][e] = (__bf16)0.0f;
    }
  }

  // LDS offsets: row reads of K and V (A operands of S^T and G^T) and transpose reads of
  // K (A operand of dQ^T), as in the forward kernel
  const int k_x = half ^ chunk_swizzle<D>(col);
  const uint32_t k_base = (uint32_t)(col * D * 2 + 16 * (k_x & 1));
  const uint32_t k_xor = (uint32_t)(32 * (k_x >> 1));
  const int gi = lane & 15;
  const int g = lane >> 4;
  int t_off[2][DM];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int row = 8 * r + 4 * half + (gi >> 2);
    const int sw = chunk_swizzle<D>(row);
#pragma unroll
    for (int dm = 0; dm < DM; ++dm) {
      const int lchunk = 4 * dm + 2 * (g & 1) + ((gi & 3) >> 1);
      t_off[r][dm] = row * D + ((lchunk ^ sw) << 3) + 4 * (gi & 1);
    }
  }

  f32x16 dq[DM];
#pragma unroll
  for (int dm = 0; dm < DM; ++dm)
#pragma unroll
    for (int e = 0; e < 16; ++e) dq[dm][e] = 0.0f;

  auto compute_tile = [&](const __bf16* kt, const __bf16* vt, int kv0) __attribute__((always_inline)) {
    f32x16 s[MB], gg[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[mb][e] = gg[mb][e] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const uint32_t o = (k_base + ((32u * ks) ^ k_xor)) + mb * 32 * D * 2;
        const bf16x8 ak = *(const bf16x8*)((const char*)kt + o);
        const bf16x8 av = *(const bf16x8*)((const char*)vt + o);
        s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qf[ks], s[mb], 0, 0, 0);
        gg[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, wf[ks], gg[mb], 0, 0, 0);
      }
    if (kv0 + BN - 1 > wave_kmin) {
      const int lim = kmax - kv0 - 4 * half;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (mb * 32 + 8 * i + j > lim) s[mb][4 * i + j] = -INFINITY;
    }
    // cl dS = P (cl c1 + 2 cl c2 P + cl G), bf16 in the B-operand key order
    bf16x8 dsf[PS];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float pv = fast_exp2(fmaf(c, s[mb][4 * i + j], neg_m));
          const float dsv = pv * fmaf(cc2, pv, fmaf(cl, gg[mb][4 * i + j], cc1));
          dsf[mb * 2 + (i >> 1)][(i & 1) * 4 + j] = (__bf16)dsv;
        }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int kst = 0; kst < PS; ++kst)
#pragma unroll
      for (int dm = 0; dm < DM; ++dm) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(kt + t_off[0][dm] + kst * 16 * D));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(kt + t_off[1][dm] + kst * 16 * D));
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        dq[dm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsf[kst], dq[dm], 0, 0, 0);
      }
  };

  publish_tiles();
  for (int t = 0; t < ntiles; t += 2) {
    if (t + 1 < ntiles) {
      load_tile<D, BN, NW>(kb, (t + 1) * BN, voff, k_buf1, wave);
      load_tile<D, BN, NW>(vb, (t + 1) * BN, voff, v_buf1, wave);
    }
    if (t * BN <= wave_kmax) compute_tile(k_buf0, v_buf0, t * BN);
    publish_tiles();
    if (t + 1 >= ntiles) break;
    if (t + 2 < ntiles) {
      load_tile<D, BN, NW>(kb, (t + 2) * BN, voff, k_buf0, wave);
      load_tile<D, BN, NW>(vb, (t + 2) * BN, voff, v_buf0, wave);
    }
    if ((t + 1) * BN <= wave_kmax) compute_tile(k_buf1, v_buf1, (t + 1) * BN);
    publish_tiles();
  }

  if (!live) return;
  float* out = p.dq + ri * D;
#pragma unroll
  for (int dm = 0; dm < DM; ++dm)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *(f32x4*)(out + dm * 32 + 8 * i + 4 * half) =
          f32x4{dq[dm][4 * i], dq[dm][4 * i + 1], dq[dm][4 * i + 2], dq[dm][4 * i + 3]};
}

// dk/dv: a workgroup of NW waves owns 32 * NW keys of one (b, kv head); the query rows of
// every head of the group stream through LDS in double-buffered tiles of BQ rows (q, w and
// the row constants).  VLDS: the V operand of G comes from the workgroup's V rows held in
// LDS for the whole kernel instead of from registers.
template <int D, int BQ, int NW, int OCC, bool CAUSAL, bool VLDS>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(OCC, OCC))) void polar_bwd_dkdv_mfma_kernel(
    const BwdMfmaParams p) {
  constexpr int BK = NW * 32;
  constexpr int MB = BQ / 32;
  constexpr int KS = D / 16;
  constexpr int DM = D / 32;
  constexpr int PS = BQ / 16;
  static_assert(BQ <= 64, "one wave-wide load brings the row constants of a tile");

  __shared__ __attribute__((aligned(1024))) __bf16 q_buf0[BQ * D];
  __shared__ __attribute__((aligned(1024))) __bf16 q_buf1[BQ * D];
  __shared__ __attribute__((aligned(1024))) __bf16 w_buf0[BQ * D];
  __shared__ __attribute__((aligned(1024))) __bf16 w_buf1[BQ * D];
  __shared__ __attribute__((aligned(1024))) f32x4 r_buf0[64];
  __shared__ __attribute__((aligned(1024))) f32x4 r_buf1[64];
  __shared__ __attribute__((aligned(1024))) __bf16 v_rows[VLDS ? BK * D : 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int half = lane >> 5;

  // blockIdx = (key tile * B * Hkv + (b * Hkv + kv head)) * n_split + split: the key tiles
  // that the most query rows see come first
  const int nbk = p.B * p.Hkv;
  const int sp = blockIdx.x % p.n_split;
  const int kb_i = blockIdx.x / p.n_split;
  const int kt_i = kb_i / nbk;
  const int bk = kb_i - kt_i * nbk;  // b * Hkv + kv head
  const int b = bk / p.Hkv;
  const int hk = bk - b * p.Hkv;
  const int G = p.H / p.Hkv;
  const int Tq = p.Tq, Tk = p.Tk;
  const int off = Tk - Tq;
  const int key0 = kt_i * BK;
  const int wk0 = key0 + wave * 32;
  const int key = wk0 + col;
  const bool live = key < Tk;
  const size_t kr = (size_t)bk * Tk + key;

  // K^T and V^T fragments (B operands): lane holds key `key`, dims ks * 16 + 8 * half + [0, 8)
  bf16x8 kf[KS], vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (live) {
      kf[ks] = *(const bf16x8*)(p.k + kr * D + ks * 16 + 8 * half);
      if constexpr (!VLDS) vf[ks] = *(const bf16x8*)(p.v + kr * D + ks * 16 + 8 * half);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) kf[ks][e] = vf[ks][e] = (__bf16)0.0f;
    }
  }

  const uint32_t voff = tile_lane_offset<D, NW>(wave, lane);
  const int q_x = half ^ chunk_swizzle<D>(col);
  const uint32_t q_base = (uint32_t)(col * D * 2 + 16 * (q_x & 1));
  const uint32_t q_xor = (uint32_t)(32 * (q_x >> 1));
  // the wave's 32 V rows in the swizzled LDS image: row wave * 32 + col has the swizzle of
  // row col (it repeats every 16 rows), so the row reads of the Q tile apply unchanged
  const uint32_t v_wave = (uint32_t)(wave * 32 * D * 2);
  if constexpr (VLDS) {
    // rows at or past Tk lie outside the buffer range and read as zero; the first
    // publish_tiles() of the loop below waits for these loads
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.v + (size_t)bk * Tk * D), (short)0, (uint32_t)((size_t)Tk * D * 2), 0x00020000);
    load_tile<D, BK, NW>(vrs, key0, voff, v_rows, wave);
  }
  const int gi = lane & 15;
  const int g = lane >> 4;
  // byte offsets of the transpose reads for d block 0; d block dm reads at t_byte ^ (64 dm):
  // its logical chunk 4 dm + c0 (c0 < 4) enters the swizzled chunk only through bits 2-3,
  // which sit at byte bits 6-7, and no other term of the offset (row * 2 D included) uses
  // those bits for dm < D / 32
  uint32_t t_byte[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int row = 8 * r + 4 * half + (gi >> 2);
    const int sw = chunk_swizzle<D>(row);
    const int lchunk = 2 * (g & 1) + ((gi & 3) >> 1);
    t_byte[r] = (uint32_t)(2 * (row * D + ((lchunk ^ sw) << 3) + 4 * (gi & 1)));
  }
  auto tr_read = [&](const __bf16* tile, int kst, int dm) __attribute__((always_inline)) {
    const char* base = (const char*)tile + kst * 16 * D * 2;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(base + (t_byte[0] ^ (64u * dm))));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(base + (t_byte[1] ^ (64u * dm))));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x16 dk[DM], dv[DM];
#pragma unroll
  for (int dm = 0; dm < DM; ++dm)
#pragma unroll
    for (int e = 0; e < 16; ++e) dk[dm][e] = dv[dm][e] = 0.0f;

  // first query row that sees the workgroup's first key, and the wave's key range
  const int i_begin = CAUSAL ? max(0, key0 - off) : 0;
  const int t_begin = min(i_begin / BQ, (Tq + BQ - 1) / BQ);
  const int nt_vis = (Tq + BQ - 1) / BQ - t_begin;  // query tiles per head that see the keys
  const int wave_kmax = min(wk0 + 31, Tk - 1);
  // the (head, query tile) pairs of the key tile, head-major, cut into n_split contiguous
  // runs of near-equal length; this workgroup takes run sp
  const long long items = (long long)G * nt_vis;
  const long long it_lo = items * sp / p.n_split;
  const long long it_hi = items * (sp + 1) / p.n_split;

  for (int gh = 0; gh < G; ++gh) {
    const int t_lo = t_begin + (int)max(it_lo - (long long)gh * nt_vis, 0ll);
    const int ntiles = t_begin + (int)min(it_hi - (long long)gh * nt_vis, (long long)nt_vis);
    const size_t bh = (size_t)b * p.H + hk * G + gh;
    const uint32_t head_bytes = (uint32_t)((size_t)Tq * D * 2);
    const __amdgpu_buffer_rsrc_t qb =
        __builtin_amdgcn_make_buffer_rsrc((void*)(p.q + bh * Tq * D), (short)0, head_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t wb =
        __builtin_amdgcn_make_buffer_rsrc((void*)(p.W + bh * Tq * D), (short)0, head_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb =
        __builtin_amdgcn_make_buffer_rsrc((void*)(p.R + bh * Tq), (short)0, (uint32_t)((size_t)Tq * 16), 0x00020000);
    // rows past the end read as zero: q = w = 0 and zero row constants give P = 1, dS = 0
    auto load = [&](int t, __bf16* qd, __bf16* wd, f32x4* rd) __attribute__((always_inline)) {
      load_tile<D, BQ, NW>(qb, t * BQ, voff, qd, wave);
      load_tile<D, BQ, NW>(wb, t * BQ, voff, wd, wave);
      if (wave == 0)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, POLAR_LDS(rd), 16, (uint32_t)((t * BQ + lane) * 16), 0, 0, 0);
    };

    auto compute_tile = [&](const __bf16* qt, const __bf16* wt, const f32x4* rt, int i0)
                            __attribute__((always_inline)) {
      f32x16 s[MB], gg[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[mb][e] = gg[mb][e] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const uint32_t o = (q_base + ((32u * ks) ^ q_xor)) + mb * 32 * D * 2;
          const bf16x8 aq = *(const bf16x8*)((const char*)qt + o);
          s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, kf[ks], s[mb], 0, 0, 0);
          const bf16x8 aw = *(const bf16x8*)((const char*)wt + o);
          bf16x8 bv;
          if constexpr (VLDS)
            bv = *(const bf16x8*)((const char*)v_rows + v_wave + (q_base + ((32u * ks) ^ q_xor)));
          else
            bv = vf[ks];
          gg[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw, bv, gg[mb], 0, 0, 0);
        }
      // causal: key j is visible to row i iff j <= i + off; only tiles whose first rows
      // precede the wave's last key need the mask, applied in place in a pass of its own so
      // that the other tiles carry no per-element compare
      if (CAUSAL && i0 + off < wave_kmax) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (key > i0 + mb * 32 + 8 * i + 4 * half + j + off) s[mb][4 * i + j] = -INFINITY;
      }
      bf16x8 pf[PS], dsf[PS];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = mb * 32 + 8 * i + 4 * half + j;  // query row in the tile
            const f32x4 rv = rt[r];
            const float x = s[mb][4 * i + j];
            const float pv = fast_exp2(fmaf(rv[1], x, -rv[0]));
            pf[mb * 2 + (i >> 1)][(i & 1) * 4 + j] = (__bf16)pv;
            const float dsv = pv * fmaf(rv[3], pv, fmaf(rv[1] * kLn2, gg[mb][4 * i + j], rv[2]));
            dsf[mb * 2 + (i >> 1)][(i & 1) * 4 + j] = (__bf16)dsv;
          }
      // dK^T += Q^T dS, dV^T += W^T P
#pragma unroll
      for (int kst = 0; kst < PS; ++kst)
#pragma unroll
        for (int dm = 0; dm < DM; ++dm) {
          dk[dm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_read(qt, kst, dm), dsf[kst], dk[dm], 0, 0, 0);
          dv[dm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_read(wt, kst, dm), pf[kst], dv[dm], 0, 0, 0);
        }
    };

    if (t_lo >= ntiles) continue;  // none of this head's tiles in the run (uniform)
    __syncthreads();  // the previous head's last tile is no longer read
    load(t_lo, q_buf0, w_buf0, r_buf0);
    publish_tiles();
    for (int t = t_lo; t < ntiles; t += 2) {
      if (t + 1 < ntiles) load(t + 1, q_buf1, w_buf1, r_buf1);
      if (!CAUSAL || t * BQ + BQ - 1 + off >= wk0) compute_tile(q_buf0, w_buf0, r_buf0, t * BQ);
      publish_tiles();
      if (t + 1 >= ntiles) break;
      if (t + 2 < ntiles) load(t + 2, q_buf0, w_buf0, r_buf0);
      if (!CAUSAL || (t + 1) * BQ + BQ - 1 + off >= wk0) compute_tile(q_buf1, w_buf1, r_buf1, (t + 1) * BQ);
      publish_tiles();
    }
  }

  if (!live) return;
  // a split key tile writes its run's partial sums (zero for an empty run)
  const size_t part_off = (size_t)sp * nbk * Tk * D;
  float* ok = (p.n_split > 1 ? p.dk_part + part_off : p.dk) + kr * D;
  float* ov = (p.n_split > 1 ? p.dv_part + part_off : p.dv) + kr * D;
#pragma unroll
  for (int dm = 0; dm < DM; ++dm)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *(f32x4*)(ok + dm * 32 + 8 * i + 4 * half) =
          f32x4{dk[dm][4 * i], dk[dm][4 * i + 1], dk[dm][4 * i + 2], dk[dm][4 * i + 3]};
      *(f32x4*)(ov + dm * 32 + 8 * i + 4 * half) =
          f32x4{dv[dm][4 * i], dv[dm][4 * i + 1], dv[dm][4 * i + 2], dv[dm][4 * i + 3]};
    }
}

// dk and dv of split key tiles: the sum of the n_split partial results, in split order.
__global__ __launch_bounds__(256) void polar_bwd_split_sum_kernel(const BwdMfmaParams p) {
  const long long n4 = p.part_n4;
  const long long stride = (long long)gridDim.x * 256;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < 2 * n4; i += stride) {
    const bool is_v = i >= n4;
    const long long e = is_v ? i - n4 : i;
    const f32x4* src = (const f32x4*)(is_v ? p.dv_part : p.dk_part) + e;
    f32x4 acc = src[0];
    for (int sp = 1; sp < p.n_split; ++sp) {
      const f32x4 x = src[(size_t)sp * n4];
      acc[0] += x[0];
      acc[1] += x[1];
      acc[2] += x[2];
      acc[3] += x[3];
    }
    ((f32x4*)(is_v ? p.dv : p.dk))[e] = acc;
  }
}

}  // namespace polar
