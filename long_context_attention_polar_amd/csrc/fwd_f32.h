// Polar Attention forward with fp32 inputs and fp32 arithmetic throughout.
//
// On MI355X the fp32 vector rate equals the fp32 matrix rate, so this path uses plain
// VALU FMAs.  A query row is spread over kF32Lanes = 8 neighbouring lanes, each holding
// D / 8 of its dimensions of q and of the accumulator (8 or 16 registers each, so nothing
// spills at either head dimension); a score is the sum of the 8 partial dot products,
// combined with three butterfly exchanges, after which every lane of the row holds the
// same score and forms the same weight.  K and V tiles of BK keys are staged in LDS and
// read by the workgroup as broadcasts.  The statistics follow the same streaming algebra
// as the bf16 kernel [ATMA §2.2, fused kernel]: a move of the reference maximum rescales
// sum p and acc by alpha and sum p^2 by alpha^2.  The reading variants (per-key floor,
// sliding window) are runtime choices here: this path is not the throughput path, and
// every branch on them is uniform over the row.
#pragma once

#include "polar_common.h"

namespace polar {

constexpr int kF32Lanes = 8;                             // lanes per query row
constexpr int kF32Threads = 256;                         // threads per workgroup
constexpr int kF32RowsPerBlock = kF32Threads / kF32Lanes;  // query rows per workgroup

// Sum over the kF32Lanes lanes of a row (aligned groups of 8 lanes); every lane of the
// group receives the same result, summed in the same order.
__device__ __forceinline__ float row_sum8(float x) {
  x += __shfl_xor(x, 1, 64);
  x += __shfl_xor(x, 2, 64);
  x += __shfl_xor(x, 4, 64);
  return x;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kF32Threads) void polar_fwd_f32_kernel(const FwdParams p) {
  constexpr int NT = kF32Threads;
  constexpr int BM = kF32RowsPerBlock;
  constexpr int BK = 16;
  constexpr int DL = D / kF32Lanes;  // dimensions per lane
  static_assert(DL % 4 == 0, "a lane's slice is whole float4s");
  __shared__ __attribute__((aligned(16))) float k_lds[BK * D];
  __shared__ __attribute__((aligned(16))) float v_lds[BK * D];

  const int tid = threadIdx.x;
  const int part = tid % kF32Lanes;  // which slice of the row this lane holds
  const int e0 = part * DL;
  int qt, bh;
  tile_coords(blockIdx.x, p.n_qt, p.B * p.H, qt, bh);
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int hk = h / (p.H / p.Hkv);
  const int Tq = p.Tq, Tk = p.Tk;
  const int off = Tk - Tq;
  const int q0 = qt * BM;
  const int qrow = q0 + tid / kF32Lanes;

  const float* qb = (const float*)p.q + (size_t)bh * Tq * D;
  const float* kb = (const float*)p.k + (size_t)(b * p.Hkv + hk) * Tk * D;
  const float* vb = (const float*)p.v + (size_t)(b * p.Hkv + hk) * Tk * D;

  const int hpi = h * p.hp_stride;
  const int win = CAUSAL ? p.hp.window : 0;
  int n_vis = context_count(qrow, Tq, Tk, CAUSAL, p.ctx_k);
  if (win > 0) n_vis = min(n_vis, win);
  const float lam = row_temperature(p.hp, hpi, n_vis);
  const float c = logit_scale(lam, p.scale);
  const int kmax = CAUSAL ? min(qrow + off, Tk - 1) : Tk - 1;
  const int klo = win > 0 ? qrow + off - win + 1 : 0;  // first key of the row's window
  const int kf = p.hp.key_floor;

  float q[DL];
#pragma unroll
  for (int e = 0; e < DL; e += 4) {
    const f32x4 x = qrow < Tq ? *(const f32x4*)(qb + (size_t)qrow * D + e0 + e) : f32x4{0, 0, 0, 0};
    q[e] = x[0];
    q[e + 1] = x[1];
    q[e + 2] = x[2];
    q[e + 3] = x[3];
  }
  float qq = 0.0f;
#pragma unroll
  for (int e = 0; e < DL; ++e) qq = fmaf(q[e], q[e], qq);
  qq = row_sum8(qq);
  const float sigma = p.hp.level_form == POLAR_LEVEL_QNORM ? p.scale * sqrtf(qq) : 1.0f;
  const float f = null_floor(p.hp, hpi, n_vis, lam, sigma);  // the row's floor (natural units)
  const float f2 = f * kLog2e;
  float acc[DL];
#pragma unroll
  for (int e = 0; e < DL; ++e) acc[e] = 0.0f;
  // with a per-key floor the reference starts at the floor, so e^{f - m_ref} <= 1
  float m_ref = kf != POLAR_KEY_FLOOR_NULL ? f2 : kMaxInit, m_true = kMaxInit, s1 = 0.0f, s2 = 0.0f;

  const int kv_end = CAUSAL ? min(Tk, q0 + BM + off) : Tk;
  const int kv_begin = win > 0 ? max(0, q0 + off - win + 1) / BK * BK : 0;
  for (int kv0 = kv_begin; kv0 < kv_end; kv0 += BK) {
    __syncthreads();
    for (int idx = tid * 4; idx < BK * D; idx += NT * 4) {
      const int key = kv0 + idx / D;
      const int e = idx % D;
      const f32x4 zero = {0, 0, 0, 0};
      *(f32x4*)(k_lds + idx) = key < Tk ? *(const f32x4*)(kb + (size_t)key * D + e) : zero;
      *(f32x4*)(v_lds + idx) = key < Tk ? *(const f32x4*)(vb + (size_t)key * D + e) : zero;
    }
    __syncthreads();
    float sc[BK];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < BK; ++j) {
      float r = 0.0f;
#pragma unroll
      for (int e = 0; e < DL; ++e) r = fmaf(q[e], k_lds[j * D + e0 + e], r);
      r = row_sum8(r);
      sc[j] = (kv0 + j <= kmax && kv0 + j >= klo) ? r : -INFINITY;
      tmax = fmaxf(tmax, sc[j]);
    }
    const float cm = c * tmax;
    m_true = fmaxf(m_true, cm);
    if (cm > m_ref + kRescaleSlack) {
      const float m_new = fmaxf(m_ref, cm);
      const float alpha = fast_exp2(m_ref - m_new);
      s1 *= alpha;
      s2 *= alpha * alpha;  // squared correction factor
#pragma unroll
      for (int e = 0; e < DL; ++e) acc[e] *= alpha;
      m_ref = m_new;
    }
    const float phi = fast_exp2(f2 - m_ref);  // the floor's weight, for the soft per-key floor
#pragma unroll
    for (int j = 0; j < BK; ++j) {
      const float x = c * sc[j];
      float pv = fast_exp2(x - m_ref);
      // soft floor: e^s - e^f = e^f (e^{s - f} - 1), with expm1 so that a score just above
      // the floor keeps its relative precision
      if (kf == POLAR_KEY_FLOOR_SOFT) pv = x > f2 ? phi * expm1f((x - f2) * kLn2) : 0.0f;
      if (kf == POLAR_KEY_FLOOR_GATE) pv = x > f2 ? pv : 0.0f;
      s1 += pv;
      s2 = fmaf(pv, pv, s2);
#pragma unroll
      for (int e = 0; e < DL; ++e) acc[e] = fmaf(pv, v_lds[j * D + e0 + e], acc[e]);
    }
  }

  // with a per-key floor the reference may sit above the true maximum; the sums are then
  // 0 and must not meet an overflowing factor
  const float to_true = s1 > 0.0f ? fast_exp2(m_ref - m_true) : 0.0f;
  if (qrow < Tq && p.part) {
    // partial mode: the statistics of this call's keys relative to their true maximum
    float* out = p.part + (((size_t)bh * Tq + qrow) * p.part_S + p.part_s) * (D + 3);
    if (part == 0) {
      out[0] = m_true * kLn2;
      out[1] = s1 * to_true;
      out[2] = s2 * to_true * to_true;
    }
#pragma unroll
    for (int e = 0; e < DL; ++e) out[3 + e0 + e] = acc[e] * to_true;
  } else if (qrow < Tq) {
    const float S1 = s1 * to_true;
    const float S2 = s2 * to_true * to_true;
    float nn = 0.0f;
#pragma unroll
    for (int e = 0; e < DL; ++e) nn = fmaf(acc[e], acc[e], nn);
    nn = row_sum8(nn);
    const float inv = nn == 0.0f ? 0.0f : 1.0f / sqrtf(nn);  // a NaN norm stays NaN
    const size_t row = (size_t)bh * Tq + qrow;
    float* drow = p.dir + row * D + e0;
#pragma unroll
    for (int e = 0; e < DL; e += 4) {
      const f32x4 val = {acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv};
      *(f32x4*)(drow + e) = val;
    }
    if (part == 0) {
      const float m_nat = m_true * kLn2;
      float neff, conf, count;
      magnitude_channel(p.hp, hpi, m_nat, S1, S2, f, p.floor_on != 0, neff, conf, count);
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
