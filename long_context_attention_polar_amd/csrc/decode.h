// Split-KV Polar Attention decode and the merge of split statistics.
//
// [ATMA §2.2, decode kernel]: a decode step reads the KV cache once; its cost is HBM
// traffic.  The cache of one (b, kv head) is cut into S contiguous splits; a workgroup
// streams one split with 16-byte loads, keeps the running (m, S1, S2, acc) of its keys
// and writes them as one partial row.  The merge brings the splits to a common maximum
// (w for S1 and acc, w^2 for S2 [ATMA §2.2, squared correction factors]) and forms the
// channels with the global visible count.
//
// Inside a split workgroup (NW waves), LPK = D / 8 lanes share one key (8 dims each) and
// each group of LPK lanes is a "slot" with its own running state; slots are combined
// through LDS at the end of the split.
//
// Reading variants: a sliding window moves split 0 to the window's first key; a per-key
// floor reduces each weight against the floor of the query's whole visible count (the
// floored weights are linear in e^s - e^f, so the merge is unchanged).  The floor is the
// template flag KF, so the default kernel carries no floor code.
#pragma once

#include "polar_common.h"

namespace polar {

// Sum over aligned groups of 8 or 16 lanes with DPP moves (all lanes get the sum).
template <int LPK>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LPK == 8 || LPK == 16, "group width");
  // quad_perm [1,0,3,2] and [2,3,0,1]: xor 1 and xor 2 inside each quad
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
  // row_half_mirror: lane i <-> 7 - i inside each group of 8 (quad 0 <-> quad 1)
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
  if constexpr (LPK == 16) {
    // row_mirror: lane i <-> 15 - i inside each row of 16 (half 0 <-> half 1)
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
  }
  return x;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

template <int D, int NW, int UNROLL, int KF = POLAR_KEY_FLOOR_NULL>
__global__ __launch_bounds__(NW * 64) void polar_decode_split_kernel(const DecodeParams p) {
  constexpr int LPK = D / 8;          // lanes per key
  constexpr int KPW = 64 / LPK;       // keys per wave per step
  constexpr int NSLOT = NW * KPW;     // independent running states per workgroup
  constexpr int W = D + 3;            // partial row width

  __shared__ float slot_m[NSLOT], slot_s1[NSLOT], slot_s2[NSLOT];
  __shared__ __attribute__((aligned(16))) float slot_acc[NSLOT][D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int sub = lane / LPK;          // key slot inside the wave
  const int dch = lane % LPK;          // 8-dim chunk of this lane
  const int slot = wave * KPW + sub;

  const int s = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int hk = h / (p.H / p.Hkv);
  const int Tk = p.Tk;
  const int lo = p.key0 + s * p.split_len;
  const int hi = min(lo + p.split_len, Tk);

  const __bf16* qp = (const __bf16*)p.q + ((size_t)b * p.H + h) * D;
  const __bf16* kb = (const __bf16*)p.k + ((size_t)b * p.Hkv + hk) * Tk * D;
  const __bf16* vb = (const __bf16*)p.v + ((size_t)b * p.Hkv + hk) * Tk * D;

  const int hpi = h * p.hp_stride;
  // One query per sequence: it sees every cached key (or the last `window` of them),
  // n = Tk - key0, never a per-split count.
  const int n = Tk - p.key0;
  const float lam = row_temperature(p.hp, hpi, n);
  const float c = logit_scale(lam, p.scale);

  float qv[8];
  {
    const u32x4 w = *(const u32x4*)(qp + dch * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qv[2 * e] = bf16_lo(w[e]);
      qv[2 * e + 1] = bf16_hi(w[e]);
    }
  }
  // per-key floor: the query's floor in base-2 units
  float f2 = 0.0f;
  if constexpr (KF != POLAR_KEY_FLOOR_NULL) {
    float qq = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) qq = fmaf(qv[e], qv[e], qq);
    qq = group_sum<LPK>(qq);
    const float sigma = p.hp.level_form == POLAR_LEVEL_QNORM ? p.scale * sqrtf(qq) : 1.0f;
    f2 = null_floor(p.hp, hpi, n, lam, sigma) * kLog2e;
  }

  float m = kMaxInit, s1 = 0.0f, s2 = 0.0f;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;

  for (int base = lo; base < hi; base += NSLOT * UNROLL) {
    u32x4 kr[UNROLL], vr[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int key = base + slot + u * NSLOT;
      if (key < hi) {  // each cache byte is read once: non-temporal loads
        kr[u] = __builtin_nontemporal_load((const u32x4*)(kb + (size_t)key * D + dch * 8));
        vr[u] = __builtin_nontemporal_load((const u32x4*)(vb + (size_t)key * D + dch * 8));
      } else {
        kr[u] = u32x4{0, 0, 0, 0};
        vr[u] = u32x4{0, 0, 0, 0};
      }
    }
    float x[UNROLL];
    float xmax = -INFINITY;
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      float r = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        r = fmaf(qv[2 * e], bf16_lo(kr[u][e]), r);
        r = fmaf(qv[2 * e + 1], bf16_hi(kr[u][e]), r);
      }
      r = group_sum<LPK>(r);
      const int key = base + slot + u * NSLOT;
      x[u] = key < hi ? c * r : -INFINITY;
      xmax = fmaxf(xmax, x[u]);
    }
    const float m_new = fmaxf(m, xmax);
    const float alpha = fast_exp2(m - m_new);
    s1 *= alpha;
    s2 *= alpha * alpha;  // squared correction factor
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= alpha;
    m = m_new;
    // the floor's weight (inf while m is far below the floor: every weight is then 0)
    const float phi = KF == POLAR_KEY_FLOOR_SOFT ? fast_exp2(f2 - m) : 0.0f;
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      float pv = fast_exp2(x[u] - m);
      if constexpr (KF == POLAR_KEY_FLOOR_SOFT) pv = fmaxf(pv - phi, 0.0f);
      if constexpr (KF == POLAR_KEY_FLOOR_GATE) pv = x[u] > f2 ? pv : 0.0f;
      s1 += pv;
      s2 = fmaf(pv, pv, s2);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] = fmaf(pv, bf16_lo(vr[u][e]), acc[2 * e]);
        acc[2 * e + 1] = fmaf(pv, bf16_hi(vr[u][e]), acc[2 * e + 1]);
      }
    }
  }

  // ---- combine the slots of the workgroup
  if (dch == 0) {
    slot_m[slot] = m;
    slot_s1[slot] = s1;
    slot_s2[slot] = s2;
  }
#pragma unroll
  for (int e = 0; e < 8; e += 4) {
    const f32x4 val = {acc[e], acc[e + 1], acc[e + 2], acc[e + 3]};
    *(f32x4*)(&slot_acc[slot][dch * 8 + e]) = val;
  }
  __syncthreads();
  float M = kMaxInit;
#pragma unroll 4
  for (int i = 0; i < NSLOT; ++i) M = fmaxf(M, slot_m[i]);
  float* out = p.part + (((size_t)b * p.H + h) * p.S + s) * W;
  for (int d = tid; d < D; d += NW * 64) {
    float a = 0.0f;
    for (int i = 0; i < NSLOT; ++i) a = fmaf(fast_exp2(slot_m[i] - M), slot_acc[i][d], a);
    out[3 + d] = a;
  }
  if (tid == 0) {
    float t1 = 0.0f, t2 = 0.0f;
    for (int i = 0; i < NSLOT; ++i) {
      const float w = fast_exp2(slot_m[i] - M);
      t1 = fmaf(w, slot_s1[i], t1);
      t2 = fmaf(w * w, slot_s2[i], t2);
    }
    // an empty split (no keys) keeps M at the start value: report it as -inf
    out[0] = (hi > lo) ? M * kLn2 : -INFINITY;
    out[1] = t1;
    out[2] = t2;
  }
}

// Merge of few partial rows (at most 16 splits): one wave per output row, every lane walking
// the splits in order with wave-uniform loads, then the channels.
template <int D>
__global__ __launch_bounds__(64) void polar_merge_few_kernel(const MergeParams p) {
  constexpr int W = D + 3;
  constexpr int DPL = D / 64;  // dims per lane
  const int lane = threadIdx.x;
  const size_t row = blockIdx.x;  // (b * H + h) * Tq + i
  const int i = (int)(row % p.Tq);
  const int h = (int)((row / p.Tq) % p.H);
  const float* part = p.part + row * p.S * W;

  float M = -INFINITY;
  for (int s = 0; s < p.S; ++s) M = fmaxf(M, part[s * W]);
  float S1 = 0.0f, S2 = 0.0f;
  float acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.0f;
  for (int s = 0; s < p.S; ++s) {
    const float ms = part[s * W];
    if (ms == -INFINITY) continue;  // a split without keys contributes nothing
    const float w = expf(ms - M);
    S1 = fmaf(w, part[s * W + 1], S1);
    S2 = fmaf(w * w, part[s * W + 2], S2);  // squared correction factor
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] = fmaf(w, part[s * W + 3 + lane + 64 * e], acc[e]);
  }
  float nn = 0.0f;
#pragma unroll
  for (int e = 0; e < DPL; ++e) nn = fmaf(acc[e], acc[e], nn);
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) nn += __shfl_xor(nn, sh, 64);
  const float inv = nn == 0.0f ? 0.0f : 1.0f / sqrtf(nn);  // a NaN norm stays NaN
#pragma unroll
  for (int e = 0; e < DPL; ++e) p.dir[row * D + lane + 64 * e] = acc[e] * inv;
  // the data-adaptive floor level needs the norm of the row's q (all lanes take part)
  float sigma = 1.0f;
  if (p.hp.level_form == POLAR_LEVEL_QNORM && p.q) {
    float qq = 0.0f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      const float x = (float)p.q[row * D + lane + 64 * e];
      qq = fmaf(x, x, qq);
    }
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) qq += __shfl_xor(qq, sh, 64);
    sigma = p.scale * sqrtf(qq);
  }
  if (lane == 0) {
    const int hpi = h * p.hp_stride;
    int n = visible_keys(i, p.Tq, p.Tk, p.causal != 0);
    if (p.lens) n = min(max(p.lens[row / ((size_t)p.H * p.Tq)], 0), p.Tk);
    if (p.hp.window > 0) n = min(n, p.hp.window);
    float neff = 0.0f, conf = 0.0f, count = 0.0f;
    if (n > 0 && M > -INFINITY) {
      const float lam = row_temperature(p.hp, hpi, n);
      const float f = null_floor(p.hp, hpi, n, lam, sigma);
      magnitude_channel(p.hp, hpi, M, S1, S2, f, p.floor_on != 0, neff, conf, count);
    }  // a row that saw no key: direction 0 and all channels 0
    p.neff[row] = neff;
    if (p.conf) p.conf[row] = conf;
    if (p.count) p.count[row] = count;
    if (p.stats) {
      p.stats[row * 3 + 0] = M;
      p.stats[row * 3 + 1] = S1;
      p.stats[row * 3 + 2] = S2;
    }
  }
}

// Merge of S partial rows into one output row, and its channels.  NW waves per row: the
// common maximum and the weighted S1, S2 are taken over the splits in parallel (split s by
// thread s, s + 64 NW, ...),
// the value sums by wave w over the splits w, w + NW, ... (each lane holding D / 64 dims),
// and the NW partial vectors are added in wave order through LDS, so every result is the
// same on every run.  Used past 16 splits (polar_merge_few_kernel below that): one wave,
// four past 64.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void polar_merge_kernel(const MergeParams p) {
  constexpr int W = D + 3;
  constexpr int DPL = D / 64;  // dims per lane
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const size_t row = blockIdx.x;  // (b * H + h) * Tq + i
  const int i = (int)(row % p.Tq);
  const int h = (int)((row / p.Tq) % p.H);
  const float* part = p.part + row * p.S * W;
  __shared__ float red[2][NW];
  __shared__ float acc_w[NW > 1 ? NW : 1][D];

  // the common maximum; a thread's first split keeps its (m, S1, S2) in registers for the
  // sums below, so they take no second round of loads
  float m0 = -INFINITY, a0 = 0.0f, b0 = 0.0f;
  if (tid < p.S) {
    m0 = part[(size_t)tid * W];
    a0 = part[(size_t)tid * W + 1];
    b0 = part[(size_t)tid * W + 2];
  }
  float M = m0;
  for (int s = tid + NW * 64; s < p.S; s += NW * 64) M = fmaxf(M, part[(size_t)s * W]);
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) M = fmaxf(M, __shfl_xor(M, sh, 64));
  if constexpr (NW > 1) {
    if (lane == 0) red[0][wave] = M;
    __syncthreads();
    M = red[0][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, red[0][w]);
    __syncthreads();
  }
  // S1 and S2 brought to it (w for S1, w^2 for S2)
  float S1 = 0.0f, S2 = 0.0f;
  auto add_split = [&](float ms, float s1, float s2) __attribute__((always_inline)) {
    if (ms == -INFINITY) return;  // a split without keys contributes nothing
    const float w = expf(ms - M);
    S1 = fmaf(w, s1, S1);
    S2 = fmaf(w * w, s2, S2);  // squared correction factor
  };
  if (tid < p.S) add_split(m0, a0, b0);
  for (int s = tid + NW * 64; s < p.S; s += NW * 64) {
    const float* ps = part + (size_t)s * W;
    add_split(ps[0], ps[1], ps[2]);
  }
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) {
    S1 += __shfl_xor(S1, sh, 64);
    S2 += __shfl_xor(S2, sh, 64);
  }
  if constexpr (NW > 1) {
    if (lane == 0) {
      red[0][wave] = S1;
      red[1][wave] = S2;
    }
    __syncthreads();
    S1 = red[0][0];
    S2 = red[1][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      S1 += red[0][w];
      S2 += red[1][w];
    }
  }
  // the value sums
  float acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.0f;
  // A wave's splits are s = wave, wave + NW, ...  It loads the values of CH of them before
  // it adds any, so those loads are in flight together, and adds them in split order.
  constexpr int CH = 16;
  for (int s0 = wave; s0 < p.S; s0 += NW * CH) {
    float msv[CH], val[CH][DPL];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int s = s0 + c * NW;
      msv[c] = -INFINITY;
#pragma unroll
      for (int e = 0; e < DPL; ++e) val[c][e] = 0.0f;
      if (s < p.S) {  // the same for the whole wave
        const float* ps = part + (size_t)s * W;
        msv[c] = ps[0];
#pragma unroll
        for (int e = 0; e < DPL; ++e) val[c][e] = ps[3 + lane + 64 * e];
      }
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (msv[c] == -INFINITY) continue;  // no keys, or past the last split
      const float w = expf(msv[c] - M);
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] = fmaf(w, val[c][e], acc[e]);
    }
  }
  if constexpr (NW > 1) {
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc_w[wave][lane + 64 * e] = acc[e];
    __syncthreads();
    if (wave != 0) return;  // wave 0 finishes the row
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      float a = acc_w[0][lane + 64 * e];
#pragma unroll
      for (int w = 1; w < NW; ++w) a += acc_w[w][lane + 64 * e];
      acc[e] = a;
    }
  }
  float nn = 0.0f;
#pragma unroll
  for (int e = 0; e < DPL; ++e) nn = fmaf(acc[e], acc[e], nn);
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) nn += __shfl_xor(nn, sh, 64);
  const float inv = nn == 0.0f ? 0.0f : 1.0f / sqrtf(nn);  // a NaN norm stays NaN
#pragma unroll
  for (int e = 0; e < DPL; ++e) p.dir[row * D + lane + 64 * e] = acc[e] * inv;
  // the data-adaptive floor level needs the norm of the row's q (all lanes take part)
  float sigma = 1.0f;
  if (p.hp.level_form == POLAR_LEVEL_QNORM && p.q) {
    float qq = 0.0f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      const float x = (float)p.q[row * D + lane + 64 * e];
      qq = fmaf(x, x, qq);
    }
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) qq += __shfl_xor(qq, sh, 64);
    sigma = p.scale * sqrtf(qq);
  }
  if (lane == 0) {
    const int hpi = h * p.hp_stride;
    int n = visible_keys(i, p.Tq, p.Tk, p.causal != 0);
    if (p.lens) n = min(max(p.lens[row / ((size_t)p.H * p.Tq)], 0), p.Tk);
    if (p.hp.window > 0) n = min(n, p.hp.window);
    float neff = 0.0f, conf = 0.0f, count = 0.0f;
    if (n > 0 && M > -INFINITY) {
      const float lam = row_temperature(p.hp, hpi, n);
      const float f = null_floor(p.hp, hpi, n, lam, sigma);
      magnitude_channel(p.hp, hpi, M, S1, S2, f, p.floor_on != 0, neff, conf, count);
    }  // a row that saw no key: direction 0 and all channels 0
    p.neff[row] = neff;
    if (p.conf) p.conf[row] = conf;
    if (p.count) p.count[row] = count;
    if (p.stats) {
      p.stats[row * 3 + 0] = M;
      p.stats[row * 3 + 1] = S1;
      p.stats[row * 3 + 2] = S2;
    }
  }
}

}  // namespace polar
