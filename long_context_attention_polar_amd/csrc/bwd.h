// Backward pass of the Polar Attention forward: dq, dk, dv for upstream gradients of
// the direction, n_eff, the confidence and the count.
//
// The ATMA summary trains models with the operator [ATMA §3] but gives no backward pass;
// the gradient is the derivative of the forward definition [ATMA §2.1] by the chain rule
// through u = A / ||A||, n_eff = Z1^2 / Z2, conf = Z1 / (Z1 + e^f) and
// count = conf tanh(ln n_eff / kappa), with absolute weights P_j = e^{s_j}, Z1 = sum P,
// Z2 = sum P^2, A = sum P v.  Per query row, with weights p_j relative to the row maximum
// (S1 = sum p, S2 = sum p^2, acc = sum p v):
//   T = tanh(ln n_eff / kappa),  G_conf = g_c + g_k T,  G_neff = g_n + g_k conf (1 - T^2) / (kappa n_eff)
//   c1 = (2 G_neff n_eff + G_conf conf (1 - conf)) / S1,  c2 = -G_neff n_eff / S2
//   w  = (g_u - u (u . g_u)) / ||acc||
//   ds_j = p_j (c1 + 2 c2 p_j + <w, v_j>)
//   dq = lam scale sum_j ds_j k_j,   dk_j = sum_i lam_i scale ds_ij q_i,   dv_j = sum_i p_ij w_i
// (conf (1 - conf) is replaced by 0 when the floor is off, where conf = 1.)
//
// Three kernels, fp32 arithmetic on the vector ALUs (q, k, v in bf16 or fp32).  A row of
// D elements is spread over LPR = D / 32 neighbouring lanes of 32 elements each; the
// partial dot products of a row are summed across those lanes with DPP moves.
//   rows  - per query row, one pass over its visible keys for the exact maximum m, S1, S2
//           and acc, then c1, c2 and w into the workspace;
//   dq    - per query row, a second pass over the keys;
//   dk/dv - per key, one pass over the query rows of every query head of its group that
//           see it.
// K/V (or Q/w) tiles of 32 rows are staged in LDS as fp32 and read by every row of the
// workgroup.
#pragma once

#include "polar_common.h"

namespace polar {

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const float* g_dir;    // [B, H, Tq, D] or null
  const float* g_neff;   // [B, H, Tq] or null
  const float* g_conf;
  const float* g_count;
  float* W;              // workspace [B, H, Tq, D]: w of every row
  float* R;              // workspace [B, H, Tq, 4]: m (base 2), c1, c2, c = lam scale log2 e
  float* dq;             // [B, H, Tq, D]
  float* dk;             // [B, Hkv, Tk, D]
  float* dv;
  int B, H, Hkv, Tq, Tk;
  int floor_on;
  int hp_stride;
  float scale;
  HeadParams hp;
};

constexpr int kBwdThreads = 256;
constexpr int kBwdTile = 32;  // rows per LDS tile

// c1 and c2 of a row from its statistics (S1, S2 relative to e^{m_nat}) and upstream
// gradients g_n, g_c, g_k of n_eff, the confidence and the count.
__device__ __forceinline__ void row_constants(const HeadParams& hp, int hpi, bool floor_on, int n, float lam,
                                              float m_nat, float s1, float s2, float g_n, float g_c, float g_k,
                                              float& c1, float& c2) {
  const float kinv = hp.kinv[hpi];
  const float n_eff = s1 * s1 / s2;
  float conf = 1.0f, dconf = 0.0f;
  if (floor_on) {
    const float f = null_floor(hp, hpi, n, lam, 1.0f);
    conf = 1.0f / (1.0f + expf(f - m_nat - logf(s1)));
    dconf = conf * (1.0f - conf);
  }
  // count = conf tanh(x / kappa), x = ln n_eff, or ln(1 + n_eff) under the log1p saturation
  const bool l1p = hp.sat_form == POLAR_SAT_LOG1P;
  const float t = tanhf((l1p ? log1pf(n_eff) : logf(n_eff)) * kinv);
  const float g_conf = g_c + g_k * t;
  const float g_neff = g_n + g_k * conf * (1.0f - t * t) * kinv / (l1p ? 1.0f + n_eff : n_eff);
  c1 = (2.0f * g_neff * n_eff + g_conf * dconf) / s1;
  c2 = -g_neff * n_eff / s2;
}

// Sum over the LPR (1, 2 or 4) neighbouring lanes of one row.
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
  if constexpr (LPR >= 2)  // quad permutation [1, 0, 3, 2]
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  if constexpr (LPR >= 4)  // quad permutation [2, 3, 0, 1]
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
  return x;
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// 32 consecutive elements (16-byte aligned) as floats.
__device__ __forceinline__ void load32(const float* src, float* dst) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const f32x4 t = *(const f32x4*)(src + 4 * i);
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[4 * i + e] = t[e];
  }
}
__device__ __forceinline__ void load32(const __bf16* src, float* dst) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 t = *(const u32x4*)(src + 8 * i);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t x = t[e];
      dst[8 * i + 2 * e] = bf_lo(x);
      dst[8 * i + 2 * e + 1] = bf_hi(x);
    }
  }
}

// 4 consecutive elements as floats.
__device__ __forceinline__ f32x4 load4(const float* src) { return *(const f32x4*)src; }
__device__ __forceinline__ f32x4 load4(const __bf16* src) {
  const u32x2 t = *(const u32x2*)src;
  const uint32_t a = t[0], b = t[1];
  return f32x4{bf_lo(a), bf_hi(a), bf_lo(b), bf_hi(b)};
}

// Rows [r0, r0 + kBwdTile) of a row-major [rows, D] matrix into LDS as floats; rows at
// or past `rows` are stored as zero.
template <int D, typename T>
__device__ __forceinline__ void stage_tile(const T* src, int r0, int rows, float* dst) {
#pragma unroll
  for (int idx = threadIdx.x * 4; idx < kBwdTile * D; idx += kBwdThreads * 4) {
    const int r = r0 + idx / D;
    f32x4 val = {0.0f, 0.0f, 0.0f, 0.0f};
    if (r < rows) val = load4(src + (size_t)r * D + idx % D);
    *(f32x4*)(dst + idx) = val;
  }
}

template <int D, typename T, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads) void polar_bwd_rows_kernel(const BwdParams p) {
  constexpr int LPR = D / 32;
  constexpr int RPB = kBwdThreads / LPR;  // query rows per workgroup
  __shared__ __attribute__((aligned(16))) float k_t[kBwdTile * D];
  __shared__ __attribute__((aligned(16))) float v_t[kBwdTile * D];
  const int part = threadIdx.x % LPR;
  const int bh = blockIdx.y;
  const int b = bh / p.H, h = bh - b * p.H, hk = h / (p.H / p.Hkv);
  const int Tq = p.Tq, Tk = p.Tk, off = Tk - Tq;
  const int q0 = blockIdx.x * RPB;
  const int row = q0 + (int)threadIdx.x / LPR;
  const bool live = row < Tq;
  const int rc = min(row, Tq - 1);  // rows past the end compute on the last row, unused
  const size_t ri = (size_t)bh * Tq + rc;
  const int hpi = h * p.hp_stride;
  const int n = visible_keys(rc, Tq, Tk, CAUSAL);
  const float lam = row_temperature(p.hp, hpi, n);
  const float c = lam * p.scale * kLog2e;
  const int kmax = CAUSAL ? rc + off : Tk - 1;  // last visible key
  const T* kb = (const T*)p.k + (size_t)(b * p.Hkv + hk) * Tk * D;
  const T* vb = (const T*)p.v + (size_t)(b * p.Hkv + hk) * Tk * D;

  float qv[32], acc[32];
  load32((const T*)p.q + ri * D + part * 32, qv);
#pragma unroll
  for (int e = 0; e < 32; ++e) acc[e] = 0.0f;
  float m = kMaxInit, s1 = 0.0f, s2 = 0.0f;

  const int kv_end = CAUSAL ? min(Tk, q0 + RPB + off) : Tk;
  for (int kv0 = 0; kv0 < kv_end; kv0 += kBwdTile) {
    __syncthreads();
    stage_tile<D>(kb, kv0, Tk, k_t);
    stage_tile<D>(vb, kv0, Tk, v_t);
    __syncthreads();
    // scores of the tile first, then one maximum update for the whole tile
    float x[kBwdTile];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < kBwdTile; ++j) {
      float r = 0.0f;
#pragma unroll
      for (int e = 0; e < 32; ++e) r = fmaf(qv[e], k_t[j * D + part * 32 + e], r);
      r = row_sum<LPR>(r);
      x[j] = (kv0 + j <= kmax) ? c * r : -INFINITY;
      tmax = fmaxf(tmax, x[j]);
    }
    const float m_new = fmaxf(m, tmax);
    const float alpha = fast_exp2(m - m_new);
    s1 *= alpha;
    s2 *= alpha * alpha;  // squared correction factor
#pragma unroll
    for (int e = 0; e < 32; ++e) acc[e] *= alpha;
    m = m_new;
#pragma unroll
    for (int j = 0; j < kBwdTile; ++j) {
      const float pv = fast_exp2(x[j] - m);
      s1 += pv;
      s2 = fmaf(pv, pv, s2);
#pragma unroll
      for (int e = 0; e < 32; ++e) acc[e] = fmaf(pv, v_t[j * D + part * 32 + e], acc[e]);
    }
  }

  // ---- c1, c2 and w of the row
  float nn = 0.0f;
#pragma unroll
  for (int e = 0; e < 32; ++e) nn = fmaf(acc[e], acc[e], nn);
  const float a = sqrtf(row_sum<LPR>(nn));
  const float inv_a = a > 0.0f ? 1.0f / a : 0.0f;  // acc == 0: zero direction, w = 0
  float gu[32];
  if (p.g_dir) {
    load32(p.g_dir + ri * D + part * 32, gu);
  } else {
#pragma unroll
    for (int e = 0; e < 32; ++e) gu[e] = 0.0f;
  }
  float ug = 0.0f;
#pragma unroll
  for (int e = 0; e < 32; ++e) ug = fmaf(acc[e] * inv_a, gu[e], ug);
  ug = row_sum<LPR>(ug);
  if (!live) return;
  float* wr = p.W + ri * D + part * 32;
#pragma unroll
  for (int e = 0; e < 32; e += 4) {
    f32x4 val;
#pragma unroll
    for (int t = 0; t < 4; ++t) val[t] = (gu[e + t] - acc[e + t] * inv_a * ug) * inv_a;
    *(f32x4*)(wr + e) = val;
  }
  if (part == 0) {
    const float g_n = p.g_neff ? p.g_neff[ri] : 0.0f;
    const float g_c = p.g_conf ? p.g_conf[ri] : 0.0f;
    const float g_k = p.g_count ? p.g_count[ri] : 0.0f;
    float c1, c2;
    row_constants(p.hp, hpi, p.floor_on != 0, n, lam, m * kLn2, s1, s2, g_n, g_c, g_k, c1, c2);
    *(f32x4*)(p.R + ri * 4) = f32x4{m, c1, c2, c};
  }
}

template <int D, typename T, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads) void polar_bwd_dq_kernel(const BwdParams p) {
  constexpr int LPR = D / 32;
  constexpr int RPB = kBwdThreads / LPR;
  __shared__ __attribute__((aligned(16))) float k_t[kBwdTile * D];
  __shared__ __attribute__((aligned(16))) float v_t[kBwdTile * D];
  const int part = threadIdx.x % LPR;
  const int bh = blockIdx.y;
  const int b = bh / p.H, h = bh - b * p.H, hk = h / (p.H / p.Hkv);
  const int Tq = p.Tq, Tk = p.Tk, off = Tk - Tq;
  const int q0 = blockIdx.x * RPB;
  const int row = q0 + (int)threadIdx.x / LPR;
  const bool live = row < Tq;
  const int rc = min(row, Tq - 1);
  const size_t ri = (size_t)bh * Tq + rc;
  const int kmax = CAUSAL ? rc + off : Tk - 1;
  const T* kb = (const T*)p.k + (size_t)(b * p.Hkv + hk) * Tk * D;
  const T* vb = (const T*)p.v + (size_t)(b * p.Hkv + hk) * Tk * D;

  float qv[32], wv[32], dq[32];
  load32((const T*)p.q + ri * D + part * 32, qv);
  load32(p.W + ri * D + part * 32, wv);
#pragma unroll
  for (int e = 0; e < 32; ++e) dq[e] = 0.0f;
  const f32x4 rv = *(const f32x4*)(p.R + ri * 4);
  const float m = rv[0], c1 = rv[1], c2 = rv[2], c = rv[3];

  const int kv_end = CAUSAL ? min(Tk, q0 + RPB + off) : Tk;
  for (int kv0 = 0; kv0 < kv_end; kv0 += kBwdTile) {
    __syncthreads();
    stage_tile<D>(kb, kv0, Tk, k_t);
    stage_tile<D>(vb, kv0, Tk, v_t);
    __syncthreads();
#pragma unroll 4
    for (int j = 0; j < kBwdTile; ++j) {
      float r = 0.0f, gs = 0.0f;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        r = fmaf(qv[e], k_t[j * D + part * 32 + e], r);
        gs = fmaf(wv[e], v_t[j * D + part * 32 + e], gs);
      }
      r = row_sum<LPR>(r);
      gs = row_sum<LPR>(gs);
      const float pv = (kv0 + j <= kmax) ? fast_exp2(c * r - m) : 0.0f;
      const float ds = pv * (c1 + 2.0f * c2 * pv + gs);
#pragma unroll
      for (int e = 0; e < 32; ++e) dq[e] = fmaf(ds, k_t[j * D + part * 32 + e], dq[e]);
    }
  }
  if (!live) return;
  const float ls = c * kLn2;  // lam * scale
  float* out = p.dq + ri * D + part * 32;
#pragma unroll
  for (int e = 0; e < 32; e += 4) *(f32x4*)(out + e) = f32x4{dq[e] * ls, dq[e + 1] * ls, dq[e + 2] * ls, dq[e + 3] * ls};
}

template <int D, typename T, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads) void polar_bwd_dkdv_kernel(const BwdParams p) {
  constexpr int LPR = D / 32;
  constexpr int RPB = kBwdThreads / LPR;  // keys per workgroup
  __shared__ __attribute__((aligned(16))) float q_t[kBwdTile * D];
  __shared__ __attribute__((aligned(16))) float w_t[kBwdTile * D];
  __shared__ f32x4 r_t[kBwdTile];
  const int tid = threadIdx.x;
  const int part = tid % LPR;
  const int bk = blockIdx.y;  // b * Hkv + hk
  const int b = bk / p.Hkv, hk = bk - b * p.Hkv;
  const int G = p.H / p.Hkv;
  const int Tq = p.Tq, Tk = p.Tk, off = Tk - Tq;
  const int j0 = blockIdx.x * RPB;
  const int key = j0 + tid / LPR;
  const bool live = key < Tk;
  const size_t kr = (size_t)bk * Tk + min(key, Tk - 1);

  float kv[32], vv[32], dk[32], dv[32];
  load32((const T*)p.k + kr * D + part * 32, kv);
  load32((const T*)p.v + kr * D + part * 32, vv);
#pragma unroll
  for (int e = 0; e < 32; ++e) dk[e] = dv[e] = 0.0f;

  const int i_begin = CAUSAL ? max(0, j0 - off) : 0;  // first query row that sees key j0
  for (int g = 0; g < G; ++g) {
    const size_t bh = (size_t)b * p.H + hk * G + g;
    const T* qb = (const T*)p.q + bh * Tq * D;
    const float* wb = p.W + bh * Tq * D;
    for (int i0 = i_begin; i0 < Tq; i0 += kBwdTile) {
      __syncthreads();
      stage_tile<D>(qb, i0, Tq, q_t);
      stage_tile<D>(wb, i0, Tq, w_t);
      if (tid < kBwdTile)
        r_t[tid] = i0 + tid < Tq ? *(const f32x4*)(p.R + (bh * Tq + i0 + tid) * 4) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      __syncthreads();
#pragma unroll 4
      for (int i = 0; i < kBwdTile; ++i) {
        float r = 0.0f, gs = 0.0f;
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          r = fmaf(kv[e], q_t[i * D + part * 32 + e], r);
          gs = fmaf(vv[e], w_t[i * D + part * 32 + e], gs);
        }
        r = row_sum<LPR>(r);
        gs = row_sum<LPR>(gs);
        const f32x4 rv = r_t[i];
        const int qi = i0 + i;
        const bool vis = qi < Tq && (!CAUSAL || key <= qi + off);
        const float pv = vis ? fast_exp2(rv[3] * r - rv[0]) : 0.0f;
        const float ds = pv * (rv[1] + 2.0f * rv[2] * pv + gs) * (rv[3] * kLn2);
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          dk[e] = fmaf(ds, q_t[i * D + part * 32 + e], dk[e]);
          dv[e] = fmaf(pv, w_t[i * D + part * 32 + e], dv[e]);
        }
      }
    }
  }
  if (!live) return;
  float* ok = p.dk + kr * D + part * 32;
  float* ov = p.dv + kr * D + part * 32;
#pragma unroll
  for (int e = 0; e < 32; e += 4) {
    *(f32x4*)(ok + e) = f32x4{dk[e], dk[e + 1], dk[e + 2], dk[e + 3]};
    *(f32x4*)(ov + e) = f32x4{dv[e], dv[e + 1], dv[e + 2], dv[e + 3]};
  }
}

}  // namespace polar
