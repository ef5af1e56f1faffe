// Grouped split-KV decode over a contiguous or paged KV cache.
//
// [ATMA §2.2, decode kernel]: a decode step costs HBM traffic, and grouped-query
// attention cuts that traffic by the group size when every KV row is read once for all
// query heads that share it.  A workgroup here owns one (sequence b, KV head, split)
// and G of the query heads of that KV head: each 16-byte chunk of a key or value row
// is loaded once and used for all G queries.  The partial row written per query head
// is the same (m, S1, S2, acc) tuple as the ungrouped decode writes, so the same merge
// combines the splits [ATMA §2.2, squared correction factors].
//
// Paged cache: the keys of sequence b are laid out in blocks of block_size rows; entry
// (b, j) of the block table names the pool block that holds keys
// [j * block_size, (j + 1) * block_size).  The pool is [num_blocks, block_size,
// kv_heads, head_dim].  A table entry outside [0, num_blocks) is never dereferenced:
// its keys are skipped.  Each sequence has its own length (a device array); the visible
// count n of its query is that length.
//
// The arithmetic of a query does not depend on whether the cache is paged (only the row
// address differs), so paged and contiguous runs give bitwise-equal partials.
//
// Reading variants: a sliding window keeps the last `window` keys of each sequence (the
// splits cover [len - window, len)); a per-key floor reduces each weight against the
// floor of the query's visible count (the template flag KF, so the default kernels carry
// no floor code).
#pragma once

#include "decode.h"

namespace polar {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

struct GroupDecodeParams {
  const void* q;           // [B, H, D] bf16
  const void* k;           // contiguous [B, Hkv, Tk, D] or pool [num_blocks, bs, Hkv, D]
  const void* v;
  const int32_t* table;    // paged: [B, max_blocks]
  const int32_t* lens;     // paged: [B] keys per sequence
  float* part;             // [B, H, S, D + 3]
  int B, H, Hkv, Tk;       // Tk: keys of every sequence (contiguous) or the largest length (paged)
  int S;                   // splits
  int split_len;           // keys per split (the last one may be shorter)
  int chunks;              // query-head chunks of G heads per KV head
  int num_blocks, bs_log2, max_blocks;
  float scale;
  int hp_stride;
  HeadParams hp;
};

// Four query heads and no per-key floor: held to 128 registers (4 waves per SIMD), which
// they fit without spills; the other instances keep the compiler's choice.
template <int D, int G, int NW, int UNROLL, bool PAGED, int KF = POLAR_KEY_FLOOR_NULL>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(G == 4 && KF == POLAR_KEY_FLOOR_NULL ? 4
                                                                                                               : 1))) void
polar_decode_group_kernel(const GroupDecodeParams p) {
  constexpr int LPK = D / 8;          // lanes per key (8 dims each)
  constexpr int KPW = 64 / LPK;       // keys per wave per step
  constexpr int NSLOT = NW * KPW;     // independent running states per query head
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
  const int hk = blockIdx.y / p.chunks;
  const int h0 = hk * (p.H / p.Hkv) + (blockIdx.y - hk * p.chunks) * G;  // first query head
  const int b = blockIdx.z;
  int len = p.Tk;
  if constexpr (PAGED) len = min(max(p.lens[b], 0), p.Tk);
  const int start = p.hp.window > 0 ? max(0, len - p.hp.window) : 0;  // first key of the window
  const int lo = start + s * p.split_len;
  const int hi = min(lo + p.split_len, len);
  const int n = max(len - start, 1);

  // One query per sequence; it sees every cached key of its sequence (or the last
  // `window` of them), n = len - start (never a per-split count).
  uint32_t qw[G][4];
  float c[G], f2[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const u32x4 w = *(const u32x4*)((const __bf16*)p.q + ((size_t)b * p.H + h0 + g) * D + dch * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) qw[g][e] = w[e];
    const int hpi = (h0 + g) * p.hp_stride;
    const float lam = row_temperature(p.hp, hpi, n);
    c[g] = logit_scale(lam, p.scale);
    f2[g] = 0.0f;
    if constexpr (KF != POLAR_KEY_FLOOR_NULL) {
      float qq = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t x = qw[g][e];
        qq = fmaf(bf16_lo(x), bf16_lo(x), qq);
        qq = fmaf(bf16_hi(x), bf16_hi(x), qq);
      }
      qq = group_sum<LPK>(qq);
      const float sigma = p.hp.level_form == POLAR_LEVEL_QNORM ? p.scale * sqrtf(qq) : 1.0f;
      f2[g] = null_floor(p.hp, hpi, n, lam, sigma) * kLog2e;
    }
  }

  // address of the 16-byte chunk of key `key` (valid keys only)
  const __bf16* kbase = (const __bf16*)p.k;
  const __bf16* vbase = (const __bf16*)p.v;
  size_t cont_off = 0;
  if constexpr (!PAGED) cont_off = ((size_t)b * p.Hkv + hk) * p.Tk * D;
  const int32_t* trow = PAGED ? p.table + (size_t)b * p.max_blocks : nullptr;
  const int bs_mask = (1 << p.bs_log2) - 1;

  float m[G], s1[G], s2[G], acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = kMaxInit;
    s1[g] = s2[g] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.0f;
  }

  // paged: the block-table entries of an iteration's keys are loaded one iteration ahead,
  // so the K/V loads never wait on a table read
  int32_t next_blk[UNROLL];
  auto table_entries = [&](int base) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int key = base + slot + u * NSLOT;
      next_blk[u] = key < hi ? trow[key >> p.bs_log2] : 0;
    }
  };
  if constexpr (PAGED) table_entries(lo);

  for (int base = lo; base < hi; base += NSLOT * UNROLL) {
    u32x4 kr[UNROLL], vr[UNROLL];
    bool ok[UNROLL];
    int32_t blk[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) blk[u] = next_blk[u];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int key = base + slot + u * NSLOT;
      ok[u] = key < hi;
      size_t row = 0;
      if constexpr (PAGED) {
        ok[u] = ok[u] && (uint32_t)blk[u] < (uint32_t)p.num_blocks;
        row = (((size_t)(uint32_t)blk[u] << p.bs_log2) + (key & bs_mask)) * p.Hkv + hk;
      } else {
        row = (size_t)key;
      }
      if (ok[u]) {
        const size_t off = (PAGED ? row * D : cont_off + row * D) + dch * 8;
        kr[u] = __builtin_nontemporal_load((const u32x4*)(kbase + off));  // read once
        vr[u] = __builtin_nontemporal_load((const u32x4*)(vbase + off));
      } else {
        kr[u] = u32x4{0, 0, 0, 0};
        vr[u] = u32x4{0, 0, 0, 0};
      }
    }
    if constexpr (PAGED) table_entries(base + NSLOT * UNROLL);
    float vf[UNROLL][8];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vf[u][2 * e] = bf16_lo(vr[u][e]);
        vf[u][2 * e + 1] = bf16_hi(vr[u][e]);
      }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float x[UNROLL];
      float xmax = -INFINITY;
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        float r = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // copy the elements out first: a bit cast applied to a vector subscript reads
          // element 0 whatever the index (seen with this compiler)
          const uint32_t qe = qw[g][e], ke = kr[u][e];
          r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qe), __builtin_bit_cast(bf16x2_t, ke), r,
                                              false);
        }
        r = group_sum<LPK>(r);
        x[u] = ok[u] ? c[g] * r : -INFINITY;
        xmax = fmaxf(xmax, x[u]);
      }
      const float m_new = fmaxf(m[g], xmax);
      const float alpha = fast_exp2(m[g] - m_new);
      s1[g] *= alpha;
      s2[g] *= alpha * alpha;  // squared correction factor
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] *= alpha;
      m[g] = m_new;
      // the floor's weight (inf while m is far below the floor: every weight is then 0)
      const float phi = KF == POLAR_KEY_FLOOR_SOFT ? fast_exp2(f2[g] - m[g]) : 0.0f;
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        float pv = fast_exp2(x[u] - m[g]);
        if constexpr (KF == POLAR_KEY_FLOOR_SOFT) pv = fmaxf(pv - phi, 0.0f);
        if constexpr (KF == POLAR_KEY_FLOOR_GATE) pv = x[u] > f2[g] ? pv : 0.0f;
        s1[g] += pv;
        s2[g] = fmaf(pv, pv, s2[g]);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(pv, vf[u][e], acc[g][e]);
      }
    }
  }

  // ---- per query head: combine the slots of the workgroup into one partial row
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (dch == 0) {
      slot_m[slot] = m[g];
      slot_s1[slot] = s1[g];
      slot_s2[slot] = s2[g];
    }
#pragma unroll
    for (int e = 0; e < 8; e += 4) {
      const f32x4 val = {acc[g][e], acc[g][e + 1], acc[g][e + 2], acc[g][e + 3]};
      *(f32x4*)(&slot_acc[slot][dch * 8 + e]) = val;
    }
    __syncthreads();
    float M = kMaxInit;
#pragma unroll 4
    for (int i = 0; i < NSLOT; ++i) M = fmaxf(M, slot_m[i]);
    float* out = p.part + (((size_t)b * p.H + h0 + g) * p.S + s) * W;
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
      // a split that saw no key keeps M at the start value: report it as -inf
      const bool any = M > kMaxInit;
      out[0] = any ? M * kLn2 : -INFINITY;
      out[1] = any ? t1 : 0.0f;
      out[2] = any ? t2 : 0.0f;
    }
    __syncthreads();
  }
}

}  // namespace polar
