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
// With several query heads the lanes of a key (16 at head_dim 128, 8 at 64) split the
// heads between them: the sum of the G partial dots leaves each lane with one head's
// full dot (split_row_sum), so the scores, the running maximum, the exponentials and
// the sums are formed once per head instead of once per lane and head; each head's
// weight and correction factor then reach the key's lanes by DPP broadcasts for the
// value products, which every lane keeps for all G heads over its 8 dims.  The K and
// V rows of the next iteration are loaded into a second register set while the current
// one is computed.
//
// Reading variants: a sliding window keeps the last `window` keys of each sequence (the
// splits cover [len - window, len)); a per-key floor reduces each weight against the
// floor of the query's visible count (the template flag KF, so the default kernels carry
// no floor code).
#pragma once

#include "decode.h"

namespace polar {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// One reduction step of the head-split row sum: the lane keeps the first N/2 of its N live
// slots and adds to slot j the partner's slot holding the same head -- N-1-j when the
// step's lane pairing flips every live head bit of M (a mirror), j + N/2 when it flips
// only the top one (a single-bit exchange); N <= 1: a plain step on slot 0.
template <int CTRL, bool MIRROR, int N, int G>
__device__ __forceinline__ void split_step(float (&r)[G]) {
  if constexpr (N > 1) {
#pragma unroll
    for (int j = 0; j < N / 2; ++j) r[j] += dpp_move<CTRL>(r[MIRROR ? N - 1 - j : j + N / 2]);
  } else {
    r[0] += dpp_move<CTRL>(r[0]);
  }
}

// Sum over the LPK lanes of one key (8 dims per lane: 16 lanes at head_dim 128, 8 at 64)
// of the partial dots of G <= LPK query heads, split so that each lane ends with one head's
// full dot.  Slot j of lane l holds head j ^ M with M = (l mod LPK) >> (log2 LPK - log2 G):
// the top lane bits pick the head.  The steps pair lane i with 15 - i (row mirror: flips
// every lane bit; LPK = 16 only), 7 - i in its half of 8 (half mirror: flips the three low
// bits), i ^ 2 and i ^ 1.  A step whose flipped bits include the lane bit of the top live
// head bit halves the live slots, and the partner's M differs from this lane's in exactly
// the live head bits the step flips, which gives the partner slot that holds the same head
// (split_step).  After the steps slot 0 holds the dot of head M summed over all LPK lanes,
// in the same order in every lane that holds that head (each add is commutative across
// the pair).
template <int G, int LPK>
__device__ __forceinline__ float split_row_sum(float (&r)[G]) {
  if constexpr (LPK == 16) {
    split_step<0x140, true, G, G>(r);       // row_mirror
    split_step<0x141, true, G / 2, G>(r);   // row_half_mirror
    split_step<0x4E, false, G / 4, G>(r);   // quad_perm [2,3,0,1]
    split_step<0xB1, false, G / 8, G>(r);   // quad_perm [1,0,3,2]
  } else {
    split_step<0x141, true, G, G>(r);       // row_half_mirror
    split_step<0x4E, false, G / 2, G>(r);   // quad_perm [2,3,0,1]
    split_step<0xB1, false, G / 4, G>(r);   // quad_perm [1,0,3,2]
  }
  return r[0];
}

// Broadcast of lane n of each row of 16 (row_newbcast), n a compile-time value after
// unrolling.
__device__ __forceinline__ float row_bcast(float x, int n) {
  switch (n) {
    case 0: return dpp_move<0x150>(x);
    case 1: return dpp_move<0x151>(x);
    case 2: return dpp_move<0x152>(x);
    case 3: return dpp_move<0x153>(x);
    case 4: return dpp_move<0x154>(x);
    case 5: return dpp_move<0x155>(x);
    case 6: return dpp_move<0x156>(x);
    case 7: return dpp_move<0x157>(x);
    case 8: return dpp_move<0x158>(x);
    case 9: return dpp_move<0x159>(x);
    case 10: return dpp_move<0x15A>(x);
    case 11: return dpp_move<0x15B>(x);
    case 12: return dpp_move<0x15C>(x);
    case 13: return dpp_move<0x15D>(x);
    case 14: return dpp_move<0x15E>(x);
    default: return dpp_move<0x15F>(x);
  }
}

// Broadcast of lane n of each group of 8 lanes: row_newbcast from lane n into the low half
// of each row of 16 (banks 0-1) and from lane 8 + n into its high half (banks 2-3).
template <int N>
__device__ __forceinline__ float half_row_bcast(float x) {
  const int lo = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x150 + N, 0xF, 0x3, false);
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(lo, __builtin_bit_cast(int, x), 0x158 + N, 0xF, 0xC, false));
}
__device__ __forceinline__ float group8_bcast(float x, int n) {
  switch (n) {
    case 0: return half_row_bcast<0>(x);
    case 1: return half_row_bcast<1>(x);
    case 2: return half_row_bcast<2>(x);
    case 3: return half_row_bcast<3>(x);
    case 4: return half_row_bcast<4>(x);
    case 5: return half_row_bcast<5>(x);
    case 6: return half_row_bcast<6>(x);
    default: return half_row_bcast<7>(x);
  }
}

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

// Four query heads and no per-key floor: held to 168 registers (3 waves per SIMD), which
// they fit without spills (at 128 registers the two register sets spill); the other
// instances keep the compiler's choice.
template <int D, int G, int NW, int UNROLL, bool PAGED, int KF = POLAR_KEY_FLOOR_NULL>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(G == 4 && KF == POLAR_KEY_FLOOR_NULL ? 3
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
  // several query heads: the LPK lanes of a key split the heads between them for the sum
  // of the dot and for the weights (each lane one head, split_row_sum), and each head's
  // weight is then broadcast from its lanes to the key's lanes for P V.  Not for two heads
  // over 8 lanes, where the two-move broadcasts cost about what the split saves.
  constexpr bool kSplit = G > 1 && (LPK == 16 || G > 2);
  constexpr int kLog2G = G == 2 ? 1 : G == 4 ? 2 : G == 8 ? 3 : 0;
  constexpr int kLog2L = LPK == 16 ? 4 : 3;
  constexpr int kLanesPerHead = LPK >> kLog2G;
  const int hm = kSplit ? dch >> (kLog2L - kLog2G) : 0;  // the head this lane finishes (split form)
  auto head_bcast = [&](float x, int g) __attribute__((always_inline)) {
    if constexpr (LPK == 16) return row_bcast(x, g * kLanesPerHead);
    else return group8_bcast(x, g * kLanesPerHead);
  };

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
  // `window` of them), n = len - start (never a per-split count).  Slot g holds query
  // head g, or head g ^ hm in the split form.
  uint32_t qw[G][4];
  float c[G], f2[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int hg = h0 + (kSplit ? g ^ hm : g);
    const u32x4 w = *(const u32x4*)((const __bf16*)p.q + ((size_t)b * p.H + hg) * D + dch * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) qw[g][e] = w[e];
    const int hpi = hg * p.hp_stride;
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

  // The K and V rows of an iteration (UNROLL keys per slot) are loaded into one of two
  // register sets while the keys of the other set are computed, so one iteration's loads
  // are in flight during the previous iteration's arithmetic.  Paged: the block-table
  // entries of a set are loaded before the set itself is issued.
  constexpr int STEP = NSLOT * UNROLL;
  struct Rows {
    u32x4 k[UNROLL], v[UNROLL];
    bool ok[UNROLL];
  };
  int32_t tbl[UNROLL];
  auto table_entries = [&](int base) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int key = base + slot + u * NSLOT;
      tbl[u] = key < hi ? trow[key >> p.bs_log2] : 0;
    }
  };
  auto issue = [&](int base, Rows& r) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int key = base + slot + u * NSLOT;
      r.ok[u] = key < hi;
      size_t row = 0;
      if constexpr (PAGED) {
        r.ok[u] = r.ok[u] && (uint32_t)tbl[u] < (uint32_t)p.num_blocks;
        row = (((size_t)(uint32_t)tbl[u] << p.bs_log2) + (key & bs_mask)) * p.Hkv + hk;
      } else {
        row = (size_t)key;
      }
      // a key past the end (or in a skipped block) loads nothing: its score is -inf, so
      // only its V row enters the sums, times a weight of 0, and that row still holds the
      // zeros it started with or an earlier key's finite values of this sequence
      if (r.ok[u]) {
        const size_t off = (PAGED ? row * D : cont_off + row * D) + dch * 8;
        r.k[u] = __builtin_nontemporal_load((const u32x4*)(kbase + off));  // read once
        r.v[u] = __builtin_nontemporal_load((const u32x4*)(vbase + off));
      }
    }
  };
  auto compute = [&](const Rows& r) __attribute__((always_inline)) {
    float vf[UNROLL][8];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vf[u][2 * e] = bf16_lo(r.v[u][e]);
        vf[u][2 * e + 1] = bf16_hi(r.v[u][e]);
      }
    if constexpr (kSplit) {
      // this lane's head (slot 0): scores, running maximum, weights and sums
      float x[UNROLL];
      float xmax = -INFINITY;
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        float part[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float t = 0.0f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t qe = qw[g][e], ke = r.k[u][e];
            t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qe), __builtin_bit_cast(bf16x2_t, ke), t,
                                                false);
          }
          part[g] = t;
        }
        const float dot = split_row_sum<G, LPK>(part);
        x[u] = r.ok[u] ? c[0] * dot : -INFINITY;
        xmax = fmaxf(xmax, x[u]);
      }
      const float m_new = fmaxf(m[0], xmax);
      const float alpha = fast_exp2(m[0] - m_new);
      s1[0] *= alpha;
      s2[0] *= alpha * alpha;  // squared correction factor
      m[0] = m_new;
      const float phi = KF == POLAR_KEY_FLOOR_SOFT ? fast_exp2(f2[0] - m[0]) : 0.0f;
      float pw[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        float pv = fast_exp2(x[u] - m[0]);
        if constexpr (KF == POLAR_KEY_FLOOR_SOFT) pv = fmaxf(pv - phi, 0.0f);
        if constexpr (KF == POLAR_KEY_FLOOR_GATE) pv = x[u] > f2[0] ? pv : 0.0f;
        s1[0] += pv;
        s2[0] = fmaf(pv, pv, s2[0]);
        pw[u] = pv;
      }
      // every head's correction factor and weights, from the first lane holding that head
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float ag = head_bcast(alpha, g);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] *= ag;
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
          const float pg = head_bcast(pw[u], g);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(pg, vf[u][e], acc[g][e]);
        }
      }
    } else {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float x[UNROLL];
      float xmax = -INFINITY;
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        float dt = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // copy the elements out first: a bit cast applied to a vector subscript reads
          // element 0 whatever the index (seen with this compiler)
          const uint32_t qe = qw[g][e], ke = r.k[u][e];
          dt = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qe), __builtin_bit_cast(bf16x2_t, ke), dt,
                                               false);
        }
        dt = group_sum<LPK>(dt);
        x[u] = r.ok[u] ? c[g] * dt : -INFINITY;
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
  };

  Rows ra, rb;
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) ra.k[u] = ra.v[u] = rb.k[u] = rb.v[u] = u32x4{0, 0, 0, 0};
  if constexpr (PAGED) table_entries(lo);
  issue(lo, ra);
  if constexpr (PAGED) table_entries(lo + STEP);
  for (int base = lo; base < hi; base += 2 * STEP) {
    issue(base + STEP, rb);
    if constexpr (PAGED) table_entries(base + 2 * STEP);
    compute(ra);
    if (base + STEP >= hi) break;
    issue(base + 2 * STEP, ra);
    if constexpr (PAGED) table_entries(base + 3 * STEP);
    compute(rb);
  }

  // ---- per query head: combine the slots of the workgroup into one partial row
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (kSplit ? dch == g * kLanesPerHead : dch == 0) {
      slot_m[slot] = m[kSplit ? 0 : g];
      slot_s1[slot] = s1[kSplit ? 0 : g];
      slot_s2[slot] = s2[kSplit ? 0 : g];
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
