// Shared device-side definitions of the Polar Attention kernels (gfx950, wave64).
//
// Notation follows the ATMA technical summary (gist.science, paper 2606.25156):
// direction channel and magnitude channel [ATMA §2.1], fused streaming kernel and
// decode kernel [ATMA §2.2].  Inside the kernels logits are kept in base-2 units:
// x = c * <q, k> with c = lam * scale * log2(e), so exp(s - m) = exp2(x - m2).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/polar_attn.h"

namespace polar {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Start value of the running maximum (base-2 units).  Finite, so that
// exp2(x - m) with x = -inf is 0 rather than NaN before the first visible key.
constexpr float kMaxInit = -1.0e30f;
// The running reference maximum is moved only when a new score exceeds it by more
// than this (base 2), so weights stay below 2^8 between moves.  The statistics are
// exact for any reference; the true maximum is tracked on the side.
constexpr float kRescaleSlack = 8.0f;
// The bf16 prefill kernel moves its reference only when a lane's weights of one tile sum
// to more than 2^16, so every weight stays at most 2^16 between moves.  bf16 weights and
// fp32 sums round relative to their size, so the bound costs no precision, and with up to
// 2^24 keys S1 <= 2^40, S1^2 <= 2^80 and S2 <= 2^56 stay far inside fp32.  A bound this
// loose leaves the reference where the wave's first tile put it unless a row's maximum
// grows by 16 (base 2) later, which a strongly tempered row's maximum otherwise does
// often enough to make the rescale pass a measurable share of the loop.
constexpr float kWeightLimit = 65536.0f;

// Per-head parameters and the reading variant, copied by value into the kernel
// arguments.
struct HeadParams {
  float tau[POLAR_MAX_PARAM_HEADS];   // length temperature
  float beta[POLAR_MAX_PARAM_HEADS];  // null-floor offset
  float kinv[POLAR_MAX_PARAM_HEADS];  // 1 / kappa
  int lam_form;                       // polar_temperature_form
  float inv_ln_train;                 // 1 / ln L for POLAR_TEMP_TRAIN_RATIO
  int level_form;                     // polar_floor_level
  int key_floor;                      // polar_key_floor
  int sat_form;                       // polar_saturation
  int window;                         // > 0: keys per sliding window
};

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  float* dir;
  float* neff;
  float* conf;
  float* count;
  float* stats;
  int B, H, Hkv, Tq, Tk;
  int n_qt;       // query tiles per (b, h)
  int floor_on;   // null floor on
  int hp_stride;  // 1: per-head tables, 0: entry 0 serves every head
  float scale;    // softmax scale
  float* part;    // partial mode: rows [B, H, Tq, part_S, D + 3] = (m, S1, S2, acc); no channels
  int part_S, part_s;
  int ctx_k;      // > 0: a row's visible count is that of a causal row over ctx_k keys
  HeadParams hp;
};


struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  float* part;    // [B, H, S, D + 3]
  int B, H, Hkv, Tk;
  int key0;       // first key of split 0 (the start of a sliding window)
  int S;          // splits
  int split_len;  // keys per split (the last one may be shorter)
  float scale;
  int hp_stride;
  HeadParams hp;
};

struct MergeParams {
  const float* part;  // [B, H, Tq, S, D + 3]
  const __bf16* q;    // [B, H, Tq, D] for the data-adaptive floor level, else unused
  float scale;
  const int32_t* lens;  // optional [B]: visible count of sequence b (one query per sequence)
  float* dir;
  float* neff;
  float* conf;
  float* count;
  float* stats;
  int B, H, Tq, Tk, S;
  int causal;
  int floor_on;
  int hp_stride;
  HeadParams hp;
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// The per-row helpers below are compiled without floating-point contraction, so that
// every kernel instantiation that inlines them (with or without statistics, prefill,
// decode, merge) forms a row's temperature, floor and channels with the same roundings.

// Keys visible to query row `row` (rows aligned to the end of the keys when causal).
__device__ __forceinline__ int visible_keys(int row, int Tq, int Tk, bool causal) {
  int n = causal ? min(row + 1 + (Tk - Tq), Tk) : Tk;
  return max(n, 1);
}

// Visible count of query row `row` for the length temperature and the floor: its own
// count, or, in a piece of a longer causal context of ctx_k keys (chunked prefill), the
// count of that row in the whole context.
__device__ __forceinline__ int context_count(int row, int Tq, int Tk, bool causal, int ctx_k) {
  if (ctx_k > 0) return max(min(row + 1 + (ctx_k - Tq), ctx_k), 1);
  return visible_keys(row, Tq, Tk, causal);
}

// Length temperature [ATMA §2.1, direction channel], by the form of the variant:
// 1 + tau ln n (the default), tau ln n, or ln n / ln L.
__device__ __forceinline__ float row_temperature(const HeadParams& hp, int hpi, int n) {
#pragma clang fp contract(off)
  const float ln_n = logf((float)n);
  if (hp.lam_form == POLAR_TEMP_SSMAX) return hp.tau[hpi] * ln_n;
  if (hp.lam_form == POLAR_TEMP_TRAIN_RATIO) return ln_n * hp.inv_ln_train;
  return 1.0f + hp.tau[hpi] * ln_n;
}

// Base-2 logit scale c = lam * scale * log2(e).  lam may be 0 (tau ln n at n = 1); c is
// then held at a tiny positive value, so masked scores stay -inf (never 0 * -inf) while
// every visible exp2(c s - m) is exactly what c = 0 gives in fp32.
__device__ __forceinline__ float logit_scale(float lam, float scale) {
#pragma clang fp contract(off)
  return fmaxf(lam * scale * kLog2e, 1.0e-30f);
}

// Expected maximum of n standard normal logits [ATMA §2.1, extreme-value-corrected
// floor]: sqrt(2 ln n) to leading order, or the second-order Gumbel mean
// b_n + gamma a_n with r = sqrt(2 ln n), b_n = r - (ln ln n + ln 4 pi) / (2 r), a_n = 1 / r.
// One logit has mean 0.
__device__ __forceinline__ float floor_level(const HeadParams& hp, int n) {
#pragma clang fp contract(off)
  if (n <= 1) return 0.0f;
  const float ln_n = logf((float)n);
  const float r = sqrtf(2.0f * ln_n);
  if (hp.level_form == POLAR_LEVEL_GUMBEL2) {
    constexpr float kLn4Pi = 2.5310242469692907f;
    constexpr float kEulerGamma = 0.5772156649015329f;
    return r - (logf(ln_n) + kLn4Pi) / (2.0f * r) + kEulerGamma / r;
  }
  return r;
}

// Null floor f = lam sigma l(n) + beta in tempered-logit units; sigma is 1, or
// scale ||q|| for the data-adaptive level (the spread of the raw logits of the row).
__device__ __forceinline__ float null_floor(const HeadParams& hp, int hpi, int n, float lam, float sigma) {
#pragma clang fp contract(off)
  return lam * sigma * floor_level(hp, n) + hp.beta[hpi];
}

// Magnitude channel from the row statistics [ATMA §2.1]:
//   n_eff = S1^2 / S2 (participation ratio),
//   conf  = S1 / (S1 + exp(f - m)) with the null floor f (1 when the floor is off),
//   count = conf * tanh(ln(n_eff) / kappa), or tanh(ln(1 + n_eff) / kappa).
// m_nat is the row maximum in natural-log units; S1, S2 are relative to exp(m_nat).
// With a per-key floor S1 may be 0 (no key above the floor): every channel is then 0.
// A NaN in the statistics (from a NaN input the row sees) reaches every channel.
__device__ __forceinline__ void magnitude_channel(const HeadParams& hp, int hpi, float m_nat, float S1, float S2,
                                                  float f, bool floor_on, float& neff, float& conf,
                                                  float& count) {
#pragma clang fp contract(off)
  if (S1 == 0.0f) {
    neff = conf = count = 0.0f;
    return;
  }
  neff = S1 * S1 / S2;
  conf = floor_on ? 1.0f / (1.0f + expf(f - m_nat - logf(S1))) : 1.0f;
  const float x = hp.sat_form == POLAR_SAT_LOG1P ? log1pf(neff) : logf(neff);
  count = conf * tanhf(x * hp.kinv[hpi]);
}

// Block id -> (query tile, b*H + h).  Consecutive block ids are dispatched round-robin
// over the 8 XCDs; when the head count allows it, every XCD receives whole heads so a
// head's K/V tiles stay in one XCD's L2.  Within an XCD the heaviest (last, for causal)
// query tiles are issued first.  RES > 0 is the number of workgroups the chip holds at
// once; a grid that fits in one such round gives the second half of each XCD's blocks the
// lightest tiles in reverse order.  An XCD that fills its CUs in the same order twice puts
// its k-th and (c/2 + k)-th blocks on one CU, and these then sum to about the same causal
// work, instead of the heavy tiles sharing CUs with the next-heaviest ones.  Only the
// assignment of tiles to blocks changes, never a tile's arithmetic.
template <int RES = 0>
__device__ __forceinline__ void tile_coords(int bid, int n_qt, int BH, int& qt, int& bh) {
  if ((BH & 7) == 0) {
    const int hpx = BH >> 3;
    const int xcd = bid & 7;
    int local = bid >> 3;
    const int c = n_qt * hpx;  // blocks per XCD
    if (RES > 0 && c <= RES / 8 && (c & 1) == 0 && local >= c / 2) local = c - 1 - (local - c / 2);
    qt = n_qt - 1 - local / hpx;
    bh = xcd * hpx + local % hpx;
  } else {
    qt = n_qt - 1 - bid / BH;
    bh = bid % BH;
  }
}

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

}  // namespace polar
