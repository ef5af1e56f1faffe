// Host side of the Polar Attention C ABI: argument checks, per-head constants, launch
// geometry.  Every check runs before the first HIP call; the library allocates nothing
// and never synchronises.  Its one piece of mutable global state is the per-device
// address of the no-allocation decode's array, looked up once per device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <type_traits>

#include "../../include/polar_attn.h"
#include "bwd.h"
#include "bwd_mfma.h"
#include "decode.h"
#include "decode_group.h"
#include "fwd_bf16.h"
#include "fwd_bf16_pipe.h"
#include "fwd_f32.h"
#include "polar_common.h"

namespace {

using polar::DecodeParams;
using polar::FwdParams;
using polar::HeadParams;
using polar::MergeParams;

// Prefill launch geometry (one configuration per dtype and head_dim).  The macros only
// exist so that tile sweeps can rebuild the library with other values.
#ifndef POLAR_BF16_WAVES
#define POLAR_BF16_WAVES 4
#endif
#ifndef POLAR_BF16_BN_D64
#define POLAR_BF16_BN_D64 64
#endif
#ifndef POLAR_BF16_BN_D128
#define POLAR_BF16_BN_D128 64
#endif
#ifndef POLAR_BF16_NB_D64
#define POLAR_BF16_NB_D64 2
#endif
#ifndef POLAR_BF16_NB_D128
#define POLAR_BF16_NB_D128 1
#endif
#ifndef POLAR_BF16_OCC_D64
#define POLAR_BF16_OCC_D64 2
#endif
#ifndef POLAR_BF16_OCC_D128
#define POLAR_BF16_OCC_D128 2
#endif
constexpr int kBf16Waves = POLAR_BF16_WAVES;      // query rows per workgroup = 32 x waves
constexpr int kBf16Bn_d64 = POLAR_BF16_BN_D64;    // keys per LDS tile
constexpr int kBf16Bn_d128 = POLAR_BF16_BN_D128;
constexpr int kBf16Nb_d64 = POLAR_BF16_NB_D64;    // 32-row query blocks per wave
constexpr int kBf16Nb_d128 = POLAR_BF16_NB_D128;
constexpr int kBf16Occ_d64 = POLAR_BF16_OCC_D64;  // waves per SIMD the registers must allow
constexpr int kBf16Occ_d128 = POLAR_BF16_OCC_D128;
constexpr int kBf16Occ_d64_one_round = 3;           // one 32-row block per wave: 160 registers
// Decode launch geometry.
constexpr int kDecodeWaves = 4;
constexpr int kDecodeUnroll = 8;

inline bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

inline bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

inline size_t elem_bytes(int32_t dtype) { return dtype == POLAR_F32 ? 4 : 2; }

// Shape checks common to every entry point.  `empty` reports a problem with no rows.
polar_status check_shape(const polar_problem* pr, bool& empty) {
  if (!pr) return POLAR_ERR_NULL_ARG;
  if (pr->batch < 0 || pr->seq_q < 0 || pr->heads < 1 || pr->kv_heads < 1 || pr->seq_k < 1)
    return POLAR_ERR_BAD_SHAPE;
  if (pr->heads % pr->kv_heads != 0) return POLAR_ERR_BAD_SHAPE;
  if (pr->causal && pr->seq_q > pr->seq_k) return POLAR_ERR_BAD_SHAPE;
  if (pr->head_dim != 64 && pr->head_dim != 128) return POLAR_ERR_UNSUPPORTED;
  if (pr->dtype != POLAR_BF16 && pr->dtype != POLAR_F32) return POLAR_ERR_UNSUPPORTED;
  empty = (pr->batch == 0 || pr->seq_q == 0);
  return POLAR_OK;
}

// The bf16 matrix-core kernels address one head's rows through a buffer resource whose
// range and offsets are 32-bit: that head's bytes, plus a tile's worth of lane offsets,
// must stay below 4 GiB.  (The fp32 and decode kernels index with 64-bit offsets.)
bool bf16_head_fits(const polar_problem* pr, int64_t seq) {
  return pr->dtype != POLAR_BF16 || (uint64_t)seq * (uint64_t)pr->head_dim * 2u + 65536u <= 0xFFFFFFFFull;
}

// Reading variant -> kernel constants, with the checks every entry point shares.
polar_status variant_params(const polar_problem* pr, HeadParams& hp) {
  const polar_variant* v = pr->variant;
  hp.lam_form = v ? v->temperature : POLAR_TEMP_LOG;
  hp.level_form = v ? v->floor_level : POLAR_LEVEL_GAUSS;
  hp.key_floor = v ? v->key_floor : POLAR_KEY_FLOOR_NULL;
  hp.sat_form = v ? v->saturation : POLAR_SAT_LOG;
  hp.window = v ? v->window : 0;
  hp.inv_ln_train = 0.0f;
  if (hp.lam_form < POLAR_TEMP_LOG || hp.lam_form > POLAR_TEMP_TRAIN_RATIO || hp.level_form < POLAR_LEVEL_GAUSS ||
      hp.level_form > POLAR_LEVEL_QNORM || hp.key_floor < POLAR_KEY_FLOOR_NULL ||
      hp.key_floor > POLAR_KEY_FLOOR_GATE || hp.sat_form < POLAR_SAT_LOG || hp.sat_form > POLAR_SAT_LOG1P)
    return POLAR_ERR_UNSUPPORTED;
  if (hp.window < 0) return POLAR_ERR_BAD_PARAM;
  if (hp.lam_form == POLAR_TEMP_TRAIN_RATIO) {
    if (v->train_len < 2) return POLAR_ERR_BAD_PARAM;
    hp.inv_ln_train = (float)(1.0 / std::log((double)v->train_len));
  }
  // a per-key floor needs a floor
  if (hp.key_floor != POLAR_KEY_FLOOR_NULL && !pr->null_bias) return POLAR_ERR_BAD_PARAM;
  return POLAR_OK;
}

// Per-head tables -> kernel constants.  Checks the values the maths needs: finite
// parameters, kappa > 0, and a non-negative length temperature over the visible counts
// 1..seq_k, positive from n = 2 on (lam is affine in ln n, so checking n = seq_k suffices
// for 1 + tau ln n; tau ln n needs tau >= 0).
polar_status head_params(const polar_problem* pr, HeadParams& hp, int& stride, int& floor_on, float& scale) {
  const polar_status vst = variant_params(pr, hp);
  if (vst != POLAR_OK) return vst;
  const bool any = pr->len_temp || pr->null_bias || pr->count_scale;
  if (any && pr->heads > POLAR_MAX_PARAM_HEADS) return POLAR_ERR_UNSUPPORTED;
  const int n = any ? pr->heads : 1;
  stride = any ? 1 : 0;
  floor_on = pr->null_bias != nullptr;
  const double ln_tk = std::log((double)pr->seq_k);
  for (int h = 0; h < n; ++h) {
    const float tau = pr->len_temp ? pr->len_temp[h] : 0.0f;
    const float beta = pr->null_bias ? pr->null_bias[h] : 0.0f;
    const float kappa = pr->count_scale ? pr->count_scale[h] : 1.0f;
    if (!std::isfinite(tau) || !std::isfinite(beta) || !std::isfinite(kappa) || !(kappa > 0.0f))
      return POLAR_ERR_BAD_PARAM;
    if (hp.lam_form == POLAR_TEMP_LOG && !(1.0 + (double)tau * ln_tk > 0.0)) return POLAR_ERR_BAD_PARAM;
    if (hp.lam_form == POLAR_TEMP_SSMAX && !(tau >= 0.0f)) return POLAR_ERR_BAD_PARAM;
    hp.tau[h] = tau;
    hp.beta[h] = beta;
    hp.kinv[h] = 1.0f / kappa;
  }
  if (!std::isfinite(pr->softmax_scale)) return POLAR_ERR_BAD_PARAM;
  scale = pr->softmax_scale > 0.0f ? pr->softmax_scale : (float)(1.0 / std::sqrt((double)pr->head_dim));
  return POLAR_OK;
}

// Output pointer checks shared by fwd, decode and merge.
polar_status check_outputs(const polar_problem* pr, const polar_outputs* out, const void* const* ins,
                           const size_t* in_bytes, int n_in) {
  if (!out || !out->direction || !out->n_eff) return POLAR_ERR_NULL_ARG;
  if (!aligned(out->direction, 16) || !aligned(out->n_eff, 4) || !aligned(out->confidence, 4) ||
      !aligned(out->count, 4) || !aligned(out->stats, 4))
    return POLAR_ERR_MISALIGNED;
  const size_t rows = (size_t)pr->batch * pr->heads * pr->seq_q;
  const void* outs[5] = {out->direction, out->n_eff, out->confidence, out->count, out->stats};
  const size_t out_bytes[5] = {rows * pr->head_dim * 4, rows * 4, rows * 4, rows * 4, rows * 12};
  for (int o = 0; o < 5; ++o)
    for (int i = 0; i < n_in; ++i)
      if (overlaps(outs[o], out_bytes[o], ins[i], in_bytes[i])) return POLAR_ERR_ALIAS;
  for (int o = 0; o < 5; ++o)
    for (int o2 = o + 1; o2 < 5; ++o2)
      if (overlaps(outs[o], out_bytes[o], outs[o2], out_bytes[o2])) return POLAR_ERR_ALIAS;
  return POLAR_OK;
}

// One launch; the status is the launch's own (hipLaunchKernel's result), so an error left
// on the calling thread by an unrelated HIP call is neither reported nor cleared here.
template <typename Kernel, typename Params>
polar_status launch(Kernel kernel, dim3 grid, dim3 block, const Params& params, void* stream) {
  void* args[] = {const_cast<Params*>(&params)};
  const hipError_t e =
      hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, 0, (hipStream_t)stream);
  return e == hipSuccess ? POLAR_OK : POLAR_ERR_HIP;
}

// Which entry point is checking a problem's reading variant.
enum class Entry { kFwd, kPartial, kDecode, kMerge, kBwd };

// Variant checks that depend on the entry point (after head_params has validated the
// variant itself).  `have_q`: the merge can read the queries (decode), which the
// data-adaptive floor level needs.
polar_status check_entry_variant(const polar_problem* pr, const HeadParams& hp, Entry e, bool have_q) {
  switch (e) {
    case Entry::kBwd:
      // the variants that change only per-row constants (temperature, floor level from the
      // count alone, saturation); a per-key floor, a window or the q-scaled level would
      // change the gradient's form
      return hp.key_floor == POLAR_KEY_FLOOR_NULL && hp.window == 0 && hp.level_form != POLAR_LEVEL_QNORM
                 ? POLAR_OK
                 : POLAR_ERR_UNSUPPORTED;
    case Entry::kFwd:
      return hp.window > 0 && !pr->causal ? POLAR_ERR_UNSUPPORTED : POLAR_OK;
    case Entry::kPartial:
      return hp.window > 0 || hp.level_form == POLAR_LEVEL_QNORM ? POLAR_ERR_UNSUPPORTED : POLAR_OK;
    case Entry::kMerge:
      return hp.level_form == POLAR_LEVEL_QNORM && !have_q ? POLAR_ERR_UNSUPPORTED : POLAR_OK;
    default:
      return POLAR_OK;
  }
}

// Workgroups of the bf16 prefill resident at once: 256 CUs x 4 SIMDs x OCC waves per SIMD,
// kBf16Waves waves each.
template <int OCC>
constexpr int kResidentWorkgroups() {
  return 256 * 4 * OCC / kBf16Waves;
}

// bf16 prefill with the key-floor and window flags of the variant.
template <int D, bool CAUSAL, bool STATS, int KF>
polar_status launch_bf16_kf(const FwdParams& fp, unsigned blocks, void* stream) {
  constexpr int NB = D == 64 ? kBf16Nb_d64 : kBf16Nb_d128;
  constexpr int OCC = D == 64 ? kBf16Occ_d64 : kBf16Occ_d128;
  constexpr int BN = D == 64 ? kBf16Bn_d64 : kBf16Bn_d128;
  if constexpr (CAUSAL) {
    if (fp.hp.window > 0)
      return launch(polar::polar_fwd_bf16_kernel<D, BN, kBf16Waves, NB, OCC, CAUSAL, STATS, KF, true>, dim3(blocks),
                    dim3(kBf16Waves * 64), fp, stream);
  }
  if constexpr (KF == POLAR_KEY_FLOOR_NULL) {
    // A causal grid the chip holds in one round lasts as long as its heaviest query tile;
    // at d = 64 such grids take query tiles of half the rows (one 32-row block per wave,
    // 160 registers, so three waves per SIMD), which the heaviest-first order spreads over
    // more resident slots -- when the tiles' key counts differ widely (fewer keys before
    // the first row than rows), or when the half-height grid itself fits one round.  A
    // chunk of rows after a long prefix has tiles of nearly equal work, where a second
    // round of half-height tiles costs more than it saves.  Larger grids, and every
    // non-causal one (equal tiles), keep two blocks per wave, which share each K and V
    // operand read between two MFMAs.
    if constexpr (D == 64 && NB == 2 && CAUSAL) {
      if (blocks <= (unsigned)kResidentWorkgroups<OCC>() &&
          (fp.Tk - fp.Tq < fp.Tq || 2 * blocks <= (unsigned)kResidentWorkgroups<kBf16Occ_d64_one_round>())) {
        FwdParams f1 = fp;
        constexpr int BM1 = kBf16Waves * 32;
        f1.n_qt = (fp.Tq + BM1 - 1) / BM1;
        const unsigned blocks1 = (unsigned)f1.n_qt * (unsigned)(fp.B * fp.H);
        return launch(polar::polar_fwd_bf16_pipe_kernel<D, kBf16Waves, 1, kBf16Occ_d64_one_round, CAUSAL, STATS>,
                      dim3(blocks1),
                      dim3(kBf16Waves * 64), f1, stream);
      }
    }
    return launch(polar::polar_fwd_bf16_pipe_kernel<D, kBf16Waves, NB, OCC, CAUSAL, STATS>, dim3(blocks),
                  dim3(kBf16Waves * 64), fp, stream);
  }
  return launch(polar::polar_fwd_bf16_kernel<D, BN, kBf16Waves, NB, OCC, CAUSAL, STATS, KF, false>, dim3(blocks),
                dim3(kBf16Waves * 64), fp, stream);
}

template <int D, bool CAUSAL, bool STATS>
polar_status launch_bf16(const FwdParams& fp, unsigned blocks, void* stream) {
  switch (fp.hp.key_floor) {
    case POLAR_KEY_FLOOR_SOFT:
      return launch_bf16_kf<D, CAUSAL, STATS, POLAR_KEY_FLOOR_SOFT>(fp, blocks, stream);
    case POLAR_KEY_FLOOR_GATE:
      return launch_bf16_kf<D, CAUSAL, STATS, POLAR_KEY_FLOOR_GATE>(fp, blocks, stream);
    default:
      return launch_bf16_kf<D, CAUSAL, STATS, POLAR_KEY_FLOOR_NULL>(fp, blocks, stream);
  }
}

template <int D, bool CAUSAL>
polar_status launch_fwd(const polar_problem* pr, FwdParams& fp, void* stream) {
  const long long BH = (long long)pr->batch * pr->heads;
  if (pr->dtype == POLAR_BF16) {
    constexpr int NB = D == 64 ? kBf16Nb_d64 : kBf16Nb_d128;
    constexpr int BM = kBf16Waves * 32 * NB;
    fp.n_qt = (pr->seq_q + BM - 1) / BM;
    const long long blocks = (long long)fp.n_qt * BH;
    if (blocks > INT32_MAX) return POLAR_ERR_UNSUPPORTED;
    // the instantiation without statistics does not track the true row maximum
    if (fp.stats || fp.part) return launch_bf16<D, CAUSAL, true>(fp, (unsigned)blocks, stream);
    return launch_bf16<D, CAUSAL, false>(fp, (unsigned)blocks, stream);
  }
  fp.n_qt = (pr->seq_q + polar::kF32RowsPerBlock - 1) / polar::kF32RowsPerBlock;
  const long long blocks = (long long)fp.n_qt * BH;
  if (blocks > INT32_MAX) return POLAR_ERR_UNSUPPORTED;
  return launch(polar::polar_fwd_f32_kernel<D, CAUSAL>, dim3((unsigned)blocks), dim3(polar::kF32Threads), fp,
                stream);
}

// Query heads one grouped-decode workgroup serves: the largest of 8, 4, 2, 1 that divides
// the group size heads / kv_heads.
int group_chunk(const polar_problem* pr) {
  const int g = pr->heads / pr->kv_heads;
  for (int c = 8; c > 1; c >>= 1)
    if (g % c == 0) return c;
  return 1;
}

// Split workgroups the automatic split count aims for, by kernel, and the fewest keys a
// split takes.  Measured: the one-head-per-workgroup kernel ran the same from 2048 to 4096
// workgroups; the grouped kernel over a contiguous cache 1-3% faster at 2048 than at 4096;
// over a shuffled paged pool 5% faster at 6144 than at 4096 (more workgroups keep more of
// the scattered block reads in flight) while a split keeps at least 2048 keys, and 3%
// slower at 6144 workgroups of 1365 keys than at 4096 of 2048.
constexpr int kSplitTargetPlain = 4096;
constexpr int kSplitTargetGrouped = 2048;
constexpr int kSplitTargetPaged = 6144;
constexpr int kSplitMinKeys = 256;
constexpr int kSplitMinKeysPaged = 2048;
// at most this many splits: past it, fewer rows gain less from more workgroups than the
// partial rows and their merge cost (batch 1, 8 heads, 2^20 keys: 128 splits 0.634 ms,
// 512 splits 0.699 ms; 64K keys: 0.060 against 0.072 ms at 256)
constexpr int kSplitMax = 128;

int auto_splits(const polar_problem* pr, bool paged) {
  // About the target's number of split workgroups, with at least the minimum of keys per
  // split (one split when the sequence is shorter) and at most kSplitMax splits.  A
  // workgroup serves one query head, or a chunk of a query-head group when heads share a
  // KV head.
  const long long rows = (long long)pr->batch * (pr->heads / group_chunk(pr));
  if (rows <= 0) return 1;  // no rows: nothing is launched
  const long long target =
      paged ? kSplitTargetPaged : (pr->heads > pr->kv_heads ? kSplitTargetGrouped : kSplitTargetPlain);
  long long s = (target + rows - 1) / rows;
  const long long min_keys = paged ? kSplitMinKeysPaged : kSplitMinKeys;
  const long long max_by_len = (pr->seq_k + min_keys - 1) / min_keys;
  if (s > max_by_len) s = max_by_len;
  if (s > kSplitMax) s = kSplitMax;
  if (s < 1) s = 1;
  return (int)s;
}

polar_status check_decode(const polar_problem* pr, int32_t num_splits, int& splits) {
  bool empty = false;
  const polar_status st = check_shape(pr, empty);
  if (st != POLAR_OK) return st;
  if (pr->seq_q != 1 && !empty) return POLAR_ERR_UNSUPPORTED;
  if (pr->dtype != POLAR_BF16) return POLAR_ERR_UNSUPPORTED;
  if (num_splits < 0 || num_splits > pr->seq_k) return POLAR_ERR_BAD_SHAPE;
  splits = num_splits == 0 ? auto_splits(pr, false) : num_splits;
  return POLAR_OK;
}

size_t partial_bytes(const polar_problem* pr, int splits) {
  return (size_t)pr->batch * pr->heads * pr->seq_q * splits * (pr->head_dim + 3) * sizeof(float);
}

// Checks of a paged decode call that need no device memory.
polar_status check_paged(const polar_problem* pr, const polar_paged_kv* kv, int32_t num_splits, int& splits) {
  if (!kv) return POLAR_ERR_NULL_ARG;
  polar_problem flat = *pr;
  flat.causal = 0;  // the query sees every cached key of its sequence
  const polar_status st = check_decode(&flat, 0, splits);
  if (st != POLAR_OK) return st;
  const int bs = kv->block_size;
  if (bs < 1 || bs > 1024 || (bs & (bs - 1)) != 0) return POLAR_ERR_BAD_SHAPE;
  if (kv->num_blocks < 1 || kv->max_blocks < 1) return POLAR_ERR_BAD_SHAPE;
  if ((long long)kv->max_blocks * bs < pr->seq_k) return POLAR_ERR_BAD_SHAPE;
  if (num_splits < 0 || num_splits > pr->seq_k) return POLAR_ERR_BAD_SHAPE;
  splits = num_splits == 0 ? auto_splits(pr, true) : num_splits;
  return POLAR_OK;
}

template <int D, bool PAGED, int KF>
polar_status launch_group_kf(int chunk, polar::GroupDecodeParams& gp, dim3 grid, void* stream) {
  constexpr int NW = kDecodeWaves;
  switch (chunk) {
    case 1:
      return launch(polar::polar_decode_group_kernel<D, 1, NW, 8, PAGED, KF>, grid, dim3(NW * 64), gp, stream);
    case 2:
      return launch(polar::polar_decode_group_kernel<D, 2, NW, 4, PAGED, KF>, grid, dim3(NW * 64), gp, stream);
    case 4:
      return launch(polar::polar_decode_group_kernel<D, 4, NW, 4, PAGED, KF>, grid, dim3(NW * 64), gp, stream);
    default:
      return launch(polar::polar_decode_group_kernel<D, 8, NW, 2, PAGED, KF>, grid, dim3(NW * 64), gp, stream);
  }
}

template <int D, bool PAGED>
polar_status launch_group(int chunk, polar::GroupDecodeParams& gp, dim3 grid, void* stream) {
  switch (gp.hp.key_floor) {
    case POLAR_KEY_FLOOR_SOFT:
      return launch_group_kf<D, PAGED, POLAR_KEY_FLOOR_SOFT>(chunk, gp, grid, stream);
    case POLAR_KEY_FLOOR_GATE:
      return launch_group_kf<D, PAGED, POLAR_KEY_FLOOR_GATE>(chunk, gp, grid, stream);
    default:
      return launch_group_kf<D, PAGED, POLAR_KEY_FLOOR_NULL>(chunk, gp, grid, stream);
  }
}

template <int D>
polar_status launch_split(const DecodeParams& dp, dim3 grid, void* stream) {
  const dim3 block(kDecodeWaves * 64);
  switch (dp.hp.key_floor) {
    case POLAR_KEY_FLOOR_SOFT:
      return launch(polar::polar_decode_split_kernel<D, kDecodeWaves, kDecodeUnroll, POLAR_KEY_FLOOR_SOFT>, grid, block,
                    dp, stream);
    case POLAR_KEY_FLOOR_GATE:
      return launch(polar::polar_decode_split_kernel<D, kDecodeWaves, kDecodeUnroll, POLAR_KEY_FLOOR_GATE>, grid, block,
                    dp, stream);
    default:
      return launch(polar::polar_decode_split_kernel<D, kDecodeWaves, kDecodeUnroll, POLAR_KEY_FLOOR_NULL>, grid, block,
                    dp, stream);
  }
}

// Grouped split kernel over a contiguous (kv == NULL) or paged cache; fills gp's common
// fields.  The caller has validated everything.
polar_status launch_grouped_splits(const polar_problem* pr, const polar_paged_kv* kv, const void* q,
                                   const void* k, const void* v, int splits, void* workspace, void* stream) {
  polar::GroupDecodeParams gp;
  std::memset(&gp, 0, sizeof(gp));
  int floor_on = 0;
  const polar_status st = head_params(pr, gp.hp, gp.hp_stride, floor_on, gp.scale);
  if (st != POLAR_OK) return st;
  const int chunk = group_chunk(pr);
  gp.q = q;
  gp.k = k;
  gp.v = v;
  gp.part = (float*)workspace;
  gp.B = pr->batch;
  gp.H = pr->heads;
  gp.Hkv = pr->kv_heads;
  gp.Tk = pr->seq_k;
  gp.S = splits;
  // the splits cover the last min(window, seq_k) keys of the longest sequence
  const int keys = gp.hp.window > 0 && gp.hp.window < pr->seq_k ? gp.hp.window : pr->seq_k;
  gp.split_len = (keys + splits - 1) / splits;
  gp.chunks = (pr->heads / pr->kv_heads) / chunk;
  if (kv) {
    gp.table = kv->block_table;
    gp.lens = kv->seq_lens;
    gp.num_blocks = kv->num_blocks;
    gp.max_blocks = kv->max_blocks;
    int l2 = 0;
    while ((1 << l2) < kv->block_size) ++l2;
    gp.bs_log2 = l2;
  }
  const long long gy = (long long)pr->kv_heads * gp.chunks;
  if (gy > 65535 || pr->batch > 65535) return POLAR_ERR_UNSUPPORTED;
  const dim3 grid(splits, (unsigned)gy, pr->batch);
  if (pr->head_dim == 64)
    return kv ? launch_group<64, true>(chunk, gp, grid, stream) : launch_group<64, false>(chunk, gp, grid, stream);
  return kv ? launch_group<128, true>(chunk, gp, grid, stream) : launch_group<128, false>(chunk, gp, grid, stream);
}

template <int D>
polar_status launch_merge(const polar_problem* pr, MergeParams& mp, void* stream) {
  const long long rows = (long long)pr->batch * pr->heads * pr->seq_q;
  if (rows > INT32_MAX) return POLAR_ERR_UNSUPPORTED;
  // up to 16 splits every lane walks them all; then the lanes share them, and four waves
  // once they outnumber what one wave's lanes take in one pass
  if (mp.S > 64) return launch(polar::polar_merge_kernel<D, 4>, dim3((unsigned)rows), dim3(256), mp, stream);
  if (mp.S > 16) return launch(polar::polar_merge_kernel<D, 1>, dim3((unsigned)rows), dim3(64), mp, stream);
  return launch(polar::polar_merge_few_kernel<D>, dim3((unsigned)rows), dim3(64), mp, stream);
}

polar_status merge_with_lens(const polar_problem* pr, const float* partials, int32_t num_splits,
                             const int32_t* lens, const void* q, const polar_outputs* out, void* stream) {
  bool empty = false;
  polar_status st = check_shape(pr, empty);
  if (st != POLAR_OK) return st;
  if (num_splits < 1) return POLAR_ERR_BAD_SHAPE;
  MergeParams mp;
  std::memset(&mp, 0, sizeof(mp));
  st = head_params(pr, mp.hp, mp.hp_stride, mp.floor_on, mp.scale);
  if (st != POLAR_OK) return st;
  st = check_entry_variant(pr, mp.hp, Entry::kMerge, q != nullptr);
  if (st != POLAR_OK) return st;
  if (empty) return POLAR_OK;  // no rows: pointers of empty tensors may be NULL
  if (!partials) return POLAR_ERR_NULL_ARG;
  if (!aligned(partials, 4)) return POLAR_ERR_MISALIGNED;
  const void* ins[1] = {partials};
  const size_t in_bytes[1] = {partial_bytes(pr, num_splits)};
  st = check_outputs(pr, out, ins, in_bytes, 1);
  if (st != POLAR_OK) return st;
  mp.part = partials;
  mp.q = static_cast<const __bf16*>(q);
  mp.lens = lens;
  mp.dir = out->direction;
  mp.neff = out->n_eff;
  mp.conf = out->confidence;
  mp.count = out->count;
  mp.stats = out->stats;
  mp.B = pr->batch;
  mp.H = pr->heads;
  mp.Tq = pr->seq_q;
  mp.Tk = pr->seq_k;
  mp.S = num_splits;
  mp.causal = pr->causal != 0;
  return pr->head_dim == 64 ? launch_merge<64>(pr, mp, stream) : launch_merge<128>(pr, mp, stream);
}

// ---- backward

constexpr size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr int kBwdWaves = 4;  // matrix-core backward: 32 rows (or keys) per wave

// Workgroups per key tile of the matrix-core dk/dv kernels.  One workgroup per (key tile,
// kv head) gives B * Hkv * Tk / 128 workgroups, which for a long single sequence is about
// one per resident slot (256 CUs x 2); under a causal mask the first key tile has ~Tq/128
// times the work of the last, so the launch would last as long as its heaviest workgroup.
// Each key tile's (head, query tile) pairs are then cut into n contiguous runs, enough for
// four workgroups per slot (causal) or one (full mask), at most 4 per query head.
int bwd_splits(const polar_problem* pr) {
  if (pr->seq_q == 0) return 1;
  const long long base = (long long)pr->batch * pr->kv_heads * ((pr->seq_k + kBwdWaves * 32 - 1) / (kBwdWaves * 32));
  const long long target = pr->causal ? 2048 : 512;
  const long long want = (target + base - 1) / base;
  const long long cap = 4ll * (pr->heads / pr->kv_heads);
  return (int)std::max(1ll, std::min(want, cap));
}

// Backward workspace.  fp32 inputs: w and the row constants in fp32, [rows, D + 4].
// bf16 inputs: the forward's partial rows [rows, D + 3] fp32 (not when the caller passes
// them in), then w as bf16 [rows, D], then the row constants [rows] f32x4, then (split
// key tiles only) the partial dk and dv, [splits, B, Hkv, Tk, D] fp32 each; every part
// starts on a 256-byte boundary.
size_t bwd_workspace(const polar_problem* pr, bool saved = false) {
  const size_t rows = (size_t)pr->batch * pr->heads * pr->seq_q;
  const size_t D = pr->head_dim;
  if (pr->dtype == POLAR_F32) return rows * (D + 4) * sizeof(float);
  if (rows == 0) return 0;
  const size_t base =
      (saved ? 0 : align256(rows * (D + 3) * 4)) + align256(rows * D * 2) + align256(rows * 16);
  const int splits = bwd_splits(pr);
  if (splits == 1) return base;
  const size_t nk = (size_t)pr->batch * pr->kv_heads * pr->seq_k;
  return base + 2 * align256((size_t)splits * nk * D * 4);
}

// bf16 backward on the matrix cores: the forward in partial mode for the row statistics
// (unless the caller saved them), then the row constants, dq and dk/dv.
template <int D, bool CAUSAL>
polar_status launch_bwd_mfma(const polar_problem* pr, FwdParams& fp, polar::BwdMfmaParams& mp, bool run_fwd,
                             void* stream) {
  polar_status st = POLAR_OK;
  if (mp.Tq > 0) {
    if (run_fwd) {
      st = launch_fwd<D, CAUSAL>(pr, fp, stream);
      if (st != POLAR_OK) return st;
    }
    const long long rows = (long long)mp.B * mp.H * mp.Tq;
    if ((rows + 15) / 16 > INT32_MAX) return POLAR_ERR_UNSUPPORTED;
    st = launch(polar::polar_bwd_prep_kernel<D, CAUSAL>, dim3((unsigned)((rows + 15) / 16)), dim3(256), mp, stream);
    if (st != POLAR_OK) return st;
    mp.n_qt = (mp.Tq + kBwdWaves * 32 - 1) / (kBwdWaves * 32);
    const long long qblocks = (long long)mp.n_qt * mp.B * mp.H;
    if (qblocks > INT32_MAX) return POLAR_ERR_UNSUPPORTED;
    st = launch(polar::polar_bwd_dq_mfma_kernel<D, 64, kBwdWaves, CAUSAL>, dim3((unsigned)qblocks),
                dim3(kBwdWaves * 64), mp, stream);
    if (st != POLAR_OK) return st;
  }
  // with no query rows this writes zero dk and dv
  mp.n_kt = (mp.Tk + kBwdWaves * 32 - 1) / (kBwdWaves * 32);
  const long long kblocks = (long long)mp.n_kt * mp.B * mp.Hkv * mp.n_split;
  if (kblocks > INT32_MAX) return POLAR_ERR_UNSUPPORTED;
  // dk and dv in one kernel with 32-row query tiles at 2 waves per SIMD; at d = 128 the V
  // operand of G is read from the workgroup's V rows in LDS
  const dim3 grid((unsigned)kblocks), block(kBwdWaves * 64);
  st = launch(polar::polar_bwd_dkdv_mfma_kernel<D, 32, kBwdWaves, 2, CAUSAL, D == 128>, grid,
              block, mp, stream);
  if (st != POLAR_OK || mp.n_split == 1) return st;
  mp.part_n4 = (long long)mp.B * mp.Hkv * mp.Tk * D / 4;
  const long long blocks = std::min((2 * mp.part_n4 + 255) / 256, 8192ll);
  return launch(polar::polar_bwd_split_sum_kernel, dim3((unsigned)blocks), dim3(256), mp, stream);
}

template <int D, typename T, bool CAUSAL>
polar_status launch_bwd(const polar::BwdParams& bp, void* stream) {
  constexpr int kRows = polar::kBwdThreads / (D / 32);  // rows (or keys) per workgroup
  const dim3 block(polar::kBwdThreads);
  if (bp.Tq > 0) {
    const dim3 grid((bp.Tq + kRows - 1) / kRows, bp.B * bp.H);
    polar_status st = launch(polar::polar_bwd_rows_kernel<D, T, CAUSAL>, grid, block, bp, stream);
    if (st != POLAR_OK) return st;
    st = launch(polar::polar_bwd_dq_kernel<D, T, CAUSAL>, grid, block, bp, stream);
    if (st != POLAR_OK) return st;
  }
  // with no query rows this writes zero dk and dv
  const dim3 grid((bp.Tk + kRows - 1) / kRows, bp.B * bp.Hkv);
  return launch(polar::polar_bwd_dkdv_kernel<D, T, CAUSAL>, grid, block, bp, stream);
}

template <typename T>
polar_status dispatch_bwd(const polar_problem* pr, const polar::BwdParams& bp, void* stream) {
  if (pr->head_dim == 64)
    return pr->causal ? launch_bwd<64, T, true>(bp, stream) : launch_bwd<64, T, false>(bp, stream);
  return pr->causal ? launch_bwd<128, T, true>(bp, stream) : launch_bwd<128, T, false>(bp, stream);
}

// ---- no-allocation decode: the split partials live in a file-scope device array.
// Each GPU the library runs on holds its own copy of `scratch` until the process ends.
// In host code `scratch` names a host-side stand-in, never the device memory: the
// device address is taken once per device with hipGetSymbolAddress, with that device
// current, and only that address is handed to kernels.
__device__ __attribute__((aligned(256))) char scratch[POLAR_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// Device address of `scratch` on the device `stream` belongs to (the current device for
// the null stream), looked up on that device's first call.
polar_status scratch_on_stream_device(void* stream, void*& ptr) {
  int dev = -1;
  const hipError_t e = stream ? hipStreamGetDevice((hipStream_t)stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) return POLAR_ERR_HIP;
  if (dev >= kMaxDevices) return POLAR_ERR_UNSUPPORTED;
  std::call_once(g_scratch_once[dev], [dev]() {
    int cur = -1;
    hipError_t err = hipGetDevice(&cur);
    if (err == hipSuccess && cur != dev) err = hipSetDevice(dev);
    void* p = nullptr;
    if (err == hipSuccess) err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != dev) (void)hipSetDevice(cur);
    g_scratch_err[dev] = err;
    g_scratch_ptr[dev] = err == hipSuccess ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev]) return POLAR_ERR_HIP;
  ptr = g_scratch_ptr[dev];
  return POLAR_OK;
}

}  // namespace

extern "C" {

int32_t polar_abi_version(void) { return POLAR_ABI_VERSION; }

const char* polar_status_string(int32_t s) {
  // the argument is an int: a value outside polar_status is valid input here
  switch (s) {
    case POLAR_OK: return "ok";
    case POLAR_ERR_NULL_ARG: return "a required pointer is NULL";
    case POLAR_ERR_BAD_SHAPE: return "a size is negative or inconsistent";
    case POLAR_ERR_UNSUPPORTED: return "head_dim, dtype, head count or mode not supported";
    case POLAR_ERR_BAD_PARAM: return "non-finite or out-of-range tau, beta, kappa or softmax_scale";
    case POLAR_ERR_MISALIGNED: return "a pointer breaks the alignment rule";
    case POLAR_ERR_WORKSPACE: return "decode workspace missing or too small";
    case POLAR_ERR_ALIAS: return "an output overlaps an input or another output";
    case POLAR_ERR_HIP: return "the HIP runtime rejected a launch";
  }
  return "unknown status";
}

polar_status polar_attn_fwd(const polar_problem* pr, const void* q, const void* k, const void* v,
                            const polar_outputs* out, void* stream) {
  bool empty = false;
  polar_status st = check_shape(pr, empty);
  if (st != POLAR_OK) return st;
  FwdParams fp;
  std::memset(&fp, 0, sizeof(fp));
  st = head_params(pr, fp.hp, fp.hp_stride, fp.floor_on, fp.scale);
  if (st != POLAR_OK) return st;
  st = check_entry_variant(pr, fp.hp, Entry::kFwd, true);
  if (st != POLAR_OK) return st;
  if (!bf16_head_fits(pr, pr->seq_k)) return POLAR_ERR_UNSUPPORTED;
  if (empty) return POLAR_OK;  // no rows: pointers of empty tensors may be NULL
  if (!q || !k || !v) return POLAR_ERR_NULL_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16)) return POLAR_ERR_MISALIGNED;
  const size_t eb = elem_bytes(pr->dtype);
  const size_t qb = (size_t)pr->batch * pr->heads * pr->seq_q * pr->head_dim * eb;
  const size_t kvb = (size_t)pr->batch * pr->kv_heads * pr->seq_k * pr->head_dim * eb;
  const void* ins[3] = {q, k, v};
  const size_t in_bytes[3] = {qb, kvb, kvb};
  st = check_outputs(pr, out, ins, in_bytes, 3);
  if (st != POLAR_OK) return st;
  fp.q = q;
  fp.k = k;
  fp.v = v;
  fp.dir = out->direction;
  fp.neff = out->n_eff;
  fp.conf = out->confidence;
  fp.count = out->count;
  fp.stats = out->stats;
  fp.B = pr->batch;
  fp.H = pr->heads;
  fp.Hkv = pr->kv_heads;
  fp.Tq = pr->seq_q;
  fp.Tk = pr->seq_k;
  if (pr->head_dim == 64)
    return pr->causal ? launch_fwd<64, true>(pr, fp, stream) : launch_fwd<64, false>(pr, fp, stream);
  return pr->causal ? launch_fwd<128, true>(pr, fp, stream) : launch_fwd<128, false>(pr, fp, stream);
}

int32_t polar_attn_decode_num_splits(const polar_problem* pr, int32_t num_splits) {
  int splits = 0;
  if (check_decode(pr, num_splits, splits) != POLAR_OK) return 0;
  return splits;
}

size_t polar_attn_decode_workspace_bytes(const polar_problem* pr, int32_t num_splits) {
  int splits = 0;
  if (check_decode(pr, num_splits, splits) != POLAR_OK) return 0;
  return partial_bytes(pr, splits);
}

polar_status polar_attn_merge(const polar_problem* pr, const float* partials, int32_t num_splits,
                              const polar_outputs* out, void* stream) {
  return merge_with_lens(pr, partials, num_splits, nullptr, nullptr, out, stream);
}


// polar_attn_decode.  use_scratch: the partials go to the library's own device array
// (the no-allocation entry point), whose device address is looked up only after every
// check has passed; `workspace` is then ignored.
static polar_status decode_impl(const polar_problem* pr, const void* q, const void* k_cache, const void* v_cache,
                                int32_t num_splits, void* workspace, size_t workspace_bytes,
                                const polar_outputs* out, void* stream, bool use_scratch) {
  int splits = 0;
  polar_status st = check_decode(pr, num_splits, splits);
  if (st != POLAR_OK) return st;
  DecodeParams dp;
  std::memset(&dp, 0, sizeof(dp));
  int floor_on = 0;
  st = head_params(pr, dp.hp, dp.hp_stride, floor_on, dp.scale);
  if (st != POLAR_OK) return st;
  st = check_entry_variant(pr, dp.hp, Entry::kDecode, true);
  if (st != POLAR_OK) return st;
  if (pr->batch == 0 || pr->seq_q == 0) return POLAR_OK;  // no rows: pointers may be NULL
  if (!q || !k_cache || !v_cache) return POLAR_ERR_NULL_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16)) return POLAR_ERR_MISALIGNED;
  const size_t need = partial_bytes(pr, splits);
  if (use_scratch) {
    if (need > (size_t)POLAR_NOALLOC_SCRATCH_BYTES) return POLAR_ERR_WORKSPACE;
    workspace = nullptr;  // not an input of this call: the partials go to the library's array
  } else {
    if (need > 0 && (!workspace || workspace_bytes < need)) return POLAR_ERR_WORKSPACE;
    if (workspace && !aligned(workspace, 16)) return POLAR_ERR_MISALIGNED;
  }
  const size_t qb = (size_t)pr->batch * pr->heads * pr->seq_q * pr->head_dim * 2;
  const size_t kvb = (size_t)pr->batch * pr->kv_heads * pr->seq_k * pr->head_dim * 2;
  const void* ins[4] = {q, k_cache, v_cache, workspace};
  const size_t in_bytes[4] = {qb, kvb, kvb, need};
  st = check_outputs(pr, out, ins, in_bytes, 4);
  if (st != POLAR_OK) return st;
  if (overlaps(workspace, need, q, qb) || overlaps(workspace, need, k_cache, kvb) ||
      overlaps(workspace, need, v_cache, kvb))
    return POLAR_ERR_ALIAS;
  if (pr->heads > 65535 || pr->batch > 65535) return POLAR_ERR_UNSUPPORTED;
  if (use_scratch) {
    st = scratch_on_stream_device(stream, workspace);
    if (st != POLAR_OK) return st;
  }
  dp.q = q;
  dp.k = k_cache;
  dp.v = v_cache;
  dp.part = (float*)workspace;
  dp.B = pr->batch;
  dp.H = pr->heads;
  dp.Hkv = pr->kv_heads;
  dp.Tk = pr->seq_k;
  dp.S = splits;
  // the query sees the last min(window, seq_k) keys
  const int keys = dp.hp.window > 0 && dp.hp.window < pr->seq_k ? dp.hp.window : pr->seq_k;
  dp.key0 = pr->seq_k - keys;
  dp.split_len = (keys + splits - 1) / splits;
  const dim3 grid(splits, pr->heads, pr->batch);
  if (pr->heads > pr->kv_heads)  // grouped: every KV row is read once per group chunk
    st = launch_grouped_splits(pr, nullptr, q, k_cache, v_cache, splits, workspace, stream);
  else if (pr->head_dim == 64)
    st = launch_split<64>(dp, grid, stream);
  else
    st = launch_split<128>(dp, grid, stream);
  if (st != POLAR_OK) return st;
  return merge_with_lens(pr, (const float*)workspace, splits, nullptr, q, out, stream);
}

polar_status polar_attn_decode(const polar_problem* pr, const void* q, const void* k_cache, const void* v_cache,
                               int32_t num_splits, void* workspace, size_t workspace_bytes,
                               const polar_outputs* out, void* stream) {
  return decode_impl(pr, q, k_cache, v_cache, num_splits, workspace, workspace_bytes, out, stream, false);
}

polar_status polar_attn_decode_noalloc(const polar_problem* pr, const void* q, const void* k_cache,
                                       const void* v_cache, int32_t num_splits, const polar_outputs* out,
                                       void* stream) {
  return decode_impl(pr, q, k_cache, v_cache, num_splits, nullptr, 0, out, stream, true);
}

int32_t polar_attn_decode_paged_num_splits(const polar_problem* pr, const polar_paged_kv* kv, int32_t num_splits) {
  int splits = 0;
  if (!pr || check_paged(pr, kv, num_splits, splits) != POLAR_OK) return 0;
  return splits;
}

size_t polar_attn_decode_paged_workspace_bytes(const polar_problem* pr, const polar_paged_kv* kv,
                                               int32_t num_splits) {
  int splits = 0;
  if (!pr || check_paged(pr, kv, num_splits, splits) != POLAR_OK) return 0;
  return partial_bytes(pr, splits);
}

polar_status polar_attn_decode_paged(const polar_problem* pr, const void* q, const polar_paged_kv* kv,
                                     int32_t num_splits, void* workspace, size_t workspace_bytes,
                                     const polar_outputs* out, void* stream) {
  if (!pr) return POLAR_ERR_NULL_ARG;
  int splits = 0;
  polar_status st = check_paged(pr, kv, num_splits, splits);
  if (st != POLAR_OK) return st;
  {
    HeadParams hp;
    int stride = 0, floor_on = 0;
    float scale = 0.0f;
    st = head_params(pr, hp, stride, floor_on, scale);
    if (st != POLAR_OK) return st;
    st = check_entry_variant(pr, hp, Entry::kDecode, true);
    if (st != POLAR_OK) return st;
  }
  if (pr->batch == 0 || pr->seq_q == 0) return POLAR_OK;  // no rows: pointers may be NULL
  if (!q || !kv->k_pool || !kv->v_pool || !kv->block_table || !kv->seq_lens) return POLAR_ERR_NULL_ARG;
  if (!aligned(q, 16) || !aligned(kv->k_pool, 16) || !aligned(kv->v_pool, 16) || !aligned(kv->block_table, 4) ||
      !aligned(kv->seq_lens, 4))
    return POLAR_ERR_MISALIGNED;
  const size_t need = partial_bytes(pr, splits);
  if (!workspace || workspace_bytes < need) return POLAR_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return POLAR_ERR_MISALIGNED;
  const size_t qb = (size_t)pr->batch * pr->heads * pr->head_dim * 2;
  const size_t pool_b = (size_t)kv->num_blocks * kv->block_size * pr->kv_heads * pr->head_dim * 2;
  const size_t tab_b = (size_t)pr->batch * kv->max_blocks * 4;
  const size_t len_b = (size_t)pr->batch * 4;
  const void* ins[6] = {q, kv->k_pool, kv->v_pool, kv->block_table, kv->seq_lens, workspace};
  const size_t in_bytes[6] = {qb, pool_b, pool_b, tab_b, len_b, need};
  st = check_outputs(pr, out, ins, in_bytes, 6);
  if (st != POLAR_OK) return st;
  for (int i = 0; i < 5; ++i)
    if (overlaps(workspace, need, ins[i], in_bytes[i])) return POLAR_ERR_ALIAS;
  st = launch_grouped_splits(pr, kv, q, kv->k_pool, kv->v_pool, splits, workspace, stream);
  if (st != POLAR_OK) return st;
  polar_problem flat = *pr;
  flat.causal = 0;
  return merge_with_lens(&flat, (const float*)workspace, splits, kv->seq_lens, q, out, stream);
}

polar_status polar_attn_fwd_partial(const polar_problem* pr, const void* q, const void* k, const void* v,
                                    int32_t context_k, float* partials, int32_t num_splits, int32_t split,
                                    void* stream) {
  bool empty = false;
  polar_status st = check_shape(pr, empty);
  if (st != POLAR_OK) return st;
  FwdParams fp;
  std::memset(&fp, 0, sizeof(fp));
  st = head_params(pr, fp.hp, fp.hp_stride, fp.floor_on, fp.scale);
  if (st != POLAR_OK) return st;
  st = check_entry_variant(pr, fp.hp, Entry::kPartial, true);
  if (st != POLAR_OK) return st;
  if (!bf16_head_fits(pr, pr->seq_k)) return POLAR_ERR_UNSUPPORTED;
  if (num_splits < 1 || split < 0 || split >= num_splits) return POLAR_ERR_BAD_SHAPE;
  if (context_k != 0) {
    if (context_k < pr->seq_q || context_k < 0) return POLAR_ERR_BAD_SHAPE;
    // the temperature must stay positive at the longest context count
    const int nh = pr->len_temp && fp.hp.lam_form == POLAR_TEMP_LOG ? pr->heads : 0;
    for (int h = 0; h < nh; ++h)
      if (!(1.0 + (double)pr->len_temp[h] * std::log((double)context_k) > 0.0)) return POLAR_ERR_BAD_PARAM;
  }
  if (empty) return POLAR_OK;  // no rows: pointers of empty tensors may be NULL
  if (!q || !k || !v || !partials) return POLAR_ERR_NULL_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16)) return POLAR_ERR_MISALIGNED;
  if (!aligned(partials, 4)) return POLAR_ERR_MISALIGNED;
  const size_t eb = elem_bytes(pr->dtype);
  const size_t qb = (size_t)pr->batch * pr->heads * pr->seq_q * pr->head_dim * eb;
  const size_t kvb = (size_t)pr->batch * pr->kv_heads * pr->seq_k * pr->head_dim * eb;
  const size_t pb = partial_bytes(pr, num_splits);
  if (overlaps(partials, pb, q, qb) || overlaps(partials, pb, k, kvb) || overlaps(partials, pb, v, kvb))
    return POLAR_ERR_ALIAS;
  fp.q = q;
  fp.k = k;
  fp.v = v;
  fp.part = partials;
  fp.part_S = num_splits;
  fp.part_s = split;
  fp.ctx_k = context_k;
  fp.B = pr->batch;
  fp.H = pr->heads;
  fp.Hkv = pr->kv_heads;
  fp.Tq = pr->seq_q;
  fp.Tk = pr->seq_k;
  if (pr->head_dim == 64)
    return pr->causal ? launch_fwd<64, true>(pr, fp, stream) : launch_fwd<64, false>(pr, fp, stream);
  return pr->causal ? launch_fwd<128, true>(pr, fp, stream) : launch_fwd<128, false>(pr, fp, stream);
}

size_t polar_attn_bwd_workspace_bytes(const polar_problem* pr) {
  bool empty = false;
  if (check_shape(pr, empty) != POLAR_OK) return 0;
  return bwd_workspace(pr);
}

size_t polar_attn_bwd_saved_workspace_bytes(const polar_problem* pr) {
  bool empty = false;
  if (check_shape(pr, empty) != POLAR_OK || pr->dtype != POLAR_BF16) return 0;
  return bwd_workspace(pr, true);
}

// Both backward entry points.  use_saved: the rows' forward statistics come from `saved`
// ([rows, D + 3] fp32, bf16 inputs only) instead of a forward pass inside the call.
static polar_status bwd_entry(const polar_problem* pr, const void* q, const void* k, const void* v,
                              const float* saved, bool use_saved, const polar_grads* g, float* dq, float* dk,
                              float* dv, void* workspace, size_t workspace_bytes, void* stream) {
  bool empty = false;
  polar_status st = check_shape(pr, empty);
  if (st != POLAR_OK) return st;
  polar::BwdParams bp;
  std::memset(&bp, 0, sizeof(bp));
  st = head_params(pr, bp.hp, bp.hp_stride, bp.floor_on, bp.scale);
  if (st != POLAR_OK) return st;
  st = check_entry_variant(pr, bp.hp, Entry::kBwd, true);
  if (st != POLAR_OK) return st;
  if (!bf16_head_fits(pr, pr->seq_k) || !bf16_head_fits(pr, pr->seq_q)) return POLAR_ERR_UNSUPPORTED;
  if (use_saved && pr->dtype != POLAR_BF16) return POLAR_ERR_UNSUPPORTED;
  if (!g) return POLAR_ERR_NULL_ARG;
  if (pr->batch == 0) return POLAR_OK;  // nothing to write
  // fp32 path: the grid's second dimension holds (batch, head) pairs
  if (pr->dtype == POLAR_F32 && (int64_t)pr->batch * pr->heads > 65535) return POLAR_ERR_UNSUPPORTED;
  const bool rows = pr->seq_q > 0;
  const size_t ws = bwd_workspace(pr, use_saved);
  if (!k || !v || !dk || !dv) return POLAR_ERR_NULL_ARG;
  if (rows && (!q || !dq)) return POLAR_ERR_NULL_ARG;
  if (rows && use_saved && !saved) return POLAR_ERR_NULL_ARG;
  if (ws > 0 && !workspace) return POLAR_ERR_WORKSPACE;
  if (workspace_bytes < ws) return POLAR_ERR_WORKSPACE;
  const void* a16[] = {q, k, v, dq, dk, dv, workspace, g->d_direction, saved};
  for (const void* ptr : a16)
    if (!aligned(ptr, 16)) return POLAR_ERR_MISALIGNED;
  if (!aligned(g->d_n_eff, 4) || !aligned(g->d_confidence, 4) || !aligned(g->d_count, 4))
    return POLAR_ERR_MISALIGNED;
  const size_t eb = elem_bytes(pr->dtype);
  const size_t nq = (size_t)pr->batch * pr->heads * pr->seq_q;
  const size_t nk = (size_t)pr->batch * pr->kv_heads * pr->seq_k;
  const size_t D = pr->head_dim;
  const void* ins[8] = {q, k, v, g->d_direction, g->d_n_eff, g->d_confidence, g->d_count, saved};
  const size_t in_bytes[8] = {nq * D * eb, nk * D * eb, nk * D * eb, nq * D * 4, nq * 4, nq * 4, nq * 4,
                              nq * (D + 3) * 4};
  const void* outs[4] = {dq, dk, dv, workspace};
  const size_t out_bytes[4] = {nq * D * 4, nk * D * 4, nk * D * 4, ws};
  for (int o = 0; o < 4; ++o) {
    for (int i = 0; i < 8; ++i)
      if (overlaps(outs[o], out_bytes[o], ins[i], in_bytes[i])) return POLAR_ERR_ALIAS;
    for (int o2 = o + 1; o2 < 4; ++o2)
      if (overlaps(outs[o], out_bytes[o], outs[o2], out_bytes[o2])) return POLAR_ERR_ALIAS;
  }
  if (pr->dtype == POLAR_BF16) {
    const size_t part_b = use_saved ? 0 : align256(nq * (D + 3) * 4);
    const size_t w_b = align256(nq * D * 2);
    char* base = static_cast<char*>(workspace);
    polar::BwdMfmaParams mp;
    std::memset(&mp, 0, sizeof(mp));
    mp.q = static_cast<const __bf16*>(q);
    mp.k = static_cast<const __bf16*>(k);
    mp.v = static_cast<const __bf16*>(v);
    mp.part = !rows ? nullptr : use_saved ? saved : reinterpret_cast<const float*>(base);
    mp.g_dir = g->d_direction;
    mp.g_neff = g->d_n_eff;
    mp.g_conf = g->d_confidence;
    mp.g_count = g->d_count;
    mp.W = rows ? reinterpret_cast<__bf16*>(base + part_b) : nullptr;
    mp.R = rows ? reinterpret_cast<polar::f32x4*>(base + part_b + w_b) : nullptr;
    mp.n_split = bwd_splits(pr);
    if (mp.n_split > 1) {
      const size_t split_b = align256((size_t)mp.n_split * nk * D * 4);
      mp.dk_part = reinterpret_cast<float*>(base + part_b + w_b + align256(nq * 16));
      mp.dv_part = reinterpret_cast<float*>(base + part_b + w_b + align256(nq * 16) + split_b);
    }
    mp.dq = dq;
    mp.dk = dk;
    mp.dv = dv;
    mp.B = pr->batch;
    mp.H = pr->heads;
    mp.Hkv = pr->kv_heads;
    mp.Tq = pr->seq_q;
    mp.Tk = pr->seq_k;
    mp.floor_on = bp.floor_on;
    mp.hp_stride = bp.hp_stride;
    mp.scale = bp.scale;
    mp.hp = bp.hp;
    // the forward in partial mode writes every row's (m, S1, S2, acc) into the workspace
    FwdParams fp;
    std::memset(&fp, 0, sizeof(fp));
    fp.q = q;
    fp.k = k;
    fp.v = v;
    fp.part = reinterpret_cast<float*>(base);
    fp.part_S = 1;
    fp.part_s = 0;
    fp.B = pr->batch;
    fp.H = pr->heads;
    fp.Hkv = pr->kv_heads;
    fp.Tq = pr->seq_q;
    fp.Tk = pr->seq_k;
    fp.floor_on = bp.floor_on;
    fp.hp_stride = bp.hp_stride;
    fp.scale = bp.scale;
    fp.hp = bp.hp;
    const bool run_fwd = !use_saved;
    if (pr->head_dim == 64)
      return pr->causal ? launch_bwd_mfma<64, true>(pr, fp, mp, run_fwd, stream)
                        : launch_bwd_mfma<64, false>(pr, fp, mp, run_fwd, stream);
    return pr->causal ? launch_bwd_mfma<128, true>(pr, fp, mp, run_fwd, stream)
                      : launch_bwd_mfma<128, false>(pr, fp, mp, run_fwd, stream);
  }
  bp.q = q;
  bp.k = k;
  bp.v = v;
  bp.g_dir = g->d_direction;
  bp.g_neff = g->d_n_eff;
  bp.g_conf = g->d_confidence;
  bp.g_count = g->d_count;
  bp.W = static_cast<float*>(workspace);
  bp.R = rows ? static_cast<float*>(workspace) + nq * D : nullptr;
  bp.dq = dq;
  bp.dk = dk;
  bp.dv = dv;
  bp.B = pr->batch;
  bp.H = pr->heads;
  bp.Hkv = pr->kv_heads;
  bp.Tq = pr->seq_q;
  bp.Tk = pr->seq_k;
  return dispatch_bwd<float>(pr, bp, stream);
}

polar_status polar_attn_bwd(const polar_problem* pr, const void* q, const void* k, const void* v,
                            const polar_grads* g, float* dq, float* dk, float* dv, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return bwd_entry(pr, q, k, v, nullptr, false, g, dq, dk, dv, workspace, workspace_bytes, stream);
}

polar_status polar_attn_bwd_saved(const polar_problem* pr, const void* q, const void* k, const void* v,
                                  const float* saved, const polar_grads* g, float* dq, float* dk, float* dv,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_entry(pr, q, k, v, saved, true, g, dq, dk, dv, workspace, workspace_bytes, stream);
}

}  // extern "C"
