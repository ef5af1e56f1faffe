/*
 * polar_attn.h - C ABI of the Polar Attention library for AMD Instinct MI355X (gfx950).
 *
 * The operator is the fused Polar Attention forward of ATMA, as described in the
 * technical summary "ATMA: Length-Invariant Language Modeling via Polar Attention and
 * Gated-Delta Compression Memory" (gist.science, paper 2606.25156), cited below as
 * [ATMA §x]:
 *   - the direction channel projects the attention-weighted sum of the values onto the
 *     unit sphere, with a per-head length temperature that sharpens the logits as the
 *     context grows and an extreme-value-corrected null floor that calibrates them
 *     against noise [ATMA §2.1, direction channel];
 *   - the magnitude channel is the participation ratio (inverse Simpson index)
 *     n_eff = (sum p)^2 / sum p^2 of the attention weights, gated by the confidence of
 *     signal detection and mapped through a bounded saturating tanh-of-log
 *     [ATMA §2.1, magnitude channel];
 *   - the fused kernel streams the running sums with squared correction factors and
 *     never holds the T x T score matrix; decode reads the KV cache directly
 *     [ATMA §2.2, hardware-software co-design].
 *
 * Per batch b, head h and query row i (query head h reads key/value head
 * h / (heads / kv_heads)):
 *   n_i   = keys visible to row i: i + 1 + (seq_k - seq_q) when causal, seq_k otherwise
 *   lam_i = 1 + tau_h ln n_i                          (length temperature)
 *   s_ij  = lam_i * softmax_scale * <q_i, k_j>,   m_i = max_j s_ij,   p_ij = exp(s_ij - m_i)
 *   S1    = sum_j p_ij,   S2 = sum_j p_ij^2,   acc = sum_j p_ij v_j
 *   direction = acc / ||acc||_2 (zero vector when acc == 0),   n_eff = S1^2 / S2
 *   null floor f_i = lam_i sqrt(2 ln n_i) + beta_h;  confidence = S1 / (S1 + exp(f_i - m_i))
 *              (confidence = 1 when the floor is off)
 *   count = confidence * tanh(ln(n_eff) / kappa_h)
 * The exact forms of the temperature, floor, confidence and saturation are readings
 * of the summary, which names these parts without formulas.
 *
 * Conventions shared by every entry point
 *   Layout     q [B, heads, seq_q, head_dim], k and v [B, kv_heads, seq_k, head_dim],
 *              contiguous row-major.  Outputs are contiguous fp32.
 *   Pointers   "DEVICE" pointers are HIP device memory owned by the caller; "HOST"
 *              pointers are read during the call only.  q, k, v, direction and
 *              workspace must be 16-byte aligned; other outputs 4-byte aligned.
 *              Outputs must not overlap the inputs.
 *   Streams    `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *              enqueues work; results are valid once the caller synchronises the stream.
 *   Memory     The library allocates nothing.  Its only mutable global state is the
 *              per-device address of the array polar_attn_decode_noalloc uses, set
 *              once per device on first use.  Calls on different streams may run
 *              concurrently, except polar_attn_decode_noalloc calls on one GPU.
 *   Errors     All argument checks run before the first HIP call; a call rejected by
 *              them (any status but POLAR_OK and POLAR_ERR_HIP) has enqueued nothing.
 *              POLAR_ERR_HIP is the failure of a kernel launch as the launch itself
 *              reports it (an error an unrelated HIP call left on the thread is neither
 *              reported nor cleared); kernels the call launched before the failing one
 *              stay enqueued.  Faults inside a kernel surface at the caller's next
 *              synchronisation.
 *   Empty      batch == 0 or seq_q == 0 is valid and enqueues nothing; the data
 *              pointers of such a call may be NULL (polar_attn_bwd with seq_q == 0
 *              still writes zero dk and dv).
 *   Values     The operator is defined for finite q, k, v; the library does not
 *              inspect values.  A NaN propagates through the forward and decode entry
 *              points: a NaN in q_i makes every output channel of row i NaN; one in
 *              k_j, every channel of every row that sees key j; one in v_j, the
 *              direction of every row that sees key j, and possibly the direction of
 *              earlier rows computed in the same query tile (a zero weight times NaN),
 *              while n_eff, confidence and count do not depend on v.  In the
 *              statistics of an affected row S1 and S2 are NaN and m is unspecified.
 *              Every other row is exactly what it is without the NaN.  Infinite inputs
 *              give unspecified values in the rows they reach and leave the other rows
 *              unchanged.  The backward entry points make no statement on them.
 */
#ifndef POLAR_ATTN_H
#define POLAR_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define POLAR_ABI_VERSION 7
/* Per-head parameter tables (len_temp, null_bias, count_scale) are supported up to
 * this many heads; with all three tables NULL any head count is accepted. */
#define POLAR_MAX_PARAM_HEADS 128

typedef enum polar_status {
  POLAR_OK = 0,
  POLAR_ERR_NULL_ARG = 1,     /* a required pointer is NULL                                */
  POLAR_ERR_BAD_SHAPE = 2,    /* a size is negative or inconsistent                        */
  POLAR_ERR_UNSUPPORTED = 3,  /* head_dim, dtype, head count or mode not built             */
  POLAR_ERR_BAD_PARAM = 4,    /* non-finite or out-of-range tau, beta, kappa or scale      */
  POLAR_ERR_MISALIGNED = 5,   /* a pointer breaks the alignment rule                       */
  POLAR_ERR_WORKSPACE = 6,    /* decode workspace missing or too small                     */
  POLAR_ERR_ALIAS = 7,        /* an output overlaps an input                               */
  POLAR_ERR_HIP = 8           /* the HIP runtime rejected a launch                         */
} polar_status;

typedef enum polar_dtype {
  POLAR_BF16 = 0,             /* bf16 q, k, v; fp32 accumulation                           */
  POLAR_F32 = 1               /* fp32 q, k, v; fp32 arithmetic throughout                  */
} polar_dtype;

/* Reading variants.  The summary names the length temperature, the extreme-value-
 * corrected null floor, the confidence gate and the saturation without formulas
 * [ATMA §2.1], and its ablation compares sliding-window attention [ATMA §3.1].  The
 * definition above is one reading of each (reading R, all fields 0); these select
 * alternatives.  n below is the row's visible count.
 *   temperature  POLAR_TEMP_LOG          lam = 1 + tau_h ln n                 (reading R)
 *                POLAR_TEMP_SSMAX        lam = tau_h ln n      (tau_h >= 0)
 *                POLAR_TEMP_TRAIN_RATIO  lam = ln n / ln train_len (train_len >= 2; tau unused)
 *   floor_level  POLAR_LEVEL_GAUSS       l(n) = sqrt(2 ln n)                  (reading R)
 *                POLAR_LEVEL_GUMBEL2     l(n) = b_n + gamma a_n, the second-order expected
 *                                        maximum of n standard normals, r = sqrt(2 ln n),
 *                                        b_n = r - (ln ln n + ln 4 pi) / (2 r), a_n = 1 / r
 *                POLAR_LEVEL_QNORM       l(n) = sqrt(2 ln n) scaled by sigma_i =
 *                                        softmax_scale ||q_i||_2 (the spread of the row's
 *                                        raw logits for unit-variance keys)
 *                the floor is f_i = lam_i sigma_i l(n_i) + beta_h (sigma_i = 1 unless QNORM;
 *                l(1) = 0)
 *   key_floor    POLAR_KEY_FLOOR_NULL    the floor is a null slot in the normaliser (R)
 *                POLAR_KEY_FLOOR_SOFT    each key's weight is max(e^{s_ij} - e^{f_i}, 0)
 *                POLAR_KEY_FLOOR_GATE    each key's weight is e^{s_ij} when s_ij > f_i, else 0
 *                S1, S2 and acc sum the floored weights; confidence = S1 / (S1 + e^{f - m});
 *                a row with no weight left gets a zero direction and zero n_eff,
 *                confidence and count.  Needs null_bias (the floor on).
 *   saturation   POLAR_SAT_LOG           count = conf tanh(ln n_eff / kappa)  (reading R)
 *                POLAR_SAT_LOG1P         count = conf tanh(ln(1 + n_eff) / kappa)
 *   window       0 = none; W > 0: key j is visible to row i iff
 *                i + seq_k - seq_q - W < j <= i + seq_k - seq_q, so n_i = min(W, causal count)
 *                (prefill needs causal; decode sees the last W keys of each sequence).
 * Where an entry point does not support a variant it returns POLAR_ERR_UNSUPPORTED;
 * an enum value out of range is POLAR_ERR_UNSUPPORTED, a negative window or a
 * train_len < 2 with POLAR_TEMP_TRAIN_RATIO is POLAR_ERR_BAD_PARAM. */
typedef enum polar_temperature_form {
  POLAR_TEMP_LOG = 0,
  POLAR_TEMP_SSMAX = 1,
  POLAR_TEMP_TRAIN_RATIO = 2
} polar_temperature_form;

typedef enum polar_floor_level {
  POLAR_LEVEL_GAUSS = 0,
  POLAR_LEVEL_GUMBEL2 = 1,
  POLAR_LEVEL_QNORM = 2
} polar_floor_level;

typedef enum polar_key_floor {
  POLAR_KEY_FLOOR_NULL = 0,
  POLAR_KEY_FLOOR_SOFT = 1,
  POLAR_KEY_FLOOR_GATE = 2
} polar_key_floor;

typedef enum polar_saturation {
  POLAR_SAT_LOG = 0,
  POLAR_SAT_LOG1P = 1
} polar_saturation;

typedef struct polar_variant {
  int32_t temperature;        /* polar_temperature_form                                     */
  int32_t train_len;          /* L of POLAR_TEMP_TRAIN_RATIO                                 */
  int32_t floor_level;        /* polar_floor_level                                          */
  int32_t key_floor;          /* polar_key_floor                                            */
  int32_t saturation;         /* polar_saturation                                           */
  int32_t window;             /* sliding window in keys, 0 = none                           */
} polar_variant;

typedef struct polar_problem {
  int32_t batch;              /* B >= 0                                                     */
  int32_t heads;              /* query heads >= 1                                           */
  int32_t kv_heads;           /* key/value heads >= 1, heads % kv_heads == 0                */
  int32_t seq_q;              /* query rows >= 0                                            */
  int32_t seq_k;              /* keys >= 1; causal requires seq_q <= seq_k                  */
  int32_t head_dim;           /* 64 or 128                                                  */
  int32_t causal;             /* nonzero: key j visible to row i iff j <= i + seq_k - seq_q */
  int32_t dtype;              /* a polar_dtype                                              */
  float softmax_scale;        /* <= 0 selects 1/sqrt(head_dim); must be finite              */
  const float* len_temp;      /* HOST [heads] tau_h, NULL = 0; needs 1 + tau_h ln(seq_k) > 0 */
  const float* null_bias;     /* HOST [heads] beta_h (finite), NULL = null floor off        */
  const float* count_scale;   /* HOST [heads] kappa_h > 0, NULL = 1                          */
  const polar_variant* variant; /* HOST, NULL = reading R (the definition above)             */
} polar_problem;

typedef struct polar_outputs {
  float* direction;           /* DEVICE [B, heads, seq_q, head_dim], required               */
  float* n_eff;               /* DEVICE [B, heads, seq_q], required                          */
  float* confidence;          /* DEVICE [B, heads, seq_q], optional (NULL = not written)     */
  float* count;               /* DEVICE [B, heads, seq_q], optional                          */
  float* stats;               /* DEVICE [B, heads, seq_q, 3] = (m, S1, S2), optional; m is the
                                 row maximum of the tempered logits in natural-log units and
                                 S1, S2 are taken relative to it                             */
} polar_outputs;

/* Fused Polar Attention forward (prefill) [ATMA §2.2, fused kernel].
 * One pass over the visible keys per query tile: tiled Q K^T and P V on the matrix
 * cores with an online softmax that also streams sum p^2 (rescaled by the square of
 * each correction factor).  Supports bf16 and fp32, head_dim 64 and 128, causal and
 * non-causal, seq_q <= seq_k when causal (rows aligned to the end of the keys).  Every
 * reading variant (a sliding window needs causal).  bf16: one head's K (and V) of
 * seq_k * head_dim * 2 bytes plus 64 KiB must fit the 32-bit range of the kernel's buffer
 * loads (seq_k <= 16,776,959 at head_dim 128, 33,553,919 at 64); beyond it
 * POLAR_ERR_UNSUPPORTED. */
polar_status polar_attn_fwd(const polar_problem* problem, const void* q, const void* k,
                            const void* v, const polar_outputs* out, void* stream);

/* Partial forward for chunked prefill [ATMA §2.2: the streaming statistics of disjoint
 * key ranges merge with weights w and w^2].  Same inputs and masking as polar_attn_fwd
 * (causal: key j of this call visible to row i iff j <= i + seq_k - seq_q), but instead
 * of the channels it writes, for every query row, the statistics (m, S1, S2, acc) of the
 * keys of this call into slot `split` of DEVICE `partials` [B, heads, seq_q, num_splits,
 * head_dim + 3] fp32 (the layout polar_attn_merge reads; m in natural-log units, S1, S2
 * and acc relative to exp(m)).  context_k > 0 says this call is one piece of a causal
 * context of context_k keys ending at the last query row: the length temperature of row
 * i then uses that context's visible count i + 1 + context_k - seq_q, so pieces computed
 * separately (a cached prefix without mask, the new chunk with the causal mask) merge
 * into exactly what one pass over the whole context computes; merge them with a
 * problem of seq_k = context_k, causal.  context_k = 0 uses the row's own visible count.
 * Requires context_k >= seq_q when nonzero and 1 + tau_h ln(context_k) > 0.  Slots other
 * than `split` are not touched; a slot that never receives a piece must hold m = -inf.
 * Reading variants: all but a sliding window and POLAR_LEVEL_QNORM (the merge that
 * finishes the pieces has no queries); a per-key floor uses the floor of the row's count
 * in the whole context.  The same bf16 size limit as polar_attn_fwd. */
polar_status polar_attn_fwd_partial(const polar_problem* problem, const void* q, const void* k, const void* v,
                                    int32_t context_k, float* partials, int32_t num_splits, int32_t split,
                                    void* stream);

/* Split count the decode will use for `num_splits` (0 = automatic choice); 0 when the
 * problem is invalid for decode. */
int32_t polar_attn_decode_num_splits(const polar_problem* problem, int32_t num_splits);

/* Bytes of device workspace polar_attn_decode needs for `num_splits` (0 = automatic):
 * the per-split partials [B, heads, seq_q, S, head_dim + 3] fp32.  0 when the problem
 * is invalid for decode. */
size_t polar_attn_decode_workspace_bytes(const polar_problem* problem, int32_t num_splits);

/* Split-KV decode [ATMA §2.2, decode kernel].  Requires seq_q == 1 (one new query per
 * sequence) and bf16.  The cache of seq_k keys is cut into S contiguous splits; one
 * kernel writes the statistics (m, S1, S2, acc) of every split into `workspace` (layout
 * as for polar_attn_merge), and a second kernel on the same stream merges them with
 * the global visible count n = seq_k.  1 <= num_splits <= seq_k, or 0 for automatic.
 * When heads > kv_heads, a workgroup serves up to 8 query heads of a group and reads
 * each K and V row once for all of them.  Every reading variant; a sliding window of W
 * keys keeps the last min(W, seq_k) keys (n = that count). */
polar_status polar_attn_decode(const polar_problem* problem, const void* q, const void* k_cache,
                               const void* v_cache, int32_t num_splits, void* workspace,
                               size_t workspace_bytes, const polar_outputs* out, void* stream);

/* Size of the device array the no-allocation decode keeps its split partials in: one
 * array per GPU, held from the first call on that GPU until the process ends. */
#define POLAR_NOALLOC_SCRATCH_BYTES (8u << 20)

/* Split-KV decode that allocates nothing, for callers that cannot call hipMalloc or
 * take a workspace: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same problem rules, arguments, kernels and results as
 * polar_attn_decode (bitwise equal for the same num_splits), but the per-split partials
 * go to a library-owned device array of POLAR_NOALLOC_SCRATCH_BYTES bytes on the GPU
 * that `stream` belongs to (the current device for the NULL stream), instead of a
 * caller workspace.  Partials above that size ([B, heads, S, head_dim + 3] fp32 for the
 * split count S the call uses) are rejected with POLAR_ERR_WORKSPACE before any HIP
 * call.  The first call on a GPU looks up the array's device address (briefly making
 * that GPU current if it is not); a failure of that lookup is POLAR_ERR_HIP.  Every
 * call on one GPU shares that GPU's array, which keeps the last call's contents: calls
 * that overlap on one GPU (concurrent streams, or host threads) race and must be
 * serialised by the caller.  No call needs the array cleared: every partial row is
 * written before it is read. */
polar_status polar_attn_decode_noalloc(const polar_problem* problem, const void* q, const void* k_cache,
                                       const void* v_cache, int32_t num_splits, const polar_outputs* out,
                                       void* stream);

/* Paged KV cache for polar_attn_decode_paged.  The keys of sequence b are stored in
 * blocks of block_size rows: block_table[b * max_blocks + j] is the pool block holding
 * keys [j * block_size, (j + 1) * block_size) of that sequence.  k_pool and v_pool are
 * DEVICE [num_blocks, block_size, kv_heads, head_dim] bf16, contiguous, 16-byte
 * aligned.  block_table is DEVICE int32 [batch, max_blocks]; seq_lens is DEVICE int32
 * [batch], the number of cached keys of each sequence.  Both are read by the kernels
 * only (the call never waits for them): a length outside [0, problem->seq_k] is clamped
 * into it, and a table entry outside [0, num_blocks) is never dereferenced -- its keys
 * are skipped, and the results of that sequence are then unspecified.  A sequence with
 * no keys gets a zero direction and zero n_eff, confidence and count. */
typedef struct polar_paged_kv {
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  const int32_t* seq_lens;
  int32_t num_blocks;         /* >= 1                                                       */
  int32_t block_size;         /* a power of two, 1 .. 1024                                  */
  int32_t max_blocks;         /* table columns; max_blocks * block_size >= problem->seq_k   */
} polar_paged_kv;

/* Split count and workspace bytes polar_attn_decode_paged uses for `num_splits`
 * (0 = automatic); 0 when the call is invalid. */
int32_t polar_attn_decode_paged_num_splits(const polar_problem* problem, const polar_paged_kv* kv,
                                           int32_t num_splits);
size_t polar_attn_decode_paged_workspace_bytes(const polar_problem* problem, const polar_paged_kv* kv,
                                               int32_t num_splits);

/* Grouped split-KV decode over a paged cache [ATMA §2.2, decode kernel; grouped-query
 * attention reads each KV row once per group].  Requires seq_q == 1 and bf16; q is
 * DEVICE [batch, heads, head_dim].  problem->seq_k is the largest sequence length the
 * call may see (it sizes the splits); causal is ignored: each query sees every cached
 * key of its sequence, and its visible count n is that sequence's length.  One
 * workgroup serves a (sequence, KV head, split) and up to 8 query heads of the group,
 * loading each K and V row once for all of them.  Writes the same per-split partials
 * as polar_attn_decode into `workspace` ([batch, heads, S, head_dim + 3] fp32) and then
 * merges them on the same stream.  Every reading variant; a sliding window of W keys
 * keeps the last min(W, length) keys of each sequence (n = that count). */
polar_status polar_attn_decode_paged(const polar_problem* problem, const void* q, const polar_paged_kv* kv,
                                     int32_t num_splits, void* workspace, size_t workspace_bytes,
                                     const polar_outputs* out, void* stream);

/* Merge of split statistics [ATMA §2.2: streaming accumulators with squared correction
 * factors].  partials: DEVICE [B, heads, seq_q, num_splits, head_dim + 3] fp32, each row
 * (m, S1, S2, acc[head_dim]) with m in natural-log units and S1, S2, acc relative to
 * exp(m); a split with no keys has m = -inf.  Each split is brought to the common
 * maximum m* with w = exp(m_s - m*) (S1 and acc scale by w, S2 by w^2), then the
 * channels are formed with the visible count of the problem's row i (seq_k when not
 * causal, i + 1 + seq_k - seq_q when causal; min(W, that count) under a sliding window of
 * W keys).  dtype is ignored.  Reading variants: all but POLAR_LEVEL_QNORM, which needs
 * the queries (POLAR_ERR_UNSUPPORTED). */
polar_status polar_attn_merge(const polar_problem* problem, const float* partials,
                              int32_t num_splits, const polar_outputs* out, void* stream);

/* Upstream gradients of the four forward channels for polar_attn_bwd.  Each is a DEVICE
 * fp32 array laid out like the matching forward output (d_direction [B, heads, seq_q,
 * head_dim], 16-byte aligned; the others [B, heads, seq_q], 4-byte aligned); NULL means
 * zero. */
typedef struct polar_grads {
  const float* d_direction;
  const float* d_n_eff;
  const float* d_confidence;
  const float* d_count;
} polar_grads;

/* Bytes of device workspace polar_attn_bwd needs.  fp32 inputs: B * heads * seq_q *
 * (head_dim + 4) fp32 (per query row, the vector w and four row constants).  bf16 inputs:
 * per query row the forward's statistics (head_dim + 3 fp32), w (head_dim bf16) and four
 * row constants (fp32), in three parts each padded to 256 bytes; then, when the key
 * side's work is split into n > 1 runs per 128-key tile, n partial dk and n partial dv
 * (n * B * kv_heads * seq_k * head_dim fp32 each, padded to 256 bytes).  n depends on the
 * shape only: for B * kv_heads * ceil(seq_k / 128) = t key tiles, n = ceil(2048 / t)
 * (causal) or ceil(512 / t) (full mask), clamped to [1, 4 * heads / kv_heads].  0 when
 * the problem is invalid (or has no query rows). */
size_t polar_attn_bwd_workspace_bytes(const polar_problem* problem);

/* Backward of polar_attn_fwd: the gradients of
 *   L = sum d_direction . direction + sum d_n_eff n_eff + sum d_confidence confidence
 *       + sum d_count count
 * with respect to q, k and v, by the chain rule through the definition above (the ATMA
 * summary trains with the operator [ATMA §3] but gives no backward; the length
 * temperature and the null floor depend on the visible count only, so they carry no
 * gradient).  Per row i, with weights p_ij = exp(s_ij - m_i), S1, S2, acc and u as in
 * the forward:
 *   T = tanh(ln n_eff / kappa),  G_conf = d_confidence + d_count T,
 *   G_neff = d_n_eff + d_count confidence (1 - T^2) / (kappa n_eff),
 *   c1 = (2 G_neff n_eff + G_conf confidence (1 - confidence)) / S1  (the second term is
 *        0 when the floor is off),   c2 = -G_neff n_eff / S2,
 *   w  = (d_direction - u (u . d_direction)) / ||acc||  (0 when acc == 0),
 *   ds_ij = p_ij (c1 + 2 c2 p_ij + <w, v_j>),
 *   dq_i = lam_i scale sum_j ds_ij k_j,  dk_j = sum_i lam_i scale ds_ij q_i,  dv_j = sum_i p_ij w_i,
 * dk and dv summed over the query heads that share a KV head.  Same problem rules as
 * polar_attn_fwd (bf16 or fp32 inputs, head_dim 64 or 128, causal or not).  fp32 inputs
 * run in fp32 on the vector ALUs (batch * heads <= 65535).  bf16 inputs run on the
 * matrix cores: the row statistics come from the forward kernel in partial mode, and
 * P, dS and w enter the products as bf16 with fp32 sums.  Reading variants: every
 * temperature form, the floor levels POLAR_LEVEL_GAUSS and POLAR_LEVEL_GUMBEL2 (they
 * depend on the count only, like lam) and either saturation (POLAR_SAT_LOG1P: T = tanh(ln(1
 * + n_eff) / kappa), and the 1 / n_eff in G_neff becomes 1 / (1 + n_eff)); a per-key
 * floor, a window or POLAR_LEVEL_QNORM returns POLAR_ERR_UNSUPPORTED.  Outputs are DEVICE fp32, 16-byte aligned and
 * overwritten: dq [B, heads, seq_q, head_dim], dk and dv [B, kv_heads, seq_k, head_dim].
 * `workspace` (DEVICE, 16-byte aligned, polar_attn_bwd_workspace_bytes bytes) is
 * scratch owned by the call until the stream reaches its end.  No output or the
 * workspace may overlap an input or another output.  batch == 0 enqueues nothing;
 * seq_q == 0 (q, dq and workspace may then be NULL) writes zero dk and dv.  The kernels
 * (three for fp32; four to six for bf16, the last summing split partial dk and dv in a
 * fixed order, so results are deterministic) run in order on `stream`.  bf16: the size
 * limit of polar_attn_fwd applies to seq_k and to seq_q (one head's Q). */
polar_status polar_attn_bwd(const polar_problem* problem, const void* q, const void* k, const void* v,
                            const polar_grads* grads, float* dq, float* dk, float* dv, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Backward from saved forward statistics: polar_attn_bwd for bf16 inputs without its
 * forward pass.  A training step that runs its forward as polar_attn_fwd_partial
 * (num_splits = 1, split = 0, context_k = 0, then polar_attn_merge for the channels) has
 * every row's (m, S1, S2, acc) already; passing them as DEVICE `saved` [B, heads, seq_q,
 * head_dim + 3] fp32 (16-byte aligned, that layout, computed for the same problem and
 * inputs) skips the forward kernel the backward would otherwise run for them.  The
 * results are then bitwise those of polar_attn_bwd.  Same arguments and rules as
 * polar_attn_bwd otherwise; `saved` is an input (no output or the workspace may overlap
 * it) and may be NULL when seq_q == 0.  fp32 inputs: POLAR_ERR_UNSUPPORTED (their
 * vector-ALU backward forms its own row statistics).  The workspace, of
 * polar_attn_bwd_saved_workspace_bytes bytes (0 for an invalid or fp32 problem), is that
 * of polar_attn_bwd without the room for the statistics. */
size_t polar_attn_bwd_saved_workspace_bytes(const polar_problem* problem);
polar_status polar_attn_bwd_saved(const polar_problem* problem, const void* q, const void* k, const void* v,
                                  const float* saved, const polar_grads* grads, float* dq, float* dk, float* dv,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* Static description of a status code: any int32 value is accepted (a value that is no
 * polar_status gives "unknown status"; the parameter is an int32_t so that such a value
 * is well-defined input in C and C++ alike). */
const char* polar_status_string(int32_t status);

/* POLAR_ABI_VERSION of the built library. */
int32_t polar_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* POLAR_ATTN_H */
