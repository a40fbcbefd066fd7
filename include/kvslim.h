/*
 * kvslim.h — C ABI of the KVSlimmer asymmetric KV-merge path for AMD MI355X (gfx950).
 *
 * One merge round on a KV cache, per (batch, kv-head), then decode attention over the
 * merged cache:
 *
 *   kvs_score          window attention statistics (lse, o) and the forward-only
 *                      Hessian-norm sums g_self / g_cross, plus adjacent-key cosine
 *   kvs_score_merge    kvs_score + kvs_merge_weights + kvs_merge_compact in one call
 *   kvs_score_merge_stats  the same round given the window statistics (lse, O) from the
 *                      prefill attention that already computed them: no first scorer pass
 *   kvs_merge_weights  pair selection (top-M adjacent pairs by cosine) and the
 *                      closed-form key-merge weights
 *   kvs_merge_compact  key merge, lossless value-slot merge, stream compaction
 *   kvs_decode_attn    GQA decode attention over a (merged) cache
 *   kvs_decode_attn_static  the same with a library-owned scratch (no workspace argument)
 *   kvs_append         write raw tokens (count 1) into a cache: a prefill chunk or a decode step
 *   kvs_exact_e_diag   diagnostics: exact-gradient scalars and weights against the forward-only ones
 *   kvs_spectral_modes analysis: per-eigen-mode split of adjacent-key cosines
 *
 * Sources.  The operations follow the KVSlimmer deep-dive "论文专题讲解：KVSlimmer：
 * 非对称 KV 合并的数学与工程" (charles2530.github.io), sections 数学主线二 (merging an adjacent
 * key pair by a second-order objective), 数学主线三 (single-query attention and its exact
 * Hessian), 数学主线四 (forward-only vectors c11, c22, c12 and the closed-form k*),
 * 实验设置 / 工程上怎么用 (preserved initial "sink" tokens and a recent window) and
 * 局限与边界 (local adjacent merging, one uniform ratio for every head); and the AsymKV
 * abstract ("Homogeneous Keys, Heterogeneous Values", in the related-papers list of the
 * fugumt.com KVSlimmer page) for lossless value handling.
 *
 * Conventions for every entry point.
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The kvs_cache and
 *    kvs_round structs are host memory, read during the call only.
 *  - The library allocates no memory and keeps no state: scratch space is the caller's
 *    `workspace` (size from kvs_workspace_bytes).  Calls on different streams are
 *    independent; outputs must not alias inputs.  The one exception is
 *    kvs_decode_attn_static, whose scratch is a static device array of the library.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and the call
 *    returns without synchronising.  Output lengths are host-computable up front.
 *  - Arguments are validated before anything is enqueued; on a validation error nothing is
 *    written.  A failed kernel launch returns KVS_ERR_HIP; outputs are then undefined.
 *    kvs_last_error() gives a message for the last failure on the calling thread.
 *  - Floating point: inputs bf16 or fp32; every sum and statistic accumulates in fp32.  On
 *    bf16 caches the matrix products take 16-bit operands: Q, K and V as given, P (decode)
 *    and -2O (second scorer pass) as bf16 hi + lo pairs (~16 significant bits), and in the
 *    scorer's first pass, which forms the window output O, P and V as f16 (11 significant
 *    bits; O within ~3e-4 of exact, relative to the row's largest element).  V must then
 *    be finite with |v| <= 65504 (f16's range); values below 2^-14 keep f16's absolute
 *    precision of 2^-24.
 *
 * Cache layout (kvs_cache).  K and V of one (batch b, kv-head h) are n_slots rows of
 * head_dim contiguous elements, starting at element offset b*stride_b + h*stride_h.
 * Slot counts n and compaction indices src use the same row indexing with strides
 * stride_b/head_dim and stride_h/head_dim (one int32 per row).  A slot holds a key, the
 * MEAN of the values it stands for and the count n of raw tokens merged into it; its
 * attention logit carries + ln n.  n == NULL means every count is 1.
 */
#ifndef KVSLIM_H
#define KVSLIM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVS_OK = 0,
  KVS_ERR_NULL = 1,        /* a required pointer is NULL */
  KVS_ERR_SHAPE = 2,       /* bad sizes: head_dim not 64/128, n_q_heads % n_kv_heads, group > 8, ... */
  KVS_ERR_DTYPE = 3,       /* unknown dtype or unsupported dtype combination */
  KVS_ERR_STRIDE = 4,      /* strides not multiples of head_dim, or negative */
  KVS_ERR_ALIGN = 5,       /* K/V/output base pointers not 16-byte aligned */
  KVS_ERR_INFEASIBLE = 6,  /* n_merge < 0 or n_merge > number of candidate pairs */
  KVS_ERR_WORKSPACE = 7,   /* workspace / selection-state buffer missing or too small */
  KVS_ERR_HIP = 8,         /* a HIP launch failed */
  KVS_STATUS_INT32_LO_ = -0x7fffffff - 1, /* range markers: every int32_t is a value of the type */
  KVS_STATUS_INT32_HI_ = 0x7fffffff
} kvs_status;

/* Element types.  Every public enum spans the whole int32_t range, so an unknown value
 * passed from C or another language is a valid argument that the call rejects
 * (KVS_ERR_DTYPE here, 0 bytes for an unknown kvs_op), not undefined behaviour. */
typedef enum {
  KVS_BF16 = 0,
  KVS_F32 = 1,
  KVS_DTYPE_INT32_LO_ = -0x7fffffff - 1,
  KVS_DTYPE_INT32_HI_ = 0x7fffffff
} kvs_dtype;

/* Size limits (KVS_ERR_SHAPE beyond them): B * H_q <= 2^20 query heads, n_slots <= 2^31 - 1,
 * and B * H_kv * n_slots <= 2^36 slots in all, which keeps every launch grid and index of
 * the kernels in range; a cache at the limit would take 16 TB at head_dim 128 in bf16. */
typedef struct {
  int32_t batch;       /* B */
  int32_t n_kv_heads;  /* H_kv */
  int32_t n_q_heads;   /* H_q, a multiple of H_kv; query head hq reads kv head hq / (H_q/H_kv) */
  int32_t head_dim;    /* D: 64 or 128 */
  int64_t n_slots;     /* N: slots per (batch, kv-head) */
  int64_t stride_b;    /* elements between batch items of K and V (multiple of head_dim) */
  int64_t stride_h;    /* elements between kv heads of K and V (multiple of head_dim) */
} kvs_cache;

typedef struct {
  int32_t window;      /* W: observation-window queries per query head, 1..65536 */
  int64_t n_sink;      /* S: leading slots never merged */
  int64_t n_recent;    /* R: trailing slots never merged */
  int64_t n_merge;     /* M: pairs merged in this round, the same for every (b, h); 0 <= M <= P */
  float sm_scale;      /* softmax scale, 1/sqrt(head_dim) for standard attention */
} kvs_round;

/* Operation ids for kvs_workspace_bytes. */
typedef enum {
  KVS_OP_SCORE = 0,      /* workspace of kvs_score */
  KVS_OP_SELECT = 1,     /* workspace of kvs_merge_weights */
  KVS_OP_SEL_STATE = 2,  /* size of the selection-state buffer (kvs_merge_weights -> kvs_merge_compact) */
  KVS_OP_DECODE = 3,     /* workspace of kvs_decode_attn */
  KVS_OP_SCORE_MERGE = 4, /* workspace of kvs_score_merge (equals KVS_OP_SCORE when n_merge is 0 or P) */
  KVS_OP_STATS_MERGE = 5, /* workspace of kvs_score_merge_stats */
  KVS_OP_INT32_LO_ = -0x7fffffff - 1,
  KVS_OP_INT32_HI_ = 0x7fffffff
} kvs_op;

/* Number of candidate pairs P = floor((N - S - R) / 2) (0 if negative).  Pair p is the
 * adjacent, disjoint slot pair (S + 2p, S + 2p + 1); an odd leftover slot before the
 * recent window is kept.  Adjacent merging: deep-dive section 数学主线二; sinks and recent
 * window: sections 实验设置 and 工程上怎么用. */
int64_t kvs_num_pairs(int64_t n_slots, int64_t n_sink, int64_t n_recent);

/* Bytes of workspace (or of the selection state) `op` needs for these shapes; 0 if none.
 * `round` may be NULL for KVS_OP_DECODE. */
size_t kvs_workspace_bytes(kvs_op op, const kvs_cache* cache, const kvs_round* round);

/*
 * kvs_score — window attention statistics and forward-only Hessian-norm sums.
 *
 * For every batch b and query head hq (kv head h = hq / G, G = H_q / H_kv), and every
 * window query w of Qw[b, hq, w, :] ([B, H_q, W, D], dtype `dtype`), over all N slots of
 * kv head h (deep-dive 数学主线三, single-query attention, with the + ln n slot bias):
 *   e_{w,i} = sm_scale * (q_w . k_i) + ln n_i
 *   lse[b, hq, w]   = log sum_i exp(e_{w,i})                     (fp32, [B, H_q, W])
 *   O[b, hq, w, :]  = sum_i exp(e_{w,i} - lse) v_i               (fp32, [B, H_q, W, D])
 * With alpha_{w,i} = exp(e_{w,i} - lse_w), summed over the G*W window queries of kv head h
 * (deep-dive 数学主线四, norms of c11, c22 and c12):
 *   g_self[b, h, i]  = sum_w alpha_{w,i} |1 - 2 alpha_{w,i}| ||v_i - o_w||       ([B, H_kv, N])
 *   g_cross[b, h, p] = sum_w alpha_{w,m} alpha_{w,m+1} ||v_m + v_{m+1} - 2 o_w||, m = S + 2p
 *                                                                                ([B, H_kv, P])
 *   cos[b, h, p]     = k_m . k_{m+1} / (||k_m|| ||k_{m+1}||)  (nullable output; 1 if both
 *                      keys are equal and a norm is 0, else 0 when a norm is 0)   ([B, H_kv, P])
 * All statistics arrays are dense row-major fp32.  Requires N >= 1 and W >= 1.
 * `n` is NULL or int32 counts >= 1 (cache row indexing).  K, V, Qw 16-byte aligned.
 */
kvs_status kvs_score(const kvs_cache* cache, kvs_dtype dtype,
                     const void* K, const void* V, const int32_t* n,
                     const void* Qw, const kvs_round* round,
                     float* lse, float* O, float* g_self, float* g_cross, float* cos,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * kvs_score_merge — one whole merge round in one call: the statistics of kvs_score (lse,
 * O, g_self, g_cross), the selection of kvs_merge_weights and the outputs of
 * kvs_merge_compact (K_out, V_out, n_out, src_out), computed with the same arithmetic, so
 * every output equals that of kvs_score -> kvs_merge_weights -> kvs_merge_compact bit for
 * bit.  0 <= n_merge <= P.  For 0 < n_merge < P the cosine and the selection state live in
 * the workspace (they are not outputs); for n_merge == P every pair merges and for
 * n_merge == 0 none does, and no cosine is computed.  For bf16 caches with head_dim 64 or
 * 128 and at most 128 window queries per kv head (G * window <= 128), the selection runs
 * between the scorer's two passes and the merge runs inside the second pass on the K/V
 * tiles it has already loaded, which saves one read of the cache; other shapes run the
 * passes one after the other.  Arguments as in kvs_score and kvs_merge_compact;
 * workspace: kvs_workspace_bytes(KVS_OP_SCORE_MERGE).  Errors as theirs.
 */
kvs_status kvs_score_merge(const kvs_cache* cache, kvs_dtype dtype,
                           const void* K, const void* V, const int32_t* n, const void* Qw,
                           const kvs_round* round, float* lse, float* O, float* g_self, float* g_cross,
                           const kvs_cache* out, kvs_dtype out_dtype,
                           void* K_out, void* V_out, int32_t* n_out, int32_t* src_out,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * kvs_score_merge_stats — kvs_score_merge for a caller that already holds the window
 * statistics: lse [B, H_q, W] (natural log) and O [B, H_q, W, D] (fp32), the attention of
 * the window queries Qw over the cache's N slots with the + ln n slot bias (deep-dive
 * 数学主线三, as kvs_score defines them).  The prefill attention of the chunk that ends
 * with the window computes exactly these (with the slot bias over a merged cache), so the
 * round skips the scorer's first pass and reads the cache once for the statistics plus,
 * for 0 < n_merge < P, the keys once for the cosine.  g_self, g_cross and the merged cache
 * are as in kvs_score_merge; given the lse and O that kvs_score writes, every output equals
 * kvs_score_merge's bit for bit.  lse and O are read only.  Workspace:
 * kvs_workspace_bytes(KVS_OP_STATS_MERGE).  Errors as kvs_score_merge's; O must be 16-byte
 * aligned.
 */
kvs_status kvs_score_merge_stats(const kvs_cache* cache, kvs_dtype dtype,
                                 const void* K, const void* V, const int32_t* n, const void* Qw,
                                 const kvs_round* round, const float* lse, const float* O,
                                 float* g_self, float* g_cross,
                                 const kvs_cache* out, kvs_dtype out_dtype,
                                 void* K_out, void* V_out, int32_t* n_out, int32_t* src_out,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * kvs_merge_weights — pair selection and closed-form weights.
 *
 * Selection (deep-dive 数学主线二 "adjacent" pairs; 局限与边界: one uniform ratio): in every
 * (b, h) independently, the round->n_merge candidate pairs with the largest cos[b, h, p],
 * ties to the smaller p.  The result is written to `sel_state` (an opaque device buffer of
 * kvs_workspace_bytes(KVS_OP_SEL_STATE) bytes) that kvs_merge_compact consumes; optionally
 * also as one flag byte per pair, selected[b, h, p] in {0, 1} ([B, H_kv, P], nullable).
 * `cos` may be NULL only when n_merge is 0 or P (nothing to choose).  In that case, when
 * neither `w` nor `selected` is requested, nothing is enqueued and `sel_state` is left
 * untouched (kvs_merge_compact does not read it for such rounds).
 *
 * Weights (deep-dive 数学主线四, closed-form forward-only k*), for every pair p, m = S + 2p:
 *   A = g_self[m] - 2 g_cross[p] + g_self[m+1]
 *   w[b, h, p, 0] = (g_self[m]   - g_cross[p]) / A
 *   w[b, h, p, 1] = (g_self[m+1] - g_cross[p]) / A
 * and the plain average (1/2, 1/2) of section 数学主线二 when A is not finite or
 * A <= 1e-6 (g_self[m] + g_self[m+1] + 2 g_cross[p]).  `w` ([B, H_kv, P, 2] fp32) is nullable.
 */
kvs_status kvs_merge_weights(const kvs_cache* cache, const kvs_round* round,
                             const float* g_self, const float* g_cross, const float* cos,
                             float* w, uint8_t* selected,
                             void* sel_state, size_t sel_state_bytes,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * kvs_merge_compact — key merge, lossless value merge and stream compaction.
 *
 * For each selected pair p (m = S + 2p), with the weights of kvs_merge_weights computed
 * inline from g_self and g_cross:
 *   k* = w_0 k_m + w_1 k_{m+1}                                (deep-dive 数学主线四)
 *   v* = (n_m v_m + n_{m+1} v_{m+1}) / (n_m + n_{m+1}),   n* = n_m + n_{m+1}
 * (values are not merged by the key rule: the merged slot keeps the count-weighted mean
 * value and the count, so attention with + ln n reproduces the two separate values
 * exactly — the lossless value handling of the AsymKV abstract).  Every other slot is
 * copied unchanged.  Slots keep their order: the output has T = N - M slots and
 * src_out[j] is the input slot of the first token of output slot j.
 *
 * `sel_state` comes from kvs_merge_weights for the same shapes and round; it is read only
 * when 0 < n_merge < P (n_merge == P merges every pair, n_merge == 0 copies), and may be
 * NULL otherwise.  The kernel
 * recomputes each pair's cosine with the same routine kvs_score uses and tests it
 * against the selection threshold.  `out` describes the K_out/V_out layout: same batch,
 * heads and head_dim as `cache`, n_slots == N - M, its own strides.  n_out and src_out
 * (int32, required) use the row indexing of `out`.  in_dtype/out_dtype: any of
 * bf16/fp32 (fp32 output keeps the full fp32 result; bf16 output is its round-to-nearest-
 * even).
 */
kvs_status kvs_merge_compact(const kvs_cache* cache, kvs_dtype in_dtype,
                             const void* K, const void* V, const int32_t* n,
                             const float* g_self, const float* g_cross,
                             const kvs_round* round, const void* sel_state,
                             const kvs_cache* out, kvs_dtype out_dtype,
                             void* K_out, void* V_out, int32_t* n_out, int32_t* src_out,
                             void* stream);

/*
 * kvs_exact_e_diag — measures the one approximation of the forward-only weights.  Given
 * an upstream gradient E [B, H_q, W, D] (fp32, dL/do of each window query) and the window
 * statistics lse [B, H_q, W], O [B, H_q, W, D] (fp32, as kvs_score writes them), with
 * alpha = exp(sm_scale q.k + ln n - lse) and, per window query w,
 *   c_ii = alpha_i (1 - 2 alpha_i)(v_i - o_w),  c12 = -alpha_m alpha_{m+1}(v_m + v_{m+1} - 2 o_w)
 * (deep-dive 数学主线四; the exact Hessian block of 数学主线三 is (E_w . c) q q^T / d_k):
 *   slot_out[b, h, i, :] = ( sum_w E_w . c_ii,  sum_w |E_w| |c_ii|,  sum_w |c_ii| )      [B, H_kv, N, 3]
 *   pair_out[b, h, p, :] = ( sum_w E_w . c12,   sum_w |E_w| |c12|,   sum_w |c12|,
 *                            exact w_m, w_{m+1}  (stationary point of 数学主线二 in the exact
 *                            scalars; (1/2, 1/2) when g11 + 2 g12 + g22 is not finite or at
 *                            most 1e-6 (|g11| + 2|g12| + |g22|) in magnitude),
 *                            forward-only w_m, w_{m+1}  (as kvs_merge_weights),
 *                            loss at each k*: |k_m - k_{m+1}|^2 (g11 w_{m+1}^2 - 2 g12 w_m w_{m+1}
 *                            + g22 w_m^2) in the exact scalars )                       [B, H_kv, P, 9]
 * Column 0 over column 1 is a norm-weighted cos(E, c); the forward-only weights assume
 * cos(E, c11) = cos(E, c22) = -cos(E, c12).  round: window, n_sink, n_recent, sm_scale
 * (n_merge is not used but must be feasible).  fp32 arithmetic on the vector units; a
 * diagnostic, not part of a merge round.  Errors as kvs_score's.
 */
kvs_status kvs_exact_e_diag(const kvs_cache* cache, kvs_dtype dtype,
                            const void* K, const void* V, const int32_t* n, const void* Qw,
                            const kvs_round* round, const float* E, const float* lse, const float* O,
                            float* slot_out, float* pair_out, void* stream);

/*
 * kvs_spectral_modes — the per-mode split of adjacent-key similarity of the deep-dive's
 * section 数学主线一.  Keys are y_t = x_t W; with the eigen-pairs (u_i, l_i) of W W^T,
 * p_{t,i} = x_t . u_i and
 *   contrib[t, i] = l_i p_{t,i} p_{t+1,i} / (|y_t| |y_{t+1}|),  |y_t|^2 = sum_i l_i p_{t,i}^2,
 *   cos[t] = sum_i contrib[t, i] = cos(y_t, y_{t+1}),
 * zero when a norm is zero.  X: [n_tokens, d_model] bf16 token states (rows contiguous);
 * modes: [n_modes, d_model] bf16, the eigenvectors as rows (the n_modes = d_k modes of
 * nonzero eigenvalue suffice: the left singular vectors of W), eigvals [n_modes] fp32.
 * Outputs (fp32, caller-owned): proj [n_tokens, n_modes] = the p_{t,i}; contrib
 * [n_tokens - 1, n_modes] (nullable); cos [n_tokens - 1].  The projections run on the
 * matrix cores with fp32 accumulation.  An analysis tool, not part of a merge round.
 * Errors: KVS_ERR_DTYPE unless bf16; KVS_ERR_SHAPE unless n_tokens >= 1, d_model is a
 * positive multiple of 64 and 1 <= n_modes <= 4096; KVS_ERR_ALIGN unless X and modes are
 * 16-byte aligned.
 */
kvs_status kvs_spectral_modes(kvs_dtype dtype, const void* X, int64_t n_tokens, int32_t d_model,
                              const void* modes, const float* eigvals, int32_t n_modes,
                              float* proj, float* contrib, float* cos, void* stream);

/*
 * kvs_append — the cache write of new raw tokens (a prefill chunk in the chunked regime of
 * the deep-dive's section 实验设置, or a decode step): for every (b, h), rows
 * [from, from + count) of the source (K_new, V_new; layout `src`, its n_slots = the rows
 * it holds) are copied to rows [at, at + count) of the cache (K, V; layout `cache`, its
 * n_slots = the rows allocated), and n[b, h, at .. at + count) = 1 (a raw token is a slot
 * of count 1, as in kvs_score); n is nullable.  Both layouts share batch, n_kv_heads,
 * head_dim and `dtype`; the source and destination rows must not overlap.  Errors:
 * KVS_ERR_SHAPE if at + count exceeds the cache rows, from + count the source rows, or the
 * layouts differ; KVS_ERR_ALIGN unless K, V, K_new, V_new are 16-byte aligned;
 * KVS_ERR_NULL for missing pointers when count > 0.  Enqueued on `stream`.
 */
kvs_status kvs_append(const kvs_cache* cache, kvs_dtype dtype, void* K, void* V, int32_t* n, int64_t at,
                      const kvs_cache* src, const void* K_new, const void* V_new, int64_t from, int64_t count,
                      void* stream);

/*
 * kvs_decode_attn — decode attention over a (merged) cache (deep-dive 数学主线三
 * attention with the + ln n slot bias):
 *   out[b, hq, :] = sum_j softmax_j(sm_scale * q[b, hq] . k_j + ln n_j) v_j
 * over the cache->n_slots slots of kv head hq / G.  q: [B, H_q, D] in `dtype`;
 * out: [B, H_q, D] fp32.  Requires N >= 1 and G = H_q / H_kv in {1, 2, 4, 8}.
 * Workspace: kvs_workspace_bytes(KVS_OP_DECODE) bytes (split partial records).
 */
kvs_status kvs_decode_attn(const kvs_cache* cache, kvs_dtype dtype,
                           const void* K, const void* V, const int32_t* n,
                           const void* q, float sm_scale, float* out,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * kvs_decode_attn_static — kvs_decode_attn for callers that cannot allocate device memory
 * or pass a workspace: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, arithmetic and outputs as kvs_decode_attn (the same
 * kernels, bit for bit), without the workspace: its scratch is a library-owned static
 * device array of KVS_STATIC_SCRATCH_BYTES bytes, one per GPU, held from the first call on
 * that GPU until the process ends.  The call itself allocates and frees nothing.  Nothing
 * in the scratch needs clearing: every call writes each record it reads.  All calls on one
 * GPU share that GPU's scratch, so calls that overlap in time on one GPU (on different
 * streams, or from different threads) race and must be serialised by the caller; the
 * stream must belong to the current device.  Errors: as kvs_decode_attn; KVS_ERR_WORKSPACE
 * when kvs_workspace_bytes(KVS_OP_DECODE) for these shapes exceeds
 * KVS_STATIC_SCRATCH_BYTES (nothing is enqueued); KVS_ERR_HIP if the scratch address cannot
 * be obtained on the first call on a device.
 */
#define KVS_STATIC_SCRATCH_BYTES (8u << 20)
kvs_status kvs_decode_attn_static(const kvs_cache* cache, kvs_dtype dtype,
                                  const void* K, const void* V, const int32_t* n,
                                  const void* q, float sm_scale, float* out, void* stream);

/* Kernel timing marks (instrumentation, off by default).
 *
 * kvs_marks_begin(max_launches, label): from now on, on the calling thread, the library
 * times each of its kernel launches whose label equals `label` (every launch if `label` is
 * NULL or ""), for the first `max_launches` such launches: a marked launch goes through
 * hipExtLaunchKernelGGL with a start and a stop HIP event, which the runtime records at the
 * kernel's own dispatch boundaries on the launch's stream.  Labels: "score_pass1",
 * "score_pass2", "score_pass2_merge", "combine", "qsum", "pair_cos", "select",
 * "merge_compact", "decode", "append", "pack", "exact_e", "spectral_proj",
 * "spectral_pair".  The events are owned by
 * the library (a per-thread pool created with hipEventDisableSystemFence, grown on demand
 * and kept until the process ends).  Errors: KVS_ERR_SHAPE if max_launches is outside
 * [1, 65536] or the label is longer than 63 bytes; KVS_ERR_HIP if an event cannot be made.
 * kvs_marks_end() stops recording and returns the number of launches marked.
 * After kvs_marks_end: kvs_mark_name(k) is the k-th marked launch's label (static string,
 * "" if k is out of range) and kvs_mark_ms(k) its duration in milliseconds (waits for
 * that launch to finish; -1 if k is out of range or the events fail).
 * A new kvs_marks_begin discards earlier marks. */
kvs_status kvs_marks_begin(int32_t max_launches, const char* label);
int32_t kvs_marks_end(void);
const char* kvs_mark_name(int32_t k);
float kvs_mark_ms(int32_t k);

/* Human-readable name of a status code (static string). */
const char* kvs_status_str(kvs_status s);

/* Message describing the last non-OK status returned on the calling thread. */
const char* kvs_last_error(void);

/* ABI version of this library (major * 100 + minor). */
int32_t kvs_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVSLIM_H */
