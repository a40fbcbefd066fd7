// C ABI of libkvslim (declared in include/kvslim.h): argument validation, workspace
// sizing and launches on the caller's stream.  No device memory is allocated here; the
// only state is a per-thread message for the last error and the per-thread timing-mark
// event pool (created on first use of kvs_marks_begin).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../include/kvslim.h"
#include "kvs_internal.h"
#include "kvs_score_impl.h"

namespace {

thread_local char g_msg[512] = "";

kvs_status fail(kvs_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return s;
}

kvs_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return KVS_OK;
  return fail(KVS_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t pairs_of(int64_t N, int64_t S, int64_t R) {
  const int64_t r = N - S - R;
  return r > 0 ? r / 2 : 0;
}

// Size limits of a cache (stated in kvslim.h): they keep every grid size and 32-bit block
// count of the launches in range.
constexpr int64_t kMaxQueryHeads = int64_t(1) << 20;
constexpr int64_t kMaxSlots = int64_t(1) << 36;

// Validates the cache description; fills the kernel shape.
kvs_status check_cache(const kvs_cache* c, int dtype, kvs::Shape& s) {
  if (!c) return fail(KVS_ERR_NULL, "cache is NULL");
  if (dtype != KVS_BF16 && dtype != KVS_F32) return fail(KVS_ERR_DTYPE, "unknown dtype %d", dtype);
  if (c->batch < 1 || c->n_kv_heads < 1 || c->n_q_heads < 1)
    return fail(KVS_ERR_SHAPE, "batch, n_kv_heads and n_q_heads must be >= 1");
  if (c->n_q_heads % c->n_kv_heads != 0)
    return fail(KVS_ERR_SHAPE, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)", c->n_q_heads, c->n_kv_heads);
  if (c->head_dim != 64 && c->head_dim != 128) return fail(KVS_ERR_SHAPE, "head_dim %d not in {64, 128}", c->head_dim);
  if (c->n_slots < 0) return fail(KVS_ERR_SHAPE, "n_slots < 0");
  if (c->n_slots > (int64_t)INT32_MAX) return fail(KVS_ERR_SHAPE, "n_slots above 2^31 - 1");
  if ((int64_t)c->batch * c->n_q_heads > kMaxQueryHeads)
    return fail(KVS_ERR_SHAPE, "batch x n_q_heads above 2^20");
  if ((int64_t)c->batch * c->n_kv_heads * c->n_slots > kMaxSlots)
    return fail(KVS_ERR_SHAPE, "batch x n_kv_heads x n_slots above 2^36");
  if (c->stride_b < 0 || c->stride_h < 0 || c->stride_b % c->head_dim || c->stride_h % c->head_dim)
    return fail(KVS_ERR_STRIDE, "strides must be non-negative multiples of head_dim");
  s.B = c->batch;
  s.Hkv = c->n_kv_heads;
  s.Hq = c->n_q_heads;
  s.G = c->n_q_heads / c->n_kv_heads;
  s.D = c->head_dim;
  s.N = c->n_slots;
  s.sb = c->stride_b;
  s.sh = c->stride_h;
  s.bf16 = dtype == KVS_BF16;
  return KVS_OK;
}

constexpr int32_t kMaxWindow = 65536;   // keeps every query-indexed grid and workspace size in range

kvs_status check_round(const kvs_round* r, const kvs::Shape& s, kvs::RoundP& rp, bool need_window) {
  if (!r) return fail(KVS_ERR_NULL, "round is NULL");
  if (need_window && (r->window < 1 || r->window > kMaxWindow))
    return fail(KVS_ERR_SHAPE, "window must be in [1, %d]", kMaxWindow);
  if (r->n_sink < 0 || r->n_recent < 0) return fail(KVS_ERR_SHAPE, "n_sink and n_recent must be >= 0");
  if (!std::isfinite(r->sm_scale)) return fail(KVS_ERR_SHAPE, "sm_scale is not finite");
  rp.W = r->window;
  rp.S = r->n_sink;
  rp.R = r->n_recent;
  rp.M = r->n_merge;
  rp.P = pairs_of(s.N, r->n_sink, r->n_recent);
  rp.scale = r->sm_scale;
  if (rp.M < 0 || rp.M > rp.P)
    return fail(KVS_ERR_INFEASIBLE, "n_merge %lld outside [0, P = %lld]", (long long)rp.M, (long long)rp.P);
  return KVS_OK;
}

// timing marks (kvs_marks_begin): library-owned HIP events, thread-local, off by default
constexpr int kMaxMarks = 1 << 16;
struct Marks {
  std::vector<hipEvent_t> ev;           // 2 per marked launch: start, stop
  std::vector<const char*> names;
  int cap = 0;                          // launches that fit the event pool
  int k = 0;                            // launches marked so far
  bool on = false;
  char filter[64] = {0};                // mark only launches with this label ("" = all)
};
thread_local Marks g_marks;

}  // namespace

namespace kvs {

void mark_events(const char* name, hipEvent_t* start, hipEvent_t* stop) {
  Marks& m = g_marks;
  *start = *stop = nullptr;
  if (!m.on || m.k >= m.cap) return;
  if (m.filter[0] && std::strcmp(m.filter, name) != 0) return;
  *start = m.ev[2 * m.k];
  *stop = m.ev[2 * m.k + 1];
  m.names[m.k] = name;
}

void mark_commit() { ++g_marks.k; }

}  // namespace kvs

extern "C" {

kvs_status kvs_marks_begin(int32_t max_launches, const char* label) {
  Marks& m = g_marks;
  if (max_launches < 1 || max_launches > kMaxMarks)
    return fail(KVS_ERR_SHAPE, "max_launches %d outside [1, %d]", (int)max_launches, kMaxMarks);
  if (label && std::strlen(label) >= sizeof(m.filter)) return fail(KVS_ERR_SHAPE, "label too long");
  while ((int)m.ev.size() < 2 * max_launches) {
    hipEvent_t e;
    const hipError_t err = hipEventCreateWithFlags(&e, hipEventDisableSystemFence);
    if (err != hipSuccess) return fail(KVS_ERR_HIP, "hipEventCreateWithFlags: %s", hipGetErrorString(err));
    m.ev.push_back(e);
  }
  m.names.assign(max_launches, "");
  m.cap = max_launches;
  m.k = 0;
  std::snprintf(m.filter, sizeof(m.filter), "%s", label ? label : "");
  m.on = true;
  return KVS_OK;
}

int32_t kvs_marks_end(void) {
  Marks& m = g_marks;
  m.on = false;
  return m.k;
}

const char* kvs_mark_name(int32_t k) {
  const Marks& m = g_marks;
  return (!m.on && k >= 0 && k < m.k) ? m.names[k] : "";
}

float kvs_mark_ms(int32_t k) {
  const Marks& m = g_marks;
  if (m.on || k < 0 || k >= m.k) return -1.0f;
  if (hipEventSynchronize(m.ev[2 * k + 1]) != hipSuccess) return -1.0f;
  float ms = -1.0f;
  if (hipEventElapsedTime(&ms, m.ev[2 * k], m.ev[2 * k + 1]) != hipSuccess) return -1.0f;
  return ms;
}

int64_t kvs_num_pairs(int64_t n_slots, int64_t n_sink, int64_t n_recent) {
  if (n_slots < 0 || n_sink < 0 || n_recent < 0) return 0;
  return pairs_of(n_slots, n_sink, n_recent);
}

// kvs_score_merge workspace: the scorer's, then for a partial round (0 < M < P) the
// cosine [B*Hkv, P] and the selection state, each 256-byte aligned.
static size_t align256(size_t x) { return (x + 255) / 256 * 256; }
static bool partial_round(const kvs::RoundP& r) { return r.M > 0 && r.M < r.P; }
static size_t score_merge_bytes(const kvs::Shape& s, const kvs::RoundP& r) {
  const size_t b = kvs::score_workspace_bytes(s, r);
  if (!partial_round(r)) return b;
  return align256(b) + align256((size_t)s.B * s.Hkv * r.P * sizeof(float)) +
         (size_t)s.B * s.Hkv * kvs::sel_stride_ints(r.P) * sizeof(int32_t);
}

// kvs_score_merge_stats workspace: the pass-2 operand pack when the fused pass takes the
// shape, then for a partial round the cosine and the selection state, 256-byte aligned.
static size_t stats_merge_bytes(const kvs::Shape& s, const kvs::RoundP& r) {
  size_t b = kvs::use_mfma_scorer(s) ? align256(kvs::stats_pack_bytes(s, r)) : 0;
  if (partial_round(r))
    b += align256((size_t)s.B * s.Hkv * r.P * sizeof(float)) +
         (size_t)s.B * s.Hkv * kvs::sel_stride_ints(r.P) * sizeof(int32_t);
  return b;
}

size_t kvs_workspace_bytes(kvs_op op, const kvs_cache* cache, const kvs_round* round) {
  kvs::Shape s;
  if (check_cache(cache, KVS_BF16, s) != KVS_OK) return 0;
  kvs::RoundP r{};
  switch (op) {
    case KVS_OP_SCORE: {
      // the size depends on the element type; report the larger of the two
      if (!round || check_round(round, s, r, true) != KVS_OK) return 0;
      const size_t bf = kvs::score_workspace_bytes(s, r);
      s.bf16 = false;
      const size_t f32 = kvs::score_workspace_bytes(s, r);
      return bf > f32 ? bf : f32;
    }
    case KVS_OP_SCORE_MERGE: {
      if (!round || check_round(round, s, r, true) != KVS_OK) return 0;
      const size_t bf = score_merge_bytes(s, r);
      s.bf16 = false;
      const size_t f32 = score_merge_bytes(s, r);
      return bf > f32 ? bf : f32;
    }
    case KVS_OP_STATS_MERGE: {
      if (!round || check_round(round, s, r, true) != KVS_OK) return 0;
      const size_t bf = stats_merge_bytes(s, r);
      s.bf16 = false;
      const size_t f32 = stats_merge_bytes(s, r);
      return bf > f32 ? bf : f32;
    }
    case KVS_OP_SELECT:
      return 0;
    case KVS_OP_SEL_STATE:
      if (!round) return 0;
      r.P = pairs_of(s.N, round->n_sink, round->n_recent);
      return (size_t)s.B * s.Hkv * kvs::sel_stride_ints(r.P) * sizeof(int32_t);
    case KVS_OP_DECODE:
      return kvs::decode_workspace_bytes(s);
    default:
      break;
  }
  return 0;
}

kvs_status kvs_score(const kvs_cache* cache, kvs_dtype dtype, const void* K, const void* V, const int32_t* n,
                     const void* Qw, const kvs_round* round, float* lse, float* O, float* g_self, float* g_cross,
                     float* cos, void* workspace, size_t workspace_bytes, void* stream) {
  kvs::Shape s;
  kvs::RoundP r;
  kvs_status st = check_cache(cache, dtype, s);
  if (st) return st;
  if ((st = check_round(round, s, r, true))) return st;
  if (s.N < 1) return fail(KVS_ERR_SHAPE, "kvs_score needs n_slots >= 1");
  if (!K || !V || !Qw || !lse || !O || !g_self || (r.P > 0 && !g_cross))
    return fail(KVS_ERR_NULL, "kvs_score: K, V, Qw, lse, O, g_self and g_cross are required");
  if (!aligned16(K) || !aligned16(V) || !aligned16(Qw)) return fail(KVS_ERR_ALIGN, "K, V, Qw must be 16-byte aligned");
  const size_t need = kvs::score_workspace_bytes(s, r);
  if (workspace_bytes < need || (need && !workspace))
    return fail(KVS_ERR_WORKSPACE, "kvs_score needs %zu workspace bytes, got %zu", need, workspace_bytes);
  return hip_status(kvs::launch_score(s, r, K, V, n, Qw, lse, O, g_self, g_cross, cos, workspace,
                                      static_cast<hipStream_t>(stream)),
                    "kvs_score");
}

kvs_status kvs_score_merge(const kvs_cache* cache, kvs_dtype dtype, const void* K, const void* V, const int32_t* n,
                           const void* Qw, const kvs_round* round, float* lse, float* O, float* g_self,
                           float* g_cross, const kvs_cache* out, kvs_dtype out_dtype, void* K_out, void* V_out,
                           int32_t* n_out, int32_t* src_out, void* workspace, size_t workspace_bytes, void* stream) {
  kvs::Shape s, so;
  kvs::RoundP r;
  kvs_status st = check_cache(cache, dtype, s);
  if (st) return st;
  if ((st = check_round(round, s, r, true))) return st;
  if (s.N < 1) return fail(KVS_ERR_SHAPE, "kvs_score_merge needs n_slots >= 1");
  if (!K || !V || !Qw || !lse || !O || !g_self || (r.P > 0 && !g_cross))
    return fail(KVS_ERR_NULL, "kvs_score_merge: K, V, Qw, lse, O, g_self and g_cross are required");
  if (!out) return fail(KVS_ERR_NULL, "kvs_score_merge: out layout is NULL");
  if ((st = check_cache(out, out_dtype, so))) return st;
  if (so.B != s.B || so.Hkv != s.Hkv || so.D != s.D)
    return fail(KVS_ERR_SHAPE, "out layout must match batch, n_kv_heads and head_dim of the input");
  if (so.N != s.N - r.M)
    return fail(KVS_ERR_SHAPE, "out n_slots %lld != N - M = %lld", (long long)so.N, (long long)(s.N - r.M));
  if (!K_out || !V_out || !n_out || !src_out)
    return fail(KVS_ERR_NULL, "kvs_score_merge: K_out, V_out, n_out, src_out are required");
  if (!aligned16(K) || !aligned16(V) || !aligned16(Qw) || !aligned16(K_out) || !aligned16(V_out))
    return fail(KVS_ERR_ALIGN, "K, V, Qw, K_out, V_out must be 16-byte aligned");
  const size_t need = score_merge_bytes(s, r);
  if (workspace_bytes < need || (need && !workspace))
    return fail(KVS_ERR_WORKSPACE, "kvs_score_merge needs %zu workspace bytes, got %zu", need, workspace_bytes);
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  kvs::OutP op{so.sb, so.sh, so.bf16};
  // workspace: scorer | cosine | selection state (the last two for partial rounds only)
  uint8_t* wb = static_cast<uint8_t*>(workspace);
  const bool part = partial_round(r);
  float* cos = part ? reinterpret_cast<float*>(wb + align256(kvs::score_workspace_bytes(s, r))) : nullptr;
  int32_t* sel = part ? reinterpret_cast<int32_t*>(reinterpret_cast<uint8_t*>(cos) +
                                                    align256((size_t)s.B * s.Hkv * r.P * sizeof(float)))
                      : nullptr;
  if (kvs::fused_round_ok(s, r))
    return hip_status(kvs::launch_score_merge_mfma(s, r, K, V, n, Qw, lse, O, g_self, g_cross, workspace, cos, sel,
                                                   op, K_out, V_out, n_out, src_out, hs),
                      "kvs_score_merge");
  // the same round as separate passes on the GPU (scorer, selection, merge pass)
  hipError_t e = kvs::launch_score(s, r, K, V, n, Qw, lse, O, g_self, g_cross, cos, workspace, hs);
  if (e == hipSuccess && part) e = kvs::launch_select(s, r, g_self, g_cross, cos, nullptr, nullptr, sel, hs);
  if (e == hipSuccess) e = kvs::launch_merge(s, r, K, V, n, g_self, g_cross, sel, op, K_out, V_out, n_out, src_out, hs);
  return hip_status(e, "kvs_score_merge");
}

kvs_status kvs_score_merge_stats(const kvs_cache* cache, kvs_dtype dtype, const void* K, const void* V,
                                 const int32_t* n, const void* Qw, const kvs_round* round, const float* lse,
                                 const float* O, float* g_self, float* g_cross, const kvs_cache* out,
                                 kvs_dtype out_dtype, void* K_out, void* V_out, int32_t* n_out, int32_t* src_out,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  kvs::Shape s, so;
  kvs::RoundP r;
  kvs_status st = check_cache(cache, dtype, s);
  if (st) return st;
  if ((st = check_round(round, s, r, true))) return st;
  if (s.N < 1) return fail(KVS_ERR_SHAPE, "kvs_score_merge_stats needs n_slots >= 1");
  if (!K || !V || !Qw || !lse || !O || !g_self || (r.P > 0 && !g_cross))
    return fail(KVS_ERR_NULL, "kvs_score_merge_stats: K, V, Qw, lse, O, g_self and g_cross are required");
  if (!out) return fail(KVS_ERR_NULL, "kvs_score_merge_stats: out layout is NULL");
  if ((st = check_cache(out, out_dtype, so))) return st;
  if (so.B != s.B || so.Hkv != s.Hkv || so.D != s.D)
    return fail(KVS_ERR_SHAPE, "out layout must match batch, n_kv_heads and head_dim of the input");
  if (so.N != s.N - r.M)
    return fail(KVS_ERR_SHAPE, "out n_slots %lld != N - M = %lld", (long long)so.N, (long long)(s.N - r.M));
  if (!K_out || !V_out || !n_out || !src_out)
    return fail(KVS_ERR_NULL, "kvs_score_merge_stats: K_out, V_out, n_out, src_out are required");
  if (!aligned16(K) || !aligned16(V) || !aligned16(Qw) || !aligned16(K_out) || !aligned16(V_out) ||
      !aligned16(O))
    return fail(KVS_ERR_ALIGN, "K, V, Qw, O, K_out, V_out must be 16-byte aligned");
  const size_t need = stats_merge_bytes(s, r);
  if (workspace_bytes < need || (need && !workspace))
    return fail(KVS_ERR_WORKSPACE, "kvs_score_merge_stats needs %zu workspace bytes, got %zu", need,
                workspace_bytes);
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  kvs::OutP op{so.sb, so.sh, so.bf16};
  const bool mfma = kvs::use_mfma_scorer(s);
  // workspace: [operand pack] | cosine | selection state (the last two for partial rounds)
  uint8_t* wb = static_cast<uint8_t*>(workspace);
  const bool part = partial_round(r);
  float* cos = part ? reinterpret_cast<float*>(wb + (mfma ? align256(kvs::stats_pack_bytes(s, r)) : 0)) : nullptr;
  int32_t* sel = part ? reinterpret_cast<int32_t*>(reinterpret_cast<uint8_t*>(cos) +
                                                    align256((size_t)s.B * s.Hkv * r.P * sizeof(float)))
                      : nullptr;
  if (mfma)
    return hip_status(kvs::launch_stats_merge_mfma(s, r, K, V, n, Qw, lse, O, g_self, g_cross, workspace, cos, sel,
                                                   op, K_out, V_out, n_out, src_out, hs),
                      "kvs_score_merge_stats");
  // fp32 caches: the cosine and the selection, the VALU pass 2, the merge pass
  hipError_t e = hipSuccess;
  if (part) {
    kvs::CosArgs ca;
    ca.K = K;
    ca.cos = cos;
    ca.S = r.S;
    ca.P = r.P;
    ca.sb = s.sb;
    ca.sh = s.sh;
    ca.Hkv = s.Hkv;
    e = kvs::launch_pair_cos(s, ca, r.P, hs);
    if (e == hipSuccess) e = kvs::launch_select(s, r, g_self, g_cross, cos, nullptr, nullptr, sel, hs);
  }
  if (e == hipSuccess) e = kvs::launch_pass2_valu(s, r, K, V, n, Qw, lse, O, g_self, g_cross, hs);
  if (e == hipSuccess) e = kvs::launch_merge(s, r, K, V, n, g_self, g_cross, sel, op, K_out, V_out, n_out, src_out, hs);
  return hip_status(e, "kvs_score_merge_stats");
}

kvs_status kvs_exact_e_diag(const kvs_cache* cache, kvs_dtype dtype, const void* K, const void* V, const int32_t* n,
                            const void* Qw, const kvs_round* round, const float* E, const float* lse, const float* O,
                            float* slot_out, float* pair_out, void* stream) {
  kvs::Shape s;
  kvs::RoundP r;
  kvs_status st = check_cache(cache, dtype, s);
  if (st) return st;
  if ((st = check_round(round, s, r, true))) return st;
  if (s.N < 1) return fail(KVS_ERR_SHAPE, "kvs_exact_e_diag needs n_slots >= 1");
  if (!K || !V || !Qw || !E || !lse || !O || !slot_out || (r.P > 0 && !pair_out))
    return fail(KVS_ERR_NULL, "kvs_exact_e_diag: K, V, Qw, E, lse, O, slot_out and pair_out are required");
  if (!aligned16(K) || !aligned16(V) || !aligned16(Qw))
    return fail(KVS_ERR_ALIGN, "K, V, Qw must be 16-byte aligned");
  return hip_status(kvs::launch_exact_e(s, r, K, V, n, Qw, E, lse, O, slot_out, pair_out,
                                        static_cast<hipStream_t>(stream)),
                    "kvs_exact_e_diag");
}

kvs_status kvs_spectral_modes(kvs_dtype dtype, const void* X, int64_t n_tokens, int32_t d_model, const void* modes,
                              const float* eigvals, int32_t n_modes, float* proj, float* contrib, float* cos,
                              void* stream) {
  if (dtype != KVS_BF16) return fail(KVS_ERR_DTYPE, "kvs_spectral_modes takes bf16 token states and modes");
  if (n_tokens < 1 || d_model < 64 || d_model % 64 || n_modes < 1 || n_modes > 4096)
    return fail(KVS_ERR_SHAPE, "kvs_spectral_modes: n_tokens >= 1, d_model a positive multiple of 64, "
                               "1 <= n_modes <= 4096");
  if (!X || !modes || !eigvals || !proj || (n_tokens > 1 && !cos))
    return fail(KVS_ERR_NULL, "kvs_spectral_modes: X, modes, eigvals, proj and cos are required");
  if (!aligned16(X) || !aligned16(modes)) return fail(KVS_ERR_ALIGN, "X and modes must be 16-byte aligned");
  return hip_status(kvs::launch_spectral(X, n_tokens, d_model, modes, eigvals, n_modes, proj, contrib, cos,
                                         static_cast<hipStream_t>(stream)),
                    "kvs_spectral_modes");
}

kvs_status kvs_append(const kvs_cache* cache, kvs_dtype dtype, void* K, void* V, int32_t* n, int64_t at,
                      const kvs_cache* src, const void* K_new, const void* V_new, int64_t from, int64_t count,
                      void* stream) {
  kvs::Shape s, ss;
  kvs_status st = check_cache(cache, dtype, s);
  if (st) return st;
  if ((st = check_cache(src, dtype, ss))) return st;
  if (ss.B != s.B || ss.Hkv != s.Hkv || ss.D != s.D)
    return fail(KVS_ERR_SHAPE, "kvs_append: source and cache must share batch, n_kv_heads and head_dim");
  if (at < 0 || from < 0 || count < 0) return fail(KVS_ERR_SHAPE, "kvs_append: at, from and count must be >= 0");
  if (at + count > s.N)
    return fail(KVS_ERR_SHAPE, "kvs_append: rows [%lld, %lld) exceed the cache's %lld rows", (long long)at,
                (long long)(at + count), (long long)s.N);
  if (from + count > ss.N)
    return fail(KVS_ERR_SHAPE, "kvs_append: source rows [%lld, %lld) exceed its %lld rows", (long long)from,
                (long long)(from + count), (long long)ss.N);
  if (count == 0) return KVS_OK;
  if (!K || !V || !K_new || !V_new) return fail(KVS_ERR_NULL, "kvs_append: K, V, K_new and V_new are required");
  if (!aligned16(K) || !aligned16(V) || !aligned16(K_new) || !aligned16(V_new))
    return fail(KVS_ERR_ALIGN, "kvs_append: K, V, K_new, V_new must be 16-byte aligned");
  return hip_status(kvs::launch_append(s, ss, K, V, n, at, K_new, V_new, from, count,
                                       static_cast<hipStream_t>(stream)),
                    "kvs_append");
}

kvs_status kvs_merge_weights(const kvs_cache* cache, const kvs_round* round, const float* g_self,
                             const float* g_cross, const float* cos, float* w, uint8_t* selected, void* sel_state,
                             size_t sel_state_bytes, void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  kvs::Shape s;
  kvs::RoundP r;
  kvs_status st = check_cache(cache, KVS_BF16, s);
  if (st) return st;
  if ((st = check_round(round, s, r, false))) return st;
  if (!sel_state) return fail(KVS_ERR_NULL, "kvs_merge_weights: sel_state is required");
  const bool choose = r.M != 0 && r.M != r.P;
  if (choose && !cos) return fail(KVS_ERR_NULL, "kvs_merge_weights: cos is required when 0 < n_merge < P");
  if (w && (!g_self || (r.P > 0 && !g_cross)))
    return fail(KVS_ERR_NULL, "kvs_merge_weights: weights need g_self and g_cross");
  const size_t need = (size_t)s.B * s.Hkv * kvs::sel_stride_ints(r.P) * sizeof(int32_t);
  if (sel_state_bytes < need)
    return fail(KVS_ERR_WORKSPACE, "sel_state needs %zu bytes, got %zu", need, sel_state_bytes);
  if (!choose && !w && !selected) return KVS_OK;   // nothing to choose, nothing requested
  return hip_status(kvs::launch_select(s, r, g_self, g_cross, choose ? cos : nullptr, w, selected,
                                       static_cast<int32_t*>(sel_state), static_cast<hipStream_t>(stream)),
                    "kvs_merge_weights");
}

kvs_status kvs_merge_compact(const kvs_cache* cache, kvs_dtype in_dtype, const void* K, const void* V,
                             const int32_t* n, const float* g_self, const float* g_cross, const kvs_round* round,
                             const void* sel_state, const kvs_cache* out, kvs_dtype out_dtype, void* K_out,
                             void* V_out, int32_t* n_out, int32_t* src_out, void* stream) {
  kvs::Shape s, so;
  kvs::RoundP r;
  kvs_status st = check_cache(cache, in_dtype, s);
  if (st) return st;
  if ((st = check_round(round, s, r, false))) return st;
  if (!out) return fail(KVS_ERR_NULL, "kvs_merge_compact: out layout is NULL");
  if ((st = check_cache(out, out_dtype, so))) return st;
  if (so.B != s.B || so.Hkv != s.Hkv || so.D != s.D)
    return fail(KVS_ERR_SHAPE, "out layout must match batch, n_kv_heads and head_dim of the input");
  if (so.N != s.N - r.M)
    return fail(KVS_ERR_SHAPE, "out n_slots %lld != N - M = %lld", (long long)so.N, (long long)(s.N - r.M));
  if (s.N == 0) return KVS_OK;
  if (!K || !V || !K_out || !V_out || !n_out || !src_out)
    return fail(KVS_ERR_NULL, "kvs_merge_compact: K, V, K_out, V_out, n_out, src_out are required");
  if (r.M > 0 && (!g_self || !g_cross)) return fail(KVS_ERR_NULL, "kvs_merge_compact: g_self and g_cross are required");
  if (!sel_state && r.M != r.P && r.M != 0)
    return fail(KVS_ERR_NULL, "kvs_merge_compact: sel_state is required when 0 < n_merge < P");
  if (!aligned16(K) || !aligned16(V) || !aligned16(K_out) || !aligned16(V_out))
    return fail(KVS_ERR_ALIGN, "K, V, K_out, V_out must be 16-byte aligned");
  kvs::OutP op{so.sb, so.sh, so.bf16};
  return hip_status(kvs::launch_merge(s, r, K, V, n, g_self, g_cross, static_cast<const int32_t*>(sel_state), op, K_out,
                                      V_out, n_out, src_out, static_cast<hipStream_t>(stream)),
                    "kvs_merge_compact");
}

static kvs_status check_decode(const kvs_cache* cache, kvs_dtype dtype, const void* K, const void* V, const void* q,
                               float sm_scale, const float* out, kvs::Shape& s, const char* name) {
  kvs_status st = check_cache(cache, dtype, s);
  if (st) return st;
  if (s.N < 1) return fail(KVS_ERR_SHAPE, "%s needs n_slots >= 1", name);
  if (s.G != 1 && s.G != 2 && s.G != 4 && s.G != 8)
    return fail(KVS_ERR_SHAPE, "%s supports n_q_heads / n_kv_heads in {1, 2, 4, 8}, got %d", name, s.G);
  if (!std::isfinite(sm_scale)) return fail(KVS_ERR_SHAPE, "sm_scale is not finite");
  if (!K || !V || !q || !out) return fail(KVS_ERR_NULL, "%s: K, V, q, out are required", name);
  if (!aligned16(K) || !aligned16(V) || !aligned16(q)) return fail(KVS_ERR_ALIGN, "K, V, q must be 16-byte aligned");
  return KVS_OK;
}

kvs_status kvs_decode_attn(const kvs_cache* cache, kvs_dtype dtype, const void* K, const void* V, const int32_t* n,
                           const void* q, float sm_scale, float* out, void* workspace, size_t workspace_bytes,
                           void* stream) {
  kvs::Shape s;
  kvs_status st = check_decode(cache, dtype, K, V, q, sm_scale, out, s, "kvs_decode_attn");
  if (st) return st;
  const size_t need = kvs::decode_workspace_bytes(s);
  if (workspace_bytes < need || !workspace)
    return fail(KVS_ERR_WORKSPACE, "kvs_decode_attn needs %zu workspace bytes, got %zu", need, workspace_bytes);
  return hip_status(kvs::launch_decode(s, K, V, n, q, sm_scale, out, workspace, static_cast<hipStream_t>(stream)),
                    "kvs_decode_attn");
}

kvs_status kvs_decode_attn_static(const kvs_cache* cache, kvs_dtype dtype, const void* K, const void* V,
                                  const int32_t* n, const void* q, float sm_scale, float* out, void* stream) {
  kvs::Shape s;
  kvs_status st = check_decode(cache, dtype, K, V, q, sm_scale, out, s, "kvs_decode_attn_static");
  if (st) return st;
  const size_t need = kvs::decode_workspace_bytes(s);
  if (need > KVS_STATIC_SCRATCH_BYTES)
    return fail(KVS_ERR_WORKSPACE,
                "kvs_decode_attn_static: these shapes need %zu bytes of scratch, above the library's %zu; use "
                "kvs_decode_attn with a workspace",
                need, (size_t)KVS_STATIC_SCRATCH_BYTES);
  void* ws = nullptr;
  hipError_t e = kvs::static_scratch(&ws);
  if (e != hipSuccess) return hip_status(e, "kvs_decode_attn_static (scratch address)");
  return hip_status(kvs::launch_decode(s, K, V, n, q, sm_scale, out, ws, static_cast<hipStream_t>(stream)),
                    "kvs_decode_attn_static");
}

const char* kvs_status_str(kvs_status s) {
  switch (s) {
    case KVS_OK: return "KVS_OK";
    case KVS_ERR_NULL: return "KVS_ERR_NULL";
    case KVS_ERR_SHAPE: return "KVS_ERR_SHAPE";
    case KVS_ERR_DTYPE: return "KVS_ERR_DTYPE";
    case KVS_ERR_STRIDE: return "KVS_ERR_STRIDE";
    case KVS_ERR_ALIGN: return "KVS_ERR_ALIGN";
    case KVS_ERR_INFEASIBLE: return "KVS_ERR_INFEASIBLE";
    case KVS_ERR_WORKSPACE: return "KVS_ERR_WORKSPACE";
    case KVS_ERR_HIP: return "KVS_ERR_HIP";
    default: break;
  }
  return "KVS_ERR_UNKNOWN";
}

const char* kvs_last_error(void) { return g_msg; }

int32_t kvs_version(void) { return 100; }

}  // extern "C"
