// Host-side validation of the C ABI, built with AddressSanitizer and UndefinedBehaviorSanitizer
// on the host code only.  Every call below fails validation (or only sizes a workspace), so no
// kernel is launched and no GPU is needed.  Exit status: the number of failed checks.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "kvslim.h"

static int g_fail = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++g_fail;                                                       \
    }                                                                 \
  } while (0)

static void* const FAKE = reinterpret_cast<void*>(4096);          // aligned, never dereferenced
static void* const MISALIGNED = reinterpret_cast<void*>(4100);

static kvs_cache cache(int B = 1, int H = 8, int Hq = 32, int D = 128, int64_t N = 32768, int64_t sb = -1,
                       int64_t sh = -1) {
  kvs_cache c;
  c.batch = B;
  c.n_kv_heads = H;
  c.n_q_heads = Hq;
  c.head_dim = D;
  c.n_slots = N;
  c.stride_h = sh < 0 ? N * D : sh;
  c.stride_b = sb < 0 ? H * c.stride_h : sb;
  return c;
}

static kvs_round rnd(int W, int64_t S, int64_t R, int64_t M, float scale) {
  kvs_round r;
  r.window = W;
  r.n_sink = S;
  r.n_recent = R;
  r.n_merge = M;
  r.sm_scale = scale;
  return r;
}

static kvs_status score(const kvs_cache* c, const kvs_round* r, int dtype = KVS_BF16, void* K = FAKE,
                        float* gc = static_cast<float*>(FAKE), size_t wsb = size_t(1) << 30) {
  float* f = static_cast<float*>(FAKE);
  return kvs_score(c, static_cast<kvs_dtype>(dtype), K, FAKE, nullptr, FAKE, r, f, f, f, gc, nullptr, FAKE, wsb,
                   nullptr);
}

int main() {
  // pairs and workspace sizes
  CHECK(kvs_num_pairs(512, 0, 0) == 256);
  CHECK(kvs_num_pairs(32768, 0, 32) == 16368);
  CHECK(kvs_num_pairs(33, 32, 0) == 0);
  CHECK(kvs_num_pairs(-1, 0, 0) == 0);
  const kvs_cache c2 = cache();
  const kvs_round r2 = rnd(32, 0, 32, 16368, 0.0883883f);
  for (int op = 0; op <= 5; ++op) (void)kvs_workspace_bytes(static_cast<kvs_op>(op), &c2, &r2);
  CHECK(kvs_workspace_bytes(KVS_OP_SCORE, &c2, &r2) > 0);
  CHECK(kvs_workspace_bytes(KVS_OP_DECODE, &c2, nullptr) > 0);
  const kvs_round r384 = rnd(48, 2, 5, 300, 0.1f);    // three 128-query blocks per kv head
  const kvs_cache c384 = cache(1, 2, 16, 128, 3001);
  CHECK(kvs_workspace_bytes(KVS_OP_SCORE, &c384, &r384) > kvs_workspace_bytes(KVS_OP_SCORE, &c384, &r2) / 64);
  const kvs_cache bad_d = cache(1, 8, 32, 96);
  CHECK(kvs_workspace_bytes(KVS_OP_SCORE, &bad_d, &r2) == 0);
  CHECK(kvs_workspace_bytes(KVS_OP_SCORE, nullptr, &r2) == 0);

  // kvs_score
  CHECK(score(nullptr, &r2) == KVS_ERR_NULL);
  CHECK(score(&c2, nullptr) == KVS_ERR_NULL);
  CHECK(score(&bad_d, &r2) == KVS_ERR_SHAPE);
  const kvs_cache bad_g = cache(1, 8, 30);
  CHECK(score(&bad_g, &r2) == KVS_ERR_SHAPE);
  const kvs_cache bad_stride = cache(1, 8, 32, 128, 32768, -1, 32768 * 128 + 1);
  CHECK(score(&bad_stride, &r2) == KVS_ERR_STRIDE);
  CHECK(score(&c2, &r2, 7) == KVS_ERR_DTYPE);
  CHECK(score(&c2, &r2, KVS_BF16, nullptr) == KVS_ERR_NULL);
  CHECK(score(&c2, &r2, KVS_BF16, FAKE, nullptr) == KVS_ERR_NULL);
  CHECK(score(&c2, &r2, KVS_BF16, MISALIGNED) == KVS_ERR_ALIGN);
  CHECK(score(&c2, &r2, KVS_BF16, FAKE, static_cast<float*>(FAKE), 16) == KVS_ERR_WORKSPACE);
  const kvs_round too_many = rnd(32, 0, 32, 16369, 0.1f), negative = rnd(32, 0, 32, -1, 0.1f);
  CHECK(score(&c2, &too_many) == KVS_ERR_INFEASIBLE);
  CHECK(score(&c2, &negative) == KVS_ERR_INFEASIBLE);
  const kvs_round w0 = rnd(0, 0, 32, 10, 0.1f), wbig = rnd(65537, 0, 32, 10, 0.1f);
  CHECK(score(&c2, &w0) == KVS_ERR_SHAPE);
  CHECK(score(&c2, &wbig) == KVS_ERR_SHAPE);
  const kvs_cache n0 = cache(1, 8, 32, 128, 0);
  const kvs_round r0 = rnd(32, 0, 0, 0, 0.1f);
  CHECK(score(&n0, &r0) == KVS_ERR_SHAPE);
  const kvs_round nan_scale = rnd(32, 0, 32, 10, std::nanf(""));
  CHECK(score(&c2, &nan_scale) == KVS_ERR_SHAPE);
  CHECK(std::strlen(kvs_last_error()) > 0);

  // kvs_merge_weights
  const kvs_round r100 = rnd(32, 0, 32, 100, 0.1f);
  float* f = static_cast<float*>(FAKE);
  CHECK(kvs_merge_weights(&c2, &r100, f, f, f, nullptr, nullptr, nullptr, 0, nullptr, 0, nullptr) == KVS_ERR_NULL);
  CHECK(kvs_merge_weights(&c2, &r100, f, f, nullptr, nullptr, nullptr, FAKE, size_t(1) << 30, nullptr, 0,
                          nullptr) == KVS_ERR_NULL);
  CHECK(kvs_merge_weights(&c2, &r100, f, f, f, nullptr, nullptr, FAKE, 16, nullptr, 0, nullptr) ==
        KVS_ERR_WORKSPACE);

  // kvs_merge_compact
  int32_t* ip = static_cast<int32_t*>(FAKE);
  const kvs_cache good_out = cache(1, 8, 32, 128, 32768 - 16368, -1, (32768 - 16368) * 128);
  const kvs_cache wrong_len = cache(1, 8, 32, 128, 32768 - 16367, -1, (32768 - 16368) * 128);
  CHECK(kvs_merge_compact(&c2, KVS_BF16, FAKE, FAKE, nullptr, f, f, &r2, nullptr, nullptr, KVS_BF16, FAKE, FAKE, ip,
                          ip, nullptr) == KVS_ERR_NULL);
  CHECK(kvs_merge_compact(&c2, KVS_BF16, FAKE, FAKE, nullptr, f, f, &r2, nullptr, &wrong_len, KVS_BF16, FAKE, FAKE,
                          ip, ip, nullptr) == KVS_ERR_SHAPE);
  CHECK(kvs_merge_compact(&c2, KVS_BF16, MISALIGNED, FAKE, nullptr, f, f, &r2, nullptr, &good_out, KVS_BF16, FAKE,
                          FAKE, ip, ip, nullptr) == KVS_ERR_ALIGN);
  CHECK(kvs_merge_compact(&c2, KVS_BF16, FAKE, FAKE, nullptr, f, f, &r2, nullptr, &good_out, static_cast<kvs_dtype>(5),
                          FAKE, FAKE, ip, ip, nullptr) == KVS_ERR_DTYPE);
  const kvs_cache part_out = cache(1, 8, 32, 128, 32768 - 100, -1, (32768 - 100) * 128);
  CHECK(kvs_merge_compact(&c2, KVS_BF16, FAKE, FAKE, nullptr, f, f, &r100, nullptr, &part_out, KVS_BF16, FAKE, FAKE,
                          ip, ip, nullptr) == KVS_ERR_NULL);

  // kvs_score_merge and kvs_score_merge_stats
  const kvs_cache c1k = cache(1, 2, 8, 128, 1000);
  const kvs_cache o500 = cache(1, 2, 8, 128, 500), o900 = cache(1, 2, 8, 128, 900);
  const kvs_round part = rnd(8, 0, 0, 100, 0.1f), full = rnd(8, 0, 0, 500, 0.1f);
  CHECK(kvs_score_merge(&c1k, KVS_BF16, FAKE, FAKE, nullptr, FAKE, &part, f, f, f, f, &o500, KVS_BF16, FAKE, FAKE, ip,
                        ip, FAKE, size_t(1) << 30, nullptr) == KVS_ERR_SHAPE);
  CHECK(kvs_score_merge(&c1k, KVS_BF16, FAKE, FAKE, nullptr, FAKE, &part, f, f, f, f, &o900, KVS_BF16, FAKE, FAKE, ip,
                        ip, FAKE, 16, nullptr) == KVS_ERR_WORKSPACE);
  CHECK(kvs_score_merge(&c1k, KVS_BF16, FAKE, FAKE, nullptr, FAKE, &full, f, f, f, f, &o500, KVS_BF16, FAKE, FAKE,
                        nullptr, ip, FAKE, size_t(1) << 30, nullptr) == KVS_ERR_NULL);
  CHECK(kvs_score_merge_stats(&c1k, KVS_BF16, FAKE, FAKE, nullptr, FAKE, &full, f, f, f, f, &o500, KVS_BF16, FAKE,
                              FAKE, ip, ip, FAKE, 16, nullptr) == KVS_ERR_WORKSPACE);
  CHECK(kvs_score_merge_stats(&c1k, KVS_BF16, FAKE, FAKE, nullptr, FAKE, &full, nullptr, f, f, f, &o500, KVS_BF16,
                              FAKE, FAKE, ip, ip, FAKE, size_t(1) << 30, nullptr) == KVS_ERR_NULL);

  // kvs_decode_attn and kvs_decode_attn_static
  CHECK(kvs_decode_attn(&c2, KVS_BF16, FAKE, FAKE, nullptr, FAKE, 0.1f, f, FAKE, 16, nullptr) == KVS_ERR_WORKSPACE);
  const kvs_cache g3 = cache(1, 8, 24);
  CHECK(kvs_decode_attn(&g3, KVS_BF16, FAKE, FAKE, nullptr, FAKE, 0.1f, f, FAKE, size_t(1) << 30, nullptr) ==
        KVS_ERR_SHAPE);
  CHECK(kvs_decode_attn(&c2, KVS_BF16, FAKE, FAKE, nullptr, nullptr, 0.1f, f, FAKE, size_t(1) << 30, nullptr) ==
        KVS_ERR_NULL);
  const kvs_cache big = cache(8, 8, 32, 128, 65536);
  CHECK(kvs_workspace_bytes(KVS_OP_DECODE, &big, nullptr) > KVS_STATIC_SCRATCH_BYTES);
  CHECK(kvs_decode_attn_static(&big, KVS_F32, FAKE, FAKE, nullptr, FAKE, 0.1f, f, nullptr) == KVS_ERR_WORKSPACE);
  CHECK(kvs_decode_attn_static(&g3, KVS_BF16, FAKE, FAKE, nullptr, FAKE, 0.1f, f, nullptr) == KVS_ERR_SHAPE);

  // kvs_append
  const kvs_cache c200 = cache(1, 2, 8, 128, 200), src50 = cache(1, 2, 8, 128, 50);
  CHECK(kvs_append(&c200, KVS_BF16, FAKE, FAKE, nullptr, 190, &src50, FAKE, FAKE, 0, 11, nullptr) == KVS_ERR_SHAPE);
  CHECK(kvs_append(&c200, KVS_BF16, FAKE, FAKE, nullptr, 0, &src50, FAKE, FAKE, 45, 6, nullptr) == KVS_ERR_SHAPE);
  CHECK(kvs_append(&c200, KVS_BF16, MISALIGNED, FAKE, nullptr, 0, &src50, FAKE, FAKE, 0, 5, nullptr) ==
        KVS_ERR_ALIGN);

  // kvs_exact_e_diag and kvs_spectral_modes
  CHECK(kvs_exact_e_diag(&c2, KVS_BF16, FAKE, FAKE, nullptr, FAKE, &r2, nullptr, f, f, f, f, nullptr) == KVS_ERR_NULL);
  CHECK(kvs_spectral_modes(KVS_F32, FAKE, 100, 64, FAKE, f, 16, f, f, f, nullptr) == KVS_ERR_DTYPE);
  CHECK(kvs_spectral_modes(KVS_BF16, FAKE, 100, 96, FAKE, f, 16, f, f, f, nullptr) == KVS_ERR_SHAPE);
  CHECK(kvs_spectral_modes(KVS_BF16, MISALIGNED, 100, 64, FAKE, f, 16, f, f, f, nullptr) == KVS_ERR_ALIGN);

  // status strings and the timing-mark entry points without a GPU
  for (int s = 0; s <= 8; ++s) CHECK(std::strncmp(kvs_status_str(static_cast<kvs_status>(s)), "KVS_", 4) == 0);
  CHECK(std::strlen(kvs_status_str(static_cast<kvs_status>(99))) > 0);
  CHECK(kvs_marks_begin(0, nullptr) == KVS_ERR_SHAPE);
  CHECK(kvs_marks_begin(1 << 17, nullptr) == KVS_ERR_SHAPE);
  char long_label[80];
  std::memset(long_label, 'x', sizeof(long_label) - 1);
  long_label[sizeof(long_label) - 1] = '\0';
  CHECK(kvs_marks_begin(4, long_label) == KVS_ERR_SHAPE);
  CHECK(kvs_marks_end() == 0);
  CHECK(kvs_mark_name(0)[0] == '\0');
  CHECK(kvs_mark_ms(0) == -1.0f);
  CHECK(kvs_version() == 100);

  std::printf("%d failed checks\n", g_fail);
  return g_fail;
}
