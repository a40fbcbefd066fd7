// Argument blocks and dispatch hooks shared by the VALU and MFMA scorer kernels.
#pragma once

#include "kvs_internal.h"

namespace kvs {

struct P1Args {
  const void* K;
  const void* V;
  const int32_t* n;
  const void* Qw;
  float* part;       // partial records [B*Hkv][GW][nsplit][D + 4]
  int64_t N, sb, sh, GW, chunk;
  int Hkv, Hq, G, W, nsplit;
  float scale;
  // MFMA pass 1 with one split per query: finish the statistics in the pass instead of the
  // combine (lse, O and the pass-2 operand pack); unused otherwise
  int fin;
  float* lse;
  float* O;
  PackP pk;
};

struct P2Args {
  const void* K;
  const void* V;
  const int32_t* n;
  const void* Qw;
  const float* lse;
  const float* O;
  float* g_self;
  float* g_cross;
  const uint4* ops;  // operand pack (MFMA pass 2 only)
  const float* qc;
  int64_t nwb;
  int64_t N, S, P, sb, sh, GW;
  int Hkv, Hq, G, W;
  float scale;
  // merge outputs of a round fused into pass 2 (kvs_score_merge); unused otherwise
  void* Ko;
  void* Vo;
  int32_t* no;
  int32_t* so;
  int64_t osb, osh;
  int64_t M;           // pairs merged (P for a full round)
  // partial rounds: the pass-1 cosine and the selection state of kvs_merge_weights
  const float* cos;
  const int32_t* sel;
  int64_t sel_stride;
  // more than one 128-query block per kv head: each block's sums go to its own slice,
  // [query block][B*Hkv][N] then [query block][B*Hkv][P], added in block order afterwards
  float* qpart;
};

struct CosArgs {
  const void* K;
  float* cos;
  int64_t S, P, sb, sh;
  int Hkv;
};

// Slot splits of the VALU pass 1 over `units` (kv head, query block) pairs: about 1024
// workgroups in all, at least 64 slots per workgroup, at most 256 splits, every split
// non-empty (many heads need few splits, which keeps the partial records small).
inline void valu_pass1_plan(int64_t N, int64_t units, int64_t& chunk, int& nsplit) {
  int64_t k = (N + 63) / 64;
  const int64_t want = (1024 + units - 1) / (units > 0 ? units : 1);
  if (k > want) k = want;
  if (k < 1) k = 1;
  if (k > 256) k = 256;
  chunk = (N + k - 1) / k;
  if (chunk < 1) chunk = 1;
  nsplit = (int)((N + chunk - 1) / chunk);
  if (nsplit < 1) nsplit = 1;
}

// Pass 2 alone on the VALU kernels from caller-supplied window statistics.
hipError_t launch_pass2_valu(const Shape& s, const RoundP& r, const void* K, const void* V, const int32_t* n,
                             const void* Qw, const float* lse, const float* O, float* g_self, float* g_cross,
                             hipStream_t st);
// Adjacent-key cosine of every candidate pair on its own (the routine pass 1 uses).
hipError_t launch_pair_cos(const Shape& s, const CosArgs& ca, int64_t P, hipStream_t st);
// A whole round given the window statistics (lse, O) instead of pass 1: operand pack,
// [cosine and selection for 0 < M < P], pass 2 with the merge and compaction folded in
// (fused_round_ok), or pass 2 then the merge pass (more than 128 window queries per kv
// head).  Requires use_mfma_scorer.
hipError_t launch_stats_merge_mfma(const Shape& s, const RoundP& r, const void* K, const void* V, const int32_t* n,
                                   const void* Qw, const float* lse, const float* O, float* g_self, float* g_cross,
                                   void* ws, float* cos, int32_t* sel_state, const OutP& o, void* K_out, void* V_out,
                                   int32_t* n_out, int32_t* src_out, hipStream_t st);
size_t stats_pack_bytes(const Shape& s, const RoundP& r);
bool use_mfma_scorer(const Shape& s);
size_t mfma_score_workspace_bytes(const Shape& s, const RoundP& r);
// Whole round fused: pass 1, combine, (for 0 < n_merge < P: the selection over the pass-1
// cosine), pass 2 with the merge and compaction folded in.  Requires use_mfma_scorer and
// at most 128 window queries per kv head.  cos ([B*Hkv, P]) and sel_state (selection
// state) are needed only for 0 < n_merge < P.
bool fused_round_ok(const Shape& s, const RoundP& r);
hipError_t launch_score_merge_mfma(const Shape& s, const RoundP& r, const void* K, const void* V, const int32_t* n,
                                   const void* Qw, float* lse, float* O, float* g_self, float* g_cross, void* ws,
                                   float* cos, int32_t* sel_state, const OutP& o, void* K_out, void* V_out,
                                   int32_t* n_out, int32_t* src_out, hipStream_t st);
hipError_t launch_score_mfma(const Shape& s, const RoundP& r, const void* K, const void* V, const int32_t* n,
                             const void* Qw, float* lse, float* O, float* g_self, float* g_cross, float* cos,
                             void* ws, hipStream_t st);

}  // namespace kvs
