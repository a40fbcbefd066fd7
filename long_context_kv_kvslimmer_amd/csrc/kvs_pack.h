// The pass-2 operand pack of one window query, written by the log-sum-exp combine or, when
// a head's window needs no combine, by the first scorer pass itself.
#pragma once

#include "kvs_common.h"
#include "kvs_internal.h"

namespace kvs {

// The 16 bytes of query row u that lane c < D / 8 copies into the pack.
template <int D>
__device__ __forceinline__ uint4 pack_query_chunk(const PackP& pk, int64_t u, int lane) {
  if (lane >= D / 8) return make_uint4(0, 0, 0, 0);
  const int64_t bh = u / pk.GW, q = u - bh * pk.GW;
  const int64_t b = bh / pk.Hkv, hk = bh - b * pk.Hkv;
  const bf16* qrow = static_cast<const bf16*>(pk.Qw) + ((b * pk.Hq + hk * pk.G) * (int64_t)pk.W + q) * D;
  return *reinterpret_cast<const uint4*>(qrow + lane * 8);
}

// The MFMA pass-2 operands of row u (as combine_kernel writes them): lane c < D / 8 of the
// calling wave packs elements 8c .. 8c + 7 of the row, fetched from the lanes that hold
// them (lane l holds elements l + 64 e in ov[e]), and stores qchunk, the lane's query
// chunk (pack_query_chunk, loaded early by the caller so that its latency overlaps other
// loads); lane 0 writes ||o||^2 and -lse log2 e.  All 64 lanes call it.
template <int D>
__device__ __forceinline__ void pack_row_wave_q(const PackP& pk, int64_t u, const float (&ov)[D / 64], float lse_u,
                                                int lane, const uint4& qchunk) {
  constexpr int nch = D / 8, KS = D / 32;
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int d = (lane * 8 + j) & (D - 1);
    float v = __shfl(ov[0], d & 63, 64);
    if constexpr (D == 128) {
      const float v1 = __shfl(ov[1], d & 63, 64);
      v = d >= 64 ? v1 : v;
    }
    x[j] = v;
  }
  const int64_t bh = u / pk.GW, q = u - bh * pk.GW;
  float on = 0.f;
  if (lane < nch) {
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float x0 = x[2 * j], x1 = x[2 * j + 1];
      on = __builtin_fmaf(x0, x0, __builtin_fmaf(x1, x1, on));
      const float m0 = -2.f * x0, m1 = -2.f * x1;
      hi[j] = pack_bf16x2(m0, m1);
      lo[j] = pack_bf16x2(m0 - bf16_lo(hi[j]), m1 - bf16_hi(hi[j]));
    }
    pk.ops[pack_ops_index(bh, pk.nwb, q, 0, lane, KS)] = qchunk;
    pk.ops[pack_ops_index(bh, pk.nwb, q, 1, lane, KS)] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    pk.ops[pack_ops_index(bh, pk.nwb, q, 2, lane, KS)] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  }
  on = group_sum<16>(on);   // lanes past nch contributed zeros
  if (lane == 0) {
    pk.qc[(bh * pk.nwb * 32 + q) * 2] = on;
    pk.qc[(bh * pk.nwb * 32 + q) * 2 + 1] = -lse_u * kLog2e;
  }
}

}  // namespace kvs
