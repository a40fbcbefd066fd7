// Scorer (kvs_score): window attention statistics and forward-only Hessian-norm sums.
//
// KVSlimmer deep-dive (charles2530.github.io):
//   section 数学主线三 — single-query attention e_i = q k_i^T / sqrt(d_k), alpha = softmax(e),
//     o = sum alpha_t v_t (here every slot's logit carries + ln n_i, n_i tokens per slot);
//   section 数学主线四 — forward-only vectors c11 = a_m (1 - 2 a_m)(v_m - o),
//     c22 = a_{m+1}(1 - 2 a_{m+1})(v_{m+1} - o), c12 = -a_m a_{m+1}(v_m + v_{m+1} - 2o), whose
//     norms (summed over the window queries) fix the closed-form merge weights.
//
// Two passes over K/V, because alpha and ||v - o|| need the final lse and o:
//   pass 1: split-N online softmax per window query -> partial (max, sum, o) records,
//           then a log-sum-exp combine -> lse, O.  Pass 1 also writes the adjacent-key
//           cosine of every candidate pair (pair_cos, the routine the merge pass reuses).
//   pass 2: alpha, residual norms, g_self / g_cross.
// This file holds the portable VALU kernels (any element type); the bf16 MFMA kernels
// live in kvs_score_mfma.hip.
#include "kvs_common.h"
#include "kvs_internal.h"
#include "kvs_score_impl.h"
#include "kvs_pack.h"

namespace kvs {

// ------------------------------------------------------------------ pass 1 (VALU) --
// grid: x = slot split, y = block of 128 window queries, z = (b, kv-head).
// Two threads per query, each owning half of the head dimension.
template <typename T, int D>
__global__ __launch_bounds__(256) void pass1_valu_kernel(P1Args a) {
  constexpr int DH = D / 2;
  constexpr int TS = 32;
  constexpr int E = Elt<T>::kPerChunk;
  __shared__ float Ks[TS][D];
  __shared__ float Vs[TS][D];
  __shared__ float lg[TS];

  const int tid = threadIdx.x;
  const int qi = tid >> 1, half = tid & 1;
  const int64_t bh = blockIdx.z;
  const int64_t b = bh / a.Hkv, h = bh - b * a.Hkv;
  const int64_t w = (int64_t)blockIdx.y * 128 + qi;
  const bool qvalid = w < a.GW;
  const T* Kp = static_cast<const T*>(a.K) + b * a.sb + h * a.sh;
  const T* Vp = static_cast<const T*>(a.V) + b * a.sb + h * a.sh;
  const int32_t* np = a.n ? a.n + (b * a.sb + h * a.sh) / D : nullptr;
  // window queries of kv head h: query heads h*G .. h*G+G-1, W rows each, contiguous
  const T* Qp = static_cast<const T*>(a.Qw) + ((b * a.Hq + h * a.G) * (int64_t)a.W) * D;

  float qs[DH];
  {
    const float c = a.scale * kLog2e;
    for (int d0 = 0; d0 < DH; d0 += E) {
      float f[E];
      if (qvalid) unpack<T>(load16(Qp + w * D + half * DH + d0), f);
#pragma unroll
      for (int e = 0; e < E; ++e) qs[d0 + e] = qvalid ? f[e] * c : 0.f;
    }
  }
  float o[DH];
#pragma unroll
  for (int d = 0; d < DH; ++d) o[d] = 0.f;
  float m = -INFINITY, l = 0.f;

  const int64_t s_begin = (int64_t)blockIdx.x * a.chunk;
  const int64_t s_end = min(a.N, s_begin + a.chunk);
  for (int64_t t0 = s_begin; t0 < s_end; t0 += TS) {
    const int nt = (int)min((int64_t)TS, s_end - t0);
    __syncthreads();
    for (int idx = tid; idx < TS * (D / E); idx += 256) {
      const int s = idx / (D / E), cch = idx % (D / E);
      float fk[E], fv[E];
      if (s < nt) {
        unpack<T>(load16(Kp + (t0 + s) * D + cch * E), fk);
        unpack<T>(load16(Vp + (t0 + s) * D + cch * E), fv);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) fk[e] = fv[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        Ks[s][cch * E + e] = fk[e];
        Vs[s][cch * E + e] = fv[e];
      }
    }
    if (tid < TS) lg[tid] = (tid < nt && np) ? __log2f((float)np[t0 + tid]) : 0.f;
    __syncthreads();
    float ev[TS];
    float mx = -INFINITY;
#pragma unroll
    for (int s = 0; s < TS; ++s) {
      float d = 0.f;
#pragma unroll
      for (int k = 0; k < DH; ++k) d = __builtin_fmaf(qs[k], Ks[s][half * DH + k], d);
      d += __shfl_xor(d, 1, 64);
      ev[s] = s < nt ? d + lg[s] : -INFINITY;
      mx = fmaxf(mx, ev[s]);
    }
    const float mn = fmaxf(m, mx);
    const float corr = exp2f(m - mn);
    l *= corr;
#pragma unroll
    for (int k = 0; k < DH; ++k) o[k] *= corr;
#pragma unroll
    for (int s = 0; s < TS; ++s) {
      const float p = exp2f(ev[s] - mn);
      l += p;
#pragma unroll
      for (int k = 0; k < DH; ++k) o[k] = __builtin_fmaf(p, Vs[s][half * DH + k], o[k]);
    }
    m = mn;
  }
  if (qvalid) {
    float* rec = a.part + ((bh * a.GW + w) * a.nsplit + blockIdx.x) * (int64_t)(D + 4);
    if (half == 0) {
      rec[0] = m;
      rec[1] = l;
    }
#pragma unroll
    for (int k = 0; k < DH; ++k) rec[4 + half * DH + k] = o[k];
  }
}

// --------------------------------------------------------- log-sum-exp combine --
// Partial records {m (log2 units), l, -, -, o[D]} of every split of a unit become the
// unit's output row; lse (natural log, nullable) is written too.
constexpr int kMaxSplit = 1024;

// One 256-thread workgroup per unit (row of `out`).  Every load of the first round is
// issued together: the thread's split maxima and sums, and the first kCombineUnroll
// records of its share of the output elements (thread t: element t % D over splits
// t / D, t / D + 256 / D, ...).  M and the weights f_s = exp2(m_s - M) are reduced in LDS,
// then each thread sums its share and the shares are added in LDS in a fixed order, so
// results do not depend on timing.  Splits beyond the first round are read in further
// rounds of kCombineUnroll.
constexpr int kCombineThreads = 256;
constexpr int kCombineUnroll = 16;
constexpr int kCombineML = kMaxSplit / kCombineThreads;

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const float* __restrict__ part, int nsplit, int D,
                                                                 float* __restrict__ lse, float* __restrict__ out,
                                                                 PackP pk) {
  __shared__ float wsh[kMaxSplit];
  __shared__ float red[8];
  __shared__ float osh[kCombineThreads];
  const int64_t u = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t rs = D + 4;
  const float* r = part + u * nsplit * rs;
  const int d = tid % D, g = tid / D, ng = kCombineThreads / D;
  // the query chunk of the operand pack does not depend on the splits: load it first
  uint4 qch = make_uint4(0, 0, 0, 0);
  if (pk.ops && tid < D / 8) {
    const int64_t bh = u / pk.GW, q = u - bh * pk.GW;
    const int64_t b = bh / pk.Hkv, hk = bh - b * pk.Hkv;
    const bf16* qrow = static_cast<const bf16*>(pk.Qw) + ((b * pk.Hq + hk * pk.G) * (int64_t)pk.W + q) * D;
    qch = *reinterpret_cast<const uint4*>(qrow + tid * 8);
  }
  float2 ml[kCombineML];
#pragma unroll
  for (int k = 0; k < kCombineML; ++k) {
    const int s = tid + k * kCombineThreads;
    ml[k] = s < nsplit ? *reinterpret_cast<const float2*>(r + s * rs) : make_float2(-INFINITY, 0.f);
  }
  float o[kCombineUnroll];
#pragma unroll
  for (int k = 0; k < kCombineUnroll; ++k) {
    const int s = g + k * ng;
    o[k] = s < nsplit ? r[s * rs + 4 + d] : 0.f;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < kCombineML; ++k) mx = fmaxf(mx, ml[k].x);
  mx = group_max<64>(mx);
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float L = 0.f;
#pragma unroll
  for (int k = 0; k < kCombineML; ++k) {
    const int s = tid + k * kCombineThreads;
    if (s < nsplit) {
      const float w = ml[k].x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml[k].x - M);
      wsh[s] = w;
      L = __builtin_fmaf(ml[k].y, w, L);
    }
  }
  L = group_sum<64>(L);
  if ((tid & 63) == 0) red[4 + (tid >> 6)] = L;
  __syncthreads();
  L = (red[4] + red[5]) + (red[6] + red[7]);
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < kCombineUnroll; ++k) {
    const int s = g + k * ng;
    if (s < nsplit) acc = __builtin_fmaf(o[k], wsh[s], acc);
  }
  for (int s0 = g + kCombineUnroll * ng; s0 < nsplit; s0 += ng * kCombineUnroll) {
#pragma unroll
    for (int k = 0; k < kCombineUnroll; ++k) {
      const int s = s0 + k * ng;
      o[k] = s < nsplit ? r[s * rs + 4 + d] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < kCombineUnroll; ++k) {
      const int s = s0 + k * ng;
      if (s < nsplit) acc = __builtin_fmaf(o[k], wsh[s], acc);
    }
  }
  osh[tid] = acc;
  __syncthreads();
  if (tid < D) {
    float v = 0.f;
    for (int k = 0; k < ng; ++k) v += osh[k * D + tid];
    const float o = v / L;
    out[u * D + tid] = o;
    osh[tid] = o;   // each thread overwrites only its own slot after reading the shares
  }
  const float lse_u = (M + __log2f(L)) * kLn2;
  if (lse && tid == 0) lse[u] = lse_u;
  if (pk.ops) {
    // operands of the MFMA pass 2: Q, and -2 O as bf16 hi + lo, in lane order
    __syncthreads();
    const int64_t bh = u / pk.GW, q = u - bh * pk.GW;
    const int nch = D / 8, KS = D / 32;
    float on = 0.f;
    if (tid < nch) {
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x0 = osh[tid * 8 + 2 * j], x1 = osh[tid * 8 + 2 * j + 1];
        on = __builtin_fmaf(x0, x0, __builtin_fmaf(x1, x1, on));
        const float m0 = -2.f * x0, m1 = -2.f * x1;
        hi[j] = pack_bf16x2(m0, m1);
        lo[j] = pack_bf16x2(m0 - bf16_lo(hi[j]), m1 - bf16_hi(hi[j]));
      }
      pk.ops[pack_ops_index(bh, pk.nwb, q, 0, tid, KS)] = qch;
      pk.ops[pack_ops_index(bh, pk.nwb, q, 1, tid, KS)] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      pk.ops[pack_ops_index(bh, pk.nwb, q, 2, tid, KS)] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }
    on = group_sum<16>(on);   // lanes past nch contributed zeros
    if (tid == 0) {
      pk.qc[(bh * pk.nwb * 32 + q) * 2] = on;
      pk.qc[(bh * pk.nwb * 32 + q) * 2 + 1] = -lse_u * kLog2e;
    }
  }
}

// Few splits and many units (many heads, short caches): one wave per unit, four units per
// workgroup, no barriers.  Lane l reads the maximum and sum of split l; the wave reduces
// them; lane l then owns output elements l (and l + 64 at D = 128) and sums the splits in
// order, the weight of split s read from lane s.  The outputs of CH splits are loaded at a
// time: 8 for up to 16 splits; 32 (every split in one round of loads) for 17 to 32 splits
// when there are enough units to fill the chip (with few units the workgroup-per-unit
// kernel is faster).
constexpr int kCombineWaveMaxSplit = 16;
constexpr int kCombineWaveMaxSplitWide = 32;
constexpr int64_t kCombineWaveWideMinUnits = 256;
constexpr int kCombineWaveUnits = 4;

template <int D, int CH>
__global__ __launch_bounds__(64 * kCombineWaveUnits) void combine_wave_kernel(const float* __restrict__ part,
                                                                             int64_t units, int nsplit,
                                                                             float* __restrict__ lse,
                                                                             float* __restrict__ out, PackP pk) {
  constexpr int E = D / 64;
  constexpr int64_t rs = D + 4;
  const int lane = threadIdx.x & 63;
  const int64_t u = (int64_t)blockIdx.x * kCombineWaveUnits + (threadIdx.x >> 6);
  if (u >= units) return;   // whole waves leave; nothing below synchronises the workgroup
  const float* r = part + u * nsplit * rs;
  // the pack's query chunk does not depend on the splits: load it with them
  const uint4 qch = pk.ops ? pack_query_chunk<D>(pk, u, lane) : make_uint4(0, 0, 0, 0);
  const float2 ml = lane < nsplit ? *reinterpret_cast<const float2*>(r + lane * rs) : make_float2(-INFINITY, 0.f);
  float o[CH][E];
#pragma unroll
  for (int k = 0; k < CH; ++k)
#pragma unroll
    for (int e = 0; e < E; ++e) o[k][e] = k < nsplit ? r[k * rs + 4 + lane + 64 * e] : 0.f;
  const float M = group_max<64>(ml.x);
  const float w = ml.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml.x - M);
  const float L = group_sum<64>(ml.y * w);
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int s0 = 0; s0 < nsplit; s0 += CH) {
    if (s0 > 0) {
#pragma unroll
      for (int k = 0; k < CH; ++k)
#pragma unroll
        for (int e = 0; e < E; ++e) o[k][e] = s0 + k < nsplit ? r[(s0 + k) * rs + 4 + lane + 64 * e] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      if (s0 + k < nsplit) {
        const float ws = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), s0 + k));
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = __builtin_fmaf(o[k][e], ws, acc[e]);
      }
    }
  }
  float ov[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    ov[e] = acc[e] / L;
    out[u * D + lane + 64 * e] = ov[e];
  }
  const float lse_u = (M + __log2f(L)) * kLn2;
  if (lse && lane == 0) lse[u] = lse_u;
  if (pk.ops) pack_row_wave_q<D>(pk, u, ov, lse_u, lane, qch);
}

// One wave per row: the MFMA pass-2 operands of window statistics the caller supplies
// (lse natural log [units], O [units, D]), packed exactly as the combine packs them.
template <int D>
__global__ __launch_bounds__(64 * kCombineWaveUnits) void pack_kernel(const float* __restrict__ lse,
                                                                     const float* __restrict__ O, int64_t units,
                                                                     PackP pk) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t u = (int64_t)blockIdx.x * kCombineWaveUnits + (threadIdx.x >> 6);
  if (u >= units) return;
  const uint4 qch = pack_query_chunk<D>(pk, u, lane);   // in flight with the loads below
  float ov[E];
#pragma unroll
  for (int e = 0; e < E; ++e) ov[e] = O[u * D + lane + 64 * e];
  pack_row_wave_q<D>(pk, u, ov, lse[u], lane, qch);
}

hipError_t launch_pack(const float* lse, const float* O, int64_t units, int D, const PackP& pk, hipStream_t st) {
  if (units == 0) return hipSuccess;
  const dim3 grid((unsigned)((units + kCombineWaveUnits - 1) / kCombineWaveUnits));
  if (D == 128)
    KVS_LAUNCH("pack", pack_kernel<128>, grid, dim3(64 * kCombineWaveUnits), 0, st, lse, O, units, pk);
  else if (D == 64)
    KVS_LAUNCH("pack", pack_kernel<64>, grid, dim3(64 * kCombineWaveUnits), 0, st, lse, O, units, pk);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_combine(const float* part, int64_t units, int nsplit, int D, float* lse, float* out,
                          hipStream_t st, const PackP* pack) {
  if (units == 0) return hipSuccess;
  if (nsplit > kMaxSplit) return hipErrorInvalidValue;
  if (D > 128) return hipErrorInvalidValue;
  PackP pk{};
  if (pack) pk = *pack;
  const bool wide = nsplit > kCombineWaveMaxSplit && nsplit <= kCombineWaveMaxSplitWide &&
                    units >= kCombineWaveWideMinUnits;
  if ((nsplit <= kCombineWaveMaxSplit || wide) && (D == 64 || D == 128)) {
    const dim3 grid((unsigned)((units + kCombineWaveUnits - 1) / kCombineWaveUnits));
    const dim3 block(64 * kCombineWaveUnits);
    if (D == 128 && wide)
      KVS_LAUNCH("combine", (combine_wave_kernel<128, 32>), grid, block, 0, st, part, units, nsplit, lse, out, pk);
    else if (D == 128)
      KVS_LAUNCH("combine", (combine_wave_kernel<128, 8>), grid, block, 0, st, part, units, nsplit, lse, out, pk);
    else if (wide)
      KVS_LAUNCH("combine", (combine_wave_kernel<64, 32>), grid, block, 0, st, part, units, nsplit, lse, out, pk);
    else
      KVS_LAUNCH("combine", (combine_wave_kernel<64, 8>), grid, block, 0, st, part, units, nsplit, lse, out, pk);
    return hipGetLastError();
  }
  KVS_LAUNCH("combine", combine_kernel, dim3((unsigned)units), dim3(kCombineThreads), 0, st, part, nsplit, D, lse, out,
             pk);
  return hipGetLastError();
}

// ------------------------------------------------------------------ pass 2 (VALU) --
// Four threads (a quad) per unit; a unit is a candidate pair (m, m+1) or a single slot
// outside the pair region.  Each thread owns a quarter of the head dimension.
template <typename T, int D, bool HAS_N>
__global__ __launch_bounds__(256) void pass2_valu_kernel(P2Args a) {
  constexpr int DQ = D / 4;
  constexpr int E = Elt<T>::kPerChunk;
  const int tid = threadIdx.x;
  const int ql = tid & 3;
  const int64_t u = (int64_t)blockIdx.x * 64 + (tid >> 2);
  const int64_t bh = blockIdx.y;
  const int64_t b = bh / a.Hkv, h = bh - b * a.Hkv;
  const int64_t n_units = a.S + a.P + (a.N - a.S - 2 * a.P);
  if (u >= n_units) return;  // whole quads leave together; only quad shuffles follow
  bool pair;
  int64_t m, p = 0;
  if (u < a.S) {
    pair = false;
    m = u;
  } else if (u < a.S + a.P) {
    pair = true;
    p = u - a.S;
    m = a.S + 2 * p;
  } else {
    pair = false;
    m = a.S + 2 * a.P + (u - a.S - a.P);
  }
  const T* Kp = static_cast<const T*>(a.K) + b * a.sb + h * a.sh;
  const T* Vp = static_cast<const T*>(a.V) + b * a.sb + h * a.sh;
  const int32_t* np = HAS_N ? a.n + (b * a.sb + h * a.sh) / D : nullptr;
  const T* Qp = static_cast<const T*>(a.Qw) + ((b * a.Hq + h * a.G) * (int64_t)a.W) * D;
  const float* Op = a.O + bh * a.GW * (int64_t)D;
  const float* Lp = a.lse + bh * a.GW;

  float k0[DQ], k1[DQ], v0[DQ], v1[DQ];
  for (int d0 = 0; d0 < DQ; d0 += E) {
    unpack<T>(load16(Kp + m * D + ql * DQ + d0), k0 + d0);
    unpack<T>(load16(Vp + m * D + ql * DQ + d0), v0 + d0);
    if (pair) {
      unpack<T>(load16(Kp + (m + 1) * D + ql * DQ + d0), k1 + d0);
      unpack<T>(load16(Vp + (m + 1) * D + ql * DQ + d0), v1 + d0);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) k1[d0 + e] = v1[d0 + e] = 0.f;
    }
  }
  const float b0 = HAS_N ? logf((float)np[m]) : 0.f;
  const float b1 = (HAS_N && pair) ? logf((float)np[m + 1]) : 0.f;
  float gs0 = 0.f, gs1 = 0.f, gx = 0.f;
  for (int64_t w = 0; w < a.GW; ++w) {
    float d0 = 0.f, d1 = 0.f, r0 = 0.f, r1 = 0.f, rc = 0.f;
    for (int c0 = 0; c0 < DQ; c0 += E) {
      float q[E];
      unpack<T>(load16(Qp + w * D + ql * DQ + c0), q);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float o = Op[w * D + ql * DQ + c0 + e];
        const float x0 = v0[c0 + e] - o, x1 = v1[c0 + e] - o, xc = x0 + x1;
        d0 = __builtin_fmaf(q[e], k0[c0 + e], d0);
        d1 = __builtin_fmaf(q[e], k1[c0 + e], d1);
        r0 = __builtin_fmaf(x0, x0, r0);
        r1 = __builtin_fmaf(x1, x1, r1);
        rc = __builtin_fmaf(xc, xc, rc);
      }
    }
    d0 = group_sum<4>(d0);
    r0 = group_sum<4>(r0);
    d1 = group_sum<4>(d1);
    r1 = group_sum<4>(r1);
    rc = group_sum<4>(rc);
    const float lw = Lp[w];
    const float a0 = expf(__builtin_fmaf(a.scale, d0, b0) - lw);
    gs0 = __builtin_fmaf(a0 * fabsf(1.f - 2.f * a0), sqrtf(r0), gs0);
    if (pair) {
      const float a1 = expf(__builtin_fmaf(a.scale, d1, b1) - lw);
      gs1 = __builtin_fmaf(a1 * fabsf(1.f - 2.f * a1), sqrtf(r1), gs1);
      gx = __builtin_fmaf(a0 * a1, sqrtf(rc), gx);
    }
  }
  if (ql == 0) {
    float* gsp = a.g_self + bh * a.N;
    gsp[m] = gs0;
    if (pair) {
      gsp[m + 1] = gs1;
      a.g_cross[bh * a.P + p] = gx;
    }
  }
}

// --------------------------------------------------------- adjacent-key cosine --
// Row layout (LPR lanes per row); every candidate pair of one (b, head) per group step.
template <typename T, int D>
__global__ __launch_bounds__(256) void pair_cos_kernel(CosArgs a) {
  constexpr int E = Elt<T>::kPerChunk;
  constexpr int LPR = D / E;
  constexpr int GPB = 256 / LPR;
  const int tid = threadIdx.x;
  const int grp = tid / LPR, j = tid % LPR;
  const int64_t bh = blockIdx.y;
  const int64_t b = bh / a.Hkv, h = bh - b * a.Hkv;
  const T* Kp = static_cast<const T*>(a.K) + b * a.sb + h * a.sh;
  const int64_t p = (int64_t)blockIdx.x * GPB + grp;
  const bool valid = p < a.P;
  float k0[E], k1[E];
  if (valid) {
    const int64_t m = a.S + 2 * p;
    unpack<T>(load16(Kp + m * D + j * E), k0);
    unpack<T>(load16(Kp + (m + 1) * D + j * E), k1);
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) k0[e] = k1[e] = 0.f;
  }
  const float c = pair_cos<E, LPR>(k0, k1);
  if (valid && j == 0) a.cos[bh * a.P + p] = c;
}

// ------------------------------------------------------------------- launchers --
hipError_t launch_pair_cos(const Shape& s, const CosArgs& ca, int64_t P, hipStream_t st) {
  if (P <= 0) return hipSuccess;
  const int64_t BH = (int64_t)s.B * s.Hkv;
  if (s.bf16) {
    constexpr int GPB128 = 256 / (128 / Elt<bf16>::kPerChunk), GPB64 = 256 / (64 / Elt<bf16>::kPerChunk);
    if (s.D == 128)
      KVS_LAUNCH("pair_cos", (pair_cos_kernel<bf16, 128>), dim3((P + GPB128 - 1) / GPB128, BH), dim3(256), 0, st, ca);
    else
      KVS_LAUNCH("pair_cos", (pair_cos_kernel<bf16, 64>), dim3((P + GPB64 - 1) / GPB64, BH), dim3(256), 0, st, ca);
  } else {
    constexpr int GPB128 = 256 / (128 / Elt<float>::kPerChunk), GPB64 = 256 / (64 / Elt<float>::kPerChunk);
    if (s.D == 128)
      KVS_LAUNCH("pair_cos", (pair_cos_kernel<float, 128>), dim3((P + GPB128 - 1) / GPB128, BH), dim3(256), 0, st, ca);
    else
      KVS_LAUNCH("pair_cos", (pair_cos_kernel<float, 64>), dim3((P + GPB64 - 1) / GPB64, BH), dim3(256), 0, st, ca);
  }
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_score_valu(const Shape& s, const RoundP& r, const P1Args& p1, const P2Args& p2,
                                    const CosArgs& ca, float* lse, float* O, hipStream_t st) {
  const int64_t BH = (int64_t)s.B * s.Hkv;
  const int nqb = (int)((p1.GW + 127) / 128);
  KVS_LAUNCH("score_pass1", (pass1_valu_kernel<T, D>), dim3(p1.nsplit, nqb, BH), dim3(256), 0, st, p1);
  hipError_t e = launch_combine(p1.part, BH * p1.GW, p1.nsplit, D, lse, O, st);
  if (e != hipSuccess) return e;
  if (ca.cos && r.P > 0) {
    constexpr int GPB = 256 / (D / Elt<T>::kPerChunk);
    KVS_LAUNCH("pair_cos", (pair_cos_kernel<T, D>), dim3((r.P + GPB - 1) / GPB, BH), dim3(256), 0, st, ca);
  }
  const int64_t units = r.S + r.P + (s.N - r.S - 2 * r.P);
  if (p2.n)
    KVS_LAUNCH("score_pass2", (pass2_valu_kernel<T, D, true>), dim3((units + 63) / 64, BH), dim3(256), 0, st, p2);
  else
    KVS_LAUNCH("score_pass2", (pass2_valu_kernel<T, D, false>), dim3((units + 63) / 64, BH), dim3(256), 0, st, p2);
  return hipGetLastError();
}

size_t score_workspace_bytes(const Shape& s, const RoundP& r) {
  if (use_mfma_scorer(s)) return mfma_score_workspace_bytes(s, r);
  const int64_t GW = (int64_t)s.G * r.W;
  int64_t chunk;
  int nsplit;
  valu_pass1_plan(s.N, (int64_t)s.B * s.Hkv * ((GW + 127) / 128), chunk, nsplit);
  return (size_t)s.B * s.Hkv * GW * nsplit * (s.D + 4) * sizeof(float);
}

// Pass 2 alone on the VALU kernels, from window statistics the caller supplies.
hipError_t launch_pass2_valu(const Shape& s, const RoundP& r, const void* K, const void* V, const int32_t* n,
                             const void* Qw, const float* lse, const float* O, float* g_self, float* g_cross,
                             hipStream_t st) {
  P2Args p2{};
  p2.K = K;
  p2.V = V;
  p2.n = n;
  p2.Qw = Qw;
  p2.lse = lse;
  p2.O = O;
  p2.g_self = g_self;
  p2.g_cross = g_cross;
  p2.N = s.N;
  p2.S = r.S;
  p2.P = r.P;
  p2.sb = s.sb;
  p2.sh = s.sh;
  p2.Hkv = s.Hkv;
  p2.Hq = s.Hq;
  p2.G = s.G;
  p2.W = r.W;
  p2.GW = (int64_t)s.G * r.W;
  p2.scale = r.scale;
  const int64_t BH = (int64_t)s.B * s.Hkv;
  const int64_t units = r.S + r.P + (s.N - r.S - 2 * r.P);
  const dim3 grid((unsigned)((units + 63) / 64), (unsigned)BH);
#define KVS_P2V(T, D)                                                                        \
  if (p2.n) KVS_LAUNCH("score_pass2", (pass2_valu_kernel<T, D, true>), grid, dim3(256), 0, st, p2); \
  else KVS_LAUNCH("score_pass2", (pass2_valu_kernel<T, D, false>), grid, dim3(256), 0, st, p2);
  if (s.bf16) {
    if (s.D == 64) { KVS_P2V(bf16, 64) } else { KVS_P2V(bf16, 128) }
  } else {
    if (s.D == 64) { KVS_P2V(float, 64) } else { KVS_P2V(float, 128) }
  }
#undef KVS_P2V
  return hipGetLastError();
}

hipError_t launch_score(const Shape& s, const RoundP& r, const void* K, const void* V, const int32_t* n,
                        const void* Qw, float* lse, float* O, float* g_self, float* g_cross, float* cos,
                        void* ws, hipStream_t st) {
  if (use_mfma_scorer(s)) return launch_score_mfma(s, r, K, V, n, Qw, lse, O, g_self, g_cross, cos, ws, st);
  P1Args p1;
  p1.K = K;
  p1.V = V;
  p1.n = n;
  p1.Qw = Qw;
  p1.part = static_cast<float*>(ws);
  p1.N = s.N;
  p1.sb = s.sb;
  p1.sh = s.sh;
  p1.Hkv = s.Hkv;
  p1.Hq = s.Hq;
  p1.G = s.G;
  p1.W = r.W;
  p1.GW = (int64_t)s.G * r.W;
  p1.scale = r.scale;
  valu_pass1_plan(s.N, (int64_t)s.B * s.Hkv * ((p1.GW + 127) / 128), p1.chunk, p1.nsplit);
  P2Args p2;
  p2.K = K;
  p2.V = V;
  p2.n = n;
  p2.Qw = Qw;
  p2.lse = lse;
  p2.O = O;
  p2.g_self = g_self;
  p2.g_cross = g_cross;
  p2.N = s.N;
  p2.S = r.S;
  p2.P = r.P;
  p2.sb = s.sb;
  p2.sh = s.sh;
  p2.Hkv = s.Hkv;
  p2.Hq = s.Hq;
  p2.G = s.G;
  p2.W = r.W;
  p2.GW = p1.GW;
  p2.scale = r.scale;
  CosArgs ca;
  ca.K = K;
  ca.cos = cos;
  ca.S = r.S;
  ca.P = r.P;
  ca.sb = s.sb;
  ca.sh = s.sh;
  ca.Hkv = s.Hkv;
  if (s.bf16)
    return s.D == 64 ? launch_score_valu<bf16, 64>(s, r, p1, p2, ca, lse, O, st)
                     : launch_score_valu<bf16, 128>(s, r, p1, p2, ca, lse, O, st);
  return s.D == 64 ? launch_score_valu<float, 64>(s, r, p1, p2, ca, lse, O, st)
                   : launch_score_valu<float, 128>(s, r, p1, p2, ca, lse, O, st);
}

}  // namespace kvs
