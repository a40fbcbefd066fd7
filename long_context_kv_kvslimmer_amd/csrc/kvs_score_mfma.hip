// bf16 MFMA scorer for gfx950 (the math is stated in kvs_score.hip).
//
// Both passes tile one (batch, kv-head) as [window queries] x [slots]; a workgroup owns a
// contiguous slot chunk and up to 128 window queries, four waves of 32 queries each, and
// stages 64-slot K and V tiles in LDS (row pitch padded to keep ds_read_b128 conflict-free).
// All contractions run on v_mfma_f32_16x16x32_bf16, always in the transposed form
// (slots or head-dim as the M side, queries as the N side) so that every lane's results
// belong to ONE query, lane % 16:
//
//   S^T[slot, q]  = K . Q^T            A = K tile rows (ds_read_b128), B = Q rows (registers)
//   pass 1:  O^T[d, q] += V^T . P^T    A = V^T via ds_read_tr16_b64 (LDS transpose read),
//                                      B = P^T straight from the S^T registers; P is split
//                                      into bf16 hi + lo parts so the product keeps ~16 bits
//   pass 2:  R^T[slot, q] = V . (-2 O)^T + ||v||^2 + ||o||^2   (accumulator pre-loaded),
//                                      giving ||v_i - o_w||^2 directly; -2 O split hi + lo
//
// Pass 1 also writes the adjacent-key cosine (the shared pair_cos routine on LDS rows in
// row layout), so the merge pass can recompute bit-identical values.
#include "kvs_common.h"
#include "kvs_score_impl.h"

namespace kvs {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kTile = 64;      // slots per LDS tile
constexpr int kQB = 128;       // window queries per workgroup (4 waves x 32)

template <int D>
struct TileCfg {
  static constexpr int KB = D / 32;          // 32-wide k blocks of the head dim
  static constexpr int DB = D / 16;          // 16-wide blocks of the head dim
  // bf16 elements per LDS row: a 32-byte pad moves consecutive rows 8 banks apart, so the
  // 16-byte row reads (8 lanes per cycle) and the 4-row transpose reads are conflict-free
  static constexpr int PITCH = D + 16;
  static constexpr int CPR = D / 8;          // 16-byte chunks per row
};

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& u) {
  u32x4_t v = {u.x, u.y, u.z, u.w};
  return __builtin_bit_cast(bf16x8_t, v);
}

// Finite stand-in for "no maximum yet": exp2(x - kNoMax) underflows to 0 for any finite x,
// and exp2(-inf - kNoMax) is 0 as well, so masked slots need no special case.
constexpr float kNoMax = -1e30f;

__device__ __forceinline__ f32x4_t mfma(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Split 8 floats into bf16 hi (RNE) and lo = bf16(x - hi).
__device__ __forceinline__ void split_hi_lo(const float* x, bf16x8_t& hi, bf16x8_t& lo) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const __bf16 h = (__bf16)x[j];
    hi[j] = h;
    lo[j] = (__bf16)(x[j] - (float)h);
  }
}

// Register-staged tile of K and V rows [t0, t0 + 64): each of NT threads fetches its
// 16-byte chunks (zeros outside [lo, hi)) so the loads stay in flight while the previous
// tile is computed, then commits them to LDS.
template <int D, int NT>
struct TileStage {
  using C = TileCfg<D>;
  static constexpr int NPT = kTile * C::CPR / NT;
  uint4 k[NPT], v[NPT];
  float lg;

  template <bool HAS_N>
  __device__ __forceinline__ void fetch(const bf16* Kp, const bf16* Vp, const int32_t* np, int64_t t0, int64_t lo,
                                        int64_t hi) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int it = 0; it < NPT; ++it) {
      const int idx = it * NT + tid;
      const int row = idx / C::CPR, ch = idx % C::CPR;
      const int64_t s = t0 + row;
      if (s >= lo && s < hi) {
        k[it] = load16(Kp + s * D + ch * 8);
        v[it] = load16(Vp + s * D + ch * 8);
      } else {
        k[it] = v[it] = make_uint4(0, 0, 0, 0);
      }
    }
    if (tid < kTile) {
      const int64_t s = t0 + tid;
      lg = (s >= lo && s < hi) ? (HAS_N ? __log2f((float)np[s]) : 0.f) : -INFINITY;
    }
  }

  __device__ __forceinline__ void commit(bf16* Kt, bf16* Vt, float* lgs) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int it = 0; it < NPT; ++it) {
      const int idx = it * NT + tid;
      const int row = idx / C::CPR, ch = idx % C::CPR;
      *reinterpret_cast<uint4*>(Kt + row * C::PITCH + ch * 8) = k[it];
      *reinterpret_cast<uint4*>(Vt + row * C::PITCH + ch * 8) = v[it];
    }
    if (tid < kTile) lgs[tid] = lg;
  }
};

// Q (or any fp32-free bf16 row block) as an MFMA operand: lane l holds
// Q[q = l%16][d = 32 kb + 8 (l/16) .. +7] of the 16 rows starting at query q.
template <int D>
__device__ __forceinline__ void load_q(const bf16* Qp, int64_t GW, int64_t q, bf16x8_t (&qop)[TileCfg<D>::KB]) {
  const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int kb = 0; kb < TileCfg<D>::KB; ++kb) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (q < GW) u = load16(Qp + q * D + kb * 32 + g * 8);
    qop[kb] = as_bf16x8(u);
  }
}

constexpr int kThreads = 512;   // 8 waves x 16 window queries

// ------------------------------------------------------------------------- pass 1 --
// grid: x = slot chunk, y = query block (128), z = (b, kv-head); eight waves of 16 queries
// share each LDS tile.  Partial records as the VALU pass 1: {m (log2 units), l, -, -, o[D]}
// per (bh, query, chunk).
template <int D, bool HAS_N>
__global__ __launch_bounds__(kThreads, 1) void p1_mfma_kernel(P1Args a, int64_t base, CosArgs ca) {
  using C = TileCfg<D>;
  __shared__ __attribute__((aligned(16))) bf16 Kt[kTile * C::PITCH];
  __shared__ __attribute__((aligned(16))) bf16 Vt[kTile * C::PITCH];
  __shared__ __attribute__((aligned(16))) float lgs[kTile];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int64_t bh = blockIdx.z;
  const int64_t b = bh / a.Hkv, h = bh - b * a.Hkv;
  const bf16* Kp = static_cast<const bf16*>(a.K) + b * a.sb + h * a.sh;
  const bf16* Vp = static_cast<const bf16*>(a.V) + b * a.sb + h * a.sh;
  const int32_t* np = HAS_N ? a.n + (b * a.sb + h * a.sh) / D : nullptr;
  const bf16* Qp = static_cast<const bf16*>(a.Qw) + ((b * a.Hq + h * a.G) * (int64_t)a.W) * D;

  const int64_t q0 = (int64_t)blockIdx.y * kQB + wv * 16;
  bf16x8_t qop[C::KB];
  load_q<D>(Qp, a.GW, q0 + c16, qop);

  const float cs = a.scale * kLog2e;
  float m = kNoMax, lsum = 0.f;
  f32x4_t acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int64_t c0 = base + (int64_t)blockIdx.x * a.chunk;
  const int64_t c1 = c0 + a.chunk;
  const int64_t lo = c0 > 0 ? c0 : 0;
  const int64_t hi = c1 < a.N ? c1 : a.N;
  const int64_t tend = c1 < a.N ? c1 : a.N;
  const bool do_cos = ca.cos != nullptr && blockIdx.y == 0;

  // two register stages keep two tiles (64 KB) of loads in flight per workgroup
  auto compute = [&](int64_t t0) {

    // adjacent-key cosine of the tile's candidate pairs (row layout: LPR lanes x 8 elements)
    if (do_cos) {
      constexpr int LPR = D / 8;
      constexpr int GPB = kThreads / LPR;
      const int grp = tid / LPR, j = tid % LPR;
#pragma unroll
      for (int pp0 = 0; pp0 < kTile / 2; pp0 += GPB) {
        const int pp = (pp0 + grp) & (kTile / 2 - 1);   // surplus groups repeat a pair and write nothing
        const int64_t m0 = t0 + 2 * pp;
        float k0[8], k1[8];
        unpack<bf16>(*reinterpret_cast<const uint4*>(Kt + (2 * pp) * C::PITCH + j * 8), k0);
        unpack<bf16>(*reinterpret_cast<const uint4*>(Kt + (2 * pp + 1) * C::PITCH + j * 8), k1);
        const float cv = pair_cos<8, LPR>(k0, k1);
        const int64_t p = (m0 - ca.S) / 2;
        if (j == 0 && pp0 + grp < kTile / 2 && m0 >= ca.S && p < ca.P && m0 >= lo && m0 + 1 < hi)
          ca.cos[bh * ca.P + p] = cv;
      }
    }

    // S^T = K . Q^T over the tile (4 slot blocks); online softmax for the lane's query
    f32x4_t st[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      st[sb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        const bf16x8_t ak =
            as_bf16x8(*reinterpret_cast<const uint4*>(Kt + (sb * 16 + c16) * C::PITCH + kb * 32 + g * 8));
        st[sb] = mfma(ak, qop[kb], st[sb]);
      }
    }
    float e[4][4];
    float mx = kNoMax;
    const bool plain = !HAS_N && t0 >= lo && t0 + kTile <= hi;   // every slot valid, count 1
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      const float4 lg4 = plain ? make_float4(0.f, 0.f, 0.f, 0.f)
                               : *reinterpret_cast<const float4*>(lgs + sb * 16 + g * 4);
      const float lgv[4] = {lg4.x, lg4.y, lg4.z, lg4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        e[sb][r] = __builtin_fmaf(st[sb][r], cs, lgv[r]);
        mx = fmaxf(mx, e[sb][r]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (mx > m) {   // rescale only when the running max grows (finite sentinel: no NaN paths)
      const float corr = __builtin_amdgcn_exp2f(m - mx);
      lsum *= corr;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) acc[db] *= corr;
      m = mx;
    }
    float p[4][4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[sb][r] = __builtin_amdgcn_exp2f(e[sb][r] - m);
        lsum += p[sb][r];
      }
    // O^T += V^T . P^T, two 32-slot halves; k index j <-> slot 32 hf + 16 (j / 4) + 4 g + j % 4
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      float pv[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pv[r] = p[2 * hf][r];
        pv[4 + r] = p[2 * hf + 1][r];
      }
      bf16x8_t phi, plo;
      split_hi_lo(pv, phi, plo);
      // transposed read: source lane i = lane % 16 points at row 32 hf + 4 g + i / 4 (+16),
      // columns 16 db + 4 (i % 4); lane t receives column 16 db + t of four consecutive rows
      const int srow = 32 * hf + 4 * g + (c16 >> 2);
      const int scol = 4 * (c16 & 3);
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;
        const bf16x4_t v0 =
            __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(Vt + srow * C::PITCH + db * 16 + scol));
        const bf16x4_t v1 =
            __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(Vt + (srow + 16) * C::PITCH + db * 16 + scol));
        const bf16x8_t vop = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        acc[db] = mfma(vop, phi, acc[db]);
        acc[db] = mfma(vop, plo, acc[db]);
      }
    }
  };
  TileStage<D, kThreads> sa, sb2;
  sa.template fetch<HAS_N>(Kp, Vp, np, c0, lo, hi);
  if (c0 + kTile < tend) sb2.template fetch<HAS_N>(Kp, Vp, np, c0 + kTile, lo, hi);
  for (int64_t t0 = c0; t0 < tend; t0 += 2 * kTile) {
    __syncthreads();
    sa.commit(Kt, Vt, lgs);
    __syncthreads();
    if (t0 + 2 * kTile < tend) sa.template fetch<HAS_N>(Kp, Vp, np, t0 + 2 * kTile, lo, hi);
    compute(t0);
    if (t0 + kTile >= tend) break;
    __syncthreads();
    sb2.commit(Kt, Vt, lgs);
    __syncthreads();
    if (t0 + 3 * kTile < tend) sb2.template fetch<HAS_N>(Kp, Vp, np, t0 + 3 * kTile, lo, hi);
    compute(t0 + kTile);
  }

  // per-query partial record: the four lane groups hold disjoint slots of the same query
  float l = lsum;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  const int64_t q = q0 + c16;
  if (q < a.GW) {
    float* rec = a.part + ((bh * a.GW + q) * a.nsplit + blockIdx.x) * (int64_t)(D + 4);
    if (g == 0) {
      rec[0] = m;
      rec[1] = l;
    }
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) rec[4 + db * 16 + g * 4 + r] = acc[db][r];
  }
}

// ------------------------------------------------------------------------- pass 2 --
// grid: x = slot chunk, y = query block (128), z = (b, kv-head); eight waves of 16 queries.
// With more than one query block the per-slot sums are accumulated with atomics (not the
// case for <= 128 window queries per kv head).
template <int D, bool HAS_N>
__global__ __launch_bounds__(kThreads, 1) void p2_mfma_kernel(P2Args a, int64_t base, int64_t chunk) {
  using C = TileCfg<D>;
  constexpr int NW = kThreads / 64;
  __shared__ __attribute__((aligned(16))) bf16 Kt[kTile * C::PITCH];
  __shared__ __attribute__((aligned(16))) bf16 Vt[kTile * C::PITCH];
  __shared__ __attribute__((aligned(16))) float lgs[kTile];
  __shared__ float vn[kTile];
  __shared__ float dv[kTile / 2];
  __shared__ float red_s[NW][kTile];
  __shared__ float red_x[NW][kTile / 2];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int64_t bh = blockIdx.z;
  const int64_t b = bh / a.Hkv, h = bh - b * a.Hkv;
  const bf16* Kp = static_cast<const bf16*>(a.K) + b * a.sb + h * a.sh;
  const bf16* Vp = static_cast<const bf16*>(a.V) + b * a.sb + h * a.sh;
  const int32_t* np = HAS_N ? a.n + (b * a.sb + h * a.sh) / D : nullptr;
  const bf16* Qp = static_cast<const bf16*>(a.Qw) + ((b * a.Hq + h * a.G) * (int64_t)a.W) * D;
  const float* Op = a.O + bh * a.GW * (int64_t)D;
  const float* Lp = a.lse + bh * a.GW;

  // the wave's 16 queries: Q and -2 O (hi + lo) as MFMA operands, ||o||^2, -lse in log2 units
  const int64_t q = (int64_t)blockIdx.y * kQB + wv * 16 + c16;
  bf16x8_t qop[C::KB], ohi[C::KB], olo[C::KB];
  load_q<D>(Qp, a.GW, q, qop);
  float on = 0.f;
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb) {
    float o8[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float ov = q < a.GW ? Op[q * D + kb * 32 + g * 8 + j] : 0.f;
      on = __builtin_fmaf(ov, ov, on);
      o8[j] = -2.f * ov;
    }
    split_hi_lo(o8, ohi[kb], olo[kb]);
  }
  on += __shfl_xor(on, 16, 64);
  on += __shfl_xor(on, 32, 64);
  const float nb = q < a.GW ? -Lp[q] * kLog2e : -INFINITY;   // padded queries get alpha = 0
  const float cs = a.scale * kLog2e;

  const int64_t c0 = base + (int64_t)blockIdx.x * chunk;
  const int64_t c1 = c0 + chunk;
  const int64_t lo = c0 > 0 ? c0 : 0;
  const int64_t hi = c1 < a.N ? c1 : a.N;
  const int64_t tend = c1 < a.N ? c1 : a.N;

  auto compute = [&](int64_t t0) {
    // per-slot ||v||^2 and per-pair ||v_m - v_{m+1}||^2: 4 threads per pair, D/4 elements each
    if (tid < 128) {
      const int pp = tid >> 2, qd = tid & 3;
      float s0 = 0.f, s1 = 0.f, sd = 0.f;
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        float x0[8], x1[8];
        unpack<bf16>(*reinterpret_cast<const uint4*>(Vt + (2 * pp) * C::PITCH + qd * (D / 4) + c * 8), x0);
        unpack<bf16>(*reinterpret_cast<const uint4*>(Vt + (2 * pp + 1) * C::PITCH + qd * (D / 4) + c * 8), x1);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          s0 = __builtin_fmaf(x0[j], x0[j], s0);
          s1 = __builtin_fmaf(x1[j], x1[j], s1);
          const float d = x0[j] - x1[j];
          sd = __builtin_fmaf(d, d, sd);
        }
      }
      s0 = group_sum<4>(s0);
      s1 = group_sum<4>(s1);
      sd = group_sum<4>(sd);
      if (qd == 0) {
        vn[2 * pp] = s0;
        vn[2 * pp + 1] = s1;
        dv[pp] = sd;
      }
    }
    __syncthreads();

    float gs[4][4], gx[4][2];
    const bool plain = !HAS_N && t0 >= lo && t0 + kTile <= hi;   // every slot valid, count 1
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      f32x4_t st = f32x4_t{0.f, 0.f, 0.f, 0.f}, rt;
#pragma unroll
      for (int r = 0; r < 4; ++r) rt[r] = vn[sb * 16 + g * 4 + r] + on;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        const bf16x8_t ak =
            as_bf16x8(*reinterpret_cast<const uint4*>(Kt + (sb * 16 + c16) * C::PITCH + kb * 32 + g * 8));
        const bf16x8_t av =
            as_bf16x8(*reinterpret_cast<const uint4*>(Vt + (sb * 16 + c16) * C::PITCH + kb * 32 + g * 8));
        st = mfma(ak, qop[kb], st);
        rt = mfma(av, ohi[kb], rt);
        rt = mfma(av, olo[kb], rt);
      }
      float al[4], r2[4];
      const float4 lg4 = plain ? make_float4(0.f, 0.f, 0.f, 0.f)
                               : *reinterpret_cast<const float4*>(lgs + sb * 16 + g * 4);
      const float lgv[4] = {lg4.x, lg4.y, lg4.z, lg4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = __builtin_fmaf(st[r], cs, lgv[r] + nb);
        al[r] = __builtin_amdgcn_exp2f(e);
        r2[r] = fmaxf(rt[r], 0.f);
        gs[sb][r] = al[r] * fabsf(__builtin_fmaf(-2.f, al[r], 1.f)) * __builtin_amdgcn_sqrtf(r2[r]);
      }
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const float rc = fmaxf(__builtin_fmaf(2.f, r2[2 * pr] + r2[2 * pr + 1], -dv[sb * 8 + g * 2 + pr]), 0.f);
        gx[sb][pr] = al[2 * pr] * al[2 * pr + 1] * __builtin_amdgcn_sqrtf(rc);
      }
    }
    // sum over the 16 queries of each lane row (DPP), then over the waves (LDS)
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) gs[sb][r] = group_sum<16>(gs[sb][r]);
      gx[sb][0] = group_sum<16>(gx[sb][0]);
      gx[sb][1] = group_sum<16>(gx[sb][1]);
    }
    if (c16 == 0) {
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) red_s[wv][sb * 16 + g * 4 + r] = gs[sb][r];
        red_x[wv][sb * 8 + g * 2] = gx[sb][0];
        red_x[wv][sb * 8 + g * 2 + 1] = gx[sb][1];
      }
    }
    __syncthreads();
    if (tid < kTile) {
      const int64_t s = t0 + tid;
      if (s >= lo && s < hi) {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) v += red_s[w][tid];
        if (gridDim.y == 1) a.g_self[bh * a.N + s] = v;
        else atomicAdd(&a.g_self[bh * a.N + s], v);
      }
    } else if (tid < kTile + kTile / 2) {
      const int pp = tid - kTile;
      const int64_t m0 = t0 + 2 * pp;
      const int64_t p = (m0 - a.S) / 2;
      if (m0 >= a.S && m0 >= lo && m0 + 1 < hi && p < a.P) {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) v += red_x[w][pp];
        if (gridDim.y == 1) a.g_cross[bh * a.P + p] = v;
        else atomicAdd(&a.g_cross[bh * a.P + p], v);
      }
    }
  };
  TileStage<D, kThreads> sa, sb2;
  sa.template fetch<HAS_N>(Kp, Vp, np, c0, lo, hi);
  if (c0 + kTile < tend) sb2.template fetch<HAS_N>(Kp, Vp, np, c0 + kTile, lo, hi);
  for (int64_t t0 = c0; t0 < tend; t0 += 2 * kTile) {
    __syncthreads();
    sa.commit(Kt, Vt, lgs);
    __syncthreads();
    if (t0 + 2 * kTile < tend) sa.template fetch<HAS_N>(Kp, Vp, np, t0 + 2 * kTile, lo, hi);
    compute(t0);
    if (t0 + kTile >= tend) break;
    __syncthreads();
    sb2.commit(Kt, Vt, lgs);
    __syncthreads();
    if (t0 + 3 * kTile < tend) sb2.template fetch<HAS_N>(Kp, Vp, np, t0 + 3 * kTile, lo, hi);
    compute(t0 + kTile);
  }
}

// -------------------------------------------------------------------- dispatch --
bool use_mfma_scorer(const Shape& s) { return s.bf16 && (s.D == 64 || s.D == 128); }

// Chunk plan shared by both passes: slot chunks are multiples of the tile, start at
// base = -(S mod 2) so that every tile starts on a candidate-pair boundary, and number
// about 2 chunks per CU over the whole grid.
static void mfma_plan(const Shape& s, const RoundP& r, int64_t& base, int64_t& chunk, int& nsplit) {
  base = -(r.S & 1);
  const int64_t span = s.N - base;
  const int64_t BH = (int64_t)s.B * s.Hkv;
  const int64_t nqb = ((int64_t)s.G * r.W + kQB - 1) / kQB;
  int64_t want = (512 + BH * nqb - 1) / (BH * nqb);   // target chunks per (bh, query block)
  if (want < 1) want = 1;
  int64_t c = (span + want - 1) / want;
  if (c < 1024) c = 1024;                               // keep partial records small
  c = (c + kTile - 1) / kTile * kTile;
  chunk = c;
  nsplit = (int)((span + c - 1) / c);
}

size_t mfma_score_workspace_bytes(const Shape& s, const RoundP& r) {
  int64_t base, chunk;
  int nsplit;
  mfma_plan(s, r, base, chunk, nsplit);
  const int64_t GW = (int64_t)s.G * r.W;
  return (size_t)s.B * s.Hkv * GW * nsplit * (s.D + 4) * sizeof(float);
}

template <int D>
static hipError_t launch_mfma_d(const Shape& s, const RoundP& r, const P1Args& p1, const P2Args& p2,
                                const CosArgs& ca, int64_t base, float* lse, float* O, hipStream_t st) {
  const int64_t BH = (int64_t)s.B * s.Hkv;
  const int nqb = (int)((p1.GW + kQB - 1) / kQB);
  const dim3 grid(p1.nsplit, nqb, (unsigned)BH);
  if (p1.n)
    hipLaunchKernelGGL((p1_mfma_kernel<D, true>), grid, dim3(kThreads), 0, st, p1, base, ca);
  else
    hipLaunchKernelGGL((p1_mfma_kernel<D, false>), grid, dim3(kThreads), 0, st, p1, base, ca);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_combine(p1.part, BH * p1.GW, p1.nsplit, D, lse, O, st);
  if (e != hipSuccess) return e;
  if (nqb > 1) {
    // several query blocks accumulate into the same sums
    e = launch_fill_zero(p2.g_self, BH * s.N, st);
    if (e == hipSuccess) e = launch_fill_zero(p2.g_cross, BH * r.P, st);
    if (e != hipSuccess) return e;
  }
  if (p2.n)
    hipLaunchKernelGGL((p2_mfma_kernel<D, true>), grid, dim3(kThreads), 0, st, p2, base, p1.chunk);
  else
    hipLaunchKernelGGL((p2_mfma_kernel<D, false>), grid, dim3(kThreads), 0, st, p2, base, p1.chunk);
  return hipGetLastError();
}

hipError_t launch_score_mfma(const Shape& s, const RoundP& r, const void* K, const void* V, const int32_t* n,
                             const void* Qw, float* lse, float* O, float* g_self, float* g_cross, float* cos,
                             void* ws, hipStream_t st) {
  int64_t base;
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
  mfma_plan(s, r, base, p1.chunk, p1.nsplit);
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
  ca.cos = r.P > 0 ? cos : nullptr;
  ca.S = r.S;
  ca.P = r.P;
  ca.sb = s.sb;
  ca.sh = s.sh;
  ca.Hkv = s.Hkv;
  return s.D == 64 ? launch_mfma_d<64>(s, r, p1, p2, ca, base, lse, O, st)
                   : launch_mfma_d<128>(s, r, p1, p2, ca, base, lse, O, st);
}

}  // namespace kvs
