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
  static constexpr int PITCH = D + 8;        // bf16 elements per LDS row (16-byte pad)
  static constexpr int CPR = D / 8;          // 16-byte chunks per row
};

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& u) {
  u32x4_t v = {u.x, u.y, u.z, u.w};
  return __builtin_bit_cast(bf16x8_t, v);
}

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

// Cooperative load of a 64-slot tile of K and V rows [t0, t0+64) into LDS (zeros outside
// [lo, hi)).  NT threads, 16-byte chunks.
template <int D, int NT>
__device__ __forceinline__ void load_tile(const bf16* Kp, const bf16* Vp, int64_t t0, int64_t lo, int64_t hi,
                                          bf16* Kt, bf16* Vt) {
  using C = TileCfg<D>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < kTile * C::CPR / NT; ++it) {
    const int idx = it * NT + tid;
    const int row = idx / C::CPR, ch = idx % C::CPR;
    const int64_t s = t0 + row;
    uint4 k = make_uint4(0, 0, 0, 0), v = make_uint4(0, 0, 0, 0);
    if (s >= lo && s < hi) {
      k = load16(Kp + s * D + ch * 8);
      v = load16(Vp + s * D + ch * 8);
    }
    *reinterpret_cast<uint4*>(Kt + row * C::PITCH + ch * 8) = k;
    *reinterpret_cast<uint4*>(Vt + row * C::PITCH + ch * 8) = v;
  }
}

// Q rows as the B operand: lane l holds Q[q = qbase + l%16][d = 32 kb + 8 (l/16) .. +7].
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

// ------------------------------------------------------------------------- pass 1 --
// grid: x = slot chunk, y = query block (128), z = (b, kv-head); eight waves of 16 queries
// share each LDS tile.  Partial records as the VALU pass 1: {m (log2 units), l, -, -, o[D]}
// per (bh, query, chunk).
template <int D, bool HAS_N>
__global__ __launch_bounds__(512, 1) void p1_mfma_kernel(P1Args a, int64_t base, CosArgs ca) {
  using C = TileCfg<D>;
  __shared__ __attribute__((aligned(16))) bf16 Kt[kTile * C::PITCH];
  __shared__ __attribute__((aligned(16))) bf16 Vt[kTile * C::PITCH];
  __shared__ float lg[kTile];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int64_t bh = blockIdx.z;
  const int64_t b = bh / a.Hkv, h = bh - b * a.Hkv;
  const bf16* Kp = static_cast<const bf16*>(a.K) + b * a.sb + h * a.sh;
  const bf16* Vp = static_cast<const bf16*>(a.V) + b * a.sb + h * a.sh;
  const int32_t* np = HAS_N ? a.n + (b * a.sb + h * a.sh) / D : nullptr;
  const bf16* Qp = static_cast<const bf16*>(a.Qw) + ((b * a.Hq + h * a.G) * (int64_t)a.W) * D;

  const int64_t q0 = (int64_t)blockIdx.y * kQB + wv * 16;
  bf16x8_t qop[1][C::KB];
  load_q<D>(Qp, a.GW, q0 + c16, qop[0]);

  const float cs = a.scale * kLog2e;
  float m[1] = {-INFINITY}, lsum[1] = {0.f};
  f32x4_t acc[1][C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[0][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int64_t c0 = base + (int64_t)blockIdx.x * a.chunk;
  const int64_t c1 = c0 + a.chunk;
  const int64_t lo = c0 > 0 ? c0 : 0;
  const int64_t hi = c1 < a.N ? c1 : a.N;
  const bool do_cos = ca.cos != nullptr && blockIdx.y == 0;

  for (int64_t t0 = c0; t0 < c1 && t0 < a.N; t0 += kTile) {
    __syncthreads();
    load_tile<D, 512>(Kp, Vp, t0, lo, hi, Kt, Vt);
    if (tid < kTile) {
      const int64_t s = t0 + tid;
      lg[tid] = (s >= lo && s < hi) ? (HAS_N ? __log2f((float)np[s]) : 0.f) : -INFINITY;
    }
    __syncthreads();

    // adjacent-key cosine of the tile's candidate pairs (row layout: 16 lanes x 8 elements)
    if (do_cos) {
      constexpr int LPR = D / 8;
      constexpr int GPB = 512 / LPR;
      const int grp = tid / LPR, j = tid % LPR;
#pragma unroll
      for (int pp0 = 0; pp0 < kTile / 2; pp0 += GPB) {
        const int pp = (pp0 + grp) & (kTile / 2 - 1);   // groups beyond the tile's pairs repeat a pair, unwritten
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

    // per query block: S^T = K . Q^T over the tile (4 slot blocks), then the online
    // softmax for the lane's query (lane % 16) over slots 16 sb + 4 g + r
    {
      constexpr int qb = 0;
      f32x4_t st[4];
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) {
        st[sb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) {
          const bf16x8_t ak =
              as_bf16x8(*reinterpret_cast<const uint4*>(Kt + (sb * 16 + c16) * C::PITCH + kb * 32 + g * 8));
          st[sb] = mfma(ak, qop[qb][kb], st[sb]);
        }
      }
      float e[4][4];
      float mx = -INFINITY;
#pragma unroll
      for (int sb = 0; sb < 4; ++sb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          e[sb][r] = __builtin_fmaf(st[sb][r], cs, lg[sb * 16 + g * 4 + r]);
          mx = fmaxf(mx, e[sb][r]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mn = fmaxf(m[qb], mx);
      const float corr = (m[qb] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[qb] - mn);
      m[qb] = mn;
      lsum[qb] *= corr;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) acc[qb][db] *= corr;
      float p[4][4];
#pragma unroll
      for (int sb = 0; sb < 4; ++sb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[sb][r] = (mn == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(e[sb][r] - mn);
          lsum[qb] += p[sb][r];
        }
      // O^T += V^T . P^T, two 32-slot halves; k index j <-> slot 32 h + 16 (j / 4) + 4 g + j % 4
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
        // source lane i = lane % 16 points at row 32 hf + 16 half2 + 4 g + i / 4, cols 16 db + 4 (i % 4)
        const int srow = 32 * hf + 4 * g + (c16 >> 2);
        const int scol = 4 * (c16 & 3);
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;
          const bf16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (lds_bf16x4*)(Vt + srow * C::PITCH + db * 16 + scol));
          const bf16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (lds_bf16x4*)(Vt + (srow + 16) * C::PITCH + db * 16 + scol));
          const bf16x8_t vop = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
          acc[qb][db] = mfma(vop, phi, acc[qb][db]);
          acc[qb][db] = mfma(vop, plo, acc[qb][db]);
        }
      }
    }
  }

  // per-query partial record: the four lane groups hold disjoint slots of the same query
  {
    constexpr int qb = 0;
    float l = lsum[qb];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int64_t q = q0 + c16;
    if (q < a.GW) {
      float* rec = a.part + ((bh * a.GW + q) * a.nsplit + blockIdx.x) * (int64_t)(D + 4);
      if (g == 0) {
        rec[0] = m[qb];
        rec[1] = l;
      }
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) rec[4 + db * 16 + g * 4 + r] = acc[qb][db][r];
    }
  }
}

// ------------------------------------------------------------------------- pass 2 --
// grid: x = slot chunk, y = query block (128), z = (b, kv-head).  With more than one query
// block the per-slot sums are accumulated with atomics (not the case for <= 128 queries).
template <int D, bool HAS_N>
__global__ __launch_bounds__(256, 2) void p2_mfma_kernel(P2Args a, int64_t base, int64_t chunk) {
  using C = TileCfg<D>;
  __shared__ __attribute__((aligned(16))) bf16 Kt[kTile * C::PITCH];
  __shared__ __attribute__((aligned(16))) bf16 Vt[kTile * C::PITCH];
  __shared__ float lg[kTile];
  __shared__ float vn[kTile];
  __shared__ float dv[kTile / 2];
  __shared__ float red_s[4][kTile];
  __shared__ float red_x[4][kTile / 2];

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

  const int64_t q0 = (int64_t)blockIdx.y * kQB + wv * 32;
  bf16x8_t qop[2][C::KB], ohi[2][C::KB], olo[2][C::KB];
  float nb[2], on[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int64_t q = q0 + qb * 16 + c16;
    load_q<D>(Qp, a.GW, q, qop[qb]);
    float s2 = 0.f;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
      float o8[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float ov = q < a.GW ? Op[q * D + kb * 32 + g * 8 + j] : 0.f;
        s2 = __builtin_fmaf(ov, ov, s2);
        o8[j] = -2.f * ov;
      }
      split_hi_lo(o8, ohi[qb][kb], olo[qb][kb]);
    }
    s2 += __shfl_xor(s2, 16, 64);
    s2 += __shfl_xor(s2, 32, 64);
    on[qb] = s2;
    // alpha = exp2(cs * s + log2 n - lse * log2e); padded queries get alpha = 0
    nb[qb] = q < a.GW ? -Lp[q] * kLog2e : -INFINITY;
  }
  const float cs = a.scale * kLog2e;

  const int64_t c0 = base + (int64_t)blockIdx.x * chunk;
  const int64_t c1 = c0 + chunk;
  const int64_t lo = c0 > 0 ? c0 : 0;
  const int64_t hi = c1 < a.N ? c1 : a.N;

  for (int64_t t0 = c0; t0 < c1 && t0 < a.N; t0 += kTile) {
    __syncthreads();
    load_tile<D, 256>(Kp, Vp, t0, lo, hi, Kt, Vt);
    if (tid < kTile) {
      const int64_t s = t0 + tid;
      lg[tid] = (s >= lo && s < hi) ? (HAS_N ? __log2f((float)np[s]) : 0.f) : -INFINITY;
    }
    __syncthreads();
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
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      f32x4_t st[2], rt[2];
      st[0] = st[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 4; ++r) rt[qb][r] = vn[sb * 16 + g * 4 + r] + on[qb];
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        const bf16x8_t ak = as_bf16x8(*reinterpret_cast<const uint4*>(Kt + (sb * 16 + c16) * C::PITCH + kb * 32 + g * 8));
        const bf16x8_t av = as_bf16x8(*reinterpret_cast<const uint4*>(Vt + (sb * 16 + c16) * C::PITCH + kb * 32 + g * 8));
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          st[qb] = mfma(ak, qop[qb][kb], st[qb]);
          rt[qb] = mfma(av, ohi[qb][kb], rt[qb]);
          rt[qb] = mfma(av, olo[qb][kb], rt[qb]);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) gs[sb][r] = 0.f;
      gx[sb][0] = gx[sb][1] = 0.f;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float al[4], r2[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = __builtin_fmaf(st[qb][r], cs, lg[sb * 16 + g * 4 + r] + nb[qb]);
          al[r] = __builtin_amdgcn_exp2f(e);
          r2[r] = fmaxf(rt[qb][r], 0.f);
          const float t = al[r] * fabsf(__builtin_fmaf(-2.f, al[r], 1.f));
          gs[sb][r] = __builtin_fmaf(t, __builtin_amdgcn_sqrtf(r2[r]), gs[sb][r]);
        }
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          const float rc = fmaxf(__builtin_fmaf(2.f, r2[2 * pr] + r2[2 * pr + 1], -dv[sb * 8 + g * 2 + pr]), 0.f);
          gx[sb][pr] = __builtin_fmaf(al[2 * pr] * al[2 * pr + 1], __builtin_amdgcn_sqrtf(rc), gx[sb][pr]);
        }
      }
    }
    // sum over the 16 queries of each lane row, then over the four waves
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
        const float v = red_s[0][tid] + red_s[1][tid] + red_s[2][tid] + red_s[3][tid];
        if (gridDim.y == 1) a.g_self[bh * a.N + s] = v;
        else atomicAdd(&a.g_self[bh * a.N + s], v);
      }
    } else if (tid < kTile + kTile / 2) {
      const int pp = tid - kTile;
      const int64_t m0 = t0 + 2 * pp;
      const int64_t p = (m0 - a.S) / 2;
      if (m0 >= a.S && m0 >= lo && m0 + 1 < hi && p < a.P) {
        const float v = red_x[0][pp] + red_x[1][pp] + red_x[2][pp] + red_x[3][pp];
        if (gridDim.y == 1) a.g_cross[bh * a.P + p] = v;
        else atomicAdd(&a.g_cross[bh * a.P + p], v);
      }
    }
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
    hipLaunchKernelGGL((p1_mfma_kernel<D, true>), grid, dim3(512), 0, st, p1, base, ca);
  else
    hipLaunchKernelGGL((p1_mfma_kernel<D, false>), grid, dim3(512), 0, st, p1, base, ca);
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
    hipLaunchKernelGGL((p2_mfma_kernel<D, true>), grid, dim3(256), 0, st, p2, base, p1.chunk);
  else
    hipLaunchKernelGGL((p2_mfma_kernel<D, false>), grid, dim3(256), 0, st, p2, base, p1.chunk);
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
