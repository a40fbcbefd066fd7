// bf16 MFMA scorer for gfx950 (the math is stated in kvs_score.hip).
//
// Both passes tile one (batch, kv-head) as [window queries] x [slots]: a workgroup owns a
// contiguous slot chunk and up to 128 window queries, and streams 32-slot K and V tiles
// through LDS rings (16-byte buffer loads written straight to LDS, rows XOR-swizzled).
// Every contraction runs in transposed form (slots or head-dim as the M side, queries as
// the N side), so each lane's results belong to one query:
//
//   pass 1 (v_mfma_f32_32x32x16):  S^T[slot, q] = K . Q^T in bf16, then
//            O^T[d, q] += V^T . P^T in f16: V^T by LDS transpose reads of the tile, which
//            the group converts to f16 in place once it has landed, P^T straight from the
//            S^T registers
//   pass 2 (v_mfma_f32_16x16x32_bf16):  S[q, slot] = Q . K^T and
//            R^T[slot, q] = V . (-2 O)^T + ||o||^2 (+ ||v||^2), giving ||v_i - o_w||^2;
//            -2 O is split into bf16 hi + lo parts so the product keeps ~16 bits
//
// Pass 1 also writes the adjacent-key cosine (the shared pair_cos routine on LDS rows in
// row layout), so the merge pass can recompute bit-identical values.
#include <type_traits>

#include "kvs_common.h"
#include "kvs_dma.h"
#include "kvs_pack.h"
#include "kvs_score_impl.h"

namespace kvs {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kChunk1Unit = 2 * kT2;   // pass-1 chunks: each tile group's half is whole tiles
constexpr int kQB = 128;               // window queries per workgroup

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

// 8 floats to f16, round to nearest even (two elements per conversion).
__device__ __forceinline__ f16x8_t to_f16x8(const float* x) {
  f16x8_t r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (_Float16)x[j];
  return r;
}

// 8 bf16 (16 bytes) to 8 f16 in the same positions: exact for |x| in f16's normal range
// [2^-14, 65504], rounded to f16's grid below it, infinite above.
__device__ __forceinline__ uint4 bf16x8_to_f16x8(const uint4& u) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  f16x8_t r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r[2 * j] = (_Float16)bf16_lo(w[j]);
    r[2 * j + 1] = (_Float16)bf16_hi(w[j]);
  }
  const u32x4_t v = __builtin_bit_cast(u32x4_t, r);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// ------------------------------------------------------------------ tiling ----
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

__device__ __forceinline__ f32x16_t mfma32(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mfma32(const f16x8_t& a, const f16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Q rows as a 32x32x16 operand: lane l holds row[q][16 ks + 8 (l / 32) .. +7] of query q.
template <int D>
__device__ __forceinline__ void load_rows32(const bf16* Qp, int64_t GW, int64_t q, bf16x8_t (&op)[D / 16]) {
  const int h = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (q < GW) u = load16(Qp + q * D + ks * 16 + h * 8);
    op[ks] = as_bf16x8(u);
  }
}

// Maximum of x over lanes l and l ^ 32 (the two halves of a 32x32 result column).
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ------------------------------------------------------------------------- pass 1 --
// Flash-style statistics of the window queries over one slot chunk.  A workgroup is two
// tile groups of four waves (512 threads, one per CU); group g streams the g-th half of
// the chunk through its own four-deep LDS ring of 32-slot tiles (16-byte buffer loads
// written straight to LDS, rows XOR-swizzled, natural slot order), and the two groups'
// softmax states are merged through LDS into one partial record per query at the end.
// A wave owns 32 window queries on 32x32x16 MFMA in transposed form, S^T = K . Q^T, so
// each lane's accumulators belong to one query.  The QK product of tile t + 1 is issued
// before the softmax of tile t so that the matrix cores run while the vector units work.
// The running maximum is raised only when it grows by more than 2^8 (P <= 256 in
// between), which makes rescales of the output accumulators rare.  O^T += V^T . P^T takes
// f16 operands: P^T from the softmax, V^T by LDS transpose reads of the tile, which the
// group converts to f16 in place in the iteration its loads land.
constexpr int kGroupWaves = 4;
constexpr int kGroups = 2;
constexpr int kGT = 64 * kGroupWaves;              // threads per group
constexpr int kThreads = kGT * kGroups;            // 512
constexpr float kLazyMax = 8.f;                    // log2 headroom of the running maximum

// grid: one workgroup per (bh, slot chunk, query block), bh fastest.  Partial records
// {m (log2 units), l, -, -, o[D]} per (bh, query, chunk).
template <int D, bool HAS_N>
__global__ __launch_bounds__(kThreads, 2 / kGroups) void p1_mfma_kernel(P1Args a, int64_t base, CosArgs ca, int BH) {
  using M = Dma<D>;
  constexpr int KS = D / 16;    // 16-wide k steps over the head dim
  constexpr int DB = D / 32;    // 32-row blocks of O^T
  // K tiles, then V tiles; after the loop the whole ring holds the records being merged
  __shared__ __attribute__((aligned(1024))) uint8_t ring[2 * kGroups * kRing2 * M::TILEB];
  __shared__ __attribute__((aligned(16))) int32_t nr[kGroups * kRing2 * kT2];
  __shared__ __attribute__((aligned(16))) float lgb[kGroups * kRing2 * kT2];   // count bias per slot
  __shared__ float xm[2 * kQB];
  static_assert(kQB * (D + 4) * 4 <= 2 * kGroups * kRing2 * M::TILEB, "record staging exceeds the ring");
  uint8_t* const kr = ring;
  uint8_t* const vr = ring + kGroups * kRing2 * M::TILEB;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wv / kGroupWaves, gw = wv % kGroupWaves, gt = tid % kGT;
  const int c32 = lane & 31, h = lane >> 5, G16 = lane >> 4, t16 = lane & 15;
  const int64_t id = blockIdx.x;
  const int64_t bh = id % BH, rest = id / BH;
  const int64_t split = rest % a.nsplit, qb = rest / a.nsplit;
  const int64_t b = bh / a.Hkv, hk = bh - b * a.Hkv;
  const int64_t hoff = b * a.sb + hk * a.sh;
  const int32_t* np = HAS_N ? a.n + hoff / D : nullptr;

  // the two halves of the chunk; group 0's half is never shorter than group 1's
  const int64_t c0 = base + split * a.chunk, half = a.chunk / kGroups;
  auto tiles_of = [&](int g) {
    const int64_t s0 = c0 + g * half;
    const int64_t l0 = s0 > 0 ? s0 : 0, h0 = s0 + half < a.N ? s0 + half : a.N;
    return h0 > l0 ? (int)((h0 - s0 + kT2 - 1) / kT2) : 0;
  };
  const int nt0 = tiles_of(0);
  const int64_t g0 = c0 + grp * half;
  const int64_t lo = g0 > 0 ? g0 : 0;
  const int64_t hi = g0 + half < a.N ? g0 + half : a.N;
  const int nt = tiles_of(grp);
  const uint32_t span = hi > lo ? (uint32_t)(hi - lo) : 0u;
  const u32x4_t rk = make_rsrc(static_cast<const bf16*>(a.K) + hoff + (hi > lo ? lo : 0) * D, span * M::ROWB);
  const u32x4_t rv = make_rsrc(static_cast<const bf16*>(a.V) + hoff + (hi > lo ? lo : 0) * D, span * M::ROWB);
  const u32x4_t rn = make_rsrc(HAS_N ? static_cast<const void*>(np + (hi > lo ? lo : 0)) : a.K, HAS_N ? span * 4u : 0u);
  uint8_t* kr_g = kr + grp * kRing2 * M::TILEB;
  uint8_t* vr_g = vr + grp * kRing2 * M::TILEB;
  int32_t* nr_g = nr + grp * kRing2 * kT2;
  float* lgb_g = lgb + grp * kRing2 * kT2;

  // K tile j (with its counts) and V tile j go to ring slot j % 4 of their own ring.  The
  // loop below issues K(t + 3) and V(t + 2) at the top of iteration t, in that order: V is
  // consumed one iteration after K, so its ring slot turns over one iteration later.
  auto issue_k = [&](int t) {
    const int buf = t % kRing2;
    const int64_t t0 = g0 + (int64_t)t * kT2;
#pragma unroll
    for (int j = 0; j < M::IPW; ++j) {
      const int u = j * kGroupWaves + gw;
      const int R = u * M::RPI + lane / M::CPR;
      const int c = (lane % M::CPR) ^ swz<D>(R);
      dma16(rk, lds_addr(kr_g + buf * M::TILEB + u * 1024), (uint32_t)((t0 + R - lo) * M::ROWB) + (uint32_t)(c << 4));
    }
    if (HAS_N && gw == 0 && lane < kT2) dma4(rn, lds_addr(nr_g + buf * kT2), (uint32_t)((t0 + lane - lo) * 4));
  };
  auto issue_v = [&](int t) {
    const int buf = t % kRing2;
    const int64_t t0 = g0 + (int64_t)t * kT2;
#pragma unroll
    for (int j = 0; j < M::IPW; ++j) {
      const int u = j * kGroupWaves + gw;
      const int R = u * M::RPI + lane / M::CPR;
      const int c = (lane % M::CPR) ^ swz<D>(R);
      dma16(rv, lds_addr(vr_g + buf * M::TILEB + u * 1024), (uint32_t)((t0 + R - lo) * M::ROWB) + (uint32_t)(c << 4));
    }
  };
  // The count bias of tile t's slots, log2 n (-inf outside the group's range), computed once
  // per slot by the wave that loads the counts (its own loads have landed) and read by
  // every wave after the next barrier.
  auto count_bias = [&](int t) {
    if (HAS_N && gw == 0 && lane < kT2) {
      const int buf = t % kRing2;
      const int64_t s = g0 + (int64_t)t * kT2 + lane;
      lgb_g[buf * kT2 + lane] = (s >= lo && s < hi) ? __log2f((float)nr_g[buf * kT2 + lane]) : -INFINITY;
    }
  };

  // Wait at the top of iteration t until V(t) has landed (and with it every earlier load,
  // K(t + 1) included: it was issued just before V(t)); issued after V(t) are K(t + 2) if
  // it exists and V(t + 1) if it exists.  V(t) is converted to f16 in this iteration.
  const bool nload = HAS_N && gw == 0;   // this wave also loads the counts with each K tile
  auto wait_top = [&](int t) {
    if (t + 1 >= nt) {
      wait_vm<0>();
    } else if (t + 2 < nt) {
      if (nload) wait_vm<2 * M::IPW + 1>();
      else wait_vm<2 * M::IPW>();
    } else {
      wait_vm<M::IPW>();
    }
  };
  // V tile t to f16 in place, element by element (the swizzled chunk positions stay), by
  // the group's threads: the O^T product takes V^T and P^T as f16 operands
  auto v_to_f16 = [&](int t) {
    uint4* V_ = reinterpret_cast<uint4*>(vr_g + (t % kRing2) * M::TILEB);
#pragma unroll
    for (int i = 0; i < M::TILEB / 16 / kGT; ++i) V_[gt + i * kGT] = bf16x8_to_f16x8(V_[gt + i * kGT]);
  };

  // K(0), K(1), V(0) and the query operands travel together (loads complete in order, so
  // waiting on the queries waits on the tiles as well); then K(2), V(1), the loads of
  // iteration -1
  {   // the first iteration reads V^T from ring slot 3 and multiplies it by a zero P^T: keep it finite
    uint4* z = reinterpret_cast<uint4*>(vr_g + (kRing2 - 1) * M::TILEB);
    for (int i = gt; i < M::TILEB / 16; i += kGT) z[i] = make_uint4(0, 0, 0, 0);
  }
  if (nt > 0) issue_k(0);
  if (nt > 1) issue_k(1);
  if (nt > 0) issue_v(0);
  const bf16* Qp = static_cast<const bf16*>(a.Qw) + ((b * a.Hq + hk * a.G) * (int64_t)a.W) * D;
  const int64_t q = qb * kQB + gw * 32 + c32;
  bf16x8_t qop[KS];
  load_rows32<D>(Qp, a.GW, q, qop);
  asm volatile("" ::"v"(qop[KS - 1]));
  if (nt > 0) count_bias(0);   // K(0) and its counts came before the queries
  if (nt > 2) issue_k(2);
  if (nt > 1) issue_v(1);

  const float cs = a.scale * kLog2e;
  float m = kNoMax, lsum = 0.f;
  f32x16_t acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
  const bool do_cos = ca.cos != nullptr && qb == 0;

  // S^T = K . Q^T of tile t: lane holds slots 8 (i / 4) + 4 h + i % 4 of query c32
  auto qk = [&](int t) {
    const uint8_t* K_ = kr_g + (t % kRing2) * M::TILEB;
    f32x16_t st;
#pragma unroll
    for (int i = 0; i < 16; ++i) st[i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      st = mfma32(as_bf16x8(*reinterpret_cast<const uint4*>(K_ + chunk_off<D>(c32, 2 * ks + h))), qop[ks], st);
    return st;
  };

  // adjacent-key cosine of the tile's candidate pairs (shared routine of the merge pass)
  auto cosines = [&](int t) {
    const uint8_t* K_ = kr_g + (t % kRing2) * M::TILEB;
    const int64_t t0 = g0 + (int64_t)t * kT2;
    if (gt < (kT2 / 2) * M::CPR) {
      const int pp = gt / M::CPR, ch = gt % M::CPR;
      float k0[8], k1[8];
      unpack<bf16>(*reinterpret_cast<const uint4*>(K_ + chunk_off<D>(2 * pp, ch)), k0);
      unpack<bf16>(*reinterpret_cast<const uint4*>(K_ + chunk_off<D>(2 * pp + 1, ch)), k1);
      const float cv = pair_cos<8, M::CPR>(k0, k1);
      const int64_t m0 = t0 + 2 * pp;
      const int64_t p = (m0 - ca.S) / 2;
      if (ch == 0 && m0 >= ca.S && p < ca.P && m0 >= lo && m0 + 1 < hi) ca.cos[bh * ca.P + p] = cv;
    }
  };

  // logits of tile t in log2 units are e[i] * sc: inside the group's range without counts
  // e = S^T and sc = scale * log2(e); otherwise e carries the scale, the count bias and
  // -inf for slots outside the range, and sc = 1
  auto logits = [&](int t, const f32x16_t& st, float (&e)[16], float& sc) {
    const int buf = t % kRing2;
    const int64_t t0 = g0 + (int64_t)t * kT2;
    if (!HAS_N && t0 >= lo && t0 + kT2 <= hi) {
#pragma unroll
      for (int i = 0; i < 16; ++i) e[i] = st[i];
      sc = cs;
    } else if (HAS_N) {
      sc = 1.f;
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        const float4 lg = *reinterpret_cast<const float4*>(lgb_g + buf * kT2 + 8 * k4 + 4 * h);
        e[4 * k4 + 0] = __builtin_fmaf(st[4 * k4 + 0], cs, lg.x);
        e[4 * k4 + 1] = __builtin_fmaf(st[4 * k4 + 1], cs, lg.y);
        e[4 * k4 + 2] = __builtin_fmaf(st[4 * k4 + 2], cs, lg.z);
        e[4 * k4 + 3] = __builtin_fmaf(st[4 * k4 + 3], cs, lg.w);
      }
    } else {
      sc = 1.f;
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t s = t0 + 8 * k4 + 4 * h + r;
          const float lg = (s >= lo && s < hi) ? 0.f : -INFINITY;
          e[4 * k4 + r] = __builtin_fmaf(st[4 * k4 + r], cs, lg);
        }
      }
    }
  };

  // softmax of one tile from its logits, with no branch, in two halves that run beside the
  // two blocks of matrix products: the reference maximum m rises only when the tile maximum
  // exceeds it by more than 2^8 (then corr = 2^(m_old - m_new) < 1, otherwise corr = 1
  // exactly); the caller rescales the output accumulators by corr.  The first half finds
  // the maximum and the first eight probabilities, the second the other eight, the sum and
  // the P^T operands in f16 for two 16-slot k steps (11-bit significands: P <= 2^8 stays in
  // f16's range, and the product keeps O within ~3e-4 of exact on these shapes).
  auto softmax_a = [&](const float (&e)[16], float sc, float (&p)[16], float& corr) {
    float mx = e[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, e[i]);
    mx = max_halves(mx) * sc;
    const float mn = mx > m + kLazyMax ? mx : m;
    corr = __builtin_amdgcn_exp2f(m - mn);
    m = mn;
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(e[i], sc, -m));
  };
  auto softmax_b = [&](const float (&e)[16], float sc, float (&p)[16], float corr, f16x8_t (&pf)[2]) {
#pragma unroll
    for (int i = 8; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(e[i], sc, -m));
    float ls = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) ls += p[i];
    lsum = __builtin_fmaf(lsum, corr, ls);
    // k index (h, j) of step ks <-> slot 16 ks + 8 (j / 4) + 4 h + j % 4: the lane's p[8 ks + j]
    pf[0] = to_f16x8(p);
    pf[1] = to_f16x8(p + 8);
  };

  // V^T operands of one 16-slot k step by transposed reads: source lane i = lane % 16 points
  // at row r0 + i / 4 (and + 8), columns 32 db + 16 (G16 % 2) + 4 (i % 4); lane t receives
  // column + t of 4 consecutive rows
  auto read_vt = [&](int t, int ks, f16x8_t (&vop)[DB]) {
    const uint8_t* V_ = vr_g + (t % kRing2) * M::TILEB;
    const int r0 = ks * 16 + 4 * h + (t16 >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      typedef __attribute__((__vector_size__(4 * sizeof(__fp16)))) __fp16 fp16x4_t;
      typedef __attribute__((address_space(3))) fp16x4_t lds_fp16x4;
      const int col = db * 32 + 16 * (G16 & 1) + 4 * (t16 & 3);
      const int cb = (col & 7) * 2;
      const f16x4_t v0 = __builtin_bit_cast(
          f16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4*)(V_ + chunk_off<D>(r0, col >> 3) + cb)));
      const f16x4_t v1 = __builtin_bit_cast(
          f16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4*)(V_ + chunk_off<D>(r0 + 8, col >> 3) + cb)));
      vop[db] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };

  // O^T += V^T . P^T of one tile (f16 operands)
  auto pv = [&](const f16x8_t (&vop)[2][DB], const f16x8_t (&pf)[2]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] = mfma32(vop[ks][db], pf[ks], acc[db]);
  };

  // Software pipeline: iteration t computes the softmax of tile t on the vector units while
  // the matrix cores run S^T of tile t + 1 and O^T += V^T . P^T of tile t - 1.  The three
  // are independent, so the scheduler interleaves the MFMAs with the softmax instructions
  // in one straight block; the first iteration multiplies a zero P^T.
  __syncthreads();   // K(0) of both groups is in (each wave waited on its own loads)
  f32x16_t s_cur;
  if (nt > 0) s_cur = qk(0);
  f16x8_t pp[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int j = 0; j < 8; ++j) pp[ks][j] = (_Float16)0.f;
  for (int t = 0; t < nt0; ++t) {
    const bool act = t < nt;
    if (act) wait_top(t);
    __syncthreads();
    if (act) {
      if (t + 1 < nt) count_bias(t + 1);   // K(t + 1) and its counts have landed
      if (t + 3 < nt) issue_k(t + 3);
      if (t + 2 < nt) issue_v(t + 2);
      if (do_cos) cosines(t);
      float e[16], sc;
      logits(t, s_cur, e, sc);
      // operands: K rows of tile t + 1 (stale past the last tile; that product is unused)
      // and V^T of tile t - 1 (stale in the first iteration, where P^T is zero)
      bf16x8_t ka[KS];
      f16x8_t vop[2][DB];
      {
        const uint8_t* K_ = kr_g + ((t + 1) % kRing2) * M::TILEB;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          ka[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(K_ + chunk_off<D>(c32, 2 * ks + h)));
      }
      read_vt(t + kRing2 - 1, 0, vop[0]);
      read_vt(t + kRing2 - 1, 1, vop[1]);
      __builtin_amdgcn_sched_barrier(0);
      // S^T of tile t + 1 (a chain of dependent products) beside the first half of the
      // softmax; the maximum starts while the operand reads land
      f32x16_t s_next;
#pragma unroll
      for (int i = 0; i < 16; ++i) s_next[i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s_next = mfma32(ka[ks], qop[ks], s_next);
      float p[16], corr;
      softmax_a(e, sc, p, corr);
      __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
#pragma unroll
      for (int i = 0; i < KS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);   // then softmax instructions
      }
      __builtin_amdgcn_sched_barrier(0);
      // O^T += V^T . P^T of tile t - 1 (independent chains) beside the second half, and
      // V(t), landed at the top of this iteration, to f16 (it is read in the next one)
      f16x8_t pf[2];
      softmax_b(e, sc, p, corr, pf);
      pv(vop, pp);
      v_to_f16(t);
#pragma unroll
      for (int i = 0; i < 2 * DB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      // the softmax results are needed here, so nothing of it sinks below the branch
      asm volatile("" ::"v"(pf[0]), "v"(pf[1]), "v"(lsum));
      if (__builtin_amdgcn_ballot_w64(corr != 1.f)) {
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] *= corr;
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) pp[ks] = pf[ks];
      s_cur = s_next;
    }
  }
  __syncthreads();   // V(nt - 1), converted in the last iteration by the whole group
  if (nt > 0) {
    f16x8_t vop[2][DB];
    read_vt(nt - 1, 0, vop[0]);
    read_vt(nt - 1, 1, vop[1]);
    pv(vop, pp);
  }

  // merge the two groups' running states through LDS, then write the partial records with
  // 16-byte stores (one record = {m, l, -, -, o[D]} is D + 4 contiguous floats)
  const float l = sum_halves(lsum);
  __syncthreads();
  float* xo = reinterpret_cast<float*>(ring);            // [128 queries][D + 4]
  constexpr int RS = D + 4;
  const int qi = gw * 32 + c32;
  if (kGroups == 2 && grp == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) xo[qi * RS + 4 + db * 32 + (i >> 2) * 8 + h * 4 + (i & 3)] = acc[db][i];
    if (h == 0) {
      xm[qi] = m;
      xm[kQB + qi] = l;
    }
  }
  __syncthreads();
  if (grp == 0) {
    const float m1 = kGroups == 2 ? xm[qi] : kNoMax, l1 = kGroups == 2 ? xm[kQB + qi] : 0.f;
    const float Mx = fmaxf(m, m1);
    const float f0 = __builtin_amdgcn_exp2f(m - Mx), f1 = __builtin_amdgcn_exp2f(m1 - Mx);
    if (h == 0) {
      xo[qi * RS] = Mx;
      xo[qi * RS + 1] = l * f0 + l1 * f1;
      xo[qi * RS + 2] = 0.f;
      xo[qi * RS + 3] = 0.f;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int d = db * 32 + (i >> 2) * 8 + h * 4 + (i & 3);
        xo[qi * RS + 4 + d] = kGroups == 2 ? acc[db][i] * f0 + xo[qi * RS + 4 + d] * f1 : acc[db][i] * f0;
      }
  }
  __syncthreads();
  const int64_t qbase = qb * kQB;
  const int nq = (int)(a.GW - qbase < kQB ? a.GW - qbase : kQB);
  if (a.fin) {
    // one split per query: what the combine does with a single record, here (o / l, the
    // log-sum-exp in natural log, the pass-2 operand pack), one wave per query row
    constexpr int E = D / 64, RPW = kQB / (kThreads / 64);   // rows per wave
    const int ln = tid & 63, w8 = tid >> 6;
    // the query chunks of all the wave's rows first, so their loads overlap
    uint4 qch[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int qq = w8 + i * (kThreads / 64);
      qch[i] = qq < nq ? pack_query_chunk<D>(a.pk, bh * a.GW + qbase + qq, ln) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int qq = w8 + i * (kThreads / 64);
      if (qq >= nq) break;   // wave-uniform
      const float* row = xo + qq * RS;
      const float mm = row[0], ll = row[1];
      float ov[E];
#pragma unroll
      for (int e = 0; e < E; ++e) ov[e] = row[4 + ln + 64 * e] / ll;
      const int64_t u = bh * a.GW + qbase + qq;
#pragma unroll
      for (int e = 0; e < E; ++e) a.O[u * D + ln + 64 * e] = ov[e];
      const float lse_u = (mm + __log2f(ll)) * kLn2;
      if (ln == 0) a.lse[u] = lse_u;
      pack_row_wave_q<D>(a.pk, u, ov, lse_u, ln, qch[i]);
    }
    return;
  }
  for (int idx = tid; idx < nq * (RS / 4); idx += kThreads) {
    const int qq = idx / (RS / 4), c = idx % (RS / 4);
    float* rec = a.part + ((bh * a.GW + qbase + qq) * a.nsplit + split) * (int64_t)RS;
    *reinterpret_cast<float4*>(rec + 4 * c) = *reinterpret_cast<const float4*>(xo + qq * RS + 4 * c);
  }
}

// ------------------------------------------------------------------------- pass 2 --
// S[q, slot] = Q . K^T and R[q, slot] = (-2 O) . V^T + ||o||^2 (+ ||v||^2) on 16x16x32 MFMA,
// with the even and the odd slots of a 32-slot tile in separate products: lane l then
// holds both slots of candidate pair l % 16 for 8 of the wave's 32 queries, so the pair
// term needs no cross-lane exchange and the sums over queries are mostly in registers.
//
// A workgroup is four waves (128 queries) over one slot chunk; two workgroups share a CU.
// K and V arrive by 16-byte buffer loads written straight into LDS (no register staging)
// as 32-slot tiles in a four-deep ring: tile t is computed while tile t - 1 is merged and
// tiles t + 1, t + 2 are in flight.  A tile's LDS row R holds slot 2 (R % 16) + R / 16
// (even slots first).  Rows are unpadded; the 16-byte chunks of row r sit at position
// c ^ swz(r), which keeps the MFMA operand reads free of bank conflicts.  ||v||^2 and
// v_m . v_{m+1} come from the diagonals of Gram products of the V operand registers, so a
// tile needs no setup pass and one barrier.  Each wave keeps its per-slot sums in LDS; the
// four waves' sums are added and written once, at the end, so the loop issues no global
// stores.  The query operands come pre-packed in lane order from the log-sum-exp combine.
constexpr int kChunk2Max = 512;      // pass-2 slots per workgroup at most

// LDS row R of a tile holds slot 2 (R % 16) + R / 16 of the tile.
__device__ __forceinline__ int row_slot(int R) { return 2 * (R & 15) + (R >> 4); }

// grid: one workgroup per (bh, slot chunk, query block), bh fastest so that the blocks of
// one head land on one XCD.
// MERGE: also merge the chunk's candidate pairs and write the compacted K/V rows (type
// TO), counts and sources, reusing the tiles already in LDS.  Without PARTIAL every pair
// merges (a full round); with PARTIAL the pairs chosen by the selection state merge and
// the others are copied, each at its compacted row.
template <int D, bool HAS_N, bool MERGE, bool PARTIAL, typename TO>
__global__ __launch_bounds__(kW2 * 64, 2) void p2_mfma_kernel(P2Args a, int64_t base, int64_t chunk, int nsplit,
                                                             int BH) {
  using M = Dma<D>;
  constexpr int KS = D / 32;                      // 32-wide k steps of 16x16x32 MFMA
  __shared__ __attribute__((aligned(1024))) uint8_t kr[kRing2 * M::TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t vr[kRing2 * M::TILEB];
  __shared__ int32_t nr[kRing2 * kT2];            // slot counts as loaded (LDS-row order)
  // per-wave sums over the wave's queries, grouped by aligned slot pair j of the chunk:
  // red[(3 j + k) kW2 + w], k = 0 the even slot, 1 the odd slot, 2 the pair term, so the
  // four waves' values of one quantity are one 16-byte read
  static_assert(kW2 == 4, "one float4 per quantity");
  __shared__ __attribute__((aligned(16))) float red[(kChunk2Max / 2) * 3 * kW2];
  // the four waves' values added in wave order (the order every reader uses)
  auto sum_waves = [](const float4& v) {
    float x = 0.f;
    x += v.x;
    x += v.y;
    x += v.z;
    x += v.w;
    return x;
  };
  // partial rounds: selection flags of the 64-pair compaction chunks the workgroup's pairs
  // fall in, and the selected pairs before each of those chunks
  constexpr int kSelChunks = kChunk2Max / 2 / kChunkPairs + 1;
  __shared__ uint64_t selm[kSelChunks];
  __shared__ int32_t selo[kSelChunks];

  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, g4 = lane >> 4;
  const int64_t id = blockIdx.x;
  const int64_t bh = id % BH;
  const int64_t rest = id / BH;
  const int64_t split = rest % nsplit, qb = rest / nsplit;
  const int64_t b = bh / a.Hkv, hk = bh - b * a.Hkv;
  const int64_t hoff = b * a.sb + hk * a.sh;

  const int64_t c0 = base + split * chunk;
  const int64_t lo = c0 > 0 ? c0 : 0;
  const int64_t hi = c0 + chunk < a.N ? c0 + chunk : a.N;
  if (hi <= lo) return;
  const int ntiles = (int)((hi - c0 + kT2 - 1) / kT2);
  const uint32_t span = (uint32_t)(hi - lo);
  const u32x4_t rk = make_rsrc(static_cast<const bf16*>(a.K) + hoff + lo * D, span * M::ROWB);
  const u32x4_t rv = make_rsrc(static_cast<const bf16*>(a.V) + hoff + lo * D, span * M::ROWB);
  const int32_t* np = HAS_N ? a.n + hoff / D + lo : nullptr;
  const u32x4_t rn = make_rsrc(HAS_N ? static_cast<const void*>(np) : a.K, HAS_N ? span * 4u : 0u);

  // tile t -> ring buffer t % kRing2; rows outside [lo, hi) read as zeros
  auto issue = [&](int t) {
    const int buf = t % kRing2;
    const int64_t t0 = c0 + (int64_t)t * kT2;
#pragma unroll
    for (int j = 0; j < M::IPW; ++j) {
      const int u = j * kW2 + wv;
      const int R = u * M::RPI + lane / M::CPR;
      const int c = (lane % M::CPR) ^ swz<D>(R);
      const uint32_t off = (uint32_t)((t0 + row_slot(R) - lo) * M::ROWB) + (uint32_t)(c << 4);
      dma16(rk, lds_addr(kr + buf * M::TILEB + u * 1024), off);
      dma16(rv, lds_addr(vr + buf * M::TILEB + u * 1024), off);
    }
    if (HAS_N && wv == 0 && lane < kT2) {
      const uint32_t off = (uint32_t)((t0 + row_slot(lane) - lo) * 4);
      dma4(rn, lds_addr(nr + buf * kT2), off);
    }
  };
  // wait for every load of a tile after which `later` (0 or 1) tiles were issued (the
  // loads complete in order; stores issued in between only make the wait stricter)
  auto wait_tile = [&](int later) {
    if (later == 0) wait_vm<0>();
    else if (HAS_N && wv == 0) wait_vm<2 * M::IPW + 1>();
    else wait_vm<2 * M::IPW>();
  };

  issue(0);

  // the wave's 32 queries as A operands (two 16-query blocks): lane l holds query
  // 16 qb2 + l % 16, head-dim chunk 4 ks + l / 16 of Q and of -2 O (bf16 hi + lo), read
  // from the operand pack in lane order (every load is 1 KB contiguous per wave); the
  // result rows of the lane are queries 16 q2 + 4 (l / 16) + r.  Queries past the window
  // (never written to the pack) are replaced by zeros and alpha = 0.
  const int64_t wb = qb * (kQB / 32) + wv;
  const int64_t wbl = wb < a.nwb ? wb : a.nwb - 1;     // blocks past the window: loads clamped, all masked
  bf16x8_t qop[2][KS], ohi[2][KS], olo[2][KS];
  float nbq[2][4];
  f32x4_t onv[2];
  {
    const uint4* opb = a.ops + (bh * a.nwb + wbl) * 2 * 3 * KS * 64 + lane;
    uint4 raw[2][3][KS];
    float4 qcr[2][2];
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
#pragma unroll
      for (int w = 0; w < 3; ++w)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) raw[q2][w][ks] = opb[((q2 * 3 + w) * KS + ks) * 64];
      const float* qcp = a.qc + ((bh * a.nwb + wbl) * 32 + q2 * 16 + 4 * g4) * 2;
      qcr[q2][0] = *reinterpret_cast<const float4*>(qcp);
      qcr[q2][1] = *reinterpret_cast<const float4*>(qcp + 4);
    }
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
      const bool va = wb * 32 + q2 * 16 + n16 < a.GW;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 zero = make_uint4(0, 0, 0, 0);
        qop[q2][ks] = as_bf16x8(va ? raw[q2][0][ks] : zero);
        ohi[q2][ks] = as_bf16x8(va ? raw[q2][1][ks] : zero);
        olo[q2][ks] = as_bf16x8(va ? raw[q2][2][ks] : zero);
      }
      const float c8[8] = {qcr[q2][0].x, qcr[q2][0].y, qcr[q2][0].z, qcr[q2][0].w,
                           qcr[q2][1].x, qcr[q2][1].y, qcr[q2][1].z, qcr[q2][1].w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool vc = wb * 32 + q2 * 16 + 4 * g4 + r < a.GW;
        onv[q2][r] = vc ? c8[2 * r] : 0.f;
        // + 1: the exponent gives twice the attention weight (see the sums below)
        nbq[q2][r] = vc ? c8[2 * r + 1] + 1.f : -INFINITY;
      }
    }
  }
  // partial rounds: wave w takes compaction chunks sel_c0 + w, sel_c0 + w + kW2, ... of the
  // pairs whose first slot lies in the workgroup's slots, reads their cosines and
  // evaluates the selection
  int64_t sel_c0 = 0;
  if constexpr (PARTIAL) {
    const int64_t pend = a.S + 2 * a.P;
    const int64_t mlo = lo > a.S ? lo : a.S, mhi = hi < pend ? hi : pend;
    const int64_t pa = (mlo - a.S + 1) / 2, pb = (mhi - a.S) / 2;   // pairs [pa, pb)
    sel_c0 = pa / kChunkPairs;
    const int nck = pb > pa ? (int)((pb - 1) / kChunkPairs - sel_c0 + 1) : 0;
    for (int k = wv; k < nck; k += kW2) {
      const int64_t cc = sel_c0 + k;
      uint64_t m = 0;
      int32_t before = 0;
      if (a.M > 0) {
        const int32_t* st = a.sel + bh * a.sel_stride;
        const SelHeader hd{(uint32_t)st[0], st[1], st[2], st[3]};
        const int64_t p = cc * kChunkPairs + lane;
        m = __ballot(p < a.P && is_selected(order_key(p < a.P ? a.cos[bh * a.P + p] : 0.f), p, hd));
        before = st[kSelHeaderInts + cc];
      }
      if (lane == 0) {
        selm[k] = m;
        selo[k] = before;
      }
    }
  }
  // tile 0 and the operands travel together; tile 1 is issued once they are in
  asm volatile("" ::"v"(olo[1][KS - 1]), "v"(nbq[1][3]));
  if (ntiles > 1) issue(1);
  const float cs = a.scale * kLog2e;
  const float ics = 1.f / cs;

  auto compute = [&](int t) {
    const int buf = t % kRing2;
    const int64_t t0 = c0 + (int64_t)t * kT2;
    const uint8_t* K_ = kr + buf * M::TILEB;
    const uint8_t* V_ = vr + buf * M::TILEB;
    // log2 n of the lane's even and odd slot (-inf outside the chunk)
    float lge = 0.f, lgo = 0.f;
    if (HAS_N || t0 < lo || t0 + kT2 > hi) {
      const int64_t se_ = t0 + 2 * n16;
      lge = (se_ >= lo && se_ < hi) ? (HAS_N ? __log2f((float)nr[buf * kT2 + n16]) : 0.f) : -INFINITY;
      lgo = (se_ + 1 >= lo && se_ + 1 < hi) ? (HAS_N ? __log2f((float)nr[buf * kT2 + 16 + n16]) : 0.f) : -INFINITY;
    }
    const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    // the slot's log2 count enters S^T through the accumulator's starting value (divided
    // by the logit scale), so each exponent argument is one fma
    const f32x4_t be = {lge * ics, lge * ics, lge * ics, lge * ics};
    const f32x4_t bo = {lgo * ics, lgo * ics, lgo * ics, lgo * ics};
    f32x4_t se[2], so[2], re[2], ro[2], gee = z, goo = z, geo = z;
    // the two workgroups that share a CU pair their waves on each SIMD: the one issuing its
    // matrix block goes first, the other fills the vector slots in between
    __builtin_amdgcn_s_setprio(1);
    // operands of k step ks: K and V rows of the even and the odd slots; the reads of step
    // ks + 1 are issued before the products of step ks, so they land while those run
    auto read_ops = [&](int ks, bf16x8_t (&op)[4]) {
      const int ch = 4 * ks + g4;
      op[0] = as_bf16x8(*reinterpret_cast<const uint4*>(K_ + chunk_off<D>(n16, ch)));
      op[1] = as_bf16x8(*reinterpret_cast<const uint4*>(K_ + chunk_off<D>(16 + n16, ch)));
      op[2] = as_bf16x8(*reinterpret_cast<const uint4*>(V_ + chunk_off<D>(n16, ch)));
      op[3] = as_bf16x8(*reinterpret_cast<const uint4*>(V_ + chunk_off<D>(16 + n16, ch)));
    };
    bf16x8_t ops2[2][4];
    read_ops(0, ops2[0]);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) read_ops(ks + 1, ops2[(ks + 1) & 1]);
      const bf16x8_t ke = ops2[ks & 1][0], ko = ops2[ks & 1][1], ve = ops2[ks & 1][2], vo = ops2[ks & 1][3];
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        se[q2] = mfma(qop[q2][ks], ke, ks == 0 ? be : se[q2]);
        so[q2] = mfma(qop[q2][ks], ko, ks == 0 ? bo : so[q2]);
        re[q2] = mfma(ohi[q2][ks], ve, ks == 0 ? onv[q2] : re[q2]);
        ro[q2] = mfma(ohi[q2][ks], vo, ks == 0 ? onv[q2] : ro[q2]);
        re[q2] = mfma(olo[q2][ks], ve, re[q2]);
        ro[q2] = mfma(olo[q2][ks], vo, ro[q2]);
      }
      // Gram blocks of the tile's values (the V registers serve as both operands):
      // their diagonals give ||v_m||^2, ||v_{m+1}||^2 and v_m . v_{m+1}
      gee = mfma(ve, ve, gee);
      goo = mfma(vo, vo, goo);
      geo = mfma(ve, vo, geo);
    }
    // order: the reads of steps 0 and 1, then each step's fifteen products followed by the
    // reads of the step after the next
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x008, 15, 0);
      if (ks + 2 < KS) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    }
    __builtin_amdgcn_s_setprio(0);
    // diagonal element n of a 16x16 result sits in lane n + 16 (n / 4), register n % 4
    const int rsel = n16 & 3;
    auto pick = [&](const f32x4_t& g) {
      return rsel == 0 ? g[0] : rsel == 1 ? g[1] : rsel == 2 ? g[2] : g[3];
    };
    const int src = n16 + 16 * (n16 >> 2);
    const float vne = __shfl(pick(gee), src, 64);
    const float vno = __shfl(pick(goo), src, 64);
    const float veo = __shfl(pick(geo), src, 64);
    const float dvp = vne + vno - 2.f * veo;          // ||v_m - v_{m+1}||^2
    // With a = 2 alpha (the exponent carries + 1): alpha |1 - 2 alpha| = |a - a^2| / 2 and
    // alpha_m alpha_{m+1} = a_m a_{m+1} / 4, one fma for the first; the factors 1/2 and
    // 1/4 (exact) are applied to the tile's sums.
    float gse = 0.f, gso = 0.f, gx = 0.f;
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ae = __builtin_amdgcn_exp2f(__builtin_fmaf(se[q2][r], cs, nbq[q2][r]));
        const float ao = __builtin_amdgcn_exp2f(__builtin_fmaf(so[q2][r], cs, nbq[q2][r]));
        const float rre = re[q2][r] + vne, rro = ro[q2][r] + vno;
        gse = __builtin_fmaf(fabsf(__builtin_fmaf(-ae, ae, ae)), __builtin_amdgcn_sqrtf(fabsf(rre)), gse);
        gso = __builtin_fmaf(fabsf(__builtin_fmaf(-ao, ao, ao)), __builtin_amdgcn_sqrtf(fabsf(rro)), gso);
        // ||v_m + v_{m+1} - 2 o||^2 = 2 r_m^2 + 2 r_{m+1}^2 - ||v_m - v_{m+1}||^2
        const float rc = __builtin_fmaf(2.f, rre + rro, -dvp);
        gx = __builtin_fmaf(ae * ao, __builtin_amdgcn_sqrtf(fabsf(rc)), gx);
      }
    // sum the four lane groups (queries 4 g + r)
    gse = 0.5f * sum_xor32(sum_xor16(gse));
    gso = 0.5f * sum_xor32(sum_xor16(gso));
    gx = 0.25f * sum_xor32(sum_xor16(gx));
    if (g4 == 0) {
      float* rp = red + (t * (kT2 / 2) + n16) * 3 * kW2 + wv;
      rp[0] = gse;
      rp[kW2] = gso;
      rp[2 * kW2] = gx;
    }
  };

  // Merge of tile tt (its g sums complete, its rows still in the ring): a merging pair
  // becomes one slot k* = w_0 k_m + w_1 k_{m+1}, v* = count-weighted mean, n* = n_m +
  // n_{m+1} at output row S + 2p - (merging pairs before p) (S + p in a full round); a pair
  // that does not merge is copied to that row and the next; protected slots are copied to
  // row i (sinks) or i - M.  Thread = (pair n, 16-byte chunk ch) of the tile; the
  // arithmetic is the merge pass's.
  auto merge_tile = [&](int tt) {
    constexpr int CPR = M::CPR, E = 8;
    if (tid >= (kT2 / 2) * CPR) return;
    const int pn = tid / CPR, ch = tid % CPR;
    const int buf = tt % kRing2;
    const int64_t m0 = c0 + (int64_t)tt * kT2 + 2 * pn;
    const uint8_t* K_ = kr + buf * M::TILEB;
    const uint8_t* V_ = vr + buf * M::TILEB;
    const int64_t hoff_o = b * a.osb + hk * a.osh;
    TO* Ko = static_cast<TO*>(a.Ko) + hoff_o;
    TO* Vo = static_cast<TO*>(a.Vo) + hoff_o;
    int32_t* no = a.no + hoff_o / D;
    int32_t* so = a.so + hoff_o / D;
    const int64_t pend = a.S + 2 * a.P;   // first slot after the candidate pairs
    const int n0 = HAS_N ? nr[buf * kT2 + pn] : 1, n1 = HAS_N ? nr[buf * kT2 + 16 + pn] : 1;
    const uint4 k0 = *reinterpret_cast<const uint4*>(K_ + chunk_off<D>(pn, ch));
    const uint4 k1 = *reinterpret_cast<const uint4*>(K_ + chunk_off<D>(16 + pn, ch));
    const uint4 v0 = *reinterpret_cast<const uint4*>(V_ + chunk_off<D>(pn, ch));
    const uint4 v1 = *reinterpret_cast<const uint4*>(V_ + chunk_off<D>(16 + pn, ch));
    // c0 - S is even, so is the tile start - S: slot m0 starts pair (m0 - S) / 2
    const bool cand = m0 >= a.S && m0 + 1 < pend && m0 >= lo && m0 + 1 < hi;
    bool mrg = cand;
    int64_t pos0;   // output row of the pair (merged) or of slot m0 (copied)
    if constexpr (PARTIAL) {
      const int64_t p = (m0 - a.S) / 2;
      const int64_t rel = p - sel_c0 * kChunkPairs;
      const int k = cand ? (int)(rel >> 6) : 0, bit = (int)(rel & 63);
      const uint64_t mk = selm[k];
      mrg = cand && ((mk >> bit) & 1ull);
      pos0 = a.S + 2 * p - (selo[k] + __popcll(mk & ((1ull << bit) - 1ull)));
    } else {
      pos0 = a.S + (m0 - a.S) / 2;
    }
    if (mrg) {
      const float4* rq = reinterpret_cast<const float4*>(red + (tt * (kT2 / 2) + pn) * 3 * kW2);
      const float g0 = sum_waves(rq[0]), g1 = sum_waves(rq[1]), gx = sum_waves(rq[2]);
      float w0, w1;
      closed_form_weights(g0, gx, g1, w0, w1);
      {   // keys, then values: half the live temporaries
        float f0[E], f1[E], o[E];
        unpack<bf16>(k0, f0);
        unpack<bf16>(k1, f1);
        merge_keys<E>(f0, f1, w0, w1, o);
        store_elems<TO, E>(Ko + pos0 * D + ch * E, o);
      }
      {
        float f0[E], f1[E], o[E];
        unpack<bf16>(v0, f0);
        unpack<bf16>(v1, f1);
        merge_values<E>(f0, f1, n0, n1, o);
        store_elems<TO, E>(Vo + pos0 * D + ch * E, o);
      }
      const int nt = n0 + n1;
      if (ch == 0) {
        no[pos0] = nt;
        so[pos0] = (int32_t)m0;
      }
    } else {
      // pairs that do not merge, and slots outside the candidate pairs, are copied
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int64_t i = m0 + r;
        if (i < lo || i >= hi || (!cand && i >= a.S && i < pend)) continue;
        const int64_t pos = cand ? pos0 + r : i < a.S ? i : i - a.M;
        const uint4 kc = r ? k1 : k0, vc = r ? v1 : v0;
        if constexpr (std::is_same<TO, bf16>::value) {   // same type: the row's bytes as they are
          *reinterpret_cast<uint4*>(Ko + pos * D + ch * E) = kc;
          *reinterpret_cast<uint4*>(Vo + pos * D + ch * E) = vc;
        } else {
          float f[E];
          unpack<bf16>(kc, f);
          store_elems<TO, E>(Ko + pos * D + ch * E, f);
          unpack<bf16>(vc, f);
          store_elems<TO, E>(Vo + pos * D + ch * E, f);
        }
        if (ch == 0) {
          no[pos] = r ? n1 : n0;
          so[pos] = (int32_t)i;
        }
      }
    }
  };

  // Iteration t: tile t is computed, tile t - 1 merged, tile t + 1 is in flight and tile
  // t + 2 goes into the slot of tile t - 2, which every wave finished reading (its compute
  // and its merge) before this iteration's barrier.  A merge reads rows and counts that
  // other waves loaded, so no slot is refilled between a barrier and a merge of it.
  for (int t = 0; t < ntiles; ++t) {
    wait_tile(t + 1 < ntiles ? 1 : 0);   // tile t landed
    __syncthreads();
    if (t + 2 < ntiles) issue(t + 2);
    if (MERGE && t > 0) {
      // the merge sits between two barriers of this workgroup: let it finish first
      __builtin_amdgcn_s_setprio(2);
      merge_tile(t - 1);
      __builtin_amdgcn_s_setprio(0);
    }
    compute(t);
  }
  __syncthreads();
  if (MERGE) merge_tile(ntiles - 1);

  // per-slot totals of the chunk -> global; with several query blocks each block writes its
  // own slice and a second kernel adds the slices in block order (no atomics, so the sums
  // do not depend on the order the blocks finish in)
  float* gs = a.g_self;
  float* gx = a.g_cross;
  if (a.qpart) {
    gs = a.qpart + qb * (int64_t)BH * (a.N + a.P);
    gx = gs + (int64_t)BH * a.N;
  }
  for (int64_t s = lo + tid; s < hi; s += kW2 * 64) {
    const int64_t ls = s - c0;
    gs[bh * a.N + s] = sum_waves(reinterpret_cast<const float4*>(red)[(ls >> 1) * 3 + (ls & 1)]);
  }
  for (int64_t pp = tid; 2 * pp < hi - c0; pp += kW2 * 64) {
    const int64_t m0 = c0 + 2 * pp;
    const int64_t p = (m0 - a.S) / 2;
    if (m0 >= a.S && m0 >= lo && m0 + 1 < hi && p < a.P)
      gx[bh * a.P + p] = sum_waves(reinterpret_cast<const float4*>(red)[pp * 3 + 2]);
  }
}

// Sums of the per-query-block slices of pass 2, added in block order: element i < BN of the
// slices goes to g_self[i], element BN + j to g_cross[j].
__global__ void qsum_kernel(const float* __restrict__ part, int nqb, int64_t BN, int64_t BP,
                            float* __restrict__ g_self, float* __restrict__ g_cross) {
  const int64_t tot = BN + BP;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < tot; i += (int64_t)gridDim.x * blockDim.x) {
    float x = part[i];
    for (int q = 1; q < nqb; ++q) x += part[q * tot + i];
    if (i < BN) g_self[i] = x;
    else g_cross[i - BN] = x;
  }
}

// -------------------------------------------------------------------- dispatch --
bool use_mfma_scorer(const Shape& s) { return s.bf16 && (s.D == 64 || s.D == 128); }

// Chunk plan of pass 1: slot chunks are multiples of the tile, start at base = -(S mod 2)
// so that every tile starts on a candidate-pair boundary, and number about one per CU over
// the whole grid (pass 1 runs one workgroup per CU).
static void mfma_plan(const Shape& s, const RoundP& r, int64_t& base, int64_t& chunk, int& nsplit) {
  base = -(r.S & 1);
  const int64_t span = s.N - base;
  const int64_t BH = (int64_t)s.B * s.Hkv;
  const int64_t nqb = ((int64_t)s.G * r.W + kQB - 1) / kQB;
  int64_t want = (256 + BH * nqb - 1) / (BH * nqb);   // target chunks per (bh, query block)
  if (want < 1) want = 1;
  int64_t c = (span + want - 1) / want;
  if (c < 512 * kGroups) c = 512 * kGroups;             // keep partial records small
  c = (c + kChunk1Unit - 1) / kChunk1Unit * kChunk1Unit;
  chunk = c;
  nsplit = (int)((span + c - 1) / c);
}

// Pass-2 chunks: multiples of the tile, at most kChunk2Max slots, about two workgroups
// per CU over the grid.
static void p2_plan(const Shape& s, const RoundP& r, int64_t& chunk, int& nsplit) {
  const int64_t span = s.N + (r.S & 1);
  const int64_t BH = (int64_t)s.B * s.Hkv;
  const int64_t nqb = ((int64_t)s.G * r.W + kQB - 1) / kQB;
  int64_t want = (512 + BH * nqb - 1) / (BH * nqb);
  if (want < 1) want = 1;
  int64_t c = (span + want - 1) / want;
  c = (c + kT2 - 1) / kT2 * kT2;
  if (c > kChunk2Max) c = kChunk2Max;
  chunk = c;
  nsplit = (int)((span + c - 1) / c);
}

// Workspace: pass-1 partial records, then (256-byte aligned) the pass-2 operand pack.
static size_t part_bytes(const Shape& s, const RoundP& r) {
  int64_t base, chunk;
  int nsplit;
  mfma_plan(s, r, base, chunk, nsplit);
  const int64_t GW = (int64_t)s.G * r.W;
  return ((size_t)s.B * s.Hkv * GW * nsplit * (s.D + 4) * sizeof(float) + 255) / 256 * 256;
}

static int64_t pack_blocks(const Shape& s, const RoundP& r) { return ((int64_t)s.G * r.W + 31) / 32; }

static size_t pack_ops_bytes(const Shape& s, const RoundP& r) {
  return ((size_t)s.B * s.Hkv * pack_blocks(s, r) * 32 * 3 * s.D * 2 + 255) / 256 * 256;
}

static size_t pack_qc_bytes(const Shape& s, const RoundP& r) {
  return ((size_t)s.B * s.Hkv * pack_blocks(s, r) * 32 * 2 * sizeof(float) + 255) / 256 * 256;
}

// Per-query-block slices of the pass-2 sums (several 128-query blocks per kv head only).
static int64_t query_blocks(const Shape& s, const RoundP& r) { return ((int64_t)s.G * r.W + kQB - 1) / kQB; }
static size_t qpart_bytes(const Shape& s, const RoundP& r) {
  const int64_t nqb = query_blocks(s, r);
  return nqb > 1 ? (size_t)nqb * s.B * s.Hkv * (s.N + r.P) * sizeof(float) : 0;
}

// Workspace: pass-1 partial records, the pass-2 operand pack, the per-query constants and
// the per-query-block slices of the sums, each 256-byte aligned.
size_t mfma_score_workspace_bytes(const Shape& s, const RoundP& r) {
  return part_bytes(s, r) + pack_ops_bytes(s, r) + pack_qc_bytes(s, r) + qpart_bytes(s, r);
}

// merge: 0 = plain pass 2; 1 = fused merge with bf16 output; 2 = fused merge with fp32 output
template <int D>
static hipError_t launch_p2_d(const Shape& s, const RoundP& r, const P2Args& p2, int64_t base, int merge,
                              hipStream_t st);

template <int D>
static hipError_t launch_mfma_d(const Shape& s, const RoundP& r, const P1Args& p1_in, const P2Args& p2,
                                const CosArgs& ca, int64_t base, float* lse, float* O, int merge, hipStream_t st) {
  const int64_t BH = (int64_t)s.B * s.Hkv;
  const int nqb = (int)((p1_in.GW + kQB - 1) / kQB);
  const dim3 grid((unsigned)(BH * p1_in.nsplit * nqb));
  PackP pk;
  pk.ops = const_cast<uint4*>(p2.ops);
  pk.qc = const_cast<float*>(p2.qc);
  pk.Qw = p1_in.Qw;
  pk.nwb = p2.nwb;
  pk.GW = p1_in.GW;
  pk.Hkv = s.Hkv;
  pk.Hq = s.Hq;
  pk.G = s.G;
  pk.W = r.W;
  // one split per query: pass 1 finishes the statistics itself and no combine runs
  P1Args p1 = p1_in;
  p1.fin = p1.nsplit == 1;
  p1.lse = lse;
  p1.O = O;
  p1.pk = pk;
  if (p1.n)
    KVS_LAUNCH("score_pass1", (p1_mfma_kernel<D, true>), grid, dim3(kThreads), 0, st, p1, base, ca, (int)BH);
  else
    KVS_LAUNCH("score_pass1", (p1_mfma_kernel<D, false>), grid, dim3(kThreads), 0, st, p1, base, ca, (int)BH);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (!p1.fin) {
    e = launch_combine(p1.part, BH * p1.GW, p1.nsplit, D, lse, O, st, &pk);
    if (e != hipSuccess) return e;
  }
  return launch_p2_d<D>(s, r, p2, base, merge, st);
}

// Pass 2 once the operand pack exists: zero the sums when several query blocks accumulate
// into them, choose the pairs of a partial fused round, then the pass itself.
template <int D>
static hipError_t launch_p2_d(const Shape& s, const RoundP& r, const P2Args& p2, int64_t base, int merge,
                              hipStream_t st) {
  const int64_t BH = (int64_t)s.B * s.Hkv;
  const int nqb = (int)((p2.GW + kQB - 1) / kQB);
  hipError_t e = hipSuccess;
  if (nqb > 1) {
    if (merge) return hipErrorInvalidValue;   // the fused merge needs every query in one workgroup
    if (!p2.qpart) return hipErrorInvalidValue;
  }
  if (merge && r.M > 0 && r.M < r.P) {
    // partial round: choose the pairs from the pass-1 cosine before pass 2 merges them
    e = launch_select(s, r, nullptr, nullptr, p2.cos, nullptr, nullptr, const_cast<int32_t*>(p2.sel), st);
    if (e != hipSuccess) return e;
  }
  int64_t chunk2;
  int nsplit2;
  p2_plan(s, r, chunk2, nsplit2);
  const dim3 grid2((unsigned)(BH * nsplit2 * nqb));
  const dim3 blk(kW2 * 64);
  const int bhi = (int)BH;
  const bool part = merge && r.M < r.P;
#define KVS_P2(NAME, HN, MG, PT, TO)                                                                        \
  KVS_LAUNCH(NAME, (p2_mfma_kernel<D, HN, MG, PT, TO>), grid2, blk, 0, st, p2, base, chunk2, nsplit2, bhi)
  if (merge == 0) {
    if (p2.n) KVS_P2("score_pass2", true, false, false, bf16);
    else KVS_P2("score_pass2", false, false, false, bf16);
  } else if (!part) {
    if (merge == 1) {
      if (p2.n) KVS_P2("score_pass2_merge", true, true, false, bf16);
      else KVS_P2("score_pass2_merge", false, true, false, bf16);
    } else {
      if (p2.n) KVS_P2("score_pass2_merge", true, true, false, float);
      else KVS_P2("score_pass2_merge", false, true, false, float);
    }
  } else {
    if (merge == 1) {
      if (p2.n) KVS_P2("score_pass2_merge", true, true, true, bf16);
      else KVS_P2("score_pass2_merge", false, true, true, bf16);
    } else {
      if (p2.n) KVS_P2("score_pass2_merge", true, true, true, float);
      else KVS_P2("score_pass2_merge", false, true, true, float);
    }
  }
#undef KVS_P2
  e = hipGetLastError();
  if (e != hipSuccess || nqb == 1) return e;
  const int64_t BN = BH * s.N, BP = BH * r.P;
  const int64_t blocks = (BN + BP + 255) / 256 < 2048 ? (BN + BP + 255) / 256 : 2048;
  KVS_LAUNCH("qsum", qsum_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p2.qpart, nqb, BN, BP, p2.g_self,
             p2.g_cross);
  return hipGetLastError();
}

static hipError_t launch_score_any(const Shape& s, const RoundP& r, const void* K, const void* V, const int32_t* n,
                                   const void* Qw, float* lse, float* O, float* g_self, float* g_cross, float* cos,
                                   void* ws, const OutP* o, int32_t* sel_state, void* K_out, void* V_out,
                                   int32_t* n_out, int32_t* src_out, hipStream_t st) {
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
  P2Args p2{};
  p2.nwb = pack_blocks(s, r);
  p2.ops = reinterpret_cast<const uint4*>(static_cast<uint8_t*>(ws) + part_bytes(s, r));
  p2.qc = reinterpret_cast<const float*>(static_cast<uint8_t*>(ws) + part_bytes(s, r) + pack_ops_bytes(s, r));
  p2.qpart = qpart_bytes(s, r) ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + part_bytes(s, r) +
                                                          pack_ops_bytes(s, r) + pack_qc_bytes(s, r))
                               : nullptr;
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
  int merge = 0;
  p2.M = r.M;
  if (o) {
    p2.Ko = K_out;
    p2.Vo = V_out;
    p2.no = n_out;
    p2.so = src_out;
    p2.osb = o->sb;
    p2.osh = o->sh;
    p2.cos = cos;
    p2.sel = sel_state;
    p2.sel_stride = sel_stride_ints(r.P);
    merge = o->bf16 ? 1 : 2;
  }
  CosArgs ca;
  ca.K = K;
  ca.cos = r.P > 0 ? cos : nullptr;
  ca.S = r.S;
  ca.P = r.P;
  ca.sb = s.sb;
  ca.sh = s.sh;
  ca.Hkv = s.Hkv;
  return s.D == 64 ? launch_mfma_d<64>(s, r, p1, p2, ca, base, lse, O, merge, st)
                   : launch_mfma_d<128>(s, r, p1, p2, ca, base, lse, O, merge, st);
}

hipError_t launch_score_mfma(const Shape& s, const RoundP& r, const void* K, const void* V, const int32_t* n,
                             const void* Qw, float* lse, float* O, float* g_self, float* g_cross, float* cos,
                             void* ws, hipStream_t st) {
  return launch_score_any(s, r, K, V, n, Qw, lse, O, g_self, g_cross, cos, ws, nullptr, nullptr, nullptr, nullptr,
                          nullptr, nullptr, st);
}

bool fused_round_ok(const Shape& s, const RoundP& r) {
  return use_mfma_scorer(s) && (int64_t)s.G * r.W <= kQB;
}

hipError_t launch_score_merge_mfma(const Shape& s, const RoundP& r, const void* K, const void* V, const int32_t* n,
                                   const void* Qw, float* lse, float* O, float* g_self, float* g_cross, void* ws,
                                   float* cos, int32_t* sel_state, const OutP& o, void* K_out, void* V_out,
                                   int32_t* n_out, int32_t* src_out, hipStream_t st) {
  const bool part = r.M > 0 && r.M < r.P;
  return launch_score_any(s, r, K, V, n, Qw, lse, O, g_self, g_cross, part ? cos : nullptr, ws, &o,
                          part ? sel_state : nullptr, K_out, V_out, n_out, src_out, st);
}

}  // namespace kvs

namespace kvs {

// Workspace of a round given the window statistics: the pass-2 operand pack and the
// per-query constants (the cosine and the selection state follow, in the API layer).
size_t stats_pack_bytes(const Shape& s, const RoundP& r) {
  return pack_ops_bytes(s, r) + pack_qc_bytes(s, r) + qpart_bytes(s, r);
}

hipError_t launch_stats_merge_mfma(const Shape& s, const RoundP& r, const void* K, const void* V, const int32_t* n,
                                   const void* Qw, const float* lse, const float* O, float* g_self, float* g_cross,
                                   void* ws, float* cos, int32_t* sel_state, const OutP& o, void* K_out, void* V_out,
                                   int32_t* n_out, int32_t* src_out, hipStream_t st) {
  const bool part = r.M > 0 && r.M < r.P;
  P2Args p2{};
  p2.nwb = pack_blocks(s, r);
  p2.ops = static_cast<const uint4*>(ws);
  p2.qc = reinterpret_cast<const float*>(static_cast<uint8_t*>(ws) + pack_ops_bytes(s, r));
  p2.qpart = qpart_bytes(s, r) ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + pack_ops_bytes(s, r) +
                                                          pack_qc_bytes(s, r))
                               : nullptr;
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
  p2.M = r.M;
  p2.Ko = K_out;
  p2.Vo = V_out;
  p2.no = n_out;
  p2.so = src_out;
  p2.osb = o.sb;
  p2.osh = o.sh;
  p2.cos = part ? cos : nullptr;
  p2.sel = part ? sel_state : nullptr;
  p2.sel_stride = sel_stride_ints(r.P);
  PackP pk;
  pk.ops = const_cast<uint4*>(p2.ops);
  pk.qc = const_cast<float*>(p2.qc);
  pk.Qw = Qw;
  pk.nwb = p2.nwb;
  pk.GW = p2.GW;
  pk.Hkv = s.Hkv;
  pk.Hq = s.Hq;
  pk.G = s.G;
  pk.W = r.W;
  hipError_t e = launch_pack(lse, O, (int64_t)s.B * s.Hkv * p2.GW, s.D, pk, st);
  if (e != hipSuccess) return e;
  if (part) {
    CosArgs ca;
    ca.K = K;
    ca.cos = cos;
    ca.S = r.S;
    ca.P = r.P;
    ca.sb = s.sb;
    ca.sh = s.sh;
    ca.Hkv = s.Hkv;
    e = launch_pair_cos(s, ca, r.P, st);
    if (e != hipSuccess) return e;
  }
  const int64_t base = -(r.S & 1);
  if (fused_round_ok(s, r)) {
    const int merge = o.bf16 ? 1 : 2;
    return s.D == 64 ? launch_p2_d<64>(s, r, p2, base, merge, st) : launch_p2_d<128>(s, r, p2, base, merge, st);
  }
  // more than 128 window queries per kv head: pass 2 alone (query blocks accumulate), the
  // selection, then the merge pass
  e = s.D == 64 ? launch_p2_d<64>(s, r, p2, base, 0, st) : launch_p2_d<128>(s, r, p2, base, 0, st);
  if (e == hipSuccess && part)
    e = launch_select(s, r, g_self, g_cross, cos, nullptr, nullptr, sel_state, st);
  if (e == hipSuccess)
    e = launch_merge(s, r, K, V, n, g_self, g_cross, part ? sel_state : nullptr, o, K_out, V_out, n_out, src_out, st);
  return e;
}

}  // namespace kvs
