// Exact-gradient diagnostics (kvs_exact_e_diag).
//
// KVSlimmer deep-dive (charles2530.github.io), section 数学主线三: with an upstream
// gradient E = dL/do the Hessian block of keys i, j is g_ij q q^T / d_k, where
// g_ij = E^T c_ij and c11 = a_m (1 - 2 a_m)(v_m - o), c22 likewise for m + 1,
// c12 = -a_m a_{m+1} (v_m + v_{m+1} - 2 o) (section 数学主线四 names the c vectors).
// Section 数学主线二 gives the stationary k* of the second-order merge loss in g11, g12,
// g22; section 数学主线四 replaces each g by a norm of c under the assumption that E
// makes the same angle with c11 and c22 and the opposite one with c12.  This pass
// computes, for a caller-supplied E per window query, the exact scalars (summed over
// the window like the norms), the norm-weighted angle sums, both closed-form weight
// pairs and the exact second-order loss of each merged key, so that the one
// approximation of the forward-only weights can be measured.  A diagnostic: plain fp32
// VALU arithmetic, four lanes per candidate pair or single slot, one pass over the
// window per unit, the window's q, o and E rows staged in LDS 16 queries at a time.
#include "kvs_common.h"
#include "kvs_internal.h"

namespace kvs {

struct DiagArgs {
  const void* K;
  const void* V;
  const int32_t* n;
  const void* Qw;
  const float* E;
  const float* lse;
  const float* O;
  float* slot_out;   // [B*Hkv, N, 3]: sum E.c_ii, sum |E||c_ii|, sum |c_ii|
  float* pair_out;   // [B*Hkv, P, 9]: the same three for c12, exact w0 w1, forward-only w0 w1,
                     //                exact loss at both k*
  int64_t N, S, P, sb, sh, GW;
  int Hkv, Hq, G, W;
  float scale;
};

// Stationary point of the loss in (g11, g12, g22); the plain average when the curvature
// g11 + 2 g12 + g22 vanishes against |g11| + 2|g12| + |g22| (1e-6) or is not finite.
__device__ __forceinline__ void exact_weights(float g11, float g12, float g22, float& w0, float& w1) {
  const float den = g11 + 2.f * g12 + g22;
  const float sc = fabsf(g11) + 2.f * fabsf(g12) + fabsf(g22);
  if (!isfinite(den) || fabsf(den) <= 1e-6f * sc) {
    w0 = w1 = 0.5f;
    return;
  }
  const float inv = 1.f / den;
  w0 = (g11 + g12) * inv;
  w1 = (g12 + g22) * inv;
}

constexpr int kDiagQB = 16;   // window queries staged in LDS at a time

__device__ __forceinline__ float elem_to_float(float x) { return x; }
__device__ __forceinline__ float elem_to_float(bf16 x) { return __uint_as_float((uint32_t)x.bits << 16); }

template <typename T, int D, bool HAS_N>
__global__ __launch_bounds__(256) void exact_e_kernel(DiagArgs a) {
  constexpr int DQ = D / 4;
  constexpr int EC = Elt<T>::kPerChunk;
  // the staged window rows: q (scaled to fp32), o and E, [kDiagQB][D] each
  __shared__ float qs[kDiagQB * D], os[kDiagQB * D], es[kDiagQB * D];
  const int tid = threadIdx.x;
  const int ql = tid & 3;
  const int64_t u = (int64_t)blockIdx.x * 64 + (tid >> 2);
  const int64_t bh = blockIdx.y;
  const int64_t b = bh / a.Hkv, h = bh - b * a.Hkv;
  const int64_t n_units = a.S + a.P + (a.N - a.S - 2 * a.P);
  const bool valid = u < n_units;   // every thread stays for the staging barriers
  bool pair = false;
  int64_t m = 0, p = 0;
  if (!valid) {
  } else if (u < a.S) {
    m = u;
  } else if (u < a.S + a.P) {
    pair = true;
    p = u - a.S;
    m = a.S + 2 * p;
  } else {
    m = a.S + 2 * a.P + (u - a.S - a.P);
  }
  const T* Kp = static_cast<const T*>(a.K) + b * a.sb + h * a.sh;
  const T* Vp = static_cast<const T*>(a.V) + b * a.sb + h * a.sh;
  const int32_t* np = HAS_N ? a.n + (b * a.sb + h * a.sh) / D : nullptr;
  const T* Qp = static_cast<const T*>(a.Qw) + ((b * a.Hq + h * a.G) * (int64_t)a.W) * D;
  const float* Op = a.O + bh * a.GW * (int64_t)D;
  const float* Ep = a.E + bh * a.GW * (int64_t)D;
  const float* Lp = a.lse + bh * a.GW;

  float k0[DQ], k1[DQ], v0[DQ], v1[DQ];
  for (int d0 = 0; d0 < DQ; d0 += EC) {
    if (valid) {
      unpack<T>(load16(Kp + m * D + ql * DQ + d0), k0 + d0);
      unpack<T>(load16(Vp + m * D + ql * DQ + d0), v0 + d0);
    } else {
#pragma unroll
      for (int e = 0; e < EC; ++e) k0[d0 + e] = v0[d0 + e] = 0.f;
    }
    if (pair) {
      unpack<T>(load16(Kp + (m + 1) * D + ql * DQ + d0), k1 + d0);
      unpack<T>(load16(Vp + (m + 1) * D + ql * DQ + d0), v1 + d0);
    } else {
#pragma unroll
      for (int e = 0; e < EC; ++e) k1[d0 + e] = v1[d0 + e] = 0.f;
    }
  }
  float dk = 0.f;   // ||k_m - k_{m+1}||^2
#pragma unroll
  for (int d = 0; d < DQ; ++d) dk = __builtin_fmaf(k0[d] - k1[d], k0[d] - k1[d], dk);
  dk = group_sum<4>(dk);
  const float b0 = (HAS_N && valid) ? logf((float)np[m]) : 0.f;
  const float b1 = (HAS_N && pair) ? logf((float)np[m + 1]) : 0.f;
  float ge0 = 0.f, ne0 = 0.f, gf0 = 0.f, ge1 = 0.f, ne1 = 0.f, gf1 = 0.f, gex = 0.f, nex = 0.f, gfx = 0.f;
  for (int64_t w0 = 0; w0 < a.GW; w0 += kDiagQB) {
    const int nq = (int)(a.GW - w0 < kDiagQB ? a.GW - w0 : kDiagQB);
    __syncthreads();   // the previous block's rows are no longer read
    for (int i = tid; i < nq * D; i += 256) {
      qs[i] = elem_to_float(Qp[w0 * D + i]);
      os[i] = Op[w0 * D + i];
      es[i] = Ep[w0 * D + i];
    }
    __syncthreads();
    for (int wi = 0; wi < nq; ++wi) {
      const float* qr = qs + wi * D + ql * DQ;
      const float* orow = os + wi * D + ql * DQ;
      const float* er = es + wi * D + ql * DQ;
      float d0 = 0.f, d1 = 0.f, r0 = 0.f, r1 = 0.f, rc = 0.f, e0 = 0.f, e1 = 0.f, ec = 0.f, ee = 0.f;
#pragma unroll
      for (int e = 0; e < DQ; ++e) {
        const float o = orow[e], g = er[e], q = qr[e];
        const float x0 = v0[e] - o, x1 = v1[e] - o, xc = x0 + x1;
        d0 = __builtin_fmaf(q, k0[e], d0);
        d1 = __builtin_fmaf(q, k1[e], d1);
        r0 = __builtin_fmaf(x0, x0, r0);
        r1 = __builtin_fmaf(x1, x1, r1);
        rc = __builtin_fmaf(xc, xc, rc);
        e0 = __builtin_fmaf(g, x0, e0);
        e1 = __builtin_fmaf(g, x1, e1);
        ec = __builtin_fmaf(g, xc, ec);
        ee = __builtin_fmaf(g, g, ee);
      }
      d0 = group_sum<4>(d0);
      d1 = group_sum<4>(d1);
      r0 = group_sum<4>(r0);
      r1 = group_sum<4>(r1);
      rc = group_sum<4>(rc);
      e0 = group_sum<4>(e0);
      e1 = group_sum<4>(e1);
      ec = group_sum<4>(ec);
      ee = group_sum<4>(ee);
      const float lw = Lp[w0 + wi];
      const float en = sqrtf(ee);
      const float a0 = expf(__builtin_fmaf(a.scale, d0, b0) - lw);
      const float s0 = a0 * (1.f - 2.f * a0);
      ge0 = __builtin_fmaf(s0, e0, ge0);
      gf0 = __builtin_fmaf(fabsf(s0), sqrtf(r0), gf0);
      ne0 = __builtin_fmaf(fabsf(s0) * sqrtf(r0), en, ne0);
      if (pair) {
        const float a1 = expf(__builtin_fmaf(a.scale, d1, b1) - lw);
        const float s1 = a1 * (1.f - 2.f * a1);
        ge1 = __builtin_fmaf(s1, e1, ge1);
        gf1 = __builtin_fmaf(fabsf(s1), sqrtf(r1), gf1);
        ne1 = __builtin_fmaf(fabsf(s1) * sqrtf(r1), en, ne1);
        const float ax = a0 * a1;
        gex = __builtin_fmaf(-ax, ec, gex);
        gfx = __builtin_fmaf(ax, sqrtf(rc), gfx);
        nex = __builtin_fmaf(ax * sqrtf(rc), en, nex);
      }
    }
  }
  if (!valid) return;
  if (ql != 0) return;
  float* so = a.slot_out + (bh * a.N + m) * 3;
  so[0] = ge0;
  so[1] = ne0;
  so[2] = gf0;
  if (!pair) return;
  so[3] = ge1;
  so[4] = ne1;
  so[5] = gf1;
  float we0, we1, wf0, wf1;
  exact_weights(ge0, gex, ge1, we0, we1);
  closed_form_weights(gf0, gfx, gf1, wf0, wf1);
  // loss at k = w0 k_m + w1 k_{m+1} (w0 + w1 = 1): ||k_m - k_{m+1}||^2 (g11 w1^2 - 2 g12 w0 w1 + g22 w0^2)
  auto loss = [&](float w0, float w1) { return dk * (ge0 * w1 * w1 - 2.f * gex * w0 * w1 + ge1 * w0 * w0); };
  float* po = a.pair_out + (bh * a.P + p) * 9;
  po[0] = gex;
  po[1] = nex;
  po[2] = gfx;
  po[3] = we0;
  po[4] = we1;
  po[5] = wf0;
  po[6] = wf1;
  po[7] = loss(we0, we1);
  po[8] = loss(wf0, wf1);
}

hipError_t launch_exact_e(const Shape& s, const RoundP& r, const void* K, const void* V, const int32_t* n,
                          const void* Qw, const float* E, const float* lse, const float* O, float* slot_out,
                          float* pair_out, hipStream_t st) {
  DiagArgs a;
  a.K = K;
  a.V = V;
  a.n = n;
  a.Qw = Qw;
  a.E = E;
  a.lse = lse;
  a.O = O;
  a.slot_out = slot_out;
  a.pair_out = pair_out;
  a.N = s.N;
  a.S = r.S;
  a.P = r.P;
  a.sb = s.sb;
  a.sh = s.sh;
  a.GW = (int64_t)s.G * r.W;
  a.Hkv = s.Hkv;
  a.Hq = s.Hq;
  a.G = s.G;
  a.W = r.W;
  a.scale = r.scale;
  const int64_t units = r.S + r.P + (s.N - r.S - 2 * r.P);
  if (units <= 0) return hipSuccess;
  const dim3 grid((unsigned)((units + 63) / 64), (unsigned)(s.B * s.Hkv));
#define KVS_DIAG(T, DD)                                                                          \
  if (n) KVS_LAUNCH("exact_e", (exact_e_kernel<T, DD, true>), grid, dim3(256), 0, st, a);       \
  else KVS_LAUNCH("exact_e", (exact_e_kernel<T, DD, false>), grid, dim3(256), 0, st, a);
  if (s.bf16) {
    if (s.D == 64) { KVS_DIAG(bf16, 64) } else { KVS_DIAG(bf16, 128) }
  } else {
    if (s.D == 64) { KVS_DIAG(float, 64) } else { KVS_DIAG(float, 128) }
  }
#undef KVS_DIAG
  return hipGetLastError();
}

}  // namespace kvs
