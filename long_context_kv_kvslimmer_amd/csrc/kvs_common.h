// Device-side helpers shared by the gfx950 kernels of libkvslim.
//
// Element types: `bf16` (raw 16-bit storage) and `float`.  Every kernel reads rows in
// 16-byte chunks: a row of D elements is LPR = D * sizeof(T) / 16 lanes, each holding
// EPL = 16 / sizeof(T) consecutive elements ("row layout").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvs {

struct bf16 {
  uint16_t bits;
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 values -> two bf16 (a in the low half), round to nearest even: one packed
// hardware conversion on gfx950.
typedef __bf16 bf16x2_hw_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2_hw_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

template <typename T>
struct Elt;

template <>
struct Elt<float> {
  static constexpr int kPerChunk = 4;
};

template <>
struct Elt<bf16> {
  static constexpr int kPerChunk = 8;
};

// One 16-byte chunk -> floats.
template <typename T>
__device__ __forceinline__ void unpack(const uint4& c, float* f);

template <>
__device__ __forceinline__ void unpack<float>(const uint4& c, float* f) {
  f[0] = __uint_as_float(c.x);
  f[1] = __uint_as_float(c.y);
  f[2] = __uint_as_float(c.z);
  f[3] = __uint_as_float(c.w);
}

template <>
__device__ __forceinline__ void unpack<bf16>(const uint4& c, float* f) {
  f[0] = bf16_lo(c.x);
  f[1] = bf16_hi(c.x);
  f[2] = bf16_lo(c.y);
  f[3] = bf16_hi(c.y);
  f[4] = bf16_lo(c.z);
  f[5] = bf16_hi(c.z);
  f[6] = bf16_lo(c.w);
  f[7] = bf16_hi(c.w);
}

__device__ __forceinline__ uint4 load16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Store E floats as type T at p (E * sizeof(T) bytes, 8- or 16-byte aligned).
template <typename T, int E>
__device__ __forceinline__ void store_elems(T* p, const float* f);

template <>
__device__ __forceinline__ void store_elems<float, 4>(float* p, const float* f) {
  *reinterpret_cast<uint4*>(p) =
      make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
}

template <>
__device__ __forceinline__ void store_elems<float, 8>(float* p, const float* f) {
  store_elems<float, 4>(p, f);
  store_elems<float, 4>(p + 4, f + 4);
}

template <>
__device__ __forceinline__ void store_elems<bf16, 4>(bf16* p, const float* f) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]));
}

template <>
__device__ __forceinline__ void store_elems<bf16, 8>(bf16* p, const float* f) {
  *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                                            pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
}

// Cross-lane moves inside a 16-lane row (DPP): lane i reads lane i^1, i^2, the mirror
// within its 8-lane half (7 - i) or within its row (15 - i).  On data that is already
// uniform over 4 (resp. 8) lanes the two mirrors pair exactly as i^4 (resp. i^8).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

// Butterfly sum over aligned groups of L lanes (L a power of two <= 64): DPP inside a
// 16-lane row, shuffles across rows.  Every lane of a group ends with the same bits
// (floating-point addition is commutative), so the result does not depend on which lane
// reads it.
template <int L>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (L >= 2) x += dpp<kDppXor1>(x);
  if constexpr (L >= 4) x += dpp<kDppXor2>(x);
  if constexpr (L >= 8) x += dpp<kDppHalfMirror>(x);
  if constexpr (L >= 16) x += dpp<kDppMirror>(x);
  if constexpr (L >= 32) x += __shfl_xor(x, 16, 64);
  if constexpr (L >= 64) x += __shfl_xor(x, 32, 64);
  return x;
}

template <int L>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (L >= 2) x = fmaxf(x, dpp<kDppXor1>(x));
  if constexpr (L >= 4) x = fmaxf(x, dpp<kDppXor2>(x));
  if constexpr (L >= 8) x = fmaxf(x, dpp<kDppHalfMirror>(x));
  if constexpr (L >= 16) x = fmaxf(x, dpp<kDppMirror>(x));
  if constexpr (L >= 32) x = fmaxf(x, __shfl_xor(x, 16, 64));
  if constexpr (L >= 64) x = fmaxf(x, __shfl_xor(x, 32, 64));
  return x;
}

// Cosine of two rows held in row layout (each lane: E elements of both rows, LPR lanes per
// row).  The one routine every kernel uses, so that the selection pass and the merge pass
// see bit-identical values.  A zero norm gives 1 if the rows are equal, else 0; -0 is
// returned as +0 so that the ordering key below is a total order consistent with ==.
// All lanes of the wave must call it together (it uses a ballot).
template <int E, int LPR>
__device__ __forceinline__ float pair_cos(const float* a, const float* b) {
  float d = 0.f, na = 0.f, nb = 0.f;
  bool eq = true;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    d = __builtin_fmaf(a[e], b[e], d);
    na = __builtin_fmaf(a[e], a[e], na);
    nb = __builtin_fmaf(b[e], b[e], nb);
    eq = eq && (a[e] == b[e]);
  }
  d = group_sum<LPR>(d);
  na = group_sum<LPR>(na);
  nb = group_sum<LPR>(nb);
  const uint64_t neq = __ballot(!eq);
  const int lane = threadIdx.x & 63;
  const uint64_t gmask = (LPR == 64 ? ~0ull : ((1ull << LPR) - 1ull)) << (lane & ~(LPR - 1));
  if (na == 0.f || nb == 0.f) return (neq & gmask) ? 0.f : 1.f;
  const float c = d * __builtin_amdgcn_rsqf(na) * __builtin_amdgcn_rsqf(nb);
  return c + 0.0f;
}

// Order-preserving unsigned image of an fp32 value: larger float -> larger key.
__device__ __forceinline__ uint32_t order_key(float c) {
  uint32_t u = __float_as_uint(c);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Closed-form forward-only merge weights from the window-summed norms
// g11 = sum ||c11||, g12 = sum ||c12||, g22 = sum ||c22|| (KVSlimmer deep-dive, section
// 数学主线四, closed-form k*), with the plain average of section 数学主线二 when the
// denominator is not finite or not clearly positive.  Explicit fma pins the rounding; one
// hardware reciprocal (v_rcp_f32, within 1 ulp; every path calls this routine, so they all
// round alike) forms 1 / A for both weights.
__device__ __forceinline__ void closed_form_weights(float g11, float g12, float g22, float& w0, float& w1) {
  const float A = __builtin_fmaf(-2.f, g12, g11) + g22;
  const float scale = __builtin_fmaf(2.f, g12, g11 + g22);
  if (!(A > 1e-6f * scale) || isinf(A)) {
    w0 = 0.5f;
    w1 = 0.5f;
  } else {
    const float inv = __builtin_amdgcn_rcpf(A);
    w0 = (g11 - g12) * inv;
    w1 = (g22 - g12) * inv;
  }
}

// One merged slot, E elements of it: k* = w0 k_m + w1 k_{m+1}; v* = the count-weighted
// mean, with weights n_m / (n_m + n_{m+1}) and n_{m+1} / (n_m + n_{m+1}) formed once per
// pair from one hardware reciprocal (exact for a power-of-two total, so without counts both
// weights are 1/2 exactly).
template <int E>
__device__ __forceinline__ void merge_keys(const float* kf0, const float* kf1, float w0, float w1, float* ko) {
#pragma unroll
  for (int e = 0; e < E; ++e) ko[e] = __builtin_fmaf(w0, kf0[e], w1 * kf1[e]);
}

template <int E>
__device__ __forceinline__ void merge_values(const float* vf0, const float* vf1, int n0, int n1, float* vo) {
  const float inv = __builtin_amdgcn_rcpf((float)(n0 + n1));
  const float u0 = (float)n0 * inv, u1 = (float)n1 * inv;
#pragma unroll
  for (int e = 0; e < E; ++e) vo[e] = __builtin_fmaf(u0, vf0[e], u1 * vf1[e]);
}

// Selection threshold of one (batch, head), written by the selection kernel.
struct SelHeader {
  uint32_t tau_key;  // order_key of the threshold cosine
  int32_t p_tau;     // among pairs whose key equals tau_key, those with p <= p_tau are selected
  int32_t n_merge;
  int32_t n_chunks;
};

__device__ __forceinline__ bool is_selected(uint32_t key, int64_t p, const SelHeader& h) {
  return key > h.tau_key || (key == h.tau_key && p <= (int64_t)h.p_tau);
}

}  // namespace kvs
