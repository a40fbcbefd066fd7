// Spectral split of adjacent-key cosines (kvs_spectral_modes).
//
// KVSlimmer deep-dive (charles2530.github.io), section 数学主线一: keys are y = x W, so
// with M = W W^T = U L U^T and p_{t,i} = x_t u_i, y_t . y_{t+1} = sum_i l_i p_{t,i} p_{t+1,i}
// and cos(y_t, y_{t+1}) splits into one term per eigen-mode,
//   c_{t,i} = l_i p_{t,i} p_{t+1,i} / (|y_t| |y_{t+1}|),  |y_t|^2 = sum_i l_i p_{t,i}^2,
// which shows how few high-eigenvalue modes carry the similarity of neighbouring keys
// (the spectral asymmetry that makes keys, not values, mergeable).  The caller supplies
// the modes with a nonzero eigenvalue (for W of d_k columns, the left singular vectors
// and squared singular values of W).  Two launches: the projections P = X U^T on the
// matrix cores (bf16 in, fp32 accumulate, the modes staged in LDS), then one wave per
// adjacent pair for the norms, the per-mode terms and their sum.
#include "kvs_common.h"
#include "kvs_internal.h"

namespace kvs {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 sp_bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float sp_f32x4_t;
typedef unsigned int sp_u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ sp_bf16x8_t sp_as_bf16x8(const uint4& u) {
  sp_u32x4_t v = {u.x, u.y, u.z, u.w};
  return __builtin_bit_cast(sp_bf16x8_t, v);
}

constexpr int kSpecBlocks = 8;   // 16-mode blocks per workgroup: 128 modes
constexpr int kSpecK = 64;       // elements of d per staged slice of the modes

// P[t, i] = x_t . u_i on v_mfma_f32_16x16x32_bf16: A = 16 tokens x 32 of d (lane l: token
// l % 16, elements 8 (l / 16) .. + 7, read straight from X: 16 contiguous bytes), B = 32 of
// d x 16 modes (lane l: mode l % 16, the same elements of its row of U); the result lane l
// holds tokens 4 (l / 16) + r of mode l % 16.  The workgroup's 128 modes are staged in LDS
// 64 elements of d at a time, double-buffered; piece c (8 elements) of mode row m sits at
// c ^ (m & 7), so the 16 lanes that read 16 different rows at one piece spread over the
// banks.  Each wave owns TB 16-token blocks: every B operand read from LDS feeds TB MFMAs
// (TB = 2 when there are tokens enough to fill the chip with 128-token workgroups).
template <int TB>
__global__ __launch_bounds__(256) void spectral_proj_kernel(const bf16* __restrict__ X, const bf16* __restrict__ U,
                                                           int64_t T, int d, int r, float* __restrict__ P) {
  constexpr int PIECES = kSpecK / 8;                    // 16-byte pieces per staged row
  constexpr int ROWS = 16 * kSpecBlocks;                // staged mode rows
  constexpr int PER_THREAD = ROWS * PIECES / 256;       // 16-byte loads per thread per slice
  __shared__ uint4 bs[2][ROWS * PIECES];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int rw = lane & 15, kc = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * (64 * TB) + 16 * TB * wv;
  const int i0 = (int)blockIdx.y * ROWS;
  const uint4 zero = make_uint4(0, 0, 0, 0);
  // A rows of the wave's token blocks; a token past T reads token 0 and is zeroed
  bool va[TB];
  const bf16* xa[TB];
#pragma unroll
  for (int h = 0; h < TB; ++h) {
    va[h] = t0 + 16 * h + rw < T;
    xa[h] = X + (va[h] ? t0 + 16 * h + rw : 0) * d + 8 * kc;
  }
  // staging loads of this thread: piece idx = tid + 256 q of the slice, row idx / PIECES
  auto stage_load = [&](int k0, uint4 (&v)[PER_THREAD]) {
#pragma unroll
    for (int q = 0; q < PER_THREAD; ++q) {
      const int idx = tid + 256 * q;
      const int row = idx / PIECES, pc = idx % PIECES;
      const int mi = i0 + row;
      v[q] = *reinterpret_cast<const uint4*>(U + (int64_t)(mi < r ? mi : 0) * d + k0 + 8 * pc);
      if (mi >= r) v[q] = zero;
    }
  };
  auto stage_store = [&](int buf, const uint4 (&v)[PER_THREAD]) {
#pragma unroll
    for (int q = 0; q < PER_THREAD; ++q) {
      const int idx = tid + 256 * q;
      const int row = idx / PIECES, pc = idx % PIECES;
      bs[buf][row * PIECES + (pc ^ (row & 7))] = v[q];
    }
  };
  sp_f32x4_t acc[TB][kSpecBlocks];
#pragma unroll
  for (int h = 0; h < TB; ++h)
#pragma unroll
    for (int j = 0; j < kSpecBlocks; ++j) acc[h][j] = sp_f32x4_t{0.f, 0.f, 0.f, 0.f};
  // the A operands of one slice: [s2][token block]; the next slice's are loaded while this
  // one's products run
  constexpr int S2 = kSpecK / 32;
  auto load_a = [&](int k0, uint4 (&a)[S2][TB]) {
#pragma unroll
    for (int s2 = 0; s2 < S2; ++s2)
#pragma unroll
      for (int h = 0; h < TB; ++h) {
        a[s2][h] = *reinterpret_cast<const uint4*>(xa[h] + k0 + 32 * s2);
        if (!va[h]) a[s2][h] = zero;
      }
  };
  uint4 nxt[PER_THREAD];
  uint4 acur[S2][TB], anxt[S2][TB];
  stage_load(0, nxt);
  load_a(0, acur);
  stage_store(0, nxt);
  __syncthreads();
  const int nk = d / kSpecK;
  for (int kb = 0; kb < nk; ++kb) {
    const int buf = kb & 1;
    const int k0 = kb * kSpecK;
    if (kb + 1 < nk) {
      stage_load(k0 + kSpecK, nxt);
      load_a(k0 + kSpecK, anxt);
    }
#pragma unroll
    for (int s2 = 0; s2 < S2; ++s2) {
#pragma unroll
      for (int j = 0; j < kSpecBlocks; ++j) {
        const int row = 16 * j + rw, pc = 4 * s2 + kc;
        const uint4 b = bs[buf][row * PIECES + (pc ^ (row & 7))];
#pragma unroll
        for (int h = 0; h < TB; ++h)
          acc[h][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sp_as_bf16x8(acur[s2][h]), sp_as_bf16x8(b), acc[h][j],
                                                              0, 0, 0);
      }
    }
#pragma unroll
    for (int s2 = 0; s2 < S2; ++s2)
#pragma unroll
      for (int h = 0; h < TB; ++h) acur[s2][h] = anxt[s2][h];
    if (kb + 1 < nk) stage_store(buf ^ 1, nxt);   // that buffer was last read before the previous barrier
    __syncthreads();
  }
#pragma unroll
  for (int h = 0; h < TB; ++h)
#pragma unroll
    for (int j = 0; j < kSpecBlocks; ++j) {
      const int mi = i0 + 16 * j + rw;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t t = t0 + 16 * h + 4 * kc + q;
        if (mi < r && t < T) P[t * r + mi] = acc[h][j][q];
      }
    }
}

// One wave per adjacent pair (t, t + 1): both weighted norms, every mode's term, the sum.
// A zero norm gives zero terms.
__global__ __launch_bounds__(256) void spectral_pair_kernel(const float* __restrict__ P, const float* __restrict__ lam,
                                                           int64_t T, int r, float* __restrict__ c,
                                                           float* __restrict__ cosv) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t + 1 >= T) return;   // whole waves leave; only wave-level reductions follow
  const float* p0 = P + t * r;
  const float* p1 = p0 + r;
  float n0 = 0.f, n1 = 0.f;
  for (int i = lane; i < r; i += 64) {
    n0 = __builtin_fmaf(lam[i] * p0[i], p0[i], n0);
    n1 = __builtin_fmaf(lam[i] * p1[i], p1[i], n1);
  }
  n0 = group_sum<64>(n0);
  n1 = group_sum<64>(n1);
  const float den = sqrtf(n0) * sqrtf(n1);
  const float inv = den > 0.f ? 1.f / den : 0.f;
  float s = 0.f;
  for (int i = lane; i < r; i += 64) {
    const float ci = lam[i] * p0[i] * p1[i] * inv;
    if (c) c[t * r + i] = ci;
    s += ci;
  }
  s = group_sum<64>(s);
  if (lane == 0) cosv[t] = s;
}

hipError_t launch_spectral(const void* X, int64_t T, int d, const void* U, const float* lam, int r, float* P,
                           float* c, float* cosv, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  const unsigned mb = (unsigned)((r + 16 * kSpecBlocks - 1) / (16 * kSpecBlocks));
  // 32 tokens per wave when 128-token workgroups still give two per CU, else 16
  if ((T + 127) / 128 * mb >= 512)
    KVS_LAUNCH("spectral_proj", spectral_proj_kernel<2>, dim3((unsigned)((T + 127) / 128), mb), dim3(256), 0, st,
               static_cast<const bf16*>(X), static_cast<const bf16*>(U), T, d, r, P);
  else
    KVS_LAUNCH("spectral_proj", spectral_proj_kernel<1>, dim3((unsigned)((T + 63) / 64), mb), dim3(256), 0, st,
               static_cast<const bf16*>(X), static_cast<const bf16*>(U), T, d, r, P);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || T < 2) return e;
  KVS_LAUNCH("spectral_pair", spectral_pair_kernel, dim3((unsigned)((T - 1 + 3) / 4)), dim3(256), 0, st, P, lam, T, r,
             c, cosv);
  return hipGetLastError();
}

}  // namespace kvs
