// Decode attention over a (merged) KV cache (kvs_decode_attn).
//
// KVSlimmer deep-dive (charles2530.github.io), section 数学主线三: softmax attention of
// one query; every slot's logit carries + ln n (n raw tokens merged into the slot, whose
// stored value is their mean), which reproduces attention over the unmerged values.
//
// Split-K over slots: a workgroup owns a contiguous slot range of one (batch, kv-head)
// and serves all G query heads of that kv head, so K and V are read once per step.  A
// row is LPR lanes x 16 bytes (row layout); each lane group keeps an online softmax
// (running max, sum, partial output) per head, updated once per block of RB rows.
// Groups are merged in LDS into one partial record per (query head, split); the shared
// log-sum-exp combine turns the records into the output.
#include "kvs_common.h"
#include "kvs_internal.h"

namespace kvs {

struct DecArgs {
  const void* K;
  const void* V;
  const int32_t* n;
  const void* q;
  float* part;
  int64_t N, sb, sh, chunk;
  int Hkv, Hq, nsplit;
  float scale;
};

// Split plan: every split is non-empty.
static void decode_plan(int64_t N, int64_t& chunk, int& nsplit) {
  int64_t c = (N + 255) / 256;
  if (c < 256) c = 256;
  c = (c + 63) / 64 * 64;
  chunk = c;
  nsplit = (int)((N + c - 1) / c);
  if (nsplit < 1) nsplit = 1;
}

template <typename T, int D, int G, bool HAS_N>
__global__ __launch_bounds__(256) void decode_kernel(DecArgs a) {
  constexpr int E = Elt<T>::kPerChunk;
  constexpr int LPR = D / E;
  constexpr int NG = 256 / LPR;
  constexpr int RB = 4;
  __shared__ float sm[NG][G];
  __shared__ float sl[NG][G];
  __shared__ float so[NG][D];

  const int tid = threadIdx.x;
  const int grp = tid / LPR, j = tid % LPR;
  const int64_t bh = blockIdx.y;
  const int64_t b = bh / a.Hkv, h = bh - b * a.Hkv;
  const T* Kp = static_cast<const T*>(a.K) + b * a.sb + h * a.sh;
  const T* Vp = static_cast<const T*>(a.V) + b * a.sb + h * a.sh;
  const int32_t* np = HAS_N ? a.n + (b * a.sb + h * a.sh) / D : nullptr;
  const T* qp = static_cast<const T*>(a.q) + (b * a.Hq + h * G) * (int64_t)D;

  float qf[G][E];
  const float c = a.scale * kLog2e;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    unpack<T>(load16(qp + g * D + j * E), qf[g]);
#pragma unroll
    for (int e = 0; e < E; ++e) qf[g][e] *= c;
  }
  float m[G], l[G], o[G][E];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) o[g][e] = 0.f;
  }

  const int64_t s_begin = (int64_t)blockIdx.x * a.chunk;
  const int64_t s_end = min(a.N, s_begin + a.chunk);
  for (int64_t base = s_begin + grp * RB; base < s_end; base += NG * RB) {
    uint4 kc[RB], vc[RB];
    float lg[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int64_t row = base + r;
      if (row < s_end) {
        kc[r] = load16(Kp + row * D + j * E);
        vc[r] = load16(Vp + row * D + j * E);
        lg[r] = HAS_N ? __log2f((float)np[row]) : 0.f;
      } else {
        kc[r] = vc[r] = make_uint4(0, 0, 0, 0);
        lg[r] = 0.f;
      }
    }
    float ev[RB][G];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      float kf[E];
      unpack<T>(kc[r], kf);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) d = __builtin_fmaf(qf[g][e], kf[e], d);
        d = group_sum<LPR>(d);
        ev[r][g] = (base + r < s_end) ? d + lg[r] : -INFINITY;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mx = ev[0][g];
#pragma unroll
      for (int r = 1; r < RB; ++r) mx = fmaxf(mx, ev[r][g]);
      const float mn = fmaxf(m[g], mx);
      const float corr = exp2f(m[g] - mn);
      l[g] *= corr;
#pragma unroll
      for (int e = 0; e < E; ++e) o[g][e] *= corr;
      m[g] = mn;
    }
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      float vf[E];
      unpack<T>(vc[r], vf);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float p = exp2f(ev[r][g] - m[g]);
        l[g] += p;
#pragma unroll
        for (int e = 0; e < E; ++e) o[g][e] = __builtin_fmaf(p, vf[e], o[g][e]);
      }
    }
  }

  if (j == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      sm[grp][g] = m[g];
      sl[grp][g] = l[g];
    }
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float Mg = -INFINITY;
    for (int k = 0; k < NG; ++k) Mg = fmaxf(Mg, sm[k][g]);
    const float f = (m[g] == -INFINITY) ? 0.f : exp2f(m[g] - Mg);
#pragma unroll
    for (int e = 0; e < E; ++e) so[grp][j * E + e] = o[g][e] * f;
    __syncthreads();
    float* rec = a.part + ((bh * G + g) * a.nsplit + blockIdx.x) * (int64_t)(D + 4);
    for (int d = tid; d < D; d += 256) {
      float acc = 0.f;
      for (int k = 0; k < NG; ++k) acc += so[k][d];
      rec[4 + d] = acc;
    }
    if (tid == 0) {
      float L = 0.f;
      for (int k = 0; k < NG; ++k)
        if (sm[k][g] != -INFINITY) L = __builtin_fmaf(sl[k][g], exp2f(sm[k][g] - Mg), L);
      rec[0] = Mg;
      rec[1] = L;
    }
    __syncthreads();
  }
}

template <typename T, int D, int G>
static hipError_t launch_dec_g(const DecArgs& a, const Shape& s, hipStream_t st) {
  const dim3 grid(a.nsplit, (unsigned)(s.B * s.Hkv));
  if (a.n)
    hipLaunchKernelGGL((decode_kernel<T, D, G, true>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((decode_kernel<T, D, G, false>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_dec_d(const DecArgs& a, const Shape& s, hipStream_t st) {
  switch (s.G) {
    case 1: return launch_dec_g<T, D, 1>(a, s, st);
    case 2: return launch_dec_g<T, D, 2>(a, s, st);
    case 4: return launch_dec_g<T, D, 4>(a, s, st);
    default: return launch_dec_g<T, D, 8>(a, s, st);
  }
}

size_t decode_workspace_bytes(const Shape& s) {
  int64_t chunk;
  int nsplit;
  decode_plan(s.N, chunk, nsplit);
  return (size_t)s.B * s.Hq * nsplit * (s.D + 4) * sizeof(float);
}

hipError_t launch_decode(const Shape& s, const void* K, const void* V, const int32_t* n, const void* q,
                         float scale, float* out, void* ws, hipStream_t st) {
  DecArgs a;
  a.K = K;
  a.V = V;
  a.n = n;
  a.q = q;
  a.part = static_cast<float*>(ws);
  a.N = s.N;
  a.sb = s.sb;
  a.sh = s.sh;
  a.Hkv = s.Hkv;
  a.Hq = s.Hq;
  a.scale = scale;
  decode_plan(s.N, a.chunk, a.nsplit);
  hipError_t e;
  if (s.bf16)
    e = s.D == 64 ? launch_dec_d<bf16, 64>(a, s, st) : launch_dec_d<bf16, 128>(a, s, st);
  else
    e = s.D == 64 ? launch_dec_d<float, 64>(a, s, st) : launch_dec_d<float, 128>(a, s, st);
  if (e != hipSuccess) return e;
  return launch_combine(a.part, (int64_t)s.B * s.Hq, a.nsplit, s.D, nullptr, out, st);
}

}  // namespace kvs
