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

// Split plan: every split is non-empty.  The bf16 MFMA kernel aims at ~512 workgroups
// over all (batch, kv-head) slices (two per CU), in multiples of 128 slots.
static void decode_plan(const Shape& s, int64_t& chunk, int& nsplit) {
  const int64_t N = s.N;
  int64_t c;
  if (s.bf16) {
    const int64_t BH = (int64_t)s.B * s.Hkv;
    c = (N * BH + 511) / 512;
    c = (c + 127) / 128 * 128;
    if (c < 128) c = 128;
  } else {
    c = (N + 255) / 256;
    if (c < 256) c = 256;
    c = (c + 63) / 64 * 64;
  }
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

// ----------------------------------------------------------------- bf16 MFMA --
// gfx950 decode for bf16 caches: v_mfma_f32_16x16x32_bf16 with the G query heads of a
// kv head as the N side (padded to 16; the padding costs MFMA cycles, which decode has
// to spare).  Each wave streams 32-slot blocks: K rows go straight from HBM into the A
// operand of S^T = K . Q^T (lane l: slot 16 sb + l % 16, 64 contiguous bytes per row per
// load), V rows are staged in a wave-private LDS tile and read back transposed
// (ds_read_tr16_b64) as the A operand of O^T += V^T . P^T, with P split into bf16 hi + lo.
// The next block's K/V registers are fetched while the current block is computed.
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 dbf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 dbf16x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float df32x4_t;
typedef unsigned int du32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ dbf16x8_t d_as_bf16x8(const uint4& u) {
  du32x4_t v = {u.x, u.y, u.z, u.w};
  return __builtin_bit_cast(dbf16x8_t, v);
}
__device__ __forceinline__ df32x4_t d_mfma(const dbf16x8_t& a, const dbf16x8_t& b, const df32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

constexpr int kDecBlock = 32;     // slots per wave step
constexpr int kDecWaves = 4;
constexpr float kDecNoMax = -1e30f;

template <int D, bool HAS_N>
struct DecBlock {
  static constexpr int KB = D / 32;
  static constexpr int CPR = D / 8;                      // 16-byte chunks per row
  static constexpr int VPL = kDecBlock * CPR / 64;       // V chunks per lane
  uint4 k[2][KB];      // A operand of S^T: slot 16 sb + l % 16, d = 32 kb + 8 (l / 16)
  uint4 v[VPL];        // V rows in row layout, staged to LDS
  int4 n[2];           // counts of slots 16 sb + 4 (l / 16) + 0..3

  __device__ __forceinline__ void fetch(const bf16* Kp, const bf16* Vp, const int32_t* np, int64_t t, int64_t end) {
    const int lane = threadIdx.x & 63, g = lane >> 4, c16 = lane & 15;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      int64_t row = t + sb * 16 + c16;
      row = row < end ? row : end - 1;   // clamped rows are masked by the bias
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) k[sb][kb] = load16(Kp + row * D + kb * 32 + g * 8);
      if (HAS_N) {
        int64_t r0 = t + sb * 16 + g * 4;
        if (r0 + 4 <= end) {
          n[sb] = *reinterpret_cast<const int4*>(np + r0);
        } else {
          n[sb].x = r0 < end ? np[r0] : 1;
          n[sb].y = r0 + 1 < end ? np[r0 + 1] : 1;
          n[sb].z = r0 + 2 < end ? np[r0 + 2] : 1;
          n[sb].w = r0 + 3 < end ? np[r0 + 3] : 1;
        }
      }
    }
#pragma unroll
    for (int it = 0; it < VPL; ++it) {
      const int idx = it * 64 + lane;
      int64_t row = t + idx / CPR;
      row = row < end ? row : end - 1;
      v[it] = load16(Vp + row * D + (idx % CPR) * 8);
    }
  }
};

template <int D, int G, bool HAS_N>
__global__ __launch_bounds__(64 * kDecWaves, 2) void decode_mfma_kernel(DecArgs a) {
  constexpr int KB = D / 32, DB = D / 16, CPR = D / 8, PITCH = D + 16;
  constexpr int VPL = DecBlock<D, HAS_N>::VPL;
  __shared__ __attribute__((aligned(16))) bf16 vt[kDecWaves][kDecBlock * PITCH];
  __shared__ float wm[kDecWaves][16], wl[kDecWaves][16];
  __shared__ float wo[kDecWaves][16][D];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int64_t bh = blockIdx.y;
  const int64_t b = bh / a.Hkv, h = bh - b * a.Hkv;
  const bf16* Kp = static_cast<const bf16*>(a.K) + b * a.sb + h * a.sh;
  const bf16* Vp = static_cast<const bf16*>(a.V) + b * a.sb + h * a.sh;
  const int32_t* np = HAS_N ? a.n + (b * a.sb + h * a.sh) / D : nullptr;
  const bf16* qp = static_cast<const bf16*>(a.q) + (b * a.Hq + h * G) * (int64_t)D;

  // B operand of S^T: lane l holds q[head l % 16][d = 32 kb + 8 (l / 16) .. +7], zero padding
  dbf16x8_t qop[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (c16 < G) u = load16(qp + c16 * D + kb * 32 + g * 8);
    qop[kb] = d_as_bf16x8(u);
  }
  const float cs = a.scale * kLog2e;
  float m = kDecNoMax, lsum = 0.f;
  df32x4_t acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = df32x4_t{0.f, 0.f, 0.f, 0.f};

  const int64_t s0 = (int64_t)blockIdx.x * a.chunk;
  const int64_t s1 = min(a.N, s0 + a.chunk);
  bf16* V_ = vt[wv];
  DecBlock<D, HAS_N> cur, nxt;
  int64_t t = s0 + (int64_t)wv * kDecBlock;
  if (t < s1) cur.fetch(Kp, Vp, np, t, s1);
  for (; t < s1; t += kDecWaves * kDecBlock) {
    const int64_t tn = t + kDecWaves * kDecBlock;
    if (tn < s1) nxt.fetch(Kp, Vp, np, tn, s1);
    // stage V rows (row layout) in the wave's LDS tile
#pragma unroll
    for (int it = 0; it < VPL; ++it) {
      const int idx = it * 64 + lane;
      *reinterpret_cast<uint4*>(V_ + (idx / CPR) * PITCH + (idx % CPR) * 8) = cur.v[it];
    }
    // S^T = K . Q^T: lane holds slots 16 sb + 4 g + r of head c16
    df32x4_t st[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      st[sb] = df32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) st[sb] = d_mfma(d_as_bf16x8(cur.k[sb][kb]), qop[kb], st[sb]);
    }
    float e[8];
    float mx = kDecNoMax;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int ns[4] = {cur.n[sb].x, cur.n[sb].y, cur.n[sb].z, cur.n[sb].w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t slot = t + sb * 16 + g * 4 + r;
        float bias = 0.f;
        if (HAS_N) bias = __log2f((float)ns[r]);
        if (slot >= s1) bias = -INFINITY;
        e[sb * 4 + r] = __builtin_fmaf(st[sb][r], cs, bias);
        mx = fmaxf(mx, e[sb * 4 + r]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (mx > m) {
      const float corr = __builtin_amdgcn_exp2f(m - mx);
      lsum *= corr;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= corr;
      m = mx;
    }
    float pv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      pv[j] = __builtin_amdgcn_exp2f(e[j] - m);
      lsum += pv[j];
    }
    // P^T operand: k index (g, j) <-> slot 16 (j / 4) + 4 g + j % 4, the lane's own pv[j]
    dbf16x8_t phi, plo;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const __bf16 hv = (__bf16)pv[j];
      phi[j] = hv;
      plo[j] = (__bf16)(pv[j] - (float)hv);
    }
    __builtin_amdgcn_wave_barrier();
    // V^T operand by transposed reads: source lane i points at row 4 g + i / 4 (and + 16),
    // columns 16 db + 4 (i % 4); lane t receives column 16 db + t of four consecutive rows
    const int srow = 4 * g + (c16 >> 2);
    const int scol = 4 * (c16 & 3);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      typedef __attribute__((address_space(3))) dbf16x4_t lds_t;
      const dbf16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_t*)(V_ + srow * PITCH + db * 16 + scol));
      const dbf16x4_t v1 =
          __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_t*)(V_ + (srow + 16) * PITCH + db * 16 + scol));
      const dbf16x8_t vop = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      acc[db] = d_mfma(vop, phi, acc[db]);
      acc[db] = d_mfma(vop, plo, acc[db]);
    }
    __builtin_amdgcn_wave_barrier();
    cur = nxt;
  }

  // merge the waves: per head c16, O^T rows d = 16 db + 4 g + r
  float l = lsum;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (g == 0) {
    wm[wv][c16] = m;
    wl[wv][c16] = l;
  }
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) wo[wv][c16][db * 16 + g * 4 + r] = acc[db][r];
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += 64 * kDecWaves) {
    const int hd = idx / D, d = idx % D;
    float M = kDecNoMax;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, wm[w][hd]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float f = __builtin_amdgcn_exp2f(wm[w][hd] - M);
      L = __builtin_fmaf(wl[w][hd], f, L);
      O = __builtin_fmaf(wo[w][hd][d], f, O);
    }
    float* rec = a.part + ((bh * G + hd) * a.nsplit + blockIdx.x) * (int64_t)(D + 4);
    rec[4 + d] = O;
    if (d == 0) {
      rec[0] = M;
      rec[1] = L;
    }
  }
}

template <typename T, int D, int G>
static hipError_t launch_dec_g(const DecArgs& a, const Shape& s, hipStream_t st) {
  const dim3 grid(a.nsplit, (unsigned)(s.B * s.Hkv));
  if (a.n)
    KVS_LAUNCH("decode", (decode_kernel<T, D, G, true>), grid, dim3(256), 0, st, a);
  else
    KVS_LAUNCH("decode", (decode_kernel<T, D, G, false>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int D, int G>
static hipError_t launch_dec_mfma_g(const DecArgs& a, const Shape& s, hipStream_t st) {
  const dim3 grid(a.nsplit, (unsigned)(s.B * s.Hkv));
  if (a.n)
    KVS_LAUNCH("decode", (decode_mfma_kernel<D, G, true>), grid, dim3(64 * kDecWaves), 0, st, a);
  else
    KVS_LAUNCH("decode", (decode_mfma_kernel<D, G, false>), grid, dim3(64 * kDecWaves), 0, st, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_dec_mfma(const DecArgs& a, const Shape& s, hipStream_t st) {
  switch (s.G) {
    case 1: return launch_dec_mfma_g<D, 1>(a, s, st);
    case 2: return launch_dec_mfma_g<D, 2>(a, s, st);
    case 4: return launch_dec_mfma_g<D, 4>(a, s, st);
    default: return launch_dec_mfma_g<D, 8>(a, s, st);
  }
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
  Shape sb = s, sf = s;
  sb.bf16 = true;
  sf.bf16 = false;
  decode_plan(sb, chunk, nsplit);
  int ns2;
  decode_plan(sf, chunk, ns2);
  if (ns2 > nsplit) nsplit = ns2;   // the workspace query does not know the element type
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
  decode_plan(s, a.chunk, a.nsplit);
  hipError_t e;
  if (s.bf16)
    e = s.D == 64 ? launch_dec_mfma<64>(a, s, st) : launch_dec_mfma<128>(a, s, st);
  else
    e = s.D == 64 ? launch_dec_d<float, 64>(a, s, st) : launch_dec_d<float, 128>(a, s, st);
  if (e != hipSuccess) return e;
  return launch_combine(a.part, (int64_t)s.B * s.Hq, a.nsplit, s.D, nullptr, out, st);
}

}  // namespace kvs
