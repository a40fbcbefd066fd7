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
#include <mutex>

#include "../../include/kvslim.h"
#include "kvs_common.h"
#include "kvs_dma.h"
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

constexpr int kDecCUs = 256;   // compute units of the chip: workgroups the bf16 decode aims at

// Split plan: every split is non-empty.  The bf16 MFMA kernel (one workgroup per CU) aims
// at about one workgroup per CU over all (batch, kv-head) slices, at least 128 slots each;
// chunks need not be whole tiles (a partial last tile is masked).
static void decode_plan(const Shape& s, int64_t& chunk, int& nsplit) {
  const int64_t N = s.N;
  int64_t c;
  if (s.bf16) {
    const int64_t BH = (int64_t)s.B * s.Hkv;
    int64_t want = kDecCUs / BH;
    if (want < 1) want = 1;
    c = (N + want - 1) / want;
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
// to spare).  S^T = K . Q^T takes K rows as the A operand (lane l: slot 16 sb + l % 16,
// 16 contiguous bytes); O^T += V^T . P^T reads V transposed from LDS (ds_read_tr16_b64)
// as the A operand, with P split into bf16 hi + lo so the probabilities keep fp32
// accuracy.
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

constexpr int kDecWaves = 4;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr float kDecNoMax = -1e30f;
constexpr float kDecLazy = 8.f;

// Tile buffers per wave: 32 KB of K + V (two 32-slot tiles at D = 128, four at D = 64), so
// the four waves of a workgroup hold 128 KB of LDS.
template <int D>
struct DecRing {
  static constexpr int R = D == 128 ? 2 : 4;
};

// One workgroup of four waves per CU over a slot chunk of one (batch, kv-head).  Each
// wave owns every fourth 32-slot tile of the chunk and streams it on its own: 16-byte
// buffer loads written straight into the wave's LDS ring (rows XOR-swizzled), completion
// tracked by the wave's own load counter, so the loop has no workgroup barrier and no
// tile is computed twice.  Per tile the wave computes S^T for all G heads, the online
// softmax (running maximum raised only when it grows by more than 2^8) and O^T over the
// whole head dimension.  At the end the four waves' (max, sum, O) are merged in LDS
// into one partial record per query head for the log-sum-exp combine.
template <int D, int G, bool HAS_N>
__global__ __launch_bounds__(kDecThreads, 1) void decode_mfma_kernel(DecArgs a, int BH) {
  using M = Dma<D>;
  constexpr int R = DecRing<D>::R;
  constexpr int KB = D / 32;                  // k steps of S^T
  constexpr int DB = D / 16;                  // 16-row blocks of O^T
  constexpr int KI = M::TILEB / 1024;         // wave-wide 16-byte loads per K (or V) tile
  constexpr int QBYTES = G * D * 2;           // the G query rows
  constexpr int QI = (QBYTES + 1023) / 1024;  // wave-wide loads for them
  constexpr int PER_TILE = 2 * KI + (HAS_N ? 1 : 0);
  constexpr int WAVEB = 2 * R * M::TILEB;     // LDS bytes of one wave's ring
  static_assert(PER_TILE * R + QI < 64, "load counter range");
  static_assert((32 + G * D) * 4 <= WAVEB, "merge area fits a wave's ring");
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kDecWaves * WAVEB];
  __shared__ __attribute__((aligned(16))) uint8_t qsh[kDecWaves * QI * 1024];
  __shared__ __attribute__((aligned(16))) int32_t nsh[kDecWaves * R * kT2];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  const int64_t id = blockIdx.x;
  const int64_t bh = id % BH, split = id / BH;
  const int64_t b = bh / a.Hkv, h = bh - b * a.Hkv;
  const int64_t hoff = b * a.sb + h * a.sh;
  const int64_t s0 = split * a.chunk;
  const int64_t s1 = s0 + a.chunk < a.N ? s0 + a.chunk : a.N;
  const int ntiles = (int)((s1 - s0 + kT2 - 1) / kT2);
  const int nmine = ntiles > wv ? (ntiles - wv + kDecWaves - 1) / kDecWaves : 0;   // tiles wv, wv + 4, ...
  const uint32_t span = (uint32_t)(s1 - s0);
  const u32x4_t rk = make_rsrc(static_cast<const bf16*>(a.K) + hoff + s0 * D, span * M::ROWB);
  const u32x4_t rv = make_rsrc(static_cast<const bf16*>(a.V) + hoff + s0 * D, span * M::ROWB);
  const int32_t* np = HAS_N ? a.n + hoff / D + s0 : nullptr;
  const u32x4_t rn = make_rsrc(HAS_N ? static_cast<const void*>(np) : a.K, HAS_N ? span * 4u : 0u);
  const bf16* qp = static_cast<const bf16*>(a.q) + (b * a.Hq + h * G) * (int64_t)D;
  const u32x4_t rq = make_rsrc(qp, (uint32_t)QBYTES);

  uint8_t* const kw = ring + wv * WAVEB;       // K buffers of this wave, then its V buffers
  uint8_t* const vw = kw + R * M::TILEB;
  int32_t* const nw = nsh + wv * R * kT2;
  uint8_t* const qw = qsh + wv * QI * 1024;

  // wave-local tile i (chunk tile wv + 4 i) -> buffer i % R; rows past the chunk read as zeros
  auto issue = [&](int i) {
    const int buf = i % R;
    const uint32_t t0 = (uint32_t)(wv + kDecWaves * i) * kT2;
#pragma unroll
    for (int u = 0; u < KI; ++u) {
      const int r = u * M::RPI + lane / M::CPR;
      const int c = (lane % M::CPR) ^ swz<D>(r);
      const uint32_t off = (t0 + r) * M::ROWB + (uint32_t)(c << 4);
      dma16(rk, lds_addr(kw + buf * M::TILEB + u * 1024), off);
      dma16(rv, lds_addr(vw + buf * M::TILEB + u * 1024), off);
    }
    if (HAS_N && lane < kT2) dma4(rn, lds_addr(nw + buf * kT2), (t0 + lane) * 4u);
  };
  // wait for wave-local tile i while `later` (0 .. R - 1) tiles issued after it are in flight
  auto wait_tile = [&](int later) {
    if (R > 3 && later >= 3) wait_vm<3 * PER_TILE>();
    else if (R > 2 && later == 2) wait_vm<2 * PER_TILE>();
    else if (later == 1) wait_vm<PER_TILE>();
    else wait_vm<0>();
  };

#pragma unroll
  for (int u = 0; u < QI; ++u) dma16(rq, lds_addr(qw + u * 1024), (uint32_t)(u * 1024 + lane * 16));
#pragma unroll
  for (int i = 0; i < R; ++i)
    if (i < nmine) issue(i);

  const float cs = a.scale * kLog2e;
  float m = kDecNoMax, lsum = 0.f;
  df32x4_t acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = df32x4_t{0.f, 0.f, 0.f, 0.f};
  // B operand of S^T: lane l holds q[head l % 16][d = 32 kb + 8 (l / 16) .. +7], zero padding
  dbf16x8_t qop[KB];

  // V^T operand by transposed reads: source lane i points at row 4 g + i / 4 (and + 16),
  // columns 16 db + 4 (i % 4); lane t receives column 16 db + t of four consecutive rows
  const int srow = 4 * g + (c16 >> 2);
  const int scol = 4 * (c16 & 3);

  for (int i = 0; i < nmine; ++i) {
    const int later = nmine - 1 - i < R - 1 ? nmine - 1 - i : R - 1;
    wait_tile(later);
    if (i == 0) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (c16 < G) u = *reinterpret_cast<const uint4*>(qw + (c16 * D + kb * 32 + g * 8) * 2);
        qop[kb] = d_as_bf16x8(u);
      }
    }
    const int buf = i % R;
    const uint8_t* K_ = kw + buf * M::TILEB;
    const uint8_t* V_ = vw + buf * M::TILEB;
    const int64_t t0 = s0 + (int64_t)(wv + kDecWaves * i) * kT2;
    // V^T operands of the whole tile first: their reads land while S^T and the softmax run
    dbf16x8_t vop[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      typedef __attribute__((address_space(3))) dbf16x4_t lds_t;
      const int col = db * 16 + scol;
      const int cb = (col & 7) * 2;
      const dbf16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_t*)(V_ + chunk_off<D>(srow, col >> 3) + cb));
      const dbf16x4_t v1 =
          __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_t*)(V_ + chunk_off<D>(srow + 16, col >> 3) + cb));
      vop[db] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    // S^T = K . Q^T: lane holds slots 16 sb + 4 g + r of head c16
    df32x4_t st[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      st[sb] = df32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        st[sb] = d_mfma(d_as_bf16x8(*reinterpret_cast<const uint4*>(K_ + chunk_off<D>(16 * sb + c16, 4 * kb + g))),
                        qop[kb], st[sb]);
    }
    float e[8];
    float mx = kDecNoMax;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      int4 n4 = make_int4(1, 1, 1, 1);
      if (HAS_N) n4 = *reinterpret_cast<const int4*>(nw + buf * kT2 + 16 * sb + 4 * g);
      const int ns[4] = {n4.x, n4.y, n4.z, n4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t slot = t0 + 16 * sb + 4 * g + r;
        float bias = HAS_N ? __log2f((float)ns[r]) : 0.f;
        if (slot >= s1) bias = -INFINITY;
        e[sb * 4 + r] = __builtin_fmaf(st[sb][r], cs, bias);
        mx = fmaxf(mx, e[sb * 4 + r]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (mx > m + kDecLazy) {
      const float corr = __builtin_amdgcn_exp2f(m - mx);
      lsum *= corr;
#pragma unroll
      for (int k = 0; k < DB; ++k) acc[k] *= corr;
      m = mx;
    }
    // P^T operand: k index (g, j) <-> slot 16 (j / 4) + 4 g + j % 4, the lane's own p[j]
    dbf16x8_t phi, plo;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = __builtin_amdgcn_exp2f(e[j] - m);
      lsum += p;
      const __bf16 hv = (__bf16)p;
      phi[j] = hv;
      plo[j] = (__bf16)(p - (float)hv);
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      acc[db] = d_mfma(vop[db], phi, acc[db]);
      acc[db] = d_mfma(vop[db], plo, acc[db]);
    }
    if (i + R < nmine) {
      wait_lds();   // this buffer's LDS reads are done before it is refilled
      issue(i + R);
    }
  }
  wait_vm<0>();

  // merge the four waves: each writes {m[16], l[16], O[G][D]} over its own ring, then the
  // workgroup forms one record {M, L, -, -, o[D]} per query head (O^T rows d = 16 db + 4 g + r)
  float l = lsum;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  float* const mine = reinterpret_cast<float*>(kw);
  if (g == 0) {
    mine[c16] = m;
    mine[16 + c16] = l;
  }
  if (c16 < G) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
      *reinterpret_cast<float4*>(mine + 32 + c16 * D + db * 16 + 4 * g) =
          make_float4(acc[db][0], acc[db][1], acc[db][2], acc[db][3]);
  }
  __syncthreads();
  const int64_t nsplit = a.nsplit;
  for (int k = tid; k < G * D; k += kDecThreads) {
    const int hh = k / D, d = k - hh * D;
    float mw[kDecWaves], Mx = kDecNoMax;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      mw[w] = reinterpret_cast<const float*>(ring + w * WAVEB)[hh];
      Mx = fmaxf(Mx, mw[w]);
    }
    float o = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float* pw = reinterpret_cast<const float*>(ring + w * WAVEB);
      const float f = __builtin_amdgcn_exp2f(mw[w] - Mx);
      o = __builtin_fmaf(f, pw[32 + hh * D + d], o);
      L = __builtin_fmaf(f, pw[16 + hh], L);
    }
    float* rec = a.part + ((bh * G + hh) * nsplit + split) * (int64_t)(D + 4);
    rec[4 + d] = o;
    if (d == 0) {
      rec[0] = Mx;
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
  const int BH = s.B * s.Hkv;
  const dim3 grid((unsigned)(a.nsplit * (int64_t)BH));
  if (a.n)
    KVS_LAUNCH("decode", (decode_mfma_kernel<D, G, true>), grid, dim3(kDecThreads), 0, st, a, BH);
  else
    KVS_LAUNCH("decode", (decode_mfma_kernel<D, G, false>), grid, dim3(kDecThreads), 0, st, a, BH);
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

// Library-owned scratch of kvs_decode_attn_static (the split partial records of a decode
// call), for callers that cannot allocate.  Every GPU the library runs on holds its own copy
// from the first use of this code object until the process ends.  Host code never uses the
// array's name as an address: static_scratch() asks HIP for the current device's address
// of it once per device and keeps it.
static __device__ __align__(256) uint8_t scratch[KVS_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

hipError_t static_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
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
