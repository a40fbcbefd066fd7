// Fused key merge, lossless value-slot merge and stream compaction (one merge round).
//
// KVSlimmer deep-dive (charles2530.github.io), section 数学主线四: a selected adjacent pair
// (k_m, k_{m+1}) is replaced by k* = w_m k_m + w_{m+1} k_{m+1} with the closed-form,
// forward-only weights; values are not merged by that rule (sections 数学主线一 and
// 本页结论: values are heterogeneous).  The merged slot keeps the count-weighted mean
// value and the count (AsymKV abstract in the fugumt.com related list: lossless value
// compression), which decode attention turns back into the exact two-value output with
// a + ln n logit bias.
//
// Work decomposition (gfx950, wave64): one wavefront owns a chunk of 64 candidate pairs
// of one (batch, kv-head).  A row of D elements is LPR lanes x 16 bytes; a wave handles
// 64/LPR pairs per step, each lane loading the same 16-byte column chunk of both rows of
// its pair, so every global load is a fully used 128-bit access and consecutive pairs
// are consecutive in memory.  There is no reuse of K/V inside a workgroup, so the rows go
// HBM -> VGPR -> HBM without an LDS round trip.  Output positions: full rounds
// (every pair merges) are arithmetic; in partial rounds the wave ballots its selection
// flags, counts the selected pairs ahead of each group with a popcount, and adds the
// chunk's offset published by the selection pass (an exclusive scan over chunks), so
// no wave waits on another.
#include "kvs_common.h"
#include "kvs_internal.h"

namespace kvs {

struct MergeArgs {
  const void* K;
  const void* V;
  const int32_t* n;
  const float* g_self;
  const float* g_cross;
  const int32_t* sel;
  void* Ko;
  void* Vo;
  int32_t* no;
  int32_t* so;
  int64_t N, S, M, P, nchunks, sel_stride;
  int64_t sb, sh, osb, osh;
  int64_t total_waves;
  int Hkv;
};

template <typename TI, typename TO, int E>
__device__ __forceinline__ void put_row_chunk(TO* dst, const uint4& raw) {
  if constexpr (sizeof(TI) == sizeof(TO)) {
    *reinterpret_cast<uint4*>(dst) = raw;
  } else {
    float f[E];
    unpack<TI>(raw, f);
    store_elems<TO, E>(dst, f);
  }
}

template <typename TI, typename TO, int D, bool PARTIAL, bool HAS_N>
__global__ __launch_bounds__(256) void merge_compact_kernel(MergeArgs a) {
  constexpr int E = Elt<TI>::kPerChunk;
  constexpr int LPR = D / E;
  constexpr int GPW = 64 / LPR;
  constexpr int STEPS = kChunkPairs / GPW;
  constexpr int U = STEPS >= 4 ? 4 : STEPS;

  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (wave >= a.total_waves) return;
  const int64_t bh = wave / a.nchunks;
  const int64_t c = wave - bh * a.nchunks;
  const int64_t b = bh / a.Hkv, h = bh - b * a.Hkv;

  const int64_t in_off = b * a.sb + h * a.sh;
  const int64_t out_off = b * a.osb + h * a.osh;
  const TI* K = static_cast<const TI*>(a.K) + in_off;
  const TI* V = static_cast<const TI*>(a.V) + in_off;
  const int32_t* n = HAS_N ? a.n + in_off / D : nullptr;
  TO* Ko = static_cast<TO*>(a.Ko) + out_off;
  TO* Vo = static_cast<TO*>(a.Vo) + out_off;
  int32_t* no = a.no + out_off / D;
  int32_t* so = a.so + out_off / D;
  const float* gs = a.g_self + bh * a.N;
  const float* gc = a.g_cross + bh * a.P;

  const int grp = lane / LPR;
  const int j = lane % LPR;
  const int64_t T = a.N - a.M;

  auto copy_row = [&](int64_t i, int64_t pos, const uint4& kc, const uint4& vc) {
    if (pos < 0 || pos >= T) return;
    put_row_chunk<TI, TO, E>(Ko + pos * D + j * E, kc);
    put_row_chunk<TI, TO, E>(Vo + pos * D + j * E, vc);
    if (j == 0) {
      no[pos] = HAS_N ? n[i] : 1;
      so[pos] = (int32_t)i;
    }
  };

  const int64_t p0 = c * kChunkPairs;
  const int64_t p1 = min(a.P, p0 + kChunkPairs);
  SelHeader hd{};
  int64_t run = 0;  // selected pairs before the current step (partial rounds)
  if constexpr (PARTIAL) {
    const int32_t* st = a.sel + bh * a.sel_stride;
    hd.tau_key = static_cast<uint32_t>(st[0]);
    hd.p_tau = st[1];
    run = st[kSelHeaderInts + c];
  }

  for (int s0 = 0; s0 < STEPS; s0 += U) {
    uint4 ka[U], kb[U], va[U], vb[U];
    float g0[U], g1[U], gx[U];
    int n0[U], n1[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t p = p0 + (int64_t)(s0 + u) * GPW + grp;
      const int64_t m = a.S + 2 * p;
      if (p < p1) {
        ka[u] = load16(K + m * D + j * E);
        kb[u] = load16(K + (m + 1) * D + j * E);
        va[u] = load16(V + m * D + j * E);
        vb[u] = load16(V + (m + 1) * D + j * E);
        g0[u] = gs[m];
        g1[u] = gs[m + 1];
        gx[u] = gc[p];
        n0[u] = HAS_N ? n[m] : 1;
        n1[u] = HAS_N ? n[m + 1] : 1;
      } else {
        ka[u] = kb[u] = va[u] = vb[u] = make_uint4(0, 0, 0, 0);
        g0[u] = g1[u] = gx[u] = 0.f;
        n0[u] = n1[u] = 1;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t p = p0 + (int64_t)(s0 + u) * GPW + grp;
      const int64_t m = a.S + 2 * p;
      const bool valid = p < p1;
      float kf0[E], kf1[E];
      unpack<TI>(ka[u], kf0);
      unpack<TI>(kb[u], kf1);
      bool sel = valid;
      int64_t pos;
      uint64_t mask = 0;
      if constexpr (PARTIAL) {
        const float cs = pair_cos<E, LPR>(kf0, kf1);
        sel = valid && is_selected(order_key(cs), p, hd);
        mask = __ballot(sel);
        const uint64_t below = grp == 0 ? 0ull : (mask & ((1ull << (grp * LPR)) - 1ull));
        pos = m - (run + (int64_t)(__popcll(below) / LPR));
      } else {
        pos = a.S + p;
      }
      if (valid) {
        if (sel) {
          if (pos >= 0 && pos < T) {
            float w0, w1;
            closed_form_weights(g0[u], gx[u], g1[u], w0, w1);
            float vf0[E], vf1[E], ko[E], vo[E];
            unpack<TI>(va[u], vf0);
            unpack<TI>(vb[u], vf1);
            merge_keys<E>(kf0, kf1, w0, w1, ko);
            merge_values<E>(vf0, vf1, n0[u], n1[u], vo);
            const int nt = n0[u] + n1[u];
            store_elems<TO, E>(Ko + pos * D + j * E, ko);
            store_elems<TO, E>(Vo + pos * D + j * E, vo);
            if (j == 0) {
              no[pos] = nt;
              so[pos] = (int32_t)m;
            }
          }
        } else {
          copy_row(m, pos, ka[u], va[u]);
          copy_row(m + 1, pos + 1, kb[u], vb[u]);
        }
      }
      if constexpr (PARTIAL) run += (int64_t)(__popcll(mask) / LPR);
    }
  }

  // Preserved leading slots (sinks) and the trailing slots after the last pair
  // (an odd leftover and the recent window) are copied; the first and last chunk do it.
  if (c == 0) {
    for (int64_t i = grp; i < a.S; i += GPW) copy_row(i, i, load16(K + i * D + j * E), load16(V + i * D + j * E));
  }
  if (c == a.nchunks - 1) {
    for (int64_t i = a.S + 2 * a.P + grp; i < a.N; i += GPW)
      copy_row(i, i - a.M, load16(K + i * D + j * E), load16(V + i * D + j * E));
  }
}

template <typename TI, typename TO, int D>
static hipError_t launch_merge_t(const MergeArgs& a, bool partial, bool has_n, hipStream_t st) {
  const int blocks = (int)((a.total_waves + 3) / 4);
  if (partial) {
    if (has_n)
      KVS_LAUNCH("merge_compact", (merge_compact_kernel<TI, TO, D, true, true>), dim3(blocks), dim3(256), 0, st, a);
    else
      KVS_LAUNCH("merge_compact", (merge_compact_kernel<TI, TO, D, true, false>), dim3(blocks), dim3(256), 0, st, a);
  } else {
    if (has_n)
      KVS_LAUNCH("merge_compact", (merge_compact_kernel<TI, TO, D, false, true>), dim3(blocks), dim3(256), 0, st, a);
    else
      KVS_LAUNCH("merge_compact", (merge_compact_kernel<TI, TO, D, false, false>), dim3(blocks), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

template <typename TI, typename TO>
static hipError_t launch_merge_d(const MergeArgs& a, int D, bool partial, bool has_n, hipStream_t st) {
  return D == 64 ? launch_merge_t<TI, TO, 64>(a, partial, has_n, st) : launch_merge_t<TI, TO, 128>(a, partial, has_n, st);
}

hipError_t launch_merge(const Shape& s, const RoundP& r, const void* K, const void* V, const int32_t* n,
                        const float* g_self, const float* g_cross, const int32_t* sel_state, const OutP& o,
                        void* K_out, void* V_out, int32_t* n_out, int32_t* src_out, hipStream_t st) {
  MergeArgs a;
  a.K = K;
  a.V = V;
  a.n = n;
  a.g_self = g_self;
  a.g_cross = g_cross;
  a.sel = sel_state;
  a.Ko = K_out;
  a.Vo = V_out;
  a.no = n_out;
  a.so = src_out;
  a.N = s.N;
  a.S = r.S;
  a.M = r.M;
  a.P = r.P;
  a.nchunks = n_chunks(r.P);
  a.sel_stride = sel_stride_ints(r.P);
  a.sb = s.sb;
  a.sh = s.sh;
  a.osb = o.sb;
  a.osh = o.sh;
  a.Hkv = s.Hkv;
  a.total_waves = (int64_t)s.B * s.Hkv * a.nchunks;
  if (s.N == 0 || a.total_waves == 0) return hipSuccess;
  // M == 0 and M == P need no threshold and never read the selection state: M == P
  // merges every pair; M == 0 is a plain copy, done as a full round over zero pairs.
  bool partial = r.M != 0 && r.M != r.P;
  if (r.M == 0 && r.P > 0) {
    a.P = 0;
    a.S = 0;
    a.nchunks = 1;
    a.total_waves = (int64_t)s.B * s.Hkv;
    partial = false;
  }
  const bool has_n = n != nullptr;
  if (s.bf16)
    return o.bf16 ? launch_merge_d<bf16, bf16>(a, s.D, partial, has_n, st)
                  : launch_merge_d<bf16, float>(a, s.D, partial, has_n, st);
  return o.bf16 ? launch_merge_d<float, bf16>(a, s.D, partial, has_n, st)
                : launch_merge_d<float, float>(a, s.D, partial, has_n, st);
}

}  // namespace kvs

namespace kvs {

// ------------------------------------------------------------------ append --
// Rows [from, from + count) of every (b, h) of the source go to rows [at, at + count) of
// the cache; their counts become 1.  One thread per 16-byte piece of a row, grid-stride.
struct AppendArgs {
  const uint8_t* Ks;
  const uint8_t* Vs;
  uint8_t* Kd;
  uint8_t* Vd;
  int32_t* n;
  int64_t at, from, count, total;
  int64_t sb, sh, dsb, dsh;   // element strides of the source and of the cache
  int Hkv, D, esz, cpr;       // element bytes, 16-byte pieces per row
};

__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < a.total; i += (int64_t)gridDim.x * 256) {
    const int64_t c = i % a.cpr, rest = i / a.cpr;
    const int64_t r = rest % a.count, bh = rest / a.count;
    const int64_t b = bh / a.Hkv, h = bh - b * a.Hkv;
    const int64_t so = ((b * a.sb + h * a.sh) + (a.from + r) * a.D) * a.esz + c * 16;
    const int64_t dro = (b * a.dsb + h * a.dsh) / a.D + a.at + r;   // cache row
    const int64_t dof = dro * a.D * a.esz + c * 16;
    *reinterpret_cast<uint4*>(a.Kd + dof) = *reinterpret_cast<const uint4*>(a.Ks + so);
    *reinterpret_cast<uint4*>(a.Vd + dof) = *reinterpret_cast<const uint4*>(a.Vs + so);
    if (a.n && c == 0) a.n[dro] = 1;
  }
}

hipError_t launch_append(const Shape& dst, const Shape& src, void* K, void* V, int32_t* n, int64_t at,
                         const void* K_new, const void* V_new, int64_t from, int64_t count, hipStream_t st) {
  AppendArgs a;
  a.Ks = static_cast<const uint8_t*>(K_new);
  a.Vs = static_cast<const uint8_t*>(V_new);
  a.Kd = static_cast<uint8_t*>(K);
  a.Vd = static_cast<uint8_t*>(V);
  a.n = n;
  a.at = at;
  a.from = from;
  a.count = count;
  a.sb = src.sb;
  a.sh = src.sh;
  a.dsb = dst.sb;
  a.dsh = dst.sh;
  a.Hkv = dst.Hkv;
  a.D = dst.D;
  a.esz = dst.bf16 ? 2 : 4;
  a.cpr = dst.D * a.esz / 16;
  a.total = (int64_t)dst.B * dst.Hkv * count * a.cpr;
  if (a.total == 0) return hipSuccess;
  int64_t blocks = (a.total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  KVS_LAUNCH("append", append_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace kvs
