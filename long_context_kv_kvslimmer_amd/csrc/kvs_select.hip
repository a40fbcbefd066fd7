// Pair selection and closed-form weights (kvs_merge_weights).
//
// Selection: in each (batch, kv-head) the n_merge candidate pairs with the largest
// adjacent-key cosine, ties to the lower pair index (KVSlimmer deep-dive, section
// 数学主线二: merge homogeneous adjacent keys; section 局限与边界: one uniform ratio for
// every head).  An MSB-first radix select over the order-preserving 32-bit image of the
// cosine finds the threshold key tau and how many keys equal to tau are taken: four
// digit passes, each a grid of workgroups of 4096 pairs over every head that adds its
// LDS histogram of one 8-bit digit into the head's global histogram (cosines of
// neighbouring pairs share their leading digits, so each wave adds its most common digit
// with one atomic); every later workgroup replays the earlier digit choices from those
// histograms.  A count pass writes, per 64-pair chunk, the keys equal to and above tau;
// one workgroup per head then scans them for the tie cut-off index and the exclusive
// offsets of the selected pairs of every chunk, which the merge pass uses for its
// compaction.  The histograms and counts live in the selection state after its header.
#include "kvs_common.h"
#include "kvs_internal.h"

namespace kvs {

constexpr int kSelThreads = 1024;                      // final workgroup (one per head)
constexpr int kHistThreads = 256;                      // histogram and count passes
constexpr int kHistKeys = 16;                          // keys per thread there
constexpr int kHistBlock = kHistThreads * kHistKeys;   // pairs per workgroup (64 chunks)

// Exclusive scan of one int per thread over a workgroup of T threads; returns the
// exclusive prefix and writes the workgroup total to *total.  Every thread must call it.
template <int T>
__device__ int block_exclusive_scan(int v, int* total, int* lds /* >= T / 64 ints */) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) lds[wv] = x;
  __syncthreads();
  int wave_pre = 0, tot = 0;
  for (int k = 0; k < T / 64; ++k) {
    const int t = lds[k];
    if (k < wv) wave_pre += t;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return wave_pre + x - v;
}

// Adds 1 to hist[d] for every lane with ok set: the digit of the wave's first such lane
// with one atomic for all lanes that share it, the other lanes one atomic each.
__device__ __forceinline__ void wave_hist_add(uint32_t* hist, bool ok, uint32_t d) {
  const uint64_t act = __ballot(ok);
  if (act == 0) return;
  const int leader = __ffsll((unsigned long long)act) - 1;
  const uint32_t ld = (uint32_t)__builtin_amdgcn_readlane((int)d, leader);
  const uint64_t same = __ballot(ok && d == ld);
  if ((int)(threadIdx.x & 63) == leader) atomicAdd(&hist[ld], (uint32_t)__popcll(same));
  if (ok && d != ld) atomicAdd(&hist[d], 1u);
}

// The radix select's state after `passes` digit passes, replayed from the head's global
// histograms: prefix = the chosen leading digits, remaining = how many keys with that
// prefix are still to be taken.  Digit s is the largest d whose count of keys >= d (among
// keys with the prefix so far) reaches `remaining`.  All T threads call it.
template <int T>
__device__ void replay_digits(const int32_t* ghist, int passes, uint32_t M, uint32_t& prefix, uint32_t& remaining,
                              uint32_t* sh /* 2 */, int* lds) {
  const int tid = threadIdx.x;
  prefix = 0;
  remaining = M;
  // every histogram count this thread needs, loaded before the first scan (one memory
  // round trip instead of one per digit); threads past 256 and digits past `passes` read
  // bin 0 of digit 0 and drop it
  uint32_t hv[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const bool ok = tid < 256 && s < passes;
    hv[s] = (uint32_t)ghist[ok ? s * 256 + 255 - tid : 0];
    if (!ok) hv[s] = 0u;
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (s >= passes) break;
    const uint32_t v = hv[s];
    int tot;
    const uint32_t x = (uint32_t)block_exclusive_scan<T>((int)v, &tot, lds) + v;   // keys with digit >= 255 - tid
    if (tid < 256 && x >= remaining && x - v < remaining) {
      sh[0] = prefix | ((uint32_t)(255 - tid) << (24 - 8 * s));
      sh[1] = remaining - (x - v);
    }
    __syncthreads();
    prefix = sh[0];
    remaining = sh[1];
    __syncthreads();
  }
}

struct SelArgs {
  const float* g_self;
  const float* g_cross;
  const float* cos;
  float* w;
  uint8_t* selected;
  int32_t* st;
  int64_t N, S, P, M, nchunks, sel_stride, hist_off, eq_off, gt_off;
};

// Clears the four digit histograms of every head.
__global__ __launch_bounds__(kHistThreads) void sel_clear_kernel(SelArgs a) {
  int32_t* h = a.st + (int64_t)blockIdx.x * a.sel_stride + a.hist_off;
  for (int i = threadIdx.x; i < 4 * 256; i += kHistThreads) h[i] = 0;
}

// Digit pass `pass` (0 = the top 8 bits) over 4096 pairs of one head: LDS histogram of
// the keys that carry the prefix chosen so far, added into the head's global histogram.
__global__ __launch_bounds__(kHistThreads) void sel_hist_kernel(SelArgs a, int pass) {
  const int64_t bh = blockIdx.y;
  const int tid = threadIdx.x;
  int32_t* st = a.st + bh * a.sel_stride;
  const float* cs = a.cos + bh * a.P;
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh[2];
  __shared__ int lds[kHistThreads / 64];
  // the keys are loaded first, so that their loads overlap the replay
  const int64_t b0 = (int64_t)blockIdx.x * kHistBlock;
  uint32_t keys[kHistKeys];
#pragma unroll
  for (int j = 0; j < kHistKeys; ++j) {
    const int64_t p = b0 + j * kHistThreads + tid;
    keys[j] = order_key(cs[p < a.P ? p : 0]);
  }
  uint32_t prefix, remaining;
  replay_digits<kHistThreads>(st + a.hist_off, pass, (uint32_t)a.M, prefix, remaining, sh, lds);
  const uint32_t mask = pass == 0 ? 0u : 0xffffffffu << (32 - 8 * pass);
  const int shift = 24 - 8 * pass;
  hist[tid] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kHistKeys; ++j) {
    const int64_t p = b0 + j * kHistThreads + tid;
    const uint32_t k = keys[j];
    wave_hist_add(hist, p < a.P && (k & mask) == prefix, (k >> shift) & 255u);
  }
  __syncthreads();
  const uint32_t v = hist[tid];
  if (v) atomicAdd(reinterpret_cast<uint32_t*>(st + a.hist_off + pass * 256 + tid), v);
}

// Per-chunk counts of keys equal to and above the threshold key tau.  Wave w at step j
// holds the 64 pairs of chunk 64 blockIdx.x + 4 j + w.
__global__ __launch_bounds__(kHistThreads) void sel_count_kernel(SelArgs a) {
  const int64_t bh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int32_t* st = a.st + bh * a.sel_stride;
  const float* cs = a.cos + bh * a.P;
  __shared__ uint32_t sh[2];
  __shared__ int lds[kHistThreads / 64];
  const int64_t b0 = (int64_t)blockIdx.x * kHistBlock;
  uint32_t keys[kHistKeys];   // loaded before the replay, as in the histogram pass
#pragma unroll
  for (int j = 0; j < kHistKeys; ++j) {
    const int64_t p = b0 + j * kHistThreads + tid;
    keys[j] = order_key(cs[p < a.P ? p : 0]);
  }
  uint32_t tau, remaining;
  replay_digits<kHistThreads>(st + a.hist_off, 4, (uint32_t)a.M, tau, remaining, sh, lds);
#pragma unroll
  for (int j = 0; j < kHistKeys; ++j) {
    const int64_t p = b0 + j * kHistThreads + tid;
    const uint32_t k = keys[j];
    const uint64_t eq = __ballot(p < a.P && k == tau);
    const uint64_t gt = __ballot(p < a.P && k > tau);
    const int64_t c = b0 / kChunkPairs + j * (kHistThreads / 64) + wv;
    if (lane == 0 && c < a.nchunks) {
      st[a.eq_off + c] = __popcll(eq);
      st[a.gt_off + c] = __popcll(gt);
    }
  }
}

// Tie cut-off index and chunk offsets of one head (one workgroup per head).
__global__ __launch_bounds__(kSelThreads) void sel_final_kernel(SelArgs a) {
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int32_t* st = a.st + bh * a.sel_stride;
  const float* cs = a.cos + bh * a.P;
  __shared__ uint32_t sh[2];
  __shared__ int lds[kSelThreads / 64];
  __shared__ int64_t sh_ct;
  __shared__ int32_t sh_rank, sh_ptau;
  uint32_t tau, remaining;
  replay_digits<kSelThreads>(st + a.hist_off, 4, (uint32_t)a.M, tau, remaining, sh, lds);
  // the chunk that holds the `remaining`-th key equal to tau, and its rank there
  if (tid == 0) {
    sh_ct = -1;
    sh_ptau = -1;
  }
  int carry = 0;
  for (int64_t c0 = 0; c0 < a.nchunks; c0 += kSelThreads) {
    const int64_t c = c0 + tid;
    const int v = c < a.nchunks ? st[a.eq_off + c] : 0;
    int tot;
    const uint32_t before = (uint32_t)(carry + block_exclusive_scan<kSelThreads>(v, &tot, lds));
    if (v > 0 && before < remaining && remaining <= before + (uint32_t)v) {
      sh_ct = c;
      sh_rank = (int32_t)(remaining - before);   // 1-based
    }
    carry += tot;
  }
  __syncthreads();
  const int64_t ct = sh_ct;
  if (wv == 0 && ct >= 0) {   // the index of that key: wave 0 reads the chunk's 64 keys
    const int64_t p = ct * kChunkPairs + lane;
    const bool e = p < a.P && order_key(cs[p]) == tau;
    const uint64_t m = __ballot(e);
    if (e && __popcll(m & ((1ull << lane) - 1ull)) + 1 == sh_rank) sh_ptau = (int32_t)p;
  }
  __syncthreads();
  SelHeader hd;
  hd.tau_key = tau;
  hd.p_tau = sh_ptau;
  hd.n_merge = (int32_t)a.M;
  hd.n_chunks = (int32_t)a.nchunks;
  // selected per chunk: every key above tau, and the keys equal to tau up to the cut-off
  carry = 0;
  for (int64_t c0 = 0; c0 < a.nchunks; c0 += kSelThreads) {
    const int64_t c = c0 + tid;
    int v = 0;
    if (c < a.nchunks) v = st[a.gt_off + c] + (c < ct ? st[a.eq_off + c] : c == ct ? sh_rank : 0);
    int tot;
    const int ex = block_exclusive_scan<kSelThreads>(v, &tot, lds);
    if (c < a.nchunks) st[kSelHeaderInts + c] = carry + ex;
    carry += tot;
  }
  if (tid == 0) {
    st[0] = (int32_t)hd.tau_key;
    st[1] = hd.p_tau;
    st[2] = hd.n_merge;
    st[3] = hd.n_chunks;
    st[kSelHeaderInts + a.nchunks] = carry;
  }
  // optional per-pair outputs
  if (a.selected || a.w) {
    for (int64_t p = tid; p < a.P; p += kSelThreads) {
      if (a.selected) a.selected[bh * a.P + p] = is_selected(order_key(cs[p]), p, hd) ? 1 : 0;
      if (a.w) {
        const int64_t m = a.S + 2 * p;
        float w0, w1;
        closed_form_weights(a.g_self[bh * a.N + m], a.g_cross[bh * a.P + p], a.g_self[bh * a.N + m + 1], w0, w1);
        a.w[(bh * a.P + p) * 2] = w0;
        a.w[(bh * a.P + p) * 2 + 1] = w1;
      }
    }
  }
}

// Heads with at most kOneWgMaxPairs candidate pairs: the whole selection of one head in one
// workgroup, its keys held in registers (KPT per thread), the four digit histograms in
// LDS, then the same header and chunk offsets as the multi-workgroup path.  Wave w at step
// j holds the 64 pairs of chunk 16 j + w; thread t owns chunk t in the scans (at most 1024
// chunks).  One launch instead of seven, for short caches (a budgeted cache between prefill
// chunks): 9 us for 256 heads x 1264 pairs against ~40.  Only one CU works per head, so
// long heads go to the multi-workgroup path (65536 pairs: 94 us here against 60).
constexpr int kOneWgMaxKeys = 16;
constexpr int kOneWgMaxPairs = kSelThreads * kOneWgMaxKeys;   // 16384 pairs, 256 chunks

template <int KPT>
__global__ __launch_bounds__(kSelThreads) void select_onewg_kernel(SelArgs a) {
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int32_t* st = a.st + bh * a.sel_stride;
  const float* cs = a.cos + bh * a.P;
  constexpr int NCH = KPT * (kSelThreads / 64);   // chunks the keys cover
  __shared__ uint32_t hist[4][256];   // one histogram per digit, cleared once
  __shared__ uint32_t sh[2];
  __shared__ int lds[kSelThreads / 64];
  __shared__ int eq_c[NCH], gt_c[NCH];
  __shared__ uint64_t eq_m[NCH];
  __shared__ int32_t sh_ct, sh_rank, sh_ptau;
  uint32_t k[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int64_t p = (int64_t)j * kSelThreads + tid;
    k[j] = p < a.P ? order_key(cs[p]) : 0u;
  }
  uint32_t prefix = 0, remaining = (uint32_t)a.M;
  static_assert(kSelThreads == 4 * 256, "one thread per histogram bin");
  reinterpret_cast<uint32_t*>(hist)[tid] = 0;
  __syncthreads();
  for (int s = 0; s < 4; ++s) {
    const uint32_t mask = s == 0 ? 0u : 0xffffffffu << (32 - 8 * s);
    const int shift = 24 - 8 * s;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int64_t p = (int64_t)j * kSelThreads + tid;
      wave_hist_add(hist[s], p < a.P && (k[j] & mask) == prefix, (k[j] >> shift) & 255u);
    }
    __syncthreads();
    // digit s: the largest d whose count of keys >= d reaches `remaining`; wave 0 alone,
    // lane l holding digits 255 - 4 l .. 252 - 4 l (counts of keys >= d by a wave scan)
    if (wv == 0) {
      uint32_t v[4], c[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = hist[s][255 - 4 * lane - j];
      c[0] = v[0];
#pragma unroll
      for (int j = 1; j < 4; ++j) c[j] = c[j - 1] + v[j];
      uint32_t x = c[3];   // inclusive scan of the lane totals
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = (uint32_t)__shfl_up((int)x, off, 64);
        if (lane >= off) x += y;
      }
      const uint32_t before = x - c[3];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t xj = before + c[j];
        if (xj >= remaining && xj - v[j] < remaining) {
          sh[0] = prefix | ((uint32_t)(255 - 4 * lane - j) << shift);
          sh[1] = remaining - (xj - v[j]);
        }
      }
    }
    __syncthreads();
    // sh is rewritten only after the next digit's barrier, which every thread reaches after
    // reading it here
    prefix = sh[0];
    remaining = sh[1];
  }
  const uint32_t tau = prefix;
  // per-chunk counts of keys equal to and above tau
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int64_t p = (int64_t)j * kSelThreads + tid;
    const uint64_t eq = __ballot(p < a.P && k[j] == tau);
    const uint64_t gt = __ballot(p < a.P && k[j] > tau);
    const int c = j * (kSelThreads / 64) + wv;
    if (lane == 0) {
      eq_c[c] = __popcll(eq);
      gt_c[c] = __popcll(gt);
      eq_m[c] = eq;
    }
  }
  if (tid == 0) {
    sh_ct = -1;
    sh_rank = 0;
    sh_ptau = -1;
  }
  __syncthreads();
  // the chunk that holds the remaining-th key equal to tau, and its rank there
  const int c = tid;
  const bool live = c < a.nchunks && c < NCH;
  const int e = live ? eq_c[c] : 0;
  int tot;
  const int before = block_exclusive_scan<kSelThreads>(e, &tot, lds);
  if (e > 0 && (uint32_t)before < remaining && remaining <= (uint32_t)(before + e)) {
    sh_ct = c;
    sh_rank = (int32_t)remaining - before;   // 1-based
  }
  __syncthreads();
  const int ct = sh_ct, rank = sh_rank;
  if (wv == 0 && ct >= 0) {   // the index of that key: wave 0 scans the chunk's flag mask
    const uint64_t m = eq_m[ct];
    const bool bit = (m >> lane) & 1ull;
    const uint64_t at = __ballot(bit && __popcll(m & ((1ull << lane) - 1ull)) + 1 == rank);
    if (lane == 0 && at) sh_ptau = (int32_t)(ct * kChunkPairs + __ffsll((unsigned long long)at) - 1);
  }
  // selected per chunk: every key above tau, and the keys equal to tau up to the cut-off
  const int v = live ? gt_c[c] + (c < ct ? e : c == ct ? rank : 0) : 0;
  const int ex = block_exclusive_scan<kSelThreads>(v, &tot, lds);
  if (live) st[kSelHeaderInts + c] = ex;
  __syncthreads();   // sh_ptau is written
  if (tid == 0) {
    st[0] = (int32_t)tau;
    st[1] = sh_ptau;
    st[2] = (int32_t)a.M;
    st[3] = (int32_t)a.nchunks;
    st[kSelHeaderInts + a.nchunks] = tot;
  }
  if (a.selected || a.w) {
    SelHeader hd;
    hd.tau_key = tau;
    hd.p_tau = sh_ptau;
    hd.n_merge = (int32_t)a.M;
    hd.n_chunks = (int32_t)a.nchunks;
    for (int64_t p = tid; p < a.P; p += kSelThreads) {
      if (a.selected) a.selected[bh * a.P + p] = is_selected(order_key(cs[p]), p, hd) ? 1 : 0;
      if (a.w) {
        const int64_t m = a.S + 2 * p;
        float w0, w1;
        closed_form_weights(a.g_self[bh * a.N + m], a.g_cross[bh * a.P + p], a.g_self[bh * a.N + m + 1], w0, w1);
        a.w[(bh * a.P + p) * 2] = w0;
        a.w[(bh * a.P + p) * 2 + 1] = w1;
      }
    }
  }
}

// M == P / M == 0 without a cosine array: thresholds are fixed, so the cosine is never read.
__global__ __launch_bounds__(kSelThreads) void select_fixed_kernel(SelArgs a) {
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x;
  int32_t* st = a.st + bh * a.sel_stride;
  const bool all = a.M == a.P && a.M > 0;
  for (int64_t c = tid; c < a.nchunks; c += kSelThreads) st[kSelHeaderInts + c] = all ? (int32_t)(c * kChunkPairs) : 0;
  if (tid == 0) {
    st[0] = all ? 0 : (int32_t)0xffffffffu;
    st[1] = all ? (int32_t)(a.P - 1) : -1;
    st[2] = (int32_t)a.M;
    st[3] = (int32_t)a.nchunks;
    st[kSelHeaderInts + a.nchunks] = (int32_t)a.M;
  }
  for (int64_t p = tid; p < a.P; p += kSelThreads) {
    if (a.selected) a.selected[bh * a.P + p] = all ? 1 : 0;
    if (a.w) {
      const int64_t m = a.S + 2 * p;
      float w0, w1;
      closed_form_weights(a.g_self[bh * a.N + m], a.g_cross[bh * a.P + p], a.g_self[bh * a.N + m + 1], w0, w1);
      a.w[(bh * a.P + p) * 2] = w0;
      a.w[(bh * a.P + p) * 2 + 1] = w1;
    }
  }
}

hipError_t launch_select(const Shape& s, const RoundP& r, const float* g_self, const float* g_cross,
                         const float* cos, float* w, uint8_t* selected, int32_t* sel_state, hipStream_t st) {
  SelArgs a;
  a.g_self = g_self;
  a.g_cross = g_cross;
  a.cos = cos;
  a.w = w;
  a.selected = selected;
  a.st = sel_state;
  a.N = s.N;
  a.S = r.S;
  a.P = r.P;
  a.M = r.M;
  a.nchunks = n_chunks(r.P);
  a.sel_stride = sel_stride_ints(r.P);
  a.hist_off = sel_hist_off(r.P);
  a.eq_off = sel_eq_off(r.P);
  a.gt_off = sel_gt_off(r.P);
  const int heads = s.B * s.Hkv;
  if (heads == 0) return hipSuccess;
  if (cos == nullptr || r.M == 0 || r.M == r.P) {
    KVS_LAUNCH("select", select_fixed_kernel, dim3(heads), dim3(kSelThreads), 0, st, a);
    return hipGetLastError();
  }
  if (r.P <= kOneWgMaxPairs) {
    const dim3 g(heads), b(kSelThreads);
    if (r.P <= 4 * kSelThreads)
      KVS_LAUNCH("select", select_onewg_kernel<4>, g, b, 0, st, a);
    else
      KVS_LAUNCH("select", select_onewg_kernel<16>, g, b, 0, st, a);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((r.P + kHistBlock - 1) / kHistBlock), (unsigned)heads);
  KVS_LAUNCH("select", sel_clear_kernel, dim3(heads), dim3(kHistThreads), 0, st, a);
  for (int pass = 0; pass < 4; ++pass)
    KVS_LAUNCH("select", sel_hist_kernel, grid, dim3(kHistThreads), 0, st, a, pass);
  KVS_LAUNCH("select", sel_count_kernel, grid, dim3(kHistThreads), 0, st, a);
  KVS_LAUNCH("select", sel_final_kernel, dim3(heads), dim3(kSelThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace kvs
