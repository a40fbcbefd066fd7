// Pair selection and closed-form weights (kvs_merge_weights).
//
// Selection: in each (batch, kv-head) the n_merge candidate pairs with the largest
// adjacent-key cosine, ties to the lower pair index (KVSlimmer deep-dive, section
// 数学主线二: merge homogeneous adjacent keys; section 局限与边界: one uniform ratio for
// every head).  One workgroup per (batch, head) runs an MSB-first radix select over the
// order-preserving 32-bit image of the cosine (four 8-bit digit passes with an LDS
// histogram), then finds the tie cut-off index with a block scan, then counts the
// selected pairs of every 64-pair chunk and publishes their exclusive scan; the merge
// pass uses those offsets for its cross-wave compaction.
#include "kvs_common.h"
#include "kvs_internal.h"

namespace kvs {

struct SelArgs {
  const float* g_self;
  const float* g_cross;
  const float* cos;
  float* w;
  uint8_t* selected;
  int32_t* st;
  int64_t N, S, P, M, nchunks, sel_stride;
};

constexpr int kSelThreads = 1024;

// Exclusive block-wide scan of one int per thread (kSelThreads threads); returns the
// exclusive prefix, writes the block total to *total (same value in every thread).
__device__ int block_exclusive_scan(int v, int* total, int* lds /* >= 16 ints */) {
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
  for (int k = 0; k < kSelThreads / 64; ++k) {
    const int t = lds[k];
    if (k < wv) wave_pre += t;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return wave_pre + x - v;
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(SelArgs a) {
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x;
  const float* cs = a.cos + bh * a.P;
  int32_t* st = a.st + bh * a.sel_stride;
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh_prefix, sh_remaining;
  __shared__ int32_t sh_ptau;
  __shared__ int scan_lds[16];

  uint32_t tau;
  int32_t p_tau;
  if (a.M == 0) {
    tau = 0xffffffffu;
    p_tau = -1;
  } else if (a.M == a.P) {
    tau = 0u;
    p_tau = (int32_t)(a.P - 1);
  } else {
    uint32_t prefix = 0, mask = 0, remaining = (uint32_t)a.M;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int d = tid; d < 256; d += kSelThreads) hist[d] = 0;
      __syncthreads();
      for (int64_t p = tid; p < a.P; p += kSelThreads) {
        const uint32_t k = order_key(cs[p]);
        if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        uint32_t cum = 0;
        int digit = 0;
        for (int d = 255; d >= 0; --d) {
          if (cum + hist[d] >= remaining) {
            digit = d;
            break;
          }
          cum += hist[d];
        }
        sh_prefix = prefix | ((uint32_t)digit << shift);
        sh_remaining = remaining - cum;
      }
      __syncthreads();
      prefix = sh_prefix;
      remaining = sh_remaining;
      mask |= 255u << shift;
    }
    tau = prefix;
    // the `remaining`-th smallest index among keys equal to tau
    if (tid == 0) sh_ptau = -1;
    __syncthreads();
    int base_count = 0;
    for (int64_t base = 0; base < a.P; base += kSelThreads) {
      const int64_t p = base + tid;
      const int f = (p < a.P && order_key(cs[p]) == tau) ? 1 : 0;
      int tot;
      const int ex = block_exclusive_scan(f, &tot, scan_lds);
      if (f && (uint32_t)(base_count + ex + 1) == remaining) sh_ptau = (int32_t)p;
      base_count += tot;
      __syncthreads();
      if (sh_ptau >= 0) break;
    }
    p_tau = sh_ptau;
  }
  SelHeader hd;
  hd.tau_key = tau;
  hd.p_tau = p_tau;
  hd.n_merge = (int32_t)a.M;
  hd.n_chunks = (int32_t)a.nchunks;

  // per-chunk selected counts -> exclusive offsets
  int carry = 0;
  for (int64_t c0 = 0; c0 < a.nchunks; c0 += kSelThreads) {
    const int64_t c = c0 + tid;
    int cnt = 0;
    if (c < a.nchunks) {
      const int64_t pe = min(a.P, (c + 1) * kChunkPairs);
      for (int64_t p = c * kChunkPairs; p < pe; ++p) cnt += is_selected(order_key(cs[p]), p, hd) ? 1 : 0;
    }
    int tot;
    const int ex = block_exclusive_scan(cnt, &tot, scan_lds);
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
      if (a.selected) {
        const bool s = (a.M == a.P) || (a.M != 0 && is_selected(order_key(cs[p]), p, hd));
        a.selected[bh * a.P + p] = s ? 1 : 0;
      }
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
  const int blocks = s.B * s.Hkv;
  if (blocks == 0) return hipSuccess;
  if (cos == nullptr)
    KVS_LAUNCH("select", select_fixed_kernel, dim3(blocks), dim3(kSelThreads), 0, st, a);
  else
    KVS_LAUNCH("select", select_kernel, dim3(blocks), dim3(kSelThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace kvs
