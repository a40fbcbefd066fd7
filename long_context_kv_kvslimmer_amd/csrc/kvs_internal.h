// Host-side launch interface between the C-ABI layer (kvs_api.cpp) and the kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvs {

// Timing marks (kvs_marks_begin): the start and stop events for the next launch of kernel
// `name`, or null when that launch is not marked; mark_commit counts the launch once it is
// issued.  A marked launch goes through hipExtLaunchKernelGGL, which records the two events
// at the kernel's own dispatch boundaries, so the events time the kernel alone.
void mark_events(const char* name, hipEvent_t* start, hipEvent_t* stop);
void mark_commit();

// Launch (with timing marks when they are on).  Used only inside functions that return
// hipError_t: a launch that fails returns its error at once, so a later successful launch
// cannot hide it.
#define KVS_LAUNCH(name, kernel, grid, block, shmem, stream, ...)                          \
  do {                                                                                    \
    hipEvent_t kvs_e0_ = nullptr, kvs_e1_ = nullptr;                                      \
    ::kvs::mark_events((name), &kvs_e0_, &kvs_e1_);                                       \
    if (kvs_e0_)                                                                          \
      hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, kvs_e0_, kvs_e1_, 0u, __VA_ARGS__); \
    else                                                                                  \
      hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);                \
    const hipError_t kvs_launch_err_ = hipGetLastError();                                 \
    if (kvs_launch_err_ != hipSuccess) return kvs_launch_err_;                            \
    if (kvs_e0_) ::kvs::mark_commit();                                                    \
  } while (0)

constexpr int kChunkPairs = 64;      // pairs per compaction chunk (one wavefront)
constexpr int kSelHeaderInts = 4;    // SelHeader size in int32

// Shapes shared by all launches (validated by the API layer).
struct Shape {
  int B, Hkv, Hq, G, D;
  int64_t N;
  int64_t sb, sh;   // element strides of K/V between batches / heads
  bool bf16;        // element type of K, V, queries
};

struct RoundP {
  int W;
  int64_t S, R, M, P;
  float scale;
};

inline int64_t n_chunks(int64_t P) { return P > 0 ? (P + kChunkPairs - 1) / kChunkPairs : 1; }
// Selection state per (b, h), in int32: header, chunk offsets (n_chunks + 1), padded to 4;
// then the selection's own scratch: four 256-bin digit histograms and, per chunk, the
// counts of keys equal to and above the threshold key.
inline int64_t sel_hist_off(int64_t P) { return ((kSelHeaderInts + n_chunks(P) + 1) + 3) / 4 * 4; }
inline int64_t sel_eq_off(int64_t P) { return sel_hist_off(P) + 4 * 256; }
inline int64_t sel_gt_off(int64_t P) { return sel_eq_off(P) + n_chunks(P); }
inline int64_t sel_stride_ints(int64_t P) { return (sel_gt_off(P) + n_chunks(P) + 3) / 4 * 4; }

// ---- scorer ----
size_t score_workspace_bytes(const Shape& s, const RoundP& r);
hipError_t launch_score(const Shape& s, const RoundP& r, const void* K, const void* V, const int32_t* n,
                        const void* Qw, float* lse, float* O, float* g_self, float* g_cross, float* cos,
                        void* ws, hipStream_t st);

// ---- selection + weights ----
hipError_t launch_select(const Shape& s, const RoundP& r, const float* g_self, const float* g_cross,
                         const float* cos, float* w, uint8_t* selected, int32_t* sel_state, hipStream_t st);

// ---- merge + compaction ----
struct OutP {
  int64_t sb, sh;
  bool bf16;
};
hipError_t launch_merge(const Shape& s, const RoundP& r, const void* K, const void* V, const int32_t* n,
                        const float* g_self, const float* g_cross, const int32_t* sel_state, const OutP& o,
                        void* K_out, void* V_out, int32_t* n_out, int32_t* src_out, hipStream_t st);

// ---- spectral split of adjacent-key cosines ----
hipError_t launch_spectral(const void* X, int64_t T, int d, const void* U, const float* lam, int r, float* P,
                           float* c, float* cosv, hipStream_t st);

// ---- exact-gradient diagnostics ----
hipError_t launch_exact_e(const Shape& s, const RoundP& r, const void* K, const void* V, const int32_t* n,
                          const void* Qw, const float* E, const float* lse, const float* O, float* slot_out,
                          float* pair_out, hipStream_t st);

// ---- append raw tokens (count 1) into a cache ----
hipError_t launch_append(const Shape& dst, const Shape& src, void* K, void* V, int32_t* n, int64_t at,
                         const void* K_new, const void* V_new, int64_t from, int64_t count, hipStream_t st);

// ---- log-sum-exp combine of split partial records {m (log2 units), l, -, -, o[D]} ----
// Optional operand pack for the bf16 MFMA pass 2 (written by the combine, read by pass 2):
// per kv head, the window queries in blocks of 32 (one wave each), two 16-query halves;
// for half q2 and 32-wide k step ks, 64 lanes x 16 bytes hold lane l = n + 16 g ->
// head-dim chunk 4 ks + g of query 16 q2 + n, as Q (bf16), hi and lo bf16 parts of -2 O.
// qc holds {||o||^2, -lse * log2(e)} per query.  Queries past GW are not written.
struct PackP {
  uint4* ops;          // [BH][nwb][2][3][KS][64]
  float* qc;           // [BH][nwb * 32][2]
  const void* Qw;      // bf16 [B, Hq, W, D]
  int64_t nwb, GW;     // 32-query blocks per kv head, window queries per kv head
  int Hkv, Hq, G, W;
};
__host__ __device__ inline int64_t pack_ops_index(int64_t bh, int64_t nwb, int64_t q, int which, int chunk, int KS) {
  const int64_t wb = q >> 5, q2 = (q >> 4) & 1, n = q & 15;
  return (((((bh * nwb + wb) * 2 + q2) * 3 + which) * KS + (chunk >> 2)) * 64) + n + 16 * (chunk & 3);
}
// units: rows of `out` ([units, D]); lse (natural log) is nullable; pack nullable.
hipError_t launch_combine(const float* part, int64_t units, int nsplit, int D, float* lse, float* out,
                          hipStream_t st, const PackP* pack = nullptr);
// The same operand pack from window statistics the caller supplies (lse natural log
// [units], O [units, D]).
hipError_t launch_pack(const float* lse, const float* O, int64_t units, int D, const PackP& pk, hipStream_t st);


// ---- decode ----
size_t decode_workspace_bytes(const Shape& s);
hipError_t launch_decode(const Shape& s, const void* K, const void* V, const int32_t* n, const void* q,
                         float scale, float* out, void* ws, hipStream_t st);
// Device address of the library's static decode scratch on the current device
// (KVS_STATIC_SCRATCH_BYTES bytes), looked up once per device.
hipError_t static_scratch(void** ptr);

}  // namespace kvs
