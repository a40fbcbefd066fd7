// Host-side launch interface between the C-ABI layer (kvs_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvs {

// Timing marks (see kvs_set_marks): before / after every kernel launch.
void mark_before(hipStream_t st, const char* name);
void mark_after(hipStream_t st);

// Launch with timing marks around it.
#define KVS_LAUNCH(name, kernel, grid, block, shmem, stream, ...)                 \
  do {                                                                           \
    ::kvs::mark_before((stream), (name));                                        \
    hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);         \
    ::kvs::mark_after((stream));                                                 \
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
// int32 per (b, h) in the selection state: header + chunk offsets (n_chunks + 1), padded to 4.
inline int64_t sel_stride_ints(int64_t P) { return ((kSelHeaderInts + n_chunks(P) + 1) + 3) / 4 * 4; }

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

// ---- log-sum-exp combine of split partial records {m (log2 units), l, -, -, o[D]} ----
// units: rows of `out` ([units, D]); lse (natural log) is nullable.
hipError_t launch_combine(const float* part, int64_t units, int nsplit, int D, float* lse, float* out,
                          hipStream_t st);

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st);

// ---- decode ----
size_t decode_workspace_bytes(const Shape& s);
hipError_t launch_decode(const Shape& s, const void* K, const void* V, const int32_t* n, const void* q,
                         float scale, float* out, void* ws, hipStream_t st);

}  // namespace kvs
