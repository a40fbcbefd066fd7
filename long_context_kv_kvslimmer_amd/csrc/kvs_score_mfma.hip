// bf16 MFMA scorer kernels for gfx950 (see kvs_score.hip for the math).
#include "kvs_common.h"
#include "kvs_score_impl.h"

namespace kvs {

bool use_mfma_scorer(const Shape&) { return false; }

size_t mfma_score_workspace_bytes(const Shape&, const RoundP&) { return 0; }

hipError_t launch_score_mfma(const Shape&, const RoundP&, const void*, const void*, const int32_t*, const void*,
                             float*, float*, float*, float*, float*, void*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace kvs
