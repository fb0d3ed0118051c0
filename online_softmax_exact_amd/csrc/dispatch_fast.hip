// Choice of the specialised kernels for a validated problem.
#include "kernels.h"

namespace attn {

bool launch_fast_fwd(const Problem& pb, int dtype, const void* q, const void* k, const void* v,
                     void* o, float* lse, int32_t* n_legal, hipStream_t stream, int* status) {
  return launch_prefill_mfma(pb, dtype, q, k, v, o, lse, n_legal, stream, status);
}

bool launch_fast_decode_partials(const Problem&, int, const void*, const void*, const void*,
                                 const SplitLayout&, float*, float*, hipStream_t, hipError_t*) {
  return false;
}

}  // namespace attn
