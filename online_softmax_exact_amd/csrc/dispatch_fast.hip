// Choice of the specialised kernels for a validated problem.
#include "kernels.h"

namespace attn {

bool launch_fast_fwd(const Problem&, int, const void*, const void*, const void*, void*,
                     float*, int32_t*, hipStream_t, int*) {
  return false;
}

bool launch_fast_decode_partials(const Problem&, int, const void*, const void*, const void*,
                                 const SplitLayout&, float*, float*, hipStream_t, hipError_t*) {
  return false;
}

}  // namespace attn
