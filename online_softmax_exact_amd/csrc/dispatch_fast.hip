// Choice of the specialised kernels for a validated problem.
#include "kernels.h"

namespace attn {

bool launch_fast_fwd(const Problem& pb, int dtype, const void* q, const void* k, const void* v,
                     void* o, float* lse, int32_t* n_legal, hipStream_t stream, int* status) {
  if (launch_fewrow_fwd(pb, dtype, q, k, v, o, lse, n_legal, stream, status)) return true;
  if (launch_prefill_mfma(pb, dtype, q, k, v, o, lse, n_legal, stream, status)) return true;
  return launch_fp32_mfma(pb, dtype, q, k, v, o, lse, n_legal, stream, status);
}

bool launch_fast_decode_partials(const Problem& pb, int dtype, const void* q, const void* k,
                                 const void* v, const SplitLayout& L, float* ws_o, float* ws_lse,
                                 hipStream_t stream, hipError_t* err) {
  return launch_fewrow_partials(pb, dtype, q, k, v, L, ws_o, ws_lse, stream, err);
}

}  // namespace attn
