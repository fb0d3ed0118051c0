// Fast-path launchers.  Each returns true when it took the problem (and then
// stores the launch status in *status / *err) and false when the problem is
// outside its specialisation, in which case the generic kernel runs.
#pragma once

#include "attn_internal.h"

namespace attn {

bool launch_fast_fwd(const Problem& pb, int dtype, const void* q, const void* k,
                     const void* v, void* o, float* lse, int32_t* n_legal,
                     hipStream_t stream, int* status);

bool launch_fast_decode_partials(const Problem& pb, int dtype, const void* q,
                                 const void* k, const void* v, const SplitLayout& L,
                                 float* ws_o, float* ws_lse, hipStream_t stream,
                                 hipError_t* err);

// MFMA prefill for fp32 (d_h and d_v in {64, 128}; no bias, window or
// variable lengths).
bool launch_fp32_mfma(const Problem& pb, int dtype, const void* q, const void* k, const void* v, void* o,
                      float* lse, int32_t* n_legal, hipStream_t stream, int* status);

// MFMA prefill (bf16, d_h and d_v in {64, 128}).
bool launch_prefill_mfma(const Problem& pb, int dtype, const void* q, const void* k,
                         const void* v, void* o, float* lse, int32_t* n_legal,
                         hipStream_t stream, int* status);

// Few-row kernel (bf16, d_h and d_v in {64, 128}, bias contiguous along keys): attn_fwd when
// H_q/H_kv * T_q <= 32, and the split-KV decode partials.
bool launch_fewrow_fwd(const Problem& pb, int dtype, const void* q, const void* k,
                       const void* v, void* o, float* lse, int32_t* n_legal,
                       hipStream_t stream, int* status);
bool launch_fewrow_partials(const Problem& pb, int dtype, const void* q, const void* k,
                            const void* v, const SplitLayout& L, float* ws_o, float* ws_lse,
                            hipStream_t stream, hipError_t* err);

// MFMA backward dQ (bf16, d_h and d_v in {64, 128}, no bias); writes D of
// every row it computes into dd.
bool launch_bwd_dq_mfma(const Problem& pb, int dtype, const void* q, const void* k, const void* v,
                        const void* o, const float* lse, const void* d_o, float* dd, void* d_q,
                        hipStream_t stream, hipError_t* err);

bool launch_bwd_dkdv_mfma(const Problem& pb, int dtype, const void* q, const void* k, const void* v,
                          const float* lse, const void* d_o, const float* dd, void* d_k, void* d_v,
                          hipStream_t stream, hipError_t* err);

}  // namespace attn
