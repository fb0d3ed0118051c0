// Merge of stored partial results (eqs 33.4-33.5 of "Chapter 33 推理计算优化"
// §33.2).  A partial (o_s, lse_s) stands for the statistics (m, l, u) =
// (lse_s, 1, o_s): e^{lse_s - m} = sum_{j in s} e^{z_j - m} and
// e^{lse_s - m} o_s = sum_{j in s} e^{z_j - m} v_j for any reference m, so
// the merged row is o = sum_s w_s o_s / sum_s w_s with w_s = e^{lse_s - m},
// m = max over the valid partials, and LSE = m + ln sum_s w_s.  A partial with
// lse_s = -inf is empty and is skipped by flag, never subtracted (§33.2
// valid-flag rule); a row with no valid partial is (+0, -inf).
//
// One wavefront per row; lanes split d_v.  HBM traffic is the partials read
// once plus the output row written once.
#include "attn_internal.h"

namespace attn {
namespace {

constexpr int kRows = 4;

template <typename TO>
__global__ __launch_bounds__(256) void merge_kernel(
    int64_t n_rows, int64_t n_states, int64_t d_v,
    const float* __restrict__ o_states, int64_t o_rs, int64_t o_ss,
    const float* __restrict__ lse_states, int64_t l_rs, int64_t l_ss,
    TO* __restrict__ out, int64_t heads, int64_t t_rows, int64_t os0,
    int64_t os1, int64_t os2, float* __restrict__ lse_out) {
  const int lane = threadIdx.x & 63;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * kRows + (threadIdx.x >> 6);
  if (r >= n_rows) return;
  const float* lrow = lse_states + r * l_rs;
  const float* orow = o_states + r * o_rs;
  const int64_t ii = r % t_rows;
  const int64_t hh = (r / t_rows) % heads;
  const int64_t bb = r / (t_rows * heads);
  TO* dst = out + bb * os0 + hh * os1 + ii * os2;

  float mx = -INFINITY;
  for (int64_t s = lane; s < n_states; s += 64) mx = fmaxf(mx, lrow[s * l_ss]);
  mx = wave_max(mx);
  if (mx == -INFINITY) {  // no valid partial: the defined masked-row output
    for (int64_t d = lane; d < d_v; d += 64) Elem<TO>::store(dst, d, 0.0f);
    if (lane == 0) lse_out[r] = -INFINITY;
    return;
  }
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float l = 0.0f;
  const float m2 = mx * kLog2e;
  for (int64_t s = 0; s < n_states; ++s) {
    const float x = lrow[s * l_ss];
    if (x == -INFINITY) continue;
    const float w = fast_exp2(fmaf(x, kLog2e, -m2));
    l += w;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int64_t d = lane + 64 * t;
      if (d < d_v) acc[t] = fmaf(w, orow[s * o_ss + d], acc[t]);
    }
  }
  const float inv = 1.0f / l;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int64_t d = lane + 64 * t;
    if (d < d_v) Elem<TO>::store(dst, d, acc[t] * inv);
  }
  if (lane == 0) lse_out[r] = mx + fast_log2(l) * kLn2;
}

}  // namespace

hipError_t launch_merge(int64_t n_rows, int64_t n_states, int64_t d_v,
                        const float* o_states, int64_t o_row_stride,
                        int64_t o_state_stride, const float* lse_states,
                        int64_t lse_row_stride, int64_t lse_state_stride,
                        int out_dtype, void* o_out, int64_t heads,
                        int64_t t_rows, const int64_t out_strides[3],
                        float* lse_out, hipStream_t stream) {
  if (n_rows == 0) return hipSuccess;
  const int64_t blocks = (n_rows + kRows - 1) / kRows;
  if (out_dtype == ATTN_F32) {
    hipLaunchKernelGGL(merge_kernel<float>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                       n_rows, n_states, d_v, o_states, o_row_stride, o_state_stride, lse_states,
                       lse_row_stride, lse_state_stride, static_cast<float*>(o_out), heads, t_rows,
                       out_strides[0], out_strides[1], out_strides[2], lse_out);
  } else {
    hipLaunchKernelGGL(merge_kernel<uint16_t>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                       n_rows, n_states, d_v, o_states, o_row_stride, o_state_stride, lse_states,
                       lse_row_stride, lse_state_stride, static_cast<uint16_t*>(o_out), heads, t_rows,
                       out_strides[0], out_strides[1], out_strides[2], lse_out);
  }
  return hipGetLastError();
}

}  // namespace attn
