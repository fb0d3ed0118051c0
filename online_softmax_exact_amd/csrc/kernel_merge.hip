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

// Partials of row r that were written: all n_states, or with per-batch KV
// lengths only the first ceil(L_b / split_size) (later ranges hold no key of
// the batch and are not written), b = r / rows_per_b.
struct StateCount {
  const int32_t* kv_lens;
  int64_t split_size, t_k, rows_per_b;
  __device__ int64_t of(int64_t r, int64_t n_states) const {
    if (kv_lens == nullptr) return n_states;
    const int64_t raw = kv_lens[r / rows_per_b];
    const int64_t len = raw < 0 ? 0 : (raw > t_k ? t_k : raw);
    const int64_t n = (len + split_size - 1) / split_size;
    return n < n_states ? n : n_states;
  }
};

template <typename TO>
__global__ __launch_bounds__(256) void merge_kernel(
    int64_t n_rows, int64_t n_states, int64_t d_v,
    const float* __restrict__ o_states, int64_t o_rs, int64_t o_ss,
    const float* __restrict__ lse_states, int64_t l_rs, int64_t l_ss,
    TO* __restrict__ out, int64_t heads, int64_t t_rows, int64_t os0,
    int64_t os1, int64_t os2, float* __restrict__ lse_out, StateCount sc) {
  const int lane = threadIdx.x & 63;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * kRows + (threadIdx.x >> 6);
  if (r >= n_rows) return;
  n_states = sc.of(r, n_states);
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

// Wide variant: one workgroup per row.  Thread (g, c) reads 16 bytes (value
// columns 4c..4c+3) of states g, g + G, g + 2G, ... so every load of a row is
// in flight at once; the per-group sums are combined in LDS.  Needs d_v % 4 ==
// 0 and 16-byte aligned rows and states.
template <typename TO>
__global__ __launch_bounds__(256) void merge_wide_kernel(
    int64_t n_states, int d_v, const float* __restrict__ o_states, int64_t o_rs, int64_t o_ss,
    const float* __restrict__ lse_states, int64_t l_rs, int64_t l_ss, TO* __restrict__ out,
    int64_t heads, int64_t t_rows, int64_t os0, int64_t os1, int64_t os2,
    float* __restrict__ lse_out, StateCount sc) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  __shared__ float red[4];
  __shared__ __attribute__((aligned(16))) float part[256 * 4];
  __shared__ float lpart[256];
  debug_poison_lds(red, sizeof(red));
  debug_poison_lds(part, sizeof(part));
  debug_poison_lds(lpart, sizeof(lpart));
  const int tid = threadIdx.x;
  const int64_t r = blockIdx.x;
  n_states = sc.of(r, n_states);
  const float* lrow = lse_states + r * l_rs;
  const float* orow = o_states + r * o_rs;

  float mx = -INFINITY;
  for (int64_t s = tid; s < n_states; s += 256) mx = fmaxf(mx, lrow[s * l_ss]);
  mx = wave_max(mx);
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

  const int chunks = d_v / 4;
  const int groups = 256 / chunks;
  const int c = tid % chunks, g = tid / chunks;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  float l = 0.0f;
  if (mx != -INFINITY && g < groups) {
    const float m2 = mx * kLog2e;
#pragma unroll 4
    for (int64_t s = g; s < n_states; s += groups) {
      const float x = lrow[s * l_ss];
      const f32x4 v = *reinterpret_cast<const f32x4*>(orow + s * o_ss + 4 * c);
      const bool valid = x != -INFINITY;       // empty states are skipped by flag
      const float w = valid ? fast_exp2(fmaf(x, kLog2e, -m2)) : 0.0f;
      if (valid) {
        acc[0] = fmaf(w, v[0], acc[0]);
        acc[1] = fmaf(w, v[1], acc[1]);
        acc[2] = fmaf(w, v[2], acc[2]);
        acc[3] = fmaf(w, v[3], acc[3]);
      }
      l += w;
    }
  }
  if (g < groups) {
    *reinterpret_cast<f32x4*>(part + 4 * tid) = acc;
    lpart[tid] = l;
  }
  __syncthreads();
  const int64_t ii = r % t_rows;
  const int64_t hh = (r / t_rows) % heads;
  const int64_t bb = r / (t_rows * heads);
  TO* dst = out + bb * os0 + hh * os1 + ii * os2;
  if (tid < chunks) {
    f32x4 sum = {0.0f, 0.0f, 0.0f, 0.0f};
    float lt = 0.0f;
    for (int gg = 0; gg < groups; ++gg) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(part + 4 * (gg * chunks + tid));
      sum[0] += x[0]; sum[1] += x[1]; sum[2] += x[2]; sum[3] += x[3];
      lt += lpart[gg * chunks + tid];
    }
    const bool live = mx != -INFINITY;
    const float inv = live ? 1.0f / lt : 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) Elem<TO>::store(dst, 4 * tid + e, live ? sum[e] * inv : 0.0f);
    if (tid == 0) lse_out[r] = live ? mx + fast_log2(lt) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_merge(int64_t n_rows, int64_t n_states, int64_t d_v,
                        const float* o_states, int64_t o_row_stride,
                        int64_t o_state_stride, const float* lse_states,
                        int64_t lse_row_stride, int64_t lse_state_stride,
                        int out_dtype, void* o_out, int64_t heads,
                        int64_t t_rows, const int64_t out_strides[3],
                        float* lse_out, hipStream_t stream, const int32_t* kv_lens,
                        int64_t split_size, int64_t t_k) {
  if (n_rows == 0) return hipSuccess;
  const StateCount sc{kv_lens, split_size > 0 ? split_size : 1, t_k, heads * t_rows};
  const bool wide = d_v % 4 == 0 && o_row_stride % 4 == 0 && o_state_stride % 4 == 0 &&
                    (reinterpret_cast<uintptr_t>(o_states) & 15) == 0 && n_rows < (int64_t(1) << 31);
  if (wide) {
    if (out_dtype == ATTN_F32)
      hipLaunchKernelGGL(merge_wide_kernel<float>, dim3(static_cast<unsigned>(n_rows)), dim3(256), 0, stream,
                         n_states, static_cast<int>(d_v), o_states, o_row_stride, o_state_stride, lse_states,
                         lse_row_stride, lse_state_stride, static_cast<float*>(o_out), heads, t_rows,
                         out_strides[0], out_strides[1], out_strides[2], lse_out, sc);
    else
      hipLaunchKernelGGL(merge_wide_kernel<uint16_t>, dim3(static_cast<unsigned>(n_rows)), dim3(256), 0, stream,
                         n_states, static_cast<int>(d_v), o_states, o_row_stride, o_state_stride, lse_states,
                         lse_row_stride, lse_state_stride, static_cast<uint16_t*>(o_out), heads, t_rows,
                         out_strides[0], out_strides[1], out_strides[2], lse_out, sc);
    return hipGetLastError();
  }
  const int64_t blocks = (n_rows + kRows - 1) / kRows;
  if (out_dtype == ATTN_F32) {
    hipLaunchKernelGGL(merge_kernel<float>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                       n_rows, n_states, d_v, o_states, o_row_stride, o_state_stride, lse_states,
                       lse_row_stride, lse_state_stride, static_cast<float*>(o_out), heads, t_rows,
                       out_strides[0], out_strides[1], out_strides[2], lse_out, sc);
  } else {
    hipLaunchKernelGGL(merge_kernel<uint16_t>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                       n_rows, n_states, d_v, o_states, o_row_stride, o_state_stride, lse_states,
                       lse_row_stride, lse_state_stride, static_cast<uint16_t*>(o_out), heads, t_rows,
                       out_strides[0], out_strides[1], out_strides[2], lse_out, sc);
  }
  return hipGetLastError();
}

}  // namespace attn
