// Internal declarations shared by the host library and the kernels.
// Device code targets gfx950 (CDNA4) only: wave64, MFMA, 160 KiB LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_mi355x.h"

namespace attn {

// ---------------------------------------------------------------------------
// Problem description after validation (plain values, passed by value to the
// kernels).  Scores are handled in the base-2 domain: z2 = z * log2(e), so a
// weight e^{z - m} is exp2(z2 - m2) on the hardware's v_exp_f32.
// ---------------------------------------------------------------------------
struct Problem {
  int64_t batch, heads_q, heads_kv, t_q, t_k, d_h, d_v, q_offset;
  int64_t qs[3], ks[3], vs[3], os[3], bs[4];
  const float* bias;
  float scale_log2;   // scale * log2(e)
  int32_t causal;
  int32_t group;      // heads_q / heads_kv
  int64_t window;     // sliding window (keys j >= q_offset + i - window + 1), 0 = none
  // Variable-length batches (device arrays, never read on the host).
  // Packed: sequence s owns rows [cu_q[s], cu_q[s+1]) and keys [cu_k[s],
  // cu_k[s+1]), row i at q_offset + (L_k - L_q) + i.  Per-batch KV lengths:
  // batch b uses keys [0, kv_lens[b]), row i at q_offset + kv_lens[b] - T_q + i.
  const int32_t* cu_q;
  const int32_t* cu_k;
  int64_t n_seqs, max_seqlen_q;
  const int32_t* kv_lens;
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Workspace layout of split-KV decode: fp32 o partials [rows, S, d_v], then
// fp32 lse partials [rows, S], where rows = B * H_q * T_q in (b, hq, i) order.
// Splits [s0, s1) hold every key some row may see: keys below the last
// causal position + 1 and at or past the first window start.  The others are
// neither computed nor merged (with per-batch KV lengths, which the host does
// not read, every split is in the range).
struct SplitLayout {
  int64_t rows, n_splits, split_size;
  int64_t s0, s1;
  size_t o_bytes, lse_offset, total;
};
SplitLayout split_layout(const Problem& pb, int64_t split_size);

// ---- launchers (return hipSuccess or the launch error) --------------------
hipError_t launch_generic(const Problem& pb, int dtype, const void* q,
                          const void* k, const void* v, void* o, float* lse,
                          int32_t* n_legal, int64_t split_size, float* ws_o,
                          float* ws_lse, hipStream_t stream);

// Backward: D_i = <dO_i, O_i>, then dQ and dK/dV (generic kernels).
hipError_t launch_bwd_rowdot(const Problem& pb, int dtype, const void* o, const void* d_o, float* ws_d,
                             hipStream_t stream);
hipError_t launch_bwd_dq_generic(const Problem& pb, int dtype, const void* q, const void* k,
                                 const void* v, const float* lse, const void* d_o, const float* ws_d,
                                 void* d_q, hipStream_t stream);
hipError_t launch_bwd_dkdv_generic(const Problem& pb, int dtype, const void* q, const void* k,
                                   const void* v, const float* lse, const void* d_o, const float* ws_d,
                                   void* d_k, void* d_v, hipStream_t stream);

hipError_t launch_merge(int64_t n_rows, int64_t n_states, int64_t d_v,
                        const float* o_states, int64_t o_row_stride,
                        int64_t o_state_stride, const float* lse_states,
                        int64_t lse_row_stride, int64_t lse_state_stride,
                        int out_dtype, void* o_out, int64_t rows_per_b,
                        int64_t rows_per_h, const int64_t out_strides[3],
                        float* lse_out, hipStream_t stream,
                        const int32_t* kv_lens = nullptr, int64_t split_size = 1,
                        int64_t t_k = 0);

// ---- device helpers -------------------------------------------------------
#if defined(__HIP_DEVICE_COMPILE__) || defined(__HIPCC__)

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest even; inputs here are finite (no NaN is ever formed).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

__device__ __forceinline__ float fast_log2(float x) {
  return __builtin_amdgcn_logf(x);
}

// Raw buffer resource over [base, base + bytes): loads at offsets >= bytes
// return zeros, which the kernels use for key rows past the end of a range.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (bytes >= 0x7fffffff ? 0x7fffffff : static_cast<int>(bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), n,
                                           0x00020000);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Packed sequences: the sequence holding packed index x of an axis whose
// offsets are cu[0..n] (the last sequence starting at or before x, by binary
// search over the offsets clamped to [0, T]), and its clamped extent [lo, hi)
// (hi >= lo).  Returns false when x lies in no sequence.
__device__ __forceinline__ bool find_seq(const int32_t* cu, int64_t n, int64_t T, int64_t x,
                                         int64_t* s, int64_t* lo, int64_t* hi) {
  auto c = [&](int64_t i) { const int64_t y = cu[i]; return y < 0 ? 0 : (y > T ? T : y); };
  int64_t a = 0, b = n - 1;
  while (a < b) {
    const int64_t mid = (a + b + 1) / 2;
    if (c(mid) <= x) a = mid; else b = mid - 1;
  }
  *s = a;
  *lo = c(a);
  const int64_t e = c(a + 1);
  *hi = e > *lo ? e : *lo;
  return x >= *lo && x < *hi;
}

// The clamped extent of sequence s of an axis with offsets cu (see find_seq).
__device__ __forceinline__ void seq_extent(const int32_t* cu, int64_t T, int64_t s, int64_t* lo, int64_t* hi) {
  auto c = [&](int64_t i) { const int64_t y = cu[i]; return y < 0 ? 0 : (y > T ? T : y); };
  *lo = c(s);
  const int64_t e = c(s + 1);
  *hi = e > *lo ? e : *lo;
}

// LDS poisoning (debug builds compiled with -DATTN_DEBUG_POISON=1): every
// kernel fills its LDS with all-one bytes when it starts, and every HBM -> LDS
// copy first fills the bytes it is about to write, so a read of LDS that no
// write of this launch (or of the current copy into a reused slot) reached
// sees a NaN (fp32 and bf16 alike) instead of zeros or an older tile.  Such a
// build gives the normal build's outputs bit for bit exactly when no such
// read happens; the GPU tests compare the two.
#ifndef ATTN_DEBUG_POISON
#define ATTN_DEBUG_POISON 0
#endif

// Whole-workgroup fill of [p, p + bytes) (4-byte aligned), then a barrier.
// Call at kernel entry, before any early return, from every thread.
__device__ __forceinline__ void debug_poison_lds(void* p, int bytes) {
  if (ATTN_DEBUG_POISON) {
    uint32_t* w = static_cast<uint32_t*>(p);
    for (int i = static_cast<int>(threadIdx.x); i < bytes / 4; i += static_cast<int>(blockDim.x)) w[i] = ~0u;
    __syncthreads();
  }
}

// One HBM -> LDS copy of BYTES (4 or 16) per lane: lane l's bytes land at
// dst + BYTES * l.  Poisoning builds fill those bytes first and wait for the
// fill, so the copy's data lands after it.
template <int BYTES>
__device__ __forceinline__ void lds_copy(__amdgpu_buffer_rsrc_t rs, __attribute__((address_space(3))) void* dst,
                                         int voffset) {
  static_assert(BYTES == 4 || BYTES == 16, "4- or 16-byte copies");
  if (ATTN_DEBUG_POISON) {
    __attribute__((address_space(3))) uint32_t* d =
        reinterpret_cast<__attribute__((address_space(3))) uint32_t*>(dst) + (BYTES / 4) * (threadIdx.x & 63);
#pragma unroll
    for (int e = 0; e < BYTES / 4; ++e) d[e] = ~0u;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
  if constexpr (BYTES == 4)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 4, voffset, 0, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, voffset, 0, 0, 0);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static float load(const float* p, int64_t i) { return p[i]; }
  __device__ static void store(float* p, int64_t i, float x) { p[i] = x; }
};
template <> struct Elem<uint16_t> {
  __device__ static float load(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  __device__ static void store(uint16_t* p, int64_t i, float x) { p[i] = f32_to_bf16(x); }
};

#endif

}  // namespace attn
