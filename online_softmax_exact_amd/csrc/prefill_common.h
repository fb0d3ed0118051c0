// Device helpers of the MFMA prefill kernel (gfx950, bf16 operands).
#pragma once

#include "attn_internal.h"

namespace attn {
namespace pf {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr float kRescale = 8.0f;   // lazy-rescale threshold, base-2 units
// Full tiles: largest sum of a lane's 16 weights (each below 2^16 then) taken
// against the lagging reference before the reference must move.
constexpr float kSumMax = 65536.0f;

// Kernel arguments (after host-side validation; positions and sizes fit 32
// bits, strides are in elements).
struct Args {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int32_t* n_legal;
  const float* bias;
  int64_t qs[3], ks[3], vs[3], os[3], bs[4];
  int64_t q_offset;
  int64_t window;   // sliding window (keys j >= q_offset + i - window + 1), 0 = none
  int32_t t_q, t_k, heads_q, group, n_qtiles, batch_heads;
  float scale_log2;
  int32_t causal;
  // Variable-length batches: packed sequences (cu_q, cu_k of n_seqs + 1
  // entries; the grid holds `rounds` query tiles per sequence and head) or
  // per-batch KV lengths (kv_lens); both NULL for a dense batch.
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* kv_lens;
  int32_t n_seqs, rounds;
  // Dense batches: 1 = batches one after the other (heads fastest, then
  // query tiles), 0 = query tiles outermost (every batch's heaviest tiles
  // first).
  int32_t batch_major;
  // Dense batches: 1 = the heads of a (query tile, batch) pair run together
  // on one XCD (the default order otherwise).
  int32_t xcd_heads;
  float scale;   // scale in natural-log units (scale_log2 = scale * log2 e)
};

// s_waitcnt vmcnt(n) for a count n <= N known once the caller is unrolled
// (the instruction takes an immediate; a runtime n becomes a chain of
// compares that waits at the largest immediate not above it).
template <int N>
__device__ __forceinline__ void wait_vm_upto(int n) {
  if constexpr (N == 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    if (n >= N) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
    else wait_vm_upto<N - 1>(n);
  }
}

// x clamped to [0, n] (device-side length and offset arrays are never trusted).
__device__ __forceinline__ int clamp_len(int x, int n) { return x < 0 ? 0 : (x > n ? n : x); }

// LDS layouts.  Tiles are written by buffer_load ... lds (each wave
// instruction fills 1 KB in lane order), so rows cannot be padded; instead the
// 16-byte chunk c of row r is stored at chunk slot c ^ swz(r).  The K swizzle
// makes the 16-byte MFMA-operand reads (16 lanes = 16 rows, one chunk each)
// hit distinct banks; the V swizzle does the same for ds_read_b64_tr_b16
// (32 lanes = 4 rows x 64 bytes).  RB is the row size in bytes (128 or 256).
template <int RB>
__device__ __forceinline__ int swz_k(int r) {
  return (r / (256 / RB)) % (RB / 16);
}
template <int RB>
__device__ __forceinline__ int swz_v(int r) {
  return RB == 256 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// Two floats to a bf16 pair (v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// i % 4 of the 8-byte rows read by lanes 4 j + i / 4, j = 0..3.
// The restrict qualifier gives the read alias information, as the K tile's
// plain loads have; without it the compiler waits for every HBM -> LDS copy
// in flight before the read, including the copy into the other ring slot
// that the barrier protocol already keeps apart.
__device__ __forceinline__ u32x2 tr_read(const lds_char* __restrict__ p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// max / sum of a value and the same value in lane ^ 32 (v_permlane32_swap
// exchanges the two 32-lane halves, so each lane sees both values).
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ int isum_xor32(int x) {
  const auto r = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(x), static_cast<unsigned>(x), false, false);
  return static_cast<int>(r[0]) + static_cast<int>(r[1]);
}

}  // namespace pf

}  // namespace attn
