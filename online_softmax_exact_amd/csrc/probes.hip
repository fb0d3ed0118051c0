// Microbenchmarks of the gfx950 units the attention kernels lean on: the
// HBM streaming read rate, the v_exp_f32 rate, the LDS read rate (16-byte
// reads and the transposed 8-byte reads), and the bf16 MFMA rate.  They give
// the measured ceilings against which the kernels' fractions are read (the
// cost model of "Chapter 33 推理计算优化" §33.1 bounds a kernel by its work
// over the rate of the unit doing it, so the rate has to be measured).  Each
// entry point launches one kernel on the caller's stream and writes a small
// result array so that no work is optimised away; the caller times it.
// Built into its own library, apart from the attention ABI.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_probes.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Every 16-byte word of [src, src + n16 * 16) read once (grid-stride), XORed
// into one word per thread.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                          unsigned* __restrict__ out) {
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  u32x4 acc = {0, 0, 0, 0};
  int64_t i = tid;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += stride) acc ^= src[i];
  out[tid] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// 8 independent chains of v_exp_f32 per thread, `iters` steps each.
__global__ __launch_bounds__(256) void exp_kernel(float* __restrict__ out, int iters, float c) {
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = -0.001f * static_cast<float>((threadIdx.x + j) & 63);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = __builtin_amdgcn_exp2f(x[j]) * c;
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += x[j];
  out[static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

// LDS reads: each wave reads the workgroup's 64 KB buffer `iters` times,
// 16-byte reads (transposed = 0) or ds_read_b64_tr_b16 (transposed = 1),
// XOR-folding one word of each into an accumulator.
template <bool TR>
__global__ __launch_bounds__(256) void lds_read_kernel(unsigned* __restrict__ out, int iters) {
  __shared__ __attribute__((aligned(16))) char buf[65536];
  for (int i = threadIdx.x; i < 65536 / 16; i += blockDim.x)
    reinterpret_cast<u32x4*>(buf)[i] = u32x4{static_cast<unsigned>(i), 1u, 2u, 3u};
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  unsigned acc = 0;
  for (int it = 0; it < iters; ++it) {
#pragma unroll 8
    for (int k = 0; k < 64; ++k) {
      // Wave w starts at a different 1 KB block; lanes read consecutive
      // 16-byte (or 8-byte) words.
      const int blk = (k + 16 * wave + it) & 63;
      if (TR) {
        const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(buf + blk * 1024 + lane * 8));
        acc ^= static_cast<unsigned>(v[0]) ^ static_cast<unsigned>(v[3]);
      } else {
        const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
            (__attribute__((address_space(3))) char*)buf + blk * 1024 + lane * 16);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
      }
    }
  }
  out[static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = acc;
}

// 4 independent accumulators of v_mfma_f32_32x32x16_bf16 per wave, `iters`
// rounds of the 4.
__global__ __launch_bounds__(256) void mfma_kernel(float* __restrict__ out, int iters) {
  const unsigned seed = threadIdx.x * 2654435761u;
  const u32x4 a = {seed, seed ^ 0x3f803f80u, seed + 1u, seed + 2u};
  const u32x4 b = {seed ^ 0x3c003c00u, seed + 3u, seed + 5u, seed + 7u};
  f32x16 c0{}, c1{}, c2{}, c3{};
  const bf16x8 av = __builtin_bit_cast(bf16x8, a & u32x4{0x3fff3fffu, 0x3fff3fffu, 0x3fff3fffu, 0x3fff3fffu});
  const bf16x8 bv = __builtin_bit_cast(bf16x8, b & u32x4{0x3fff3fffu, 0x3fff3fffu, 0x3fff3fffu, 0x3fff3fffu});
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, c3, 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  out[static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

int status(hipError_t e) { return e == hipSuccess ? 0 : -1; }

}  // namespace

extern "C" {

int attn_probe_stream_read(const void* src, size_t bytes, unsigned* out, int blocks, void* stream) {
  if (src == nullptr || out == nullptr || blocks < 1 || (reinterpret_cast<uintptr_t>(src) & 15) != 0) return -2;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), static_cast<int64_t>(bytes / 16), out);
  return status(hipGetLastError());
}

int attn_probe_exp(float* out, int blocks, int iters, void* stream) {
  if (out == nullptr || blocks < 1 || iters < 0) return -2;
  hipLaunchKernelGGL(exp_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), out, iters,
                     0.999f);
  return status(hipGetLastError());
}

int attn_probe_lds_read(unsigned* out, int blocks, int iters, int transposed, void* stream) {
  if (out == nullptr || blocks < 1 || iters < 0) return -2;
  if (transposed)
    hipLaunchKernelGGL(lds_read_kernel<true>, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), out,
                       iters);
  else
    hipLaunchKernelGGL(lds_read_kernel<false>, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), out,
                       iters);
  return status(hipGetLastError());
}

int attn_probe_mfma(float* out, int blocks, int iters, void* stream) {
  if (out == nullptr || blocks < 1 || iters < 0) return -2;
  hipLaunchKernelGGL(mfma_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), out, iters);
  return status(hipGetLastError());
}

}  // extern "C"
