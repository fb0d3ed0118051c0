// Generic backward kernels (any head size 1..256, fp32 or bf16, bias,
// window, grouped heads): gradients of the attention of attn_fwd by
// recomputing the probabilities from the saved LSE, following eqs 33.6-33.8
// of "Chapter 33 推理计算优化" §33.3 (block size, parallelism and backward
// recomputation):
//   P_ij = e^{z_ij - LSE_i} on legal keys (0 elsewhere),
//   G_V = P^T G_O, G_P = G_O V^T, (G_S)_ij = P_ij ((G_P)_ij - D_i) with
//   D_i = sum_k P_ik (G_P)_ik = <G_O_i, O_i> (Exercise 33.4),
//   G_Q = scale G_S K, G_K = scale G_S^T Q.
// Three kernels: D per query row; G_Q with one wavefront per query row (one
// lane per key of a 64-key block, like the generic forward kernel); G_K and
// G_V with one wavefront per key row (one lane per query row of a 64-row
// block, over every query head of the key's group).  All arithmetic in fp32.
#include "attn_internal.h"
#include "kernels.h"

namespace attn {
namespace {

constexpr int kWaves = 4;
constexpr int kMaxD = 256;
constexpr int kAcc = kMaxD / 64;

// D_i = <G_O_i, O_i> for every query row (b, hq, i), into ws_d (row order).
template <typename T>
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(Problem pb, const T* __restrict__ o,
                                                         const T* __restrict__ d_o,
                                                         float* __restrict__ ws_d, int64_t rows) {
  const int lane = threadIdx.x & 63;
  for (int64_t r = blockIdx.x * int64_t(kWaves) + (threadIdx.x >> 6); r < rows;
       r += int64_t(gridDim.x) * kWaves) {
    const int64_t i = r % pb.t_q, bh = r / pb.t_q;
    const int64_t hq = bh % pb.heads_q, b = bh / pb.heads_q;
    const int64_t off = b * pb.os[0] + hq * pb.os[1] + i * pb.os[2];
    float acc = 0.0f;
    for (int d = lane; d < pb.d_v; d += 64) acc = fmaf(Elem<T>::load(o + off, d), Elem<T>::load(d_o + off, d), acc);
    acc = wave_sum(acc);
    if (lane == 0) ws_d[r] = acc;
  }
}

// Legal-key range [lo, hi) of a row at logical position pos over t_k keys.
__device__ __forceinline__ void key_range(const Problem& pb, int64_t pos, int64_t t_k, int64_t* lo, int64_t* hi) {
  *lo = 0;
  *hi = t_k;
  if (pb.causal && pos + 1 < *hi) *hi = pos + 1;
  if (pb.window > 0 && pos - pb.window + 1 > *lo) *lo = pos - pb.window + 1;
}

// G_Q: one wavefront per query row.
template <typename T, bool HAS_BIAS>
__global__ __launch_bounds__(256) void bwd_dq_kernel(Problem pb, const T* __restrict__ q,
                                                     const T* __restrict__ k, const T* __restrict__ v,
                                                     const float* __restrict__ lse,
                                                     const T* __restrict__ d_o,
                                                     const float* __restrict__ ws_d, T* __restrict__ d_q,
                                                     int64_t rows) {
  __shared__ float sq[kWaves][kMaxD];
  __shared__ float sg[kWaves][kMaxD];
  debug_poison_lds(sq, sizeof(sq));
  debug_poison_lds(sg, sizeof(sg));
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  for (int64_t base = blockIdx.x * int64_t(kWaves); base < rows; base += int64_t(gridDim.x) * kWaves) {
    const int64_t r = base + wave;
    bool ok = r < rows;
    const int64_t i = ok ? r % pb.t_q : 0, bh = ok ? r / pb.t_q : 0;
    const int64_t hq = bh % pb.heads_q, b = bh / pb.heads_q;
    const int64_t kvh = hq / pb.group;
    // This row's keys [k0, k0 + t_k) and position (packed sequences: its
    // sequence's own, rows at the end of its keys; a row outside every
    // sequence is not written; per-batch KV lengths: the batch's first L_b
    // keys, rows at the end of them).
    int64_t k0 = 0, t_k = pb.t_k, pos = pb.q_offset + i;
    if (pb.cu_q != nullptr && ok) {
      int64_t sq, q0, q1, k1;
      ok = find_seq(pb.cu_q, pb.n_seqs, pb.t_q, i, &sq, &q0, &q1);
      seq_extent(pb.cu_k, pb.t_k, sq, &k0, &k1);
      t_k = k1 - k0;
      pos = pb.q_offset + t_k - (q1 - q0) + (i - q0);
    } else if (pb.kv_lens != nullptr && ok) {
      const int64_t raw = pb.kv_lens[b];
      t_k = raw < 0 ? 0 : (raw > pb.t_k ? pb.t_k : raw);
      pos = pb.q_offset + t_k - pb.t_q + i;
    }
    const T* qrow = q + b * pb.qs[0] + hq * pb.qs[1] + i * pb.qs[2];
    const T* grow = d_o + b * pb.os[0] + hq * pb.os[1] + i * pb.os[2];
    for (int d = lane; d < kMaxD; d += 64) {
      sq[wave][d] = (ok && d < pb.d_h) ? Elem<T>::load(qrow, d) : 0.0f;
      sg[wave][d] = (ok && d < pb.d_v) ? Elem<T>::load(grow, d) : 0.0f;
    }
    __syncthreads();
    if (ok) {
      const float l2 = lse[r] * kLog2e;          // -inf for a row with no legal key
      const float dd = ws_d[r];
      float acc[kAcc] = {0.0f, 0.0f, 0.0f, 0.0f};
      int64_t lo, hi;
      key_range(pb, pos, t_k, &lo, &hi);
      if (l2 == -INFINITY) hi = lo;              // no legal key: G_Q = 0
      const T* kbase = k + b * pb.ks[0] + kvh * pb.ks[1] + k0 * pb.ks[2];
      const T* vbase = v + b * pb.vs[0] + kvh * pb.vs[1] + k0 * pb.vs[2];
      const float* brow =
          HAS_BIAS ? pb.bias + b * pb.bs[0] + hq * pb.bs[1] + i * pb.bs[2] + k0 * pb.bs[3] : nullptr;
      for (int64_t kb = lo; kb < hi; kb += 64) {
        const int64_t j = kb + lane;
        float ds = 0.0f;
        if (j < hi) {
          const T* krow = kbase + j * pb.ks[2];
          const T* vrow = vbase + j * pb.vs[2];
          float dot = 0.0f, dp = 0.0f;
          for (int d = 0; d < pb.d_h; ++d) dot = fmaf(sq[wave][d], Elem<T>::load(krow, d), dot);
          for (int d = 0; d < pb.d_v; ++d) dp = fmaf(sg[wave][d], Elem<T>::load(vrow, d), dp);
          float z2 = dot * pb.scale_log2;
          bool legal = true;
          if (HAS_BIAS) {
            const float mb = brow[j * pb.bs[3]];
            if (mb == -INFINITY) legal = false;
            else z2 = fmaf(mb, kLog2e, z2);
          }
          const float p = legal ? fast_exp2(z2 - l2) : 0.0f;
          ds = p * (dp - dd);                      // eq 33.7
        }
        const int nj = (hi - kb) < 64 ? static_cast<int>(hi - kb) : 64;
        for (int jj = 0; jj < nj; ++jj) {
          const float dsj = __shfl(ds, jj, 64);
          const T* krow = kbase + (kb + jj) * pb.ks[2];
#pragma unroll
          for (int t = 0; t < kAcc; ++t) {
            const int d = lane + 64 * t;
            if (d < pb.d_h) acc[t] = fmaf(dsj, Elem<T>::load(krow, d), acc[t]);
          }
        }
      }
      const float sc = pb.scale_log2 * kLn2;      // the score scale
      T* out = d_q + b * pb.qs[0] + hq * pb.qs[1] + i * pb.qs[2];
#pragma unroll
      for (int t = 0; t < kAcc; ++t) {
        const int d = lane + 64 * t;
        if (d < pb.d_h) Elem<T>::store(out, d, acc[t] * sc);   // eq 33.8
      }
    }
    __syncthreads();
  }
}

// G_K and G_V: one wavefront per key row (b, kv head, j), over the rows of
// every query head of its group that see key j.
template <typename T, bool HAS_BIAS>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(Problem pb, const T* __restrict__ q,
                                                       const T* __restrict__ k, const T* __restrict__ v,
                                                       const float* __restrict__ lse,
                                                       const T* __restrict__ d_o,
                                                       const float* __restrict__ ws_d, T* __restrict__ d_k,
                                                       T* __restrict__ d_v, int64_t keys) {
  __shared__ float sk[kWaves][kMaxD];
  __shared__ float sv[kWaves][kMaxD];
  debug_poison_lds(sk, sizeof(sk));
  debug_poison_lds(sv, sizeof(sv));
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  for (int64_t base = blockIdx.x * int64_t(kWaves); base < keys; base += int64_t(gridDim.x) * kWaves) {
    const int64_t r = base + wave;
    bool ok = r < keys;
    const int64_t j = ok ? r % pb.t_k : 0, bh = ok ? r / pb.t_k : 0;
    const int64_t kvh = bh % pb.heads_kv, b = bh / pb.heads_kv;
    // This key's rows [q0, q0 + t_q) and its index jl among its sequence's
    // keys (packed sequences: its own sequence, whose rows sit at the end of
    // its keys; a key outside every sequence is not written).
    // Per-batch KV lengths: rows at q_offset + L_b - T_q + i; a key at or
    // past L_b is seen by no row and gets zero.
    int64_t q0 = 0, t_q = pb.t_q, jl = j, q_off = pb.q_offset;
    bool seen = true;
    if (pb.cu_q != nullptr && ok) {
      int64_t sk, k0, k1, q1;
      ok = find_seq(pb.cu_k, pb.n_seqs, pb.t_k, j, &sk, &k0, &k1);
      seq_extent(pb.cu_q, pb.t_q, sk, &q0, &q1);
      t_q = q1 - q0;
      jl = j - k0;
      q_off = pb.q_offset + (k1 - k0) - t_q;
    } else if (pb.kv_lens != nullptr && ok) {
      const int64_t raw = pb.kv_lens[b];
      const int64_t len = raw < 0 ? 0 : (raw > pb.t_k ? pb.t_k : raw);
      q_off = pb.q_offset + len - pb.t_q;
      seen = j < len;
    }
    const T* krow = k + b * pb.ks[0] + kvh * pb.ks[1] + j * pb.ks[2];
    const T* vrow = v + b * pb.vs[0] + kvh * pb.vs[1] + j * pb.vs[2];
    for (int d = lane; d < kMaxD; d += 64) {
      sk[wave][d] = (ok && d < pb.d_h) ? Elem<T>::load(krow, d) : 0.0f;
      sv[wave][d] = (ok && d < pb.d_v) ? Elem<T>::load(vrow, d) : 0.0f;
    }
    __syncthreads();
    if (ok) {
      // Rows i that see key j: q_offset + i >= j (causal) and
      // q_offset + i - W + 1 <= j (window).
      int64_t ilo = 0, ihi = seen ? t_q : 0;
      if (pb.causal && jl - q_off > ilo) ilo = jl - q_off;
      if (pb.window > 0 && jl - q_off + pb.window < ihi) ihi = jl - q_off + pb.window;
      float ak[kAcc] = {0.0f, 0.0f, 0.0f, 0.0f}, av[kAcc] = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int64_t g = 0; g < pb.group; ++g) {
        const int64_t hq = kvh * pb.group + g;
        const T* qbase = q + b * pb.qs[0] + hq * pb.qs[1] + q0 * pb.qs[2];
        const T* gbase = d_o + b * pb.os[0] + hq * pb.os[1] + q0 * pb.os[2];
        const int64_t rbase = (b * pb.heads_q + hq) * pb.t_q + q0;
        const float* bbase =
            HAS_BIAS ? pb.bias + b * pb.bs[0] + hq * pb.bs[1] + q0 * pb.bs[2] + j * pb.bs[3] : nullptr;
        for (int64_t ib = ilo; ib < ihi; ib += 64) {
          const int64_t i = ib + lane;
          float p = 0.0f, ds = 0.0f;
          if (i < ihi) {
            const float l2 = lse[rbase + i] * kLog2e;
            if (l2 != -INFINITY) {
              const T* qrow = qbase + i * pb.qs[2];
              const T* grow = gbase + i * pb.os[2];
              float dot = 0.0f, dp = 0.0f;
              for (int d = 0; d < pb.d_h; ++d) dot = fmaf(Elem<T>::load(qrow, d), sk[wave][d], dot);
              for (int d = 0; d < pb.d_v; ++d) dp = fmaf(Elem<T>::load(grow, d), sv[wave][d], dp);
              float z2 = dot * pb.scale_log2;
              bool legal = true;
              if (HAS_BIAS) {
                const float mb = bbase[i * pb.bs[2]];
                if (mb == -INFINITY) legal = false;
                else z2 = fmaf(mb, kLog2e, z2);
              }
              p = legal ? fast_exp2(z2 - l2) : 0.0f;
              ds = p * (dp - ws_d[rbase + i]);     // eq 33.7
            }
          }
          const int ni = (ihi - ib) < 64 ? static_cast<int>(ihi - ib) : 64;
          for (int ii = 0; ii < ni; ++ii) {
            const float pi = __shfl(p, ii, 64);
            const float dsi = __shfl(ds, ii, 64);
            const T* qrow = qbase + (ib + ii) * pb.qs[2];
            const T* grow = gbase + (ib + ii) * pb.os[2];
#pragma unroll
            for (int t = 0; t < kAcc; ++t) {
              const int d = lane + 64 * t;
              if (d < pb.d_v) av[t] = fmaf(pi, Elem<T>::load(grow, d), av[t]);    // eq 33.6
              if (d < pb.d_h) ak[t] = fmaf(dsi, Elem<T>::load(qrow, d), ak[t]);   // eq 33.8
            }
          }
        }
      }
      const float sc = pb.scale_log2 * kLn2;
      T* ok_row = d_k + b * pb.ks[0] + kvh * pb.ks[1] + j * pb.ks[2];
      T* ov_row = d_v + b * pb.vs[0] + kvh * pb.vs[1] + j * pb.vs[2];
#pragma unroll
      for (int t = 0; t < kAcc; ++t) {
        const int d = lane + 64 * t;
        if (d < pb.d_h) Elem<T>::store(ok_row, d, ak[t] * sc);
        if (d < pb.d_v) Elem<T>::store(ov_row, d, av[t]);
      }
    }
    __syncthreads();
  }
}

int64_t grid_for(int64_t items) {
  const int64_t wgs = (items + kWaves - 1) / kWaves;
  return wgs < 65536 ? (wgs > 0 ? wgs : 1) : 65536;
}

}  // namespace

hipError_t launch_bwd_rowdot(const Problem& pb, int dtype, const void* o, const void* d_o, float* ws_d,
                             hipStream_t stream) {
  const int64_t rows = pb.batch * pb.heads_q * pb.t_q;
  if (rows == 0) return hipSuccess;
  if (dtype == ATTN_F32)
    hipLaunchKernelGGL((bwd_rowdot_kernel<float>), dim3(grid_for(rows)), dim3(256), 0, stream, pb,
                       static_cast<const float*>(o), static_cast<const float*>(d_o), ws_d, rows);
  else
    hipLaunchKernelGGL((bwd_rowdot_kernel<uint16_t>), dim3(grid_for(rows)), dim3(256), 0, stream, pb,
                       static_cast<const uint16_t*>(o), static_cast<const uint16_t*>(d_o), ws_d, rows);
  return hipGetLastError();
}

namespace {
template <typename T, bool HAS_BIAS>
void dq_t(const Problem& pb, const void* q, const void* k, const void* v, const float* lse,
          const void* d_o, const float* ws_d, void* d_q, int64_t rows, hipStream_t stream) {
  hipLaunchKernelGGL((bwd_dq_kernel<T, HAS_BIAS>), dim3(grid_for(rows)), dim3(256), 0, stream, pb,
                     static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v), lse,
                     static_cast<const T*>(d_o), ws_d, static_cast<T*>(d_q), rows);
}
template <typename T, bool HAS_BIAS>
void dkdv_t(const Problem& pb, const void* q, const void* k, const void* v, const float* lse,
            const void* d_o, const float* ws_d, void* d_k, void* d_v, int64_t keys, hipStream_t stream) {
  hipLaunchKernelGGL((bwd_dkdv_kernel<T, HAS_BIAS>), dim3(grid_for(keys)), dim3(256), 0, stream, pb,
                     static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v), lse,
                     static_cast<const T*>(d_o), ws_d, static_cast<T*>(d_k), static_cast<T*>(d_v), keys);
}
}  // namespace

hipError_t launch_bwd_dq_generic(const Problem& pb, int dtype, const void* q, const void* k,
                                 const void* v, const float* lse, const void* d_o, const float* ws_d,
                                 void* d_q, hipStream_t stream) {
  const int64_t rows = pb.batch * pb.heads_q * pb.t_q;
  if (rows == 0) return hipSuccess;
  const bool bias = pb.bias != nullptr;
  if (dtype == ATTN_F32) {
    if (bias) dq_t<float, true>(pb, q, k, v, lse, d_o, ws_d, d_q, rows, stream);
    else dq_t<float, false>(pb, q, k, v, lse, d_o, ws_d, d_q, rows, stream);
  } else {
    if (bias) dq_t<uint16_t, true>(pb, q, k, v, lse, d_o, ws_d, d_q, rows, stream);
    else dq_t<uint16_t, false>(pb, q, k, v, lse, d_o, ws_d, d_q, rows, stream);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_generic(const Problem& pb, int dtype, const void* q, const void* k,
                                   const void* v, const float* lse, const void* d_o, const float* ws_d,
                                   void* d_k, void* d_v, hipStream_t stream) {
  const int64_t keys = pb.batch * pb.heads_kv * pb.t_k;
  if (keys == 0) return hipSuccess;
  const bool bias = pb.bias != nullptr;
  if (dtype == ATTN_F32) {
    if (bias) dkdv_t<float, true>(pb, q, k, v, lse, d_o, ws_d, d_k, d_v, keys, stream);
    else dkdv_t<float, false>(pb, q, k, v, lse, d_o, ws_d, d_k, d_v, keys, stream);
  } else {
    if (bias) dkdv_t<uint16_t, true>(pb, q, k, v, lse, d_o, ws_d, d_k, d_v, keys, stream);
    else dkdv_t<uint16_t, false>(pb, q, k, v, lse, d_o, ws_d, d_k, d_v, keys, stream);
  }
  return hipGetLastError();
}

}  // namespace attn
