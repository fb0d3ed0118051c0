// Generic exact attention kernel: one wavefront per query row, one lane per
// key of a 64-key block, VALU dot products.  It serves fp32 inputs, any head
// size 1..256, any strides and bias broadcast, and writes either final rows or
// split-KV partials.  It follows Algorithm 33.1 of "Chapter 33 推理计算优化"
// §33.2 literally per row: a block with no legal key is skipped, the first
// legal block initialises (m, l, u), later blocks merge by eqs 33.4-33.5, and
// a row that never saw a legal key is finalised as (+0, -inf).
#include "attn_internal.h"

namespace attn {
namespace {

constexpr int kWaves = 4;      // rows per workgroup
constexpr int kMaxD = 256;
constexpr int kAcc = kMaxD / 64;
#ifndef GEN_ILP
#define GEN_ILP 8          // independent partial sums of a score's dot product
#endif
#ifndef GEN_PV_UNROLL
#define GEN_PV_UNROLL 8    // keys of the P V loop unrolled (their V loads in flight together)
#endif

template <typename T, bool HAS_BIAS, bool SPLIT, bool COUNT>
__global__ __launch_bounds__(256) void generic_kernel(
    Problem pb, const T* __restrict__ q, const T* __restrict__ k,
    const T* __restrict__ v, T* __restrict__ o, float* __restrict__ lse,
    int32_t* __restrict__ n_legal, int64_t split_size, int64_t n_splits,
    int64_t row_blocks, int64_t total_blocks, float* __restrict__ ws_o,
    float* __restrict__ ws_lse) {
  __shared__ float sq[kWaves][kMaxD];
  debug_poison_lds(sq, sizeof(sq));
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  for (int64_t blk = blockIdx.x; blk < total_blocks; blk += gridDim.x) {
    // blk -> (b, hq, split, row block); the row block varies fastest.
    int64_t rest = blk;
    const int64_t rb = rest % row_blocks; rest /= row_blocks;
    const int64_t s = rest % n_splits;    rest /= n_splits;
    const int64_t hq = rest % pb.heads_q;
    const int64_t b = rest / pb.heads_q;
    const int64_t i = rb * kWaves + wave;
    bool row_ok = i < pb.t_q;
    const int64_t kvh = hq / pb.group;

    // This row's keys [k0, k0 + t_k) and logical position.  Packed sequences:
    // the sequence holding row i (binary search over the clamped row offsets;
    // a row outside every sequence is not written); per-batch KV lengths: the
    // batch's own length; rows sit at the end of their keys in both.
    int64_t k0 = 0, t_k = pb.t_k, pos = pb.q_offset + i;
    if (pb.cu_q != nullptr && row_ok) {
      int64_t sq, q0, q1, k1;
      row_ok = find_seq(pb.cu_q, pb.n_seqs, pb.t_q, i, &sq, &q0, &q1);
      seq_extent(pb.cu_k, pb.t_k, sq, &k0, &k1);
      t_k = k1 - k0;
      pos = pb.q_offset + t_k - (q1 - q0) + (i - q0);
    } else if (pb.kv_lens != nullptr) {
      const int64_t raw = pb.kv_lens[b];
      t_k = raw < 0 ? 0 : (raw > pb.t_k ? pb.t_k : raw);
      pos = pb.q_offset + t_k - pb.t_q + i;
    }

    const T* qrow = q + b * pb.qs[0] + hq * pb.qs[1] + i * pb.qs[2];
    for (int d = lane; d < kMaxD; d += 64)
      sq[wave][d] = (row_ok && d < pb.d_h) ? Elem<T>::load(qrow, d) : 0.0f;
    __syncthreads();

    if (row_ok) {
      int64_t lo = s * split_size;
      int64_t hi = split_size < t_k - lo ? lo + split_size : t_k;
      if (pb.causal && pos + 1 < hi) hi = pos + 1;  // causal block skipping
      if (pb.window > 0 && pos - pb.window + 1 > lo) lo = pos - pb.window + 1;  // sliding window
      const T* kbase = k + b * pb.ks[0] + kvh * pb.ks[1] + k0 * pb.ks[2];
      const T* vbase = v + b * pb.vs[0] + kvh * pb.vs[1] + k0 * pb.vs[2];
      const float* brow =
          HAS_BIAS ? pb.bias + b * pb.bs[0] + hq * pb.bs[1] + i * pb.bs[2] + k0 * pb.bs[3] : nullptr;

      bool has = false;        // "no legal key yet" (Algorithm 33.1)
      float m2 = 0.0f;         // running max, base-2 domain, valid iff has
      float l_lane = 0.0f;     // this lane's share of l
      float acc[kAcc] = {0.0f, 0.0f, 0.0f, 0.0f};
      int32_t count = 0;

      for (int64_t kb = lo; kb < hi; kb += 64) {
        const int64_t j = kb + lane;
        bool legal = j < hi;
        float z2 = 0.0f;
        if (legal) {
          const T* krow = kbase + j * pb.ks[2];
          // GEN_ILP independent partial sums, so consecutive loads of the key
          // row are in flight together instead of one per fma latency.
          float dotp[GEN_ILP];
#pragma unroll
          for (int e = 0; e < GEN_ILP; ++e) dotp[e] = 0.0f;
          int d = 0;
          for (; d + GEN_ILP <= pb.d_h; d += GEN_ILP) {
#pragma unroll
            for (int e = 0; e < GEN_ILP; ++e) dotp[e] = fmaf(sq[wave][d + e], Elem<T>::load(krow, d + e), dotp[e]);
          }
          for (; d < pb.d_h; ++d) dotp[0] = fmaf(sq[wave][d], Elem<T>::load(krow, d), dotp[0]);
          float dot = 0.0f;
#pragma unroll
          for (int e = 0; e < GEN_ILP; ++e) dot += dotp[e];
          z2 = dot * pb.scale_log2;
          if (HAS_BIAS) {
            const float mb = brow[j * pb.bs[3]];
            if (mb == -INFINITY) legal = false;
            else z2 = fmaf(mb, kLog2e, z2);
          }
        }
        const uint64_t ballot = __ballot(legal);
        if (ballot == 0) continue;            // fully masked block: no stats
        if (COUNT) count += __popcll(ballot);
        const float bm = wave_max(legal ? z2 : -INFINITY);
        if (!has) {
          has = true;
          m2 = bm;
        } else if (bm > m2) {                  // merge (eqs 33.4-33.5)
          const float alpha = fast_exp2(m2 - bm);
          l_lane *= alpha;
#pragma unroll
          for (int t = 0; t < kAcc; ++t) acc[t] *= alpha;
          m2 = bm;
        }
        const float p = legal ? fast_exp2(z2 - m2) : 0.0f;
        l_lane += p;
        const int nj = (hi - kb) < 64 ? static_cast<int>(hi - kb) : 64;
#pragma unroll GEN_PV_UNROLL
        for (int jj = 0; jj < nj; ++jj) {
          const float pj = __shfl(p, jj, 64);
          const T* vrow = vbase + (kb + jj) * pb.vs[2];
#pragma unroll
          for (int t = 0; t < kAcc; ++t) {
            const int dv = lane + 64 * t;
            if (dv < pb.d_v) acc[t] = fmaf(pj, Elem<T>::load(vrow, dv), acc[t]);
          }
        }
      }

      const float l = wave_sum(l_lane);
      const int64_t row = (b * pb.heads_q + hq) * pb.t_q + i;
      float inv = 0.0f, lse_val = -INFINITY;
      if (has) {
        inv = 1.0f / l;
        lse_val = (m2 + fast_log2(l)) * kLn2;
      }
      if (SPLIT) {
        float* wo = ws_o + (row * n_splits + s) * pb.d_v;
#pragma unroll
        for (int t = 0; t < kAcc; ++t) {
          const int dv = lane + 64 * t;
          if (dv < pb.d_v) wo[dv] = has ? acc[t] * inv : 0.0f;
        }
        if (lane == 0) ws_lse[row * n_splits + s] = lse_val;
      } else {
        T* orow = o + b * pb.os[0] + hq * pb.os[1] + i * pb.os[2];
#pragma unroll
        for (int t = 0; t < kAcc; ++t) {
          const int dv = lane + 64 * t;
          if (dv < pb.d_v) Elem<T>::store(orow, dv, has ? acc[t] * inv : 0.0f);
        }
        if (lane == 0) {
          lse[row] = lse_val;
          if (COUNT) n_legal[row] = count;
        }
      }
    }
    __syncthreads();  // sq is rewritten by the next block of the loop
  }
}

template <typename T, bool HAS_BIAS, bool SPLIT, bool COUNT>
hipError_t launch_t(const Problem& pb, const void* q, const void* k,
                    const void* v, void* o, float* lse, int32_t* n_legal,
                    int64_t split_size, int64_t n_splits, float* ws_o,
                    float* ws_lse, hipStream_t stream) {
  const int64_t row_blocks = (pb.t_q + kWaves - 1) / kWaves;
  const int64_t total = row_blocks * n_splits * pb.heads_q * pb.batch;
  if (total == 0) return hipSuccess;
  const int64_t grid = total < (1ll << 30) ? total : (1ll << 30);
  hipLaunchKernelGGL((generic_kernel<T, HAS_BIAS, SPLIT, COUNT>), dim3(static_cast<unsigned>(grid)),
                     dim3(256), 0, stream, pb, static_cast<const T*>(q),
                     static_cast<const T*>(k), static_cast<const T*>(v),
                     static_cast<T*>(o), lse, n_legal, split_size, n_splits,
                     row_blocks, total, ws_o, ws_lse);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch_t(const Problem& pb, const void* q, const void* k,
                      const void* v, void* o, float* lse, int32_t* n_legal,
                      int64_t split_size, float* ws_o, float* ws_lse,
                      hipStream_t stream) {
  const bool bias = pb.bias != nullptr;
  if (ws_o != nullptr) {
    const int64_t n_splits = pb.t_k > 0 ? pb.t_k / split_size + (pb.t_k % split_size != 0) : 1;
    if (bias)
      return launch_t<T, true, true, false>(pb, q, k, v, o, lse, nullptr, split_size, n_splits, ws_o, ws_lse, stream);
    return launch_t<T, false, true, false>(pb, q, k, v, o, lse, nullptr, split_size, n_splits, ws_o, ws_lse, stream);
  }
  const int64_t whole = pb.t_k > 0 ? pb.t_k : 1;
  if (bias) {
    if (n_legal) return launch_t<T, true, false, true>(pb, q, k, v, o, lse, n_legal, whole, 1, nullptr, nullptr, stream);
    return launch_t<T, true, false, false>(pb, q, k, v, o, lse, nullptr, whole, 1, nullptr, nullptr, stream);
  }
  if (n_legal) return launch_t<T, false, false, true>(pb, q, k, v, o, lse, n_legal, whole, 1, nullptr, nullptr, stream);
  return launch_t<T, false, false, false>(pb, q, k, v, o, lse, nullptr, whole, 1, nullptr, nullptr, stream);
}

}  // namespace

hipError_t launch_generic(const Problem& pb, int dtype, const void* q,
                          const void* k, const void* v, void* o, float* lse,
                          int32_t* n_legal, int64_t split_size, float* ws_o,
                          float* ws_lse, hipStream_t stream) {
  if (dtype == ATTN_F32)
    return dispatch_t<float>(pb, q, k, v, o, lse, n_legal, split_size, ws_o, ws_lse, stream);
  return dispatch_t<uint16_t>(pb, q, k, v, o, lse, n_legal, split_size, ws_o, ws_lse, stream);
}

}  // namespace attn
