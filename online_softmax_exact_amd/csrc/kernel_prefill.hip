// MFMA prefill kernel for bf16 Q/K/V/O, d_h and d_v in {64, 128}.
//
// What it computes: for every query row, Algorithm 33.1 of "Chapter 33
// 推理计算优化" §33.2 over key tiles of 64, i.e. exact softmax attention
// (eq 33.2) with the running statistics (m, l, u) of eq 33.3 merged tile by
// tile (eqs 33.4-33.5).  Tiles that no row of a wave can see are skipped and
// tiles that every row sees in full need no mask (§33.3, causal block
// skipping); every legal key of every row is processed.
//
// Mapping onto CDNA4 (gfx950):
// * A workgroup of 4 wavefronts owns 128 consecutive query rows of one
//   (batch, head); wavefront w owns rows 32w..32w+31.
// * Scores are computed transposed, S^T = K Q^T, with
//   v_mfma_f32_32x32x16_bf16: A = a 32-key slice of the K tile (read from LDS
//   with 16-byte reads), B = Q^T kept in registers for the whole kernel.  In
//   the result each lane holds 16 scores of ONE query row (lane % 32), so the
//   row maximum is an in-lane reduction plus one exchange with lane ^ 32.
// * P^T (bf16) stays in the same registers and is the B operand of
//   O^T = V^T P^T; the A operand V^T is read from a row-major V tile in LDS
//   with ds_read_b64_tr_b16, which hands each lane 4 keys of one value column.
//   The key order inside a 16-key MFMA step is the order in which the score
//   registers hold them; any order is valid for a contraction as long as both
//   operands agree.
// * K/V tiles are double-buffered in LDS: global loads of tile t + 1 are in
//   flight while tile t is computed.  Row strides are padded so that the
//   16-byte K reads and the transposed V reads are free of bank conflicts.
// * Rescaling is lazy: the reference maximum m of a row only moves when a
//   tile's maximum exceeds it by more than 8 (base-2 units); the merge rule
//   holds for any reference value, so o = u / l is unchanged, and the weights
//   stay below 2^8.
// * Scores live in the base-2 domain: p = exp2(dot * scale * log2(e) - m2) on
//   v_exp_f32; LSE is converted back to natural-log units at the end.
#include "attn_internal.h"
#include "kernels.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kBc = 64;            // keys per tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBr = 32 * kWaves;   // query rows per workgroup
constexpr float kRescale = 8.0f;   // lazy-rescale threshold, base-2 units
#ifndef PREFILL_WAVES_PER_SIMD
#define PREFILL_WAVES_PER_SIMD 2       // resident waves per SIMD the kernel is built for
#endif

template <int DH, int DV>
struct Cfg {
  static constexpr int KS = DH / 16;             // k-steps of K Q^T
  static constexpr int MO = DV / 32;             // 32-row slices of O^T
  static constexpr int K_STRIDE = DH * 2 + 16;   // bytes per K row in LDS
  static constexpr int V_STRIDE = DV * 2 + 64;   // bytes per V row in LDS
  static constexpr int K_BYTES = kBc * K_STRIDE;
  static constexpr int V_BYTES = kBc * V_STRIDE;
  static constexpr int BUF = K_BYTES + V_BYTES;
  static constexpr int K_CHUNKS = kBc * DH / 8;  // 16-byte chunks per tile
  static constexpr int V_CHUNKS = kBc * DV / 8;
  static constexpr int K_PER_T = K_CHUNKS / kThreads;
  static constexpr int V_PER_T = V_CHUNKS / kThreads;
};

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
  int32_t t_q, t_k, heads_q, group, n_qtiles, batch_heads;
  float scale_log2;
  int32_t causal;
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ u32x2 tr_read(const lds_char* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Tile classification for one wavefront.
enum : int { kSkip = 0, kFull = 1, kPartial = 2 };

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

template <int DH, int DV, bool BIAS, bool COUNT>
__global__ __launch_bounds__(kThreads, PREFILL_WAVES_PER_SIMD) void prefill_kernel(Args a) {
  using C = Cfg<DH, DV>;
  // K ring of two tiles, then V ring of two tiles.  K runs one tile ahead of
  // V: while tile t's softmax and P V run, tile t + 1's scores are computed.
  __shared__ __attribute__((aligned(16))) char smem[2 * C::K_BYTES + 2 * C::V_BYTES];
  char* const kring = smem;
  char* const vring = smem + 2 * C::K_BYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;        // which half of the wave
  const int lr = lane & 31;       // this lane's query row within the wave

  // Heaviest query tiles first (with causal masking, later tiles see more keys).
  const int bid = blockIdx.x;
  const int qt = a.n_qtiles - 1 - bid / a.batch_heads;
  const int bh = bid % a.batch_heads;
  const int b = bh / a.heads_q;
  const int hq = bh % a.heads_q;
  const int kvh = hq / a.group;

  const int row0 = qt * kBr + wave * 32;   // first row of this wave
  const int row = row0 + lr;               // this lane's row
  const bool row_ok = row < a.t_q;

  // Q^T operand: lane holds Q[row][16 ks + 8 h .. + 7] for every k-step.
  u32x4 qreg[C::KS];
  {
    const uint16_t* qp = a.q + b * a.qs[0] + hq * a.qs[1] + static_cast<int64_t>(row) * a.qs[2];
#pragma unroll
    for (int s = 0; s < C::KS; ++s)
      qreg[s] = row_ok ? *reinterpret_cast<const u32x4*>(qp + 16 * s + 8 * h) : u32x4{0, 0, 0, 0};
  }

  // Positions clamped to [-1, T_k]: every value >= T_k - 1 sees all keys.
  auto clamp_pos = [&](int64_t p) -> int {
    return p < -1 ? -1 : (p > a.t_k ? a.t_k : static_cast<int>(p));
  };
  const int pos_row = clamp_pos(a.q_offset + row);          // this lane's position
  const int pos_w_first = clamp_pos(a.q_offset + row0);     // first row of the wave
  const int pos_w_last = clamp_pos(a.q_offset + row0 + 31); // last row of the wave

  // Tiles the workgroup streams: keys [0, k_end).  Tiles the wave computes:
  // the first n_w of them (every later one is above the wave's diagonal).
  // Tiles t < t_full need no mask for any row of the wave.
  const int wg_last = clamp_pos(a.q_offset + static_cast<int64_t>(qt) * kBr + kBr - 1);
  const int k_end = a.causal ? (wg_last + 1 < a.t_k ? wg_last + 1 : a.t_k) : a.t_k;
  const int n_tiles = k_end > 0 ? (k_end + kBc - 1) / kBc : 0;
  int n_w = n_tiles;
  if (row0 >= a.t_q) {
    n_w = 0;
  } else if (a.causal) {
    const int last = pos_w_last < a.t_k - 1 ? pos_w_last : a.t_k - 1;
    const int tw = last < 0 ? 0 : last / kBc + 1;
    if (tw < n_w) n_w = tw;
  }
  int t_full = a.t_k / kBc;
  if (a.causal) {
    const int tf = (pos_w_first + 1) / kBc;   // pos_w_first >= -1
    if (tf < t_full) t_full = tf;
  }
  if (BIAS) t_full = 0;

  const uint16_t* kbase = a.k + b * a.ks[0] + kvh * a.ks[1];
  const uint16_t* vbase = a.v + b * a.vs[0] + kvh * a.vs[1];
  const int k_row_bytes = static_cast<int>(a.ks[2]) * 2;
  const int v_row_bytes = static_cast<int>(a.vs[2]) * 2;
  // Per-wave bias window for 16-byte loads: rows row0 .. last valid row of the
  // wave, keys [0, T_k) of the last one; lane offset = its row + its keys.
  const float* bias_w = nullptr;
  int64_t bias_w_bytes = 0;
  int bias_off = 0;
  if (BIAS) {
    bias_w = a.bias + b * a.bs[0] + hq * a.bs[1] + static_cast<int64_t>(row0) * a.bs[2];
    const int rows_w = a.t_q - row0 < 32 ? a.t_q - row0 : 32;
    bias_w_bytes = rows_w > 0 ? (static_cast<int64_t>(rows_w - 1) * a.bs[2] + a.t_k) * 4 : 0;
    bias_off = row_ok ? static_cast<int>(lr * a.bs[2] * 4) + 16 * h : 0;
  }

  // Per-row running statistics.
  bool has = false;        // a legal key has been seen (Algorithm 33.1)
  float m2 = 0.0f;         // reference maximum, base-2 units (valid iff has)
  float l_lane = 0.0f;     // this lane's share of l
  int32_t count = 0;
  f32x16 oacc[C::MO];
#pragma unroll
  for (int i = 0; i < C::MO; ++i) oacc[i] = f32x16{};

  // ---- tile movement: HBM -> registers (buffer loads) -> LDS ----
  // Thread tid moves 16-byte chunks c = tid + i * kThreads of a tile: row
  // c / (D / 8), column chunk c % (D / 8).  Rows past T_k read as zeros.
  u32x4 kpre[C::K_PER_T], vpre[C::V_PER_T];
  // Chunk i of this thread lies kThreads / (D / 8) rows below chunk i - 1:
  // one offset register per thread, the row step goes into the descriptor.
  const int koff = (tid / (DH / 8)) * k_row_bytes + (tid % (DH / 8)) * 16;
  const int voff = (tid / (DV / 8)) * v_row_bytes + (tid % (DV / 8)) * 16;
  constexpr int K_ROWS_PER_I = kThreads / (DH / 8);
  constexpr int V_ROWS_PER_I = kThreads / (DV / 8);
  auto gload_k = [&](int t) {
#pragma unroll
    for (int i = 0; i < C::K_PER_T; ++i) {
      const int r0i = t * kBc + i * K_ROWS_PER_I;
      const auto rs = make_rsrc(reinterpret_cast<const char*>(kbase) + static_cast<int64_t>(r0i) * k_row_bytes,
                                static_cast<int64_t>(a.t_k - r0i) * k_row_bytes);
      kpre[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, koff, 0, 0);
    }
  };
  auto gload_v = [&](int t) {
#pragma unroll
    for (int i = 0; i < C::V_PER_T; ++i) {
      const int r0i = t * kBc + i * V_ROWS_PER_I;
      const auto rs = make_rsrc(reinterpret_cast<const char*>(vbase) + static_cast<int64_t>(r0i) * v_row_bytes,
                                static_cast<int64_t>(a.t_k - r0i) * v_row_bytes);
      vpre[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, 0);
    }
  };
  auto sstore_k = [&](int slot) {
    char* kl = kring + slot * C::K_BYTES;
#pragma unroll
    for (int i = 0; i < C::K_PER_T; ++i) {
      const int c = tid + i * kThreads;
      const int r = c / (DH / 8), col = c % (DH / 8);
      *reinterpret_cast<u32x4*>(kl + r * C::K_STRIDE + col * 16) = kpre[i];
    }
  };
  auto sstore_v = [&](int slot) {
    char* vl = vring + slot * C::V_BYTES;
#pragma unroll
    for (int i = 0; i < C::V_PER_T; ++i) {
      const int c = tid + i * kThreads;
      const int r = c / (DV / 8), col = c % (DV / 8);
      *reinterpret_cast<u32x4*>(vl + r * C::V_STRIDE + col * 16) = vpre[i];
    }
  };

  // S^T of the K tile in `slot` for the two 32-key halves.
  auto scores = [&](int slot, f32x16& s0, f32x16& s1) {
    const char* kl = kring + slot * C::K_BYTES;
    s0 = f32x16{};
    s1 = f32x16{};
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      const u32x4 k0 = *reinterpret_cast<const u32x4*>(kl + lr * C::K_STRIDE + 32 * s + 16 * h);
      const u32x4 k1 = *reinterpret_cast<const u32x4*>(kl + (32 + lr) * C::K_STRIDE + 32 * s + 16 * h);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(k0), as_bf16x8(qreg[s]), s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(k1), as_bf16x8(qreg[s]), s1, 0, 0, 0);
    }
  };

  // Softmax statistics of tile t and O^T += V^T P^T.
  auto softmax_pv = [&](int t, f32x16& s0, f32x16& s1) {
    const int kb = t * kBc;
    const bool full = t < t_full;
    // Register r of half mt holds key kb + 32 mt + 8 (r / 4) + 4 h + (r % 4).
    float tmax;
    if (full) {
      float mx = fmaxf(s0[0], s0[1]);
#pragma unroll
      for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s0[r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s1[r]);
      tmax = max_xor32(mx) * a.scale_log2;
      if (COUNT) count += 32;
    } else {
      // Legal iff key < T_k, causally visible, and bias != -inf.
      int lim = a.causal ? pos_row - kb : kBc;
      if (a.t_k - 1 - kb < lim) lim = a.t_k - 1 - kb;   // keys past T_k do not exist
      if (lim < -1) lim = -1;
      if (!row_ok) lim = -1;   // rows past T_q: nothing legal, no bias read
      // Bias of this lane's row for its 32 keys (contiguous along keys):
      // 16-byte loads of the 4 consecutive keys each register group holds.
      float mb0[16], mb1[16];
      if (BIAS) {
        const auto rs = make_rsrc(bias_w + kb, bias_w_bytes - static_cast<int64_t>(kb) * 4);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 x0 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, bias_off + 32 * g, 0, 0));
          const f32x4 x1 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, bias_off + 128 + 32 * g, 0, 0));
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            mb0[4 * g + e] = x0[e];
            mb1[4 * g + e] = x1[e];
          }
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j0 = 8 * (r >> 2) + 4 * h + (r & 3);
        const int j1 = 32 + j0;
        float z0 = s0[r] * a.scale_log2, z1 = s1[r] * a.scale_log2;
        bool ok0 = j0 <= lim, ok1 = j1 <= lim;
        if (BIAS) {
          ok0 = ok0 && mb0[r] != -INFINITY;
          ok1 = ok1 && mb1[r] != -INFINITY;
          z0 = fmaf(mb0[r], kLog2e, z0);
          z1 = fmaf(mb1[r], kLog2e, z1);
        }
        if (COUNT) count += static_cast<int>(ok0) + static_cast<int>(ok1);
        s0[r] = ok0 ? z0 : -INFINITY;
        s1[r] = ok1 ? z1 : -INFINITY;
        mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
      }
      tmax = max_xor32(mx);
    }

    // Update the running reference maximum (lazy) and rescale if it moved.
    bool need = false;
    if (tmax != -INFINITY) {
      if (!has) {
        has = true;
        m2 = tmax;
      } else if (tmax > m2 + kRescale) {
        need = true;
      }
    }
    if (__ballot(need) != 0) {
      const float alpha = need ? fast_exp2(m2 - tmax) : 1.0f;
      if (need) m2 = tmax;
      l_lane *= alpha;
#pragma unroll
      for (int i = 0; i < C::MO; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
    }

    // P = exp2(z - m2); illegal entries hold -inf and give 0.  l sums the
    // fp32 weights (the LSE keeps fp32 accuracy); V is multiplied by their
    // bf16 roundings.
    unsigned pk0[8], pk1[8];
    {
      if (full) {
        const float nm = -m2;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s0[r] = fast_exp2(fmaf(s0[r], a.scale_log2, nm));
          s1[r] = fast_exp2(fmaf(s1[r], a.scale_log2, nm));
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s0[r] = fast_exp2(s0[r] - m2);
          s1[r] = fast_exp2(s1[r] - m2);
        }
      }
      float ps[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) ps[r] = s0[r] + s1[r];
#pragma unroll
      for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
        for (int r = 0; r < w; ++r) ps[r] += ps[r + w];
      l_lane += ps[0];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pk0[i] = pack_bf16(s0[2 * i], s0[2 * i + 1]);
        pk1[i] = pack_bf16(s1[2 * i], s1[2 * i + 1]);
      }
    }

    // O^T += V^T P^T over four 16-key steps.
    const lds_char* vl = (const lds_char*)(vring + (t & 1) * C::V_BYTES);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const unsigned* pk = (kk < 2) ? pk0 : pk1;
      const int off = 4 * (kk & 1);
      const u32x4 bop = {pk[off], pk[off + 1], pk[off + 2], pk[off + 3]};
      // Keys of this step for this lane: base + (0..3) and base + 8 + (0..3).
      const int key_base = 32 * (kk >> 1) + 16 * (kk & 1) + 4 * h;
      const int src_row = key_base + ((lane & 15) >> 2);
#pragma unroll
      for (int mo = 0; mo < C::MO; ++mo) {
        const int col = 32 * mo + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        const lds_char* p0 = vl + src_row * C::V_STRIDE + col * 2;
        const u32x2 lo = tr_read(p0);
        const u32x2 hi = tr_read(p0 + 8 * C::V_STRIDE);
        const u32x4 aop = {lo[0], lo[1], hi[0], hi[1]};
        oacc[mo] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(aop), as_bf16x8(bop), oacc[mo], 0, 0, 0);
      }
    }
  };

  // One pipeline step: scores of tile t + 1 (into sn) are issued before the
  // softmax and P V of tile t (in sc), so the MFMAs run while the VALU works;
  // then the tiles for the next step are stored to LDS and the global loads
  // two tiles ahead are issued.
  // With a bias the extra score registers do not fit: tile t's scores are
  // then computed right before its softmax, and K runs one tile ahead (like
  // V) instead of two.  Ring slots: K(t) and V(t) live in slot t & 1; a slot
  // is only rewritten after the barrier that follows its last reader.
  constexpr bool kPipe = !BIAS;
  constexpr int kAhead = kPipe ? 2 : 1;     // K tiles held in LDS beyond the current one
  auto step = [&](int t, f32x16& sc0, f32x16& sc1, f32x16& sn0, f32x16& sn1) {
    if (kPipe) {
      if (t + 1 < n_w) scores((t + 1) & 1, sn0, sn1);
    } else {
      if (t < n_w) scores(t & 1, sc0, sc1);
    }
    if (t < n_w) softmax_pv(t, sc0, sc1);
    // kPipe: K(t + 2) replaces K(t), read in the previous step.
    // otherwise: K(t + 1) replaces K(t - 1).  V(t + 1) replaces V(t - 1).
    if (t + kAhead < n_tiles) sstore_k((t + kAhead) & 1);
    if (t + 1 < n_tiles) sstore_v((t + 1) & 1);
    __syncthreads();
    if (t + kAhead + 1 < n_tiles) gload_k(t + kAhead + 1);
    if (t + 2 < n_tiles) gload_v(t + 2);
  };

  // Prologue: K(0 .. kAhead - 1) and V(0) in LDS; K(kAhead), V(1) in flight;
  // with the prefetch, the scores of tile 0.
  if (n_tiles > 0) {
    gload_k(0);
    sstore_k(0);
    gload_v(0);
    sstore_v(0);
  }
  if (kPipe && n_tiles > 1) {
    gload_k(1);
    sstore_k(1);
  }
  __syncthreads();
  if (n_tiles > kAhead) gload_k(kAhead);
  if (n_tiles > 1) gload_v(1);
  f32x16 sa0 = f32x16{}, sa1 = f32x16{}, sb0 = f32x16{}, sb1 = f32x16{};
  if (kPipe && n_w > 0) scores(0, sa0, sa1);
  __syncthreads();   // with the prefetch, K slot 0 is rewritten in step 0

  int t = 0;
  for (; t + 1 < n_tiles; t += 2) {
    step(t, sa0, sa1, sb0, sb1);
    step(t + 1, sb0, sb1, sa0, sa1);
  }
  if (t < n_tiles) step(t, sa0, sa1, sb0, sb1);

  // ---- finalise: o = u / l, LSE = m + ln l; rows with no legal key -> (+0, -inf) ----
  const float l_row = sum_xor32(l_lane);
  if (COUNT) count = isum_xor32(count);
  if (!row_ok) return;
  const float inv = has ? 1.0f / l_row : 0.0f;
  uint16_t* op = a.o + b * a.os[0] + hq * a.os[1] + static_cast<int64_t>(row) * a.os[2];
#pragma unroll
  for (int mo = 0; mo < C::MO; ++mo) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dv = 32 * mo + 8 * g + 4 * h;
      u32x2 w;
      w[0] = pack_bf16(oacc[mo][4 * g] * inv, oacc[mo][4 * g + 1] * inv);
      w[1] = pack_bf16(oacc[mo][4 * g + 2] * inv, oacc[mo][4 * g + 3] * inv);
      *reinterpret_cast<u32x2*>(op + dv) = w;
    }
  }
  if (h == 0) {
    const int64_t ridx = (static_cast<int64_t>(b) * a.heads_q + hq) * a.t_q + row;
    a.lse[ridx] = has ? (m2 + fast_log2(l_row)) * kLn2 : -INFINITY;
    if (COUNT) a.n_legal[ridx] = count;
  }
}

template <int DH, int DV, bool BIAS, bool COUNT>
hipError_t launch_cfg(const Args& a, int64_t blocks, hipStream_t stream) {
  hipLaunchKernelGGL((prefill_kernel<DH, DV, BIAS, COUNT>), dim3(static_cast<unsigned>(blocks)),
                     dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int DH, int DV>
hipError_t launch_dims(const Args& a, int64_t blocks, bool bias, bool count, hipStream_t s) {
  if (bias) return count ? launch_cfg<DH, DV, true, true>(a, blocks, s) : launch_cfg<DH, DV, true, false>(a, blocks, s);
  return count ? launch_cfg<DH, DV, false, true>(a, blocks, s) : launch_cfg<DH, DV, false, false>(a, blocks, s);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

// Takes bf16 problems with d_h, d_v in {64, 128}, positive scale, 16-byte
// aligned rows and sizes that fit 32-bit row/key indices.
bool launch_prefill_mfma(const Problem& pb, int dtype, const void* q, const void* k,
                         const void* v, void* o, float* lse, int32_t* n_legal,
                         hipStream_t stream, int* status) {
  if (dtype != ATTN_BF16) return false;
  if (!((pb.d_h == 64 || pb.d_h == 128) && (pb.d_v == 64 || pb.d_v == 128))) return false;
  if (!(pb.scale_log2 > 0.0f)) return false;
  if (pb.t_q >= (int64_t(1) << 30) || pb.t_k >= (int64_t(1) << 30)) return false;
  if (pb.ks[2] >= (int64_t(1) << 24) || pb.vs[2] >= (int64_t(1) << 24)) return false;  // tile < 2 GiB
  if (pb.bias != nullptr && (pb.bs[3] != 1 || pb.bs[2] * 32 >= (int64_t(1) << 28)))
    return false;   // bias must be contiguous along keys; window offsets fit 32 bits
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return false;
  for (int i = 0; i < 3; ++i)
    if ((pb.qs[i] | pb.ks[i] | pb.vs[i] | pb.os[i]) & 7) return false;
  const int64_t n_qtiles = (pb.t_q + kBr - 1) / kBr;
  const int64_t blocks = n_qtiles * pb.batch * pb.heads_q;
  if (blocks >= (int64_t(1) << 31) || pb.batch * pb.heads_q >= (int64_t(1) << 30)) return false;

  Args a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.n_legal = n_legal;
  a.bias = pb.bias;
  for (int i = 0; i < 3; ++i) {
    a.qs[i] = pb.qs[i]; a.ks[i] = pb.ks[i]; a.vs[i] = pb.vs[i]; a.os[i] = pb.os[i];
  }
  for (int i = 0; i < 4; ++i) a.bs[i] = pb.bs[i];
  a.q_offset = pb.q_offset;
  a.t_q = static_cast<int32_t>(pb.t_q);
  a.t_k = static_cast<int32_t>(pb.t_k);
  a.heads_q = static_cast<int32_t>(pb.heads_q);
  a.group = pb.group;
  a.n_qtiles = static_cast<int32_t>(n_qtiles);
  a.batch_heads = static_cast<int32_t>(pb.batch * pb.heads_q);
  a.scale_log2 = pb.scale_log2;
  a.causal = pb.causal;

  const bool bias = pb.bias != nullptr;
  const bool count = n_legal != nullptr;
  hipError_t e;
  if (pb.d_h == 128 && pb.d_v == 128) e = launch_dims<128, 128>(a, blocks, bias, count, stream);
  else if (pb.d_h == 64 && pb.d_v == 128) e = launch_dims<64, 128>(a, blocks, bias, count, stream);
  else if (pb.d_h == 128 && pb.d_v == 64) e = launch_dims<128, 64>(a, blocks, bias, count, stream);
  else e = launch_dims<64, 64>(a, blocks, bias, count, stream);
  *status = e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
  return true;
}

}  // namespace attn
