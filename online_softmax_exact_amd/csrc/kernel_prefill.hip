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

template <int DH, int DV, bool BIAS, bool COUNT>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(Args a) {
  using C = Cfg<DH, DV>;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::BUF];

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

  // Keys this workgroup may need: [0, k_end).
  int64_t k_end = a.t_k;
  if (a.causal) {
    int64_t last = a.q_offset + static_cast<int64_t>(qt) * kBr + kBr - 1;
    if (last + 1 < k_end) k_end = last + 1;
  }
  const int n_tiles = k_end > 0 ? static_cast<int>((k_end + kBc - 1) / kBc) : 0;

  const uint16_t* kbase = a.k + b * a.ks[0] + kvh * a.ks[1];
  const uint16_t* vbase = a.v + b * a.vs[0] + kvh * a.vs[1];

  // Per-row running statistics.
  bool has = false;        // a legal key has been seen (Algorithm 33.1)
  float m2 = 0.0f;         // reference maximum, base-2 units (valid iff has)
  float l_lane = 0.0f;     // this lane's share of l
  int32_t count = 0;
  f32x16 oacc[C::MO];
#pragma unroll
  for (int i = 0; i < C::MO; ++i) oacc[i] = f32x16{};

  // ---- global -> register prefetch of one tile, register -> LDS store ----
  u32x4 kpre[C::K_PER_T], vpre[C::V_PER_T];
  auto load_tile = [&](int t) {
    const int kb = t * kBc;
#pragma unroll
    for (int i = 0; i < C::K_PER_T; ++i) {
      const int c = tid + i * kThreads;
      const int r = c / (DH / 8), col = c % (DH / 8);
      const int key = kb + r;
      kpre[i] = key < a.t_k ? *reinterpret_cast<const u32x4*>(kbase + static_cast<int64_t>(key) * a.ks[2] + col * 8)
                            : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < C::V_PER_T; ++i) {
      const int c = tid + i * kThreads;
      const int r = c / (DV / 8), col = c % (DV / 8);
      const int key = kb + r;
      vpre[i] = key < a.t_k ? *reinterpret_cast<const u32x4*>(vbase + static_cast<int64_t>(key) * a.vs[2] + col * 8)
                            : u32x4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&](int buf) {
    char* kl = smem + buf * C::BUF;
    char* vl = kl + C::K_BYTES;
#pragma unroll
    for (int i = 0; i < C::K_PER_T; ++i) {
      const int c = tid + i * kThreads;
      const int r = c / (DH / 8), col = c % (DH / 8);
      *reinterpret_cast<u32x4*>(kl + r * C::K_STRIDE + col * 16) = kpre[i];
    }
#pragma unroll
    for (int i = 0; i < C::V_PER_T; ++i) {
      const int c = tid + i * kThreads;
      const int r = c / (DV / 8), col = c % (DV / 8);
      *reinterpret_cast<u32x4*>(vl + r * C::V_STRIDE + col * 16) = vpre[i];
    }
  };

  const float* brow = nullptr;
  if (BIAS) brow = a.bias + b * a.bs[0] + hq * a.bs[1] + static_cast<int64_t>(row) * a.bs[2];
  const int64_t pos_row = a.q_offset + row;                  // this lane's position
  const int64_t pos_w_first = a.q_offset + row0;             // first row of the wave
  const int64_t pos_w_last = a.q_offset + row0 + 31;         // last row of the wave

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int kb = t * kBc;
    if (t + 1 < n_tiles) load_tile(t + 1);

    // Classify the tile for this wave.
    int kind = kPartial;
    if (row0 >= a.t_q || (a.causal && kb > pos_w_last)) kind = kSkip;
    else if (!BIAS && kb + kBc <= a.t_k && (!a.causal || kb + kBc - 1 <= pos_w_first)) kind = kFull;

    if (kind != kSkip) {
      const char* kl = smem + (t & 1) * C::BUF;
      const lds_char* vl = (const lds_char*)(smem + (t & 1) * C::BUF + C::K_BYTES);

      // S^T for the two 32-key halves of the tile.
      f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
      for (int s = 0; s < C::KS; ++s) {
        const u32x4 k0 = *reinterpret_cast<const u32x4*>(kl + lr * C::K_STRIDE + 32 * s + 16 * h);
        const u32x4 k1 = *reinterpret_cast<const u32x4*>(kl + (32 + lr) * C::K_STRIDE + 32 * s + 16 * h);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(k0), as_bf16x8(qreg[s]), s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(k1), as_bf16x8(qreg[s]), s1, 0, 0, 0);
      }

      // Register r of half mt holds key kb + 32 mt + 8 (r / 4) + 4 h + (r % 4).
      float tmax;
      if (kind == kFull) {
        float mx = s0[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s0[r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s1[r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        tmax = mx * a.scale_log2;
        if (COUNT) count += 32;
      } else {
        // Legal iff key < T_k, causally visible, and bias != -inf.
        int64_t lim64 = a.causal ? pos_row - kb : int64_t(kBc);
        const int64_t kmax = a.t_k - kb;   // keys at relative index >= kmax do not exist
        if (kmax - 1 < lim64) lim64 = kmax - 1;
        int lim = lim64 < -1 ? -1 : (lim64 > kBc ? kBc : static_cast<int>(lim64));
        if (!row_ok) lim = -1;   // rows past T_q: nothing legal, no bias read
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j0 = 8 * (r >> 2) + 4 * h + (r & 3);
          const int j1 = 32 + j0;
          float z0 = s0[r] * a.scale_log2, z1 = s1[r] * a.scale_log2;
          bool ok0 = j0 <= lim, ok1 = j1 <= lim;
          if (BIAS) {
            if (ok0) {
              const float m = brow[static_cast<int64_t>(kb + j0) * a.bs[3]];
              ok0 = m != -INFINITY;
              z0 = fmaf(m, kLog2e, z0);
            }
            if (ok1) {
              const float m = brow[static_cast<int64_t>(kb + j1) * a.bs[3]];
              ok1 = m != -INFINITY;
              z1 = fmaf(m, kLog2e, z1);
            }
          }
          if (COUNT) count += static_cast<int>(ok0) + static_cast<int>(ok1);
          s0[r] = ok0 ? z0 : -INFINITY;
          s1[r] = ok1 ? z1 : -INFINITY;
          mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        tmax = mx;
      }

      // Update the running reference maximum (lazy) and rescale if it moved.
      const bool tile_has = tmax != -INFINITY;
      bool need = false;
      if (tile_has) {
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
        float p0[16], p1[16];
        if (kind == kFull) {
          const float nm = -m2;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            p0[r] = fast_exp2(fmaf(s0[r], a.scale_log2, nm));
            p1[r] = fast_exp2(fmaf(s1[r], a.scale_log2, nm));
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            p0[r] = fast_exp2(s0[r] - m2);
            p1[r] = fast_exp2(s1[r] - m2);
          }
        }
        float ls0 = 0.0f, ls1 = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          ls0 += p0[r];
          ls1 += p1[r];
        }
        l_lane += ls0 + ls1;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          pk0[i] = pack_bf16(p0[2 * i], p0[2 * i + 1]);
          pk1[i] = pack_bf16(p1[2 * i], p1[2 * i + 1]);
        }
      }

      // O^T += V^T P^T over four 16-key steps.
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
    }

    if (t + 1 < n_tiles) store_tile((t + 1) & 1);
    __syncthreads();
  }

  // ---- finalise: o = u / l, LSE = m + ln l; rows with no legal key -> (+0, -inf) ----
  const float l_row = l_lane + __shfl_xor(l_lane, 32, 64);
  if (COUNT) count += __shfl_xor(count, 32, 64);
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
