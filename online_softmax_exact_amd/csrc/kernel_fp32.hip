// MFMA prefill for fp32 Q/K/V/O, d_h and d_v in {64, 128}, with or without a
// bias and a sliding window, no variable lengths (the generic kernel serves
// the rest).
//
// What it computes: for every query row, Algorithm 33.1 of "Chapter 33
// 推理计算优化" §33.2 over key tiles of 32: exact softmax attention (eq 33.2)
// with the running statistics (m, l, u) of eq 33.3 merged tile by tile
// (eqs 33.4-33.5); a tile with no legal key for a row leaves its statistics
// unchanged and a row that never sees one is finalised as (+0, -inf).  Tiles
// past the last key any row of a wavefront can see are skipped (§33.3).
//
// Mapping onto CDNA4: the contractions run on the fp32 matrix cores
// (v_mfma_f32_32x32x2_f32, the same 157.3 TFLOP/s as the fp32 vector units but
// without their per-lane dot-product chains).  A workgroup of 4 wavefronts
// owns 128 query rows of one (batch, head); wavefront w owns rows 32w..32w+31.
// * S^T = K Q^T: step s multiplies keys x dims {2s, 2s+1}; lane l supplies
//   A = K[l % 32][2s + l / 32] from the LDS tile and B = Q[row][2s + l / 32]
//   from registers.  The result gives each lane 16 scores of one query row
//   (keys 8 (r / 4) + 4 (l / 32) + r % 4 in register r), so the row maximum is
//   an in-lane reduction plus one exchange with lane ^ 32.
// * O^T += V^T P^T: step s contracts the two keys that register s holds in
//   the two half-waves, so the B operand is the weight already in register s
//   and A = V[that key][32 mo + l % 32] comes from the LDS tile.
// * K rows in LDS are padded by one float so the 32 rows of a column read hit
//   32 different banks; V rows are read along columns, which is conflict-free.
// * Grids of fewer than FP32_SPLIT_BELOW such workgroups (the single-head
//   workload has one) take fp32_split_kernel instead: one workgroup per 32
//   rows whose wavefronts split the rows' key tiles and merge their states,
//   so the serial chain is a quarter of the tiles.
#include "attn_internal.h"
#include "kernels.h"

namespace attn {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32 * kWaves;   // query rows per workgroup
constexpr int kKeys = 32;            // keys per tile
#ifndef FP32_SPLIT_BELOW
#define FP32_SPLIT_BELOW 64          // grids below this many 128-row workgroups take fp32_split_kernel
#endif

struct F32Args {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  int32_t* n_legal;
  int64_t qs[3], ks[3], vs[3], os[3];
  int64_t q_offset;
  int64_t window;           // keys j >= q_offset + i - window + 1; 0 = none
  const float* bias;        // fp32 additive bias / mask, NULL = none
  int64_t bs[4];            // its element strides over b, hq, i, j
  int32_t t_q, t_k, heads_q, group, n_qtiles, batch_heads;
  float scale_log2;
  int32_t causal;
  int32_t split;            // 1: fp32_split_kernel (one workgroup per 32 rows, keys split over waves)
};

// Logical position clamped to [-1, T_k]: every value >= T_k - 1 sees all keys.
__device__ __forceinline__ int clamp_pos32(const F32Args& a, int64_t p) {
  return p < -1 ? -1 : (p > a.t_k ? a.t_k : static_cast<int>(p));
}

template <int DH, int DV, bool COUNT, bool BIAS>
__global__ __launch_bounds__(kThreads, 2) void fp32_prefill_kernel(F32Args a) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int KP = DH + 1;   // padded K row, in floats
  constexpr int MO = DV / 32;  // 32-row slices of O^T
  __shared__ float k_tile[kKeys * KP];
  __shared__ __attribute__((aligned(16))) float v_tile[kKeys * DV];
  debug_poison_lds(k_tile, sizeof(k_tile));
  debug_poison_lds(v_tile, sizeof(v_tile));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int lr = lane & 31;

  // Heaviest (latest, when causal) query tiles first.
  const int bid = blockIdx.x;
  const int qt = a.n_qtiles - 1 - bid / a.batch_heads;
  const int bh = bid % a.batch_heads;
  const int b = bh / a.heads_q;
  const int hq = bh % a.heads_q;
  const int kvh = hq / a.group;

  const int row0 = qt * kRows + wave * 32;
  const int row = row0 + lr;
  const bool row_ok = row < a.t_q;

  // Q^T operand of step s: Q[row][2 s + h].
  float qreg[DH / 2];
  {
    const float* qp = a.q + b * a.qs[0] + hq * a.qs[1] + static_cast<int64_t>(row) * a.qs[2];
#pragma unroll
    for (int s = 0; s < DH / 2; ++s) qreg[s] = row_ok ? qp[2 * s + h] : 0.0f;
  }

  // Keys the workgroup streams: [0, k_end); this wavefront computes the tiles
  // up to its last row's position.
  const int wg_last = (qt + 1) * kRows < a.t_q ? (qt + 1) * kRows - 1 : a.t_q - 1;
  const int pos_wg = clamp_pos32(a, a.q_offset + wg_last);
  const int k_end = a.causal ? (pos_wg + 1 < a.t_k ? pos_wg + 1 : a.t_k) : a.t_k;
  const int n_tiles = k_end > 0 ? (k_end + kKeys - 1) / kKeys : 0;
  const int w_last = row0 + 31 < a.t_q ? row0 + 31 : a.t_q - 1;
  const int pos_w = clamp_pos32(a, a.q_offset + w_last);
  int n_w = row0 < a.t_q ? n_tiles : 0;
  if (a.causal) {
    const int last = pos_w < a.t_k - 1 ? pos_w : a.t_k - 1;
    const int tw = last < 0 ? 0 : last / kKeys + 1;
    if (tw < n_w) n_w = tw;
  }
  const int pos_row = clamp_pos32(a, a.q_offset + row);
  // Sliding window: first key of this row, of the wavefront's first row and
  // of the workgroup's first row (clamped to [0, T_k]); tiles before the
  // workgroup's are never loaded, tiles before the wavefront's are skipped.
  auto win_lo = [&](int64_t r) -> int {
    if (a.window <= 0) return 0;
    const int64_t lo = a.q_offset + r - a.window + 1;
    return lo < 0 ? 0 : (lo > a.t_k ? a.t_k : static_cast<int>(lo));
  };
  const int lo_row = win_lo(row);
  const int lo_w = win_lo(row0);
  const int t_begin = win_lo(static_cast<int64_t>(qt) * kRows) / kKeys;
  const float* brow = nullptr;   // this row's bias
  if (BIAS && row_ok) brow = a.bias + b * a.bs[0] + hq * a.bs[1] + static_cast<int64_t>(row) * a.bs[2];

  const float* kbase = a.k + b * a.ks[0] + kvh * a.ks[1];
  const float* vbase = a.v + b * a.vs[0] + kvh * a.vs[1];

  bool has = false;        // a legal key has been seen (Algorithm 33.1)
  float m2 = 0.0f;         // running maximum, base-2 units (valid iff has)
  float l_lane = 0.0f;     // this lane's half of l
  int32_t count = 0;
  f32x16 oacc[MO];
#pragma unroll
  for (int i = 0; i < MO; ++i) oacc[i] = f32x16{};

  // Tile copies: thread tid moves 16-byte chunks c = tid + kThreads i of the
  // K tile (DH / 4 chunks per key) and of the V tile; consecutive threads take
  // consecutive chunks of a key row.  Tile t + 1 is loaded into registers
  // while tile t is computed; keys past T_k read as zero.
  constexpr int KN = kKeys * DH / 4 / kThreads;
  constexpr int VN = kKeys * DV / 4 / kThreads;
  f32x4 kpre[KN], vpre[VN];
  auto fetch = [&](int t) {
#pragma unroll
    for (int i = 0; i < KN; ++i) {
      const int c = tid + kThreads * i, key = t * kKeys + c / (DH / 4), d = 4 * (c % (DH / 4));
      kpre[i] = key < a.t_k ? *reinterpret_cast<const f32x4*>(kbase + static_cast<int64_t>(key) * a.ks[2] + d)
                            : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll
    for (int i = 0; i < VN; ++i) {
      const int c = tid + kThreads * i, key = t * kKeys + c / (DV / 4), d = 4 * (c % (DV / 4));
      vpre[i] = key < a.t_k ? *reinterpret_cast<const f32x4*>(vbase + static_cast<int64_t>(key) * a.vs[2] + d)
                            : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  };
  if (t_begin < n_tiles) fetch(t_begin);
  for (int t = t_begin; t < n_tiles; ++t) {
    __syncthreads();   // every wave is done reading tile t - 1
#pragma unroll
    for (int i = 0; i < KN; ++i) {
      const int c = tid + kThreads * i, kk = c / (DH / 4), d = 4 * (c % (DH / 4));
#pragma unroll
      for (int e = 0; e < 4; ++e) k_tile[kk * KP + d + e] = kpre[i][e];
    }
#pragma unroll
    for (int i = 0; i < VN; ++i) {
      const int c = tid + kThreads * i, kk = c / (DV / 4), d = 4 * (c % (DV / 4));
      *reinterpret_cast<f32x4*>(v_tile + kk * DV + d) = vpre[i];
    }
    __syncthreads();
    if (t + 1 < n_tiles) fetch(t + 1);
    const int key0 = t * kKeys;
    if (t >= n_w || key0 + kKeys <= lo_w) continue;   // wave-uniform: no row of this wavefront sees the tile

    f32x16 sacc = f32x16{};
#pragma unroll
    for (int s = 0; s < DH / 2; ++s)
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(k_tile[lr * KP + 2 * s + h], qreg[s], sacc, 0, 0, 0);

    // Legal keys of this row in the tile: j < T_k, (not causal or j <= pos),
    // inside the window, and a bias entry that is not -inf.
    int lim = a.causal ? pos_row - key0 : kKeys - 1;
    if (a.t_k - 1 - key0 < lim) lim = a.t_k - 1 - key0;
    if (!row_ok) lim = -1;
    const int first = lo_row - key0;
    float z[16];
    float mx = -INFINITY;
    bool any = false;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = 8 * (r >> 2) + 4 * h + (r & 3);
      bool legal = j <= lim && j >= first;
      float zb = 0.0f;
      if (BIAS) {
        const float mb = legal ? brow[static_cast<int64_t>(key0 + j) * a.bs[3]] : -INFINITY;
        legal = legal && mb != -INFINITY;
        zb = mb * kLog2e;
      }
      z[r] = legal ? fmaf(sacc[r], a.scale_log2, zb) : -INFINITY;
      mx = fmaxf(mx, z[r]);
      any = any || legal;
      if (COUNT) count += legal ? 1 : 0;
    }
    // Both exchanges run on every lane (a short-circuit || around one would
    // leave the partner lane out of it).
    const float tmax = fmaxf(mx, __shfl_xor(mx, 32));
    const int any_partner = __shfl_xor(static_cast<int>(any), 32);
    const bool any_row = any || any_partner != 0;
    // Merge (eqs 33.4-33.5): a tile with no legal key changes nothing.
    const float m_new = any_row ? (has ? fmaxf(m2, tmax) : tmax) : m2;
    const float alpha = (has && any_row) ? fast_exp2(m2 - m_new) : 1.0f;
    l_lane *= alpha;
#pragma unroll
    for (int i = 0; i < MO; ++i) oacc[i] *= alpha;
    if (any_row) {
      m2 = m_new;
      has = true;
    }
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = z[r] == -INFINITY ? 0.0f : fast_exp2(z[r] - m2);
      l_lane += p[r];
    }
    // O^T += V^T P^T: step s contracts keys 8 (s / 4) + (s % 4) and that + 4.
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const int key = 8 * (s >> 2) + 4 * h + (s & 3);
#pragma unroll
      for (int mo = 0; mo < MO; ++mo)
        oacc[mo] = __builtin_amdgcn_mfma_f32_32x32x2f32(v_tile[key * DV + 32 * mo + lr], p[s], oacc[mo], 0, 0, 0);
    }
  }

  // o = u / l, LSE = m + ln l; a row with no legal key gets (+0, -inf).
  const float l_row = l_lane + __shfl_xor(l_lane, 32);
  if (COUNT) count += __shfl_xor(count, 32);
  if (!row_ok) return;
  const float inv = has ? 1.0f / l_row : 0.0f;
  float* op = a.o + b * a.os[0] + hq * a.os[1] + static_cast<int64_t>(row) * a.os[2];
#pragma unroll
  for (int mo = 0; mo < MO; ++mo) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 w = {oacc[mo][4 * g] * inv, oacc[mo][4 * g + 1] * inv, oacc[mo][4 * g + 2] * inv,
                       oacc[mo][4 * g + 3] * inv};
      *reinterpret_cast<f32x4*>(op + 32 * mo + 8 * g + 4 * h) = w;
    }
  }
  if (h == 0) {
    const int64_t ridx = (static_cast<int64_t>(b) * a.heads_q + hq) * a.t_q + row;
    a.lse[ridx] = has ? (m2 + fast_log2(l_row)) * kLn2 : -INFINITY;
    if (COUNT) a.n_legal[ridx] = count;
  }
#endif
}

// Small grids (fewer workgroups than fp32_prefill_kernel would fill the CUs
// with): one workgroup per 32 query rows, whose 4 wavefronts split the
// rows' visible key tiles into 4 contiguous parts.  Each wavefront streams
// its part through its own LDS tiles (no barriers), keeps its own (m, l, u)
// per row and stores them at the end; the 4 states of a row are merged by
// eqs 33.4-33.5 (a part with no legal key contributes nothing).  The
// critical path is then a quarter of the row block's tiles instead of all
// the tiles of a 128-row block's last wavefront.
template <int DH, int DV, bool COUNT, bool BIAS>
__global__ __launch_bounds__(kThreads, 1) void fp32_split_kernel(F32Args a) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int KP = DH + 1;            // padded K row, in floats
  constexpr int MO = DV / 32;
  constexpr int K_FL = kKeys * KP;      // a multiple of 4 floats: the V tile after it stays 16-byte aligned
  constexpr int TILE_FL = K_FL + kKeys * DV;
  constexpr int MERGE_FL = kWaves * 32 * DV + 3 * kWaves * 32;
  constexpr int SMEM_FL = kWaves * TILE_FL > MERGE_FL ? kWaves * TILE_FL : MERGE_FL;
  static_assert(K_FL % 4 == 0, "V tile alignment");
  __shared__ __attribute__((aligned(16))) float smem[SMEM_FL];
  debug_poison_lds(smem, sizeof(smem));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int lr = lane & 31;

  // Heaviest (latest, when causal) row blocks first.
  const int n_rb = (a.t_q + 31) / 32;
  const int bid = blockIdx.x;
  const int rb = n_rb - 1 - bid / a.batch_heads;
  const int bh = bid % a.batch_heads;
  const int b = bh / a.heads_q;
  const int hq = bh % a.heads_q;
  const int kvh = hq / a.group;

  const int row0 = rb * 32;
  const int row = row0 + lr;
  const bool row_ok = row < a.t_q;

  // Q^T operand of step s: Q[row][2 s + h], from 16-byte loads of a valid
  // row (rows past T_q read row 0 and are zeroed: no branch per load).
  float qreg[DH / 2];
  {
    const float* qp = a.q + b * a.qs[0] + hq * a.qs[1] + static_cast<int64_t>(row_ok ? row : 0) * a.qs[2];
#pragma unroll
    for (int c = 0; c < DH / 4; ++c) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(qp + 4 * c);
      qreg[2 * c] = row_ok ? (h ? x[1] : x[0]) : 0.0f;
      qreg[2 * c + 1] = row_ok ? (h ? x[3] : x[2]) : 0.0f;
    }
  }

  auto win_lo = [&](int64_t r) -> int {
    if (a.window <= 0) return 0;
    const int64_t lo = a.q_offset + r - a.window + 1;
    return lo < 0 ? 0 : (lo > a.t_k ? a.t_k : static_cast<int>(lo));
  };
  // Key tiles some row of the block may see: [t0, t1), cut into 4 parts.
  const int last_row = row0 + 31 < a.t_q ? row0 + 31 : a.t_q - 1;
  const int pos_last = clamp_pos32(a, a.q_offset + last_row);
  const int k_end = a.causal ? (pos_last + 1 < a.t_k ? pos_last + 1 : a.t_k) : a.t_k;
  const int t0 = win_lo(row0) / kKeys;
  int t1 = (k_end + kKeys - 1) / kKeys;
  if (t1 < t0) t1 = t0;
  const int part = (t1 - t0 + kWaves - 1) / kWaves;
  const int tw0 = t0 + wave * part < t1 ? t0 + wave * part : t1;
  const int tw1 = tw0 + part < t1 ? tw0 + part : t1;

  const int pos_row = clamp_pos32(a, a.q_offset + row);
  const int lo_row = win_lo(row);
  const float* brow = nullptr;
  if (BIAS && row_ok) brow = a.bias + b * a.bs[0] + hq * a.bs[1] + static_cast<int64_t>(row) * a.bs[2];
  const float* kbase = a.k + b * a.ks[0] + kvh * a.ks[1];
  const float* vbase = a.v + b * a.vs[0] + kvh * a.vs[1];
  float* const k_tile = smem + wave * TILE_FL;
  float* const v_tile = k_tile + K_FL;

  bool has = false;
  float m2 = 0.0f;
  float l_lane = 0.0f;
  int32_t count = 0;
  f32x16 oacc[MO];
#pragma unroll
  for (int i = 0; i < MO; ++i) oacc[i] = f32x16{};

  // This wavefront's copies of tile t: lane l moves 16-byte chunks
  // c = l + 64 i; keys past T_k read as zero.
  constexpr int KN = kKeys * DH / 4 / 64;
  constexpr int VN = kKeys * DV / 4 / 64;
  f32x4 kpre[KN], vpre[VN];
  // Keys past T_k read key 0 (a tile holds at least one key below T_k) and
  // are zeroed, so every load is issued without a branch.
  auto fetch = [&](int t) {
#pragma unroll
    for (int i = 0; i < KN; ++i) {
      const int c = lane + 64 * i, key = t * kKeys + c / (DH / 4), d = 4 * (c % (DH / 4));
      const f32x4 x = *reinterpret_cast<const f32x4*>(kbase + static_cast<int64_t>(key < a.t_k ? key : 0) * a.ks[2] + d);
      kpre[i] = key < a.t_k ? x : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll
    for (int i = 0; i < VN; ++i) {
      const int c = lane + 64 * i, key = t * kKeys + c / (DV / 4), d = 4 * (c % (DV / 4));
      const f32x4 x = *reinterpret_cast<const f32x4*>(vbase + static_cast<int64_t>(key < a.t_k ? key : 0) * a.vs[2] + d);
      vpre[i] = key < a.t_k ? x : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  };
  if (tw0 < tw1) fetch(tw0);
  for (int t = tw0; t < tw1; ++t) {
    // The previous tile's operand reads were issued before these stores (LDS
    // operations of a wavefront run in order).
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < KN; ++i) {
      const int c = lane + 64 * i, kk = c / (DH / 4), d = 4 * (c % (DH / 4));
#pragma unroll
      for (int e = 0; e < 4; ++e) k_tile[kk * KP + d + e] = kpre[i][e];
    }
#pragma unroll
    for (int i = 0; i < VN; ++i) {
      const int c = lane + 64 * i, kk = c / (DV / 4), d = 4 * (c % (DV / 4));
      *reinterpret_cast<f32x4*>(v_tile + kk * DV + d) = vpre[i];
    }
    asm volatile("" ::: "memory");
    if (t + 1 < tw1) fetch(t + 1);
    const int key0 = t * kKeys;

    // Every K operand is read before the products, so the chain of products
    // waits for LDS once.
    float kop[DH / 2];
#pragma unroll
    for (int s = 0; s < DH / 2; ++s) kop[s] = k_tile[lr * KP + 2 * s + h];
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int s = 0; s < DH / 2; ++s)
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(kop[s], qreg[s], sacc, 0, 0, 0);

    int lim = a.causal ? pos_row - key0 : kKeys - 1;
    if (a.t_k - 1 - key0 < lim) lim = a.t_k - 1 - key0;
    if (!row_ok) lim = -1;
    const int first = lo_row - key0;
    float z[16];
    float mx = -INFINITY;
    bool any = false;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = 8 * (r >> 2) + 4 * h + (r & 3);
      bool legal = j <= lim && j >= first;
      float zb = 0.0f;
      if (BIAS) {
        const float mb = legal ? brow[static_cast<int64_t>(key0 + j) * a.bs[3]] : -INFINITY;
        legal = legal && mb != -INFINITY;
        zb = mb * kLog2e;
      }
      z[r] = legal ? fmaf(sacc[r], a.scale_log2, zb) : -INFINITY;
      mx = fmaxf(mx, z[r]);
      any = any || legal;
      if (COUNT) count += legal ? 1 : 0;
    }
    const float tmax = fmaxf(mx, __shfl_xor(mx, 32));
    const int any_partner = __shfl_xor(static_cast<int>(any), 32);
    const bool any_row = any || any_partner != 0;
    const float m_new = any_row ? (has ? fmaxf(m2, tmax) : tmax) : m2;
    const float alpha = (has && any_row) ? fast_exp2(m2 - m_new) : 1.0f;
    l_lane *= alpha;
#pragma unroll
    for (int i = 0; i < MO; ++i) oacc[i] *= alpha;
    if (any_row) {
      m2 = m_new;
      has = true;
    }
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = z[r] == -INFINITY ? 0.0f : fast_exp2(z[r] - m2);
      l_lane += p[r];
    }
    float vop[16][MO];
#pragma unroll
    for (int s = 0; s < 16; ++s)
#pragma unroll
      for (int mo = 0; mo < MO; ++mo) vop[s][mo] = v_tile[(8 * (s >> 2) + 4 * h + (s & 3)) * DV + 32 * mo + lr];
#pragma unroll
    for (int s = 0; s < 16; ++s)
#pragma unroll
      for (int mo = 0; mo < MO; ++mo)
        oacc[mo] = __builtin_amdgcn_mfma_f32_32x32x2f32(vop[s][mo], p[s], oacc[mo], 0, 0, 0);
  }

  // ---- merge the four wavefront states of each row ----
  const float l_row = l_lane + __shfl_xor(l_lane, 32);
  if (COUNT) count += __shfl_xor(count, 32);
  __syncthreads();                             // every wavefront is done with its tiles
  debug_poison_lds(smem, MERGE_FL * 4);        // the merge area: only stored states are read
  float* const mo_area = smem;                 // [wave][row][DV]
  float* const m_area = smem + kWaves * 32 * DV;
  float* const l_area = m_area + kWaves * 32;
  int32_t* const c_area = reinterpret_cast<int32_t*>(l_area + kWaves * 32);
  {
    float* dst = mo_area + (wave * 32 + lr) * DV;
#pragma unroll
    for (int mo = 0; mo < MO; ++mo)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 x = {oacc[mo][4 * g], oacc[mo][4 * g + 1], oacc[mo][4 * g + 2], oacc[mo][4 * g + 3]};
        *reinterpret_cast<f32x4*>(dst + 32 * mo + 8 * g + 4 * h) = x;
      }
    if (h == 0) {
      m_area[wave * 32 + lr] = has ? m2 : -INFINITY;
      l_area[wave * 32 + lr] = l_row;
      c_area[wave * 32 + lr] = count;
    }
  }
  __syncthreads();
  for (int e = tid; e < 32 * DV; e += kThreads) {
    const int r = e / DV, d = e % DV;
    const int orow = row0 + r;
    if (orow >= a.t_q) break;                  // e grows with r: no later row exists
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, m_area[w * 32 + r]);
    float num = 0.0f, den = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = m_area[w * 32 + r];
        if (mw == -INFINITY) continue;           // this part held no legal key of the row
        const float c = fast_exp2(mw - M);
        num = fmaf(c, mo_area[(w * 32 + r) * DV + d], num);
        den = fmaf(c, l_area[w * 32 + r], den);
      }
    }
    const bool live = M != -INFINITY;
    a.o[b * a.os[0] + hq * a.os[1] + static_cast<int64_t>(orow) * a.os[2] + d] = live ? num / den : 0.0f;
    if (d == 0) {
      const int64_t ridx = (static_cast<int64_t>(b) * a.heads_q + hq) * a.t_q + orow;
      a.lse[ridx] = live ? (M + fast_log2(den)) * kLn2 : -INFINITY;
      if (COUNT) {
        int32_t n = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) n += c_area[w * 32 + r];
        a.n_legal[ridx] = n;
      }
    }
  }
#endif
}

template <int DH, int DV, bool BIAS>
void launch_b(const F32Args& a, int64_t blocks, bool count, hipStream_t s) {
  if (a.split) {
    if (count)
      hipLaunchKernelGGL((fp32_split_kernel<DH, DV, true, BIAS>), dim3(static_cast<unsigned>(blocks)),
                         dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((fp32_split_kernel<DH, DV, false, BIAS>), dim3(static_cast<unsigned>(blocks)),
                         dim3(kThreads), 0, s, a);
    return;
  }
  if (count)
    hipLaunchKernelGGL((fp32_prefill_kernel<DH, DV, true, BIAS>), dim3(static_cast<unsigned>(blocks)),
                       dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((fp32_prefill_kernel<DH, DV, false, BIAS>), dim3(static_cast<unsigned>(blocks)),
                       dim3(kThreads), 0, s, a);
}

template <int DH, int DV>
hipError_t launch_dims(const F32Args& a, int64_t blocks, bool count, hipStream_t s) {
  if (a.bias != nullptr) launch_b<DH, DV, true>(a, blocks, count, s);
  else launch_b<DH, DV, false>(a, blocks, count, s);
  return hipGetLastError();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

// fp32 problems with d_h, d_v in {64, 128} (any bias and window), no
// variable lengths, 16-byte aligned tensors with strides a multiple of 4
// floats, and sizes that fit 32-bit tile indices.  Returns false when it does not
// apply (the generic kernel then runs).
bool launch_fp32_mfma(const Problem& pb, int dtype, const void* q, const void* k, const void* v, void* o,
                      float* lse, int32_t* n_legal, hipStream_t stream, int* status) {
  if (dtype != ATTN_F32 || pb.cu_q != nullptr || pb.kv_lens != nullptr) return false;
  if (!((pb.d_h == 64 || pb.d_h == 128) && (pb.d_v == 64 || pb.d_v == 128))) return false;
  if (pb.t_q >= (int64_t(1) << 30) || pb.t_k >= (int64_t(1) << 30)) return false;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return false;
  for (int i = 0; i < 3; ++i)
    if ((pb.qs[i] | pb.ks[i] | pb.vs[i] | pb.os[i]) & 3) return false;
  const int64_t n_qtiles = (pb.t_q + kRows - 1) / kRows;
  int64_t blocks = n_qtiles * pb.batch * pb.heads_q;
  if (blocks >= (int64_t(1) << 31) || pb.batch * pb.heads_q >= (int64_t(1) << 30)) return false;
  // Fewer workgroups than FP32_SPLIT_BELOW: one per 32 rows, keys split over
  // its wavefronts (4x the workgroups, a quarter of the serial tiles each).
  const bool split = blocks < FP32_SPLIT_BELOW;
  if (split) blocks = (pb.t_q + 31) / 32 * pb.batch * pb.heads_q;
  F32Args a;
  a.q = static_cast<const float*>(q);
  a.k = static_cast<const float*>(k);
  a.v = static_cast<const float*>(v);
  a.o = static_cast<float*>(o);
  a.lse = lse;
  a.n_legal = n_legal;
  for (int i = 0; i < 3; ++i) {
    a.qs[i] = pb.qs[i]; a.ks[i] = pb.ks[i]; a.vs[i] = pb.vs[i]; a.os[i] = pb.os[i];
  }
  a.q_offset = pb.q_offset;
  a.window = pb.window;
  a.bias = pb.bias;
  for (int i = 0; i < 4; ++i) a.bs[i] = pb.bs[i];
  a.t_q = static_cast<int32_t>(pb.t_q);
  a.t_k = static_cast<int32_t>(pb.t_k);
  a.heads_q = static_cast<int32_t>(pb.heads_q);
  a.group = pb.group;
  a.n_qtiles = static_cast<int32_t>(n_qtiles);
  a.batch_heads = static_cast<int32_t>(pb.batch * pb.heads_q);
  a.scale_log2 = pb.scale_log2;
  a.causal = pb.causal;
  a.split = split;
  const bool count = n_legal != nullptr;
  hipError_t e;
  if (pb.d_h == 128 && pb.d_v == 128) e = launch_dims<128, 128>(a, blocks, count, stream);
  else if (pb.d_h == 64 && pb.d_v == 128) e = launch_dims<64, 128>(a, blocks, count, stream);
  else if (pb.d_h == 128 && pb.d_v == 64) e = launch_dims<128, 64>(a, blocks, count, stream);
  else e = launch_dims<64, 64>(a, blocks, count, stream);
  *status = e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
  return true;
}

}  // namespace attn
