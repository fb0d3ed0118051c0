// MFMA backward kernels for bf16 Q/K/V/O/dO, d_h and d_v in {64, 128}, with
// or without a bias (keys contiguous): gradients of the attention of attn_fwd
// by recomputing the
// probabilities from the saved LSE, eqs 33.6-33.8 of "Chapter 33 推理计算优化"
// §33.3 (block size, parallelism and backward recomputation):
//   P_ij = e^{z_ij - LSE_i} on legal keys, dP = dO V^T,
//   dS_ij = P_ij (dP_ij - D_i) with D_i = <dO_i, O_i> (Exercise 33.4),
//   dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO.
// No running maximum is needed: the saved LSE is the exact normaliser.  With
// a bias the exponent is scale dot + M - LSE (base 2); a row whose LSE is
// -inf (no legal key; with a bias such a row can sit in a fully visible
// block) takes +inf there, so all its weights are 0 without a mask.
//
// dQ kernel: the forward kernel's mapping.  A workgroup of 4 wavefronts owns
// 128 query rows; K/V tiles of 64 keys stream HBM -> LDS (buffer_load ... lds
// into two-slot rings).  Per 32-key block: S^T = K Q^T and dP^T = V dO^T
// (A = 16-byte reads of K / V rows, B = Q^T / dO^T resident in registers),
// so each lane holds 16 entries of one query row; dS^T is packed to bf16 and
// is the B operand of dQ^T += K^T dS^T, whose A operand K^T comes from
// ds_read_b64_tr_b16 of the row-major K tile.
//
// dK/dV kernel: a workgroup of 4 wavefronts owns 128 keys of one (batch, KV
// head); wavefront w owns keys 32 w .. 32 w + 31, with K^T (and V^T for dK)
// resident in registers.  Q/dO tiles of 64 rows of every query head of the
// group stream HBM -> LDS.  Per 32-row block: S = Q K^T (and dP = dO V^T),
// so each lane holds 16 entries of one key column; P (dV) or dS (dK) is
// packed to bf16 and is the B operand of dV^T += dO^T P or dK^T += Q^T dS,
// with A = dO^T / Q^T from transposed reads of the row-major tile.  One launch
// per output (dV, then dK): each keeps one accumulator set and two operand
// sets in registers.
//
// Tiles are 64 rows; all rows of a tile use the XOR swizzle of the transposed
// reads (16-byte row reads are conflict-free with it too: 16 consecutive rows
// map chunk c to 16 distinct chunks).
//
// Work order: tiles outermost (dQ: heaviest causal tiles first; dK / dV: low
// key tiles first), every (batch, head) of a tile together; dense batches
// whose K/V exceeds the 256 MB Infinity Cache go batch after batch instead.
// Packed sequences map grid slots to (sequence, tile) from the offsets (see
// VArgs).
#include <type_traits>

#include "attn_internal.h"
#include "kernels.h"
#include "prefill_common.h"

namespace attn {
namespace {

using namespace pf;

constexpr int kW = 4;
constexpr int kThreads = 64 * kW;
constexpr int kRowsW = 32;              // rows (dQ) or keys (dK/dV) per wavefront
constexpr int kBr = kRowsW * kW;        // per workgroup
constexpr int kBc = 64;                 // streamed tile rows
#ifndef BWD_PIPE
#define BWD_PIPE 1     // dV: software-pipelined path for units whose two blocks are fully legal
#endif
#ifndef BWD_FUSED
#define BWD_FUSED 1    // dense batches without a bias: dK and dV in one launch
#endif
#ifndef BWD_READ_AHEAD
#define BWD_READ_AHEAD 1  // 1: MFMA products read their LDS operand a step ahead (where registers allow)
#endif
#ifndef BWD_SCHED
#define BWD_SCHED 0    // VALU instructions placed after each MFMA in that path (0: compiler's order)
#endif

struct BArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* d_o;
  const float* lse;
  float* dd;                // D_i = <dO_i, O_i>, [B, H_q, T_q]: written by dQ, read by dK / dV
  const uint16_t* o;        // forward output (dQ only: D from its rows)
  uint16_t* out;            // dQ, dK or dV
  int64_t qs[3], ks[3], vs[3], os[3];
  int64_t q_offset;
  int64_t window;
  int32_t t_q, t_k, heads_q, heads_kv, group, n_tiles_grid, n_units;
  float scale_log2;
  int32_t causal;
  int32_t batch_major;      // 1: batches one after the other (heads fastest, then tiles)
};

// Packed sequences: offsets of n_seqs sequences along T_q and T_k.  Packed
// instances take it as one more kernel argument; the others keep the argument
// block above (a larger block changes their code).
//
// Tile slots: sequence s owns slots [start_s, start_{s+1}) of the grid's
// n_slots = floor(T / 128) + n_seqs, with start_s = floor(cu[s] / 128) + s
// over the offsets of the tiled dimension (rows for dQ, keys for dK / dV).
// floor((a + L) / 128) - floor(a / 128) + 1 >= ceil(L / 128), so each
// sequence has a slot for every one of its tiles, found from the offsets
// alone (no host copy of them, no per-sequence bound); slots outside a
// sequence's tiles return at once.
struct VArgs {
  const int32_t* cu_q;
  const int32_t* cu_k;
  int32_t n_seqs, n_slots;
  // Per-batch KV lengths instead (cu_q NULL): batch b uses keys [0, L_b),
  // rows at q_offset + L_b - T_q + i; dense grid; keys past L_b get zero.
  const int32_t* kv_lens;
};
// Bias instances take the bias as one more trailing argument (fp32, keys
// contiguous, any broadcast over batch, head and row).
struct BBias {
  const float* bias;
  int64_t bs[3];   // element strides of b, hq, i (keys are contiguous)
};
// The trailing argument of type T (only called when one is present).
template <class T, class U, class... R>
__device__ __forceinline__ const T& pick(const U& u, const R&... r) {
  if constexpr (std::is_same_v<T, U>) return u;
  else return pick<T>(r...);
}
template <class T, class... X>
constexpr bool has_arg = (std::is_same_v<T, X> || ...);

template <int DH, int DV>
struct BCfg {
  static constexpr int KS = DH / 16;     // k-steps over d_h
  static constexpr int MS = DV / 16;     // k-steps over d_v
  static constexpr int MQ = DH / 32;     // 32-wide slices of d_h
  static constexpr int MV = DV / 32;     // 32-wide slices of d_v
  static constexpr int H_RB = DH * 2;    // bytes per row of a d_h-wide tile
  static constexpr int V_RB = DV * 2;    // bytes per row of a d_v-wide tile
  static constexpr int H_BYTES = kBc * H_RB;
  static constexpr int V_BYTES = kBc * V_RB;
  static constexpr int H_DMA = H_BYTES / 1024 / kW;   // 1 KB copies per wavefront per tile
  static constexpr int V_DMA = V_BYTES / 1024 / kW;
};

// Position helpers: logical position clamped to [-1, T_k].
__device__ __forceinline__ int clamp_pos(const BArgs& a, int64_t p) {
  return p < -1 ? -1 : (p > a.t_k ? a.t_k : static_cast<int>(p));
}
// First key inside the window of logical row r (0 without a window), in [0, T_k].
__device__ __forceinline__ int win_lo(const BArgs& a, int64_t r) {
  if (a.window <= 0) return 0;
  const int64_t lo = a.q_offset + r - a.window + 1;
  return lo < 0 ? 0 : (lo > a.t_k ? a.t_k : static_cast<int>(lo));
}

// Byte offsets (relative to a tile's first row) of the 16-byte chunks one
// wavefront copies: copy j, lane l fills LDS bytes [1024 (wave n + j) + 16 l, +16)
// of the slot, i.e. row r, chunk slot sl, which holds chunk sl ^ swz(r).
template <int RB, int N>
__device__ __forceinline__ void dma_offsets(int wave, int lane, int row_bytes, int* off) {
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const int byte = (wave * N + j) * 1024 + lane * 16;
    const int r = byte / RB, sl = (byte % RB) / 16;
    off[j] = r * row_bytes + (sl ^ swz_v<RB>(r)) * 16;
  }
}

template <int RB, int N>
__device__ __forceinline__ void dma_tile(const void* base, int64_t first_row, int64_t n_rows, int row_bytes,
                                         char* slot, int wave, const int* off) {
  const auto rs = make_rsrc(static_cast<const char*>(base) + first_row * row_bytes,
                            (n_rows - first_row) * row_bytes);
#pragma unroll
  for (int j = 0; j < N; ++j)
    lds_copy<16>(rs, (__attribute__((address_space(3))) void*)(slot + (wave * N + j) * 1024), off[j]);
}

// Address of the 16-byte chunk holding elements 16 s + 8 h .. + 7 of row r of
// a swizzled tile (A operand of a 32x32x16 MFMA: lane = row, 8 elements).
template <int RB>
__device__ __forceinline__ const lds_char* row_chunk(const char* tile, int r, int s, int h) {
  return (const lds_char*)tile + r * RB + (((2 * s + h) ^ swz_v<RB>(r)) << 4);
}

// Transposed-read address for operand step kk2 of rows base .. base + 15 and
// output slice mo (32 columns) of a swizzled row-major tile: rows
// src + 8 e with src = 16 kk2 + 4 h + (lane % 16) / 4 (+ base), byte column
// 64 mo + 32 ((lane / 16) % 2) + 8 (lane % 4).
template <int RB>
__device__ __forceinline__ const lds_char* tr_addr(const char* tile, int base, int kk2, int mo, int e, int lane) {
  const int h = lane >> 5;
  const int src = base + 16 * kk2 + 4 * h + ((lane & 15) >> 2) + 8 * e;
  const int cb = 64 * mo + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);
  return (const lds_char*)tile + src * RB + (((cb >> 4) ^ swz_v<RB>(src)) << 4) + (cb & 15);
}

// Tile slot -> (sequence, tile): the last s with start_s <= slot (a binary
// search over the clamped offsets cu of the tiled dimension of size n).
// Entries out of order (outside the contract) still give an s in range.
__device__ __forceinline__ int slot_seq(const int32_t* cu, int n_seqs, int n, int slot, int* tile) {
  int lo = 0, hi = n_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (clamp_len(cu[mid], n) / kBr + mid <= slot) lo = mid;
    else hi = mid - 1;
  }
  *tile = slot - (clamp_len(cu[lo], n) / kBr + lo);
  return lo;
}

// Moves the row pointers (q, d_o and, for dQ, o and the output) to sequence sq's
// first row and the key pointers (k, v and, for dK / dV, the output) to its
// first key, and makes the sizes and q_offset the sequence's own, with its
// rows at the end of its keys.  *row_base and *key_base are the packed row
// and key of the sequence's row 0 and key 0 (LSE, D and the bias keep the
// packed layout).
template <bool OUT_ROWS>
__device__ __forceinline__ void enter_seq(BArgs& a, const VArgs& va, int sq, int64_t out_row_stride,
                                          int32_t* row_base, int32_t* key_base) {
  const int q0 = clamp_len(va.cu_q[sq], a.t_q);
  const int q1 = max(q0, clamp_len(va.cu_q[sq + 1], a.t_q));
  const int k0 = clamp_len(va.cu_k[sq], a.t_k);
  const int k1 = max(k0, clamp_len(va.cu_k[sq + 1], a.t_k));
  a.q += static_cast<int64_t>(q0) * a.qs[2];
  a.d_o += static_cast<int64_t>(q0) * a.os[2];
  if (OUT_ROWS) a.o += static_cast<int64_t>(q0) * a.os[2];   // dQ also reads O (for D)
  a.k += static_cast<int64_t>(k0) * a.ks[2];
  a.v += static_cast<int64_t>(k0) * a.vs[2];
  a.out += static_cast<int64_t>(OUT_ROWS ? q0 : k0) * out_row_stride;
  *row_base = q0;
  *key_base = k0;
  a.q_offset += (k1 - k0) - (q1 - q0);
  a.t_q = q1 - q0;
  a.t_k = k1 - k0;
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
template <int DH, int DV, class... Extra>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_mfma_kernel(BArgs a, Extra... ex) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr bool VAR = has_arg<VArgs, Extra...>;
  constexpr bool BIAS = has_arg<BBias, Extra...>;
  using C = BCfg<DH, DV>;
  // Products read their LDS operand a step ahead (BWD_READ_AHEAD), so each
  // waits for a read issued a product earlier rather than for its own: at
  // d_h = d_v = 128 without a bias (backward B1 H32 T8192 1.87 -> 1.82 ms;
  // its extra registers spill outside the tile loop only).  With a bias the
  // spills land inside the loop, and at d_h = 64 it measured no gain.
  constexpr bool kDqAhead = BWD_READ_AHEAD && DH == 128 && DV == 128 && !BIAS;
  __shared__ __attribute__((aligned(1024))) char smem[2 * C::H_BYTES + 2 * C::V_BYTES];
  debug_poison_lds(smem, sizeof(smem));
  char* const kring = smem;
  char* const vring = smem + 2 * C::H_BYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int lr = lane & 31;

  // Heaviest query tiles first (packed sequences: slots in descending order,
  // so each sequence's last tile first).
  const int bid = blockIdx.x;
  int qt = a.n_tiles_grid - 1 - bid / a.n_units;
  int bh = bid % a.n_units;
  if (!VAR && a.batch_major) {
    const int i2 = bid / a.heads_q;
    qt = a.n_tiles_grid - 1 - i2 % a.n_tiles_grid;
    bh = (i2 / a.n_tiles_grid) * a.heads_q + bid % a.heads_q;
  }
  const int b = bh / a.heads_q;
  const int hq = bh % a.heads_q;
  const int kvh = hq / a.group;
  int64_t ridx_base = (static_cast<int64_t>(b) * a.heads_q + hq) * a.t_q;   // LSE / D index of row 0
  int32_t row_base = 0, key_base = 0;
  if constexpr (VAR) {
    const VArgs& va = pick<VArgs>(ex...);
    if (va.cu_q != nullptr) {
      const int sq = slot_seq(va.cu_q, va.n_seqs, a.t_q, qt, &qt);
      enter_seq<true>(a, va, sq, a.qs[2], &row_base, &key_base);
      if (qt < 0 || qt * kBr >= a.t_q) return;   // whole workgroup: a slot outside the sequence's tiles
      ridx_base += row_base;
    } else {
      const int len = clamp_len(va.kv_lens[b], a.t_k);
      a.q_offset += len - a.t_q;
      a.t_k = len;
    }
  }

  const int row0 = qt * kBr + wave * kRowsW;
  const int row = row0 + lr;
  const bool row_ok = row < a.t_q;
  const int64_t ridx = ridx_base + row;

  // Q^T and dO^T operands of this lane's row.
  u32x4 qreg[C::KS], greg[C::MS];
  {
    const uint16_t* qp = a.q + b * a.qs[0] + hq * a.qs[1] + static_cast<int64_t>(row) * a.qs[2];
    const uint16_t* gp = a.d_o + b * a.os[0] + hq * a.os[1] + static_cast<int64_t>(row) * a.os[2];
#pragma unroll
    for (int s = 0; s < C::KS; ++s)
      qreg[s] = row_ok ? *reinterpret_cast<const u32x4*>(qp + 16 * s + 8 * h) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < C::MS; ++s)
      greg[s] = row_ok ? *reinterpret_cast<const u32x4*>(gp + 16 * s + 8 * h) : u32x4{0, 0, 0, 0};
  }
  float lse2 = row_ok ? a.lse[ridx] * kLog2e : -INFINITY;
  // A row with no legal key has every weight 0; with a bias a full block can
  // hold such a row (all its entries -inf), so its LSE acts as +inf there.
  if (BIAS && lse2 == -INFINITY) lse2 = INFINITY;
  // Bias rows of this wavefront (keys contiguous): 16 values per lane and
  // block through a buffer that ends at the wavefront's last row and key.
  const float* bias_w = nullptr;
  int64_t bias_w_bytes = 0;
  int bias_off = 0;
  if constexpr (BIAS) {
    const BBias& bb = pick<BBias>(ex...);
    bias_w = bb.bias + b * bb.bs[0] + hq * bb.bs[1] + static_cast<int64_t>(row_base + row0) * bb.bs[2] + key_base;
    const int rows_w = a.t_q - row0 < kRowsW ? a.t_q - row0 : kRowsW;
    bias_w_bytes = rows_w > 0 ? (static_cast<int64_t>(rows_w - 1) * bb.bs[2] + a.t_k) * 4 : 0;
    bias_off = row_ok ? static_cast<int>(lr * bb.bs[2] * 4) + 16 * h : 0;
  }
  // D_i = <dO_i, O_i> (Exercise 33.4): this lane's half of the row from the
  // dO operand already in registers and the same chunks of O, the halves
  // joined by one exchange; stored for the dK / dV launches.
  float dd = 0.0f;
  {
    const uint16_t* orow = a.o + b * a.os[0] + hq * a.os[1] + static_cast<int64_t>(row) * a.os[2];
#pragma unroll
    for (int s = 0; s < C::MS; ++s) {
      const u32x4 ov = row_ok ? *reinterpret_cast<const u32x4*>(orow + 16 * s + 8 * h) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        dd = fmaf(__uint_as_float(greg[s][w] << 16), __uint_as_float(ov[w] << 16), dd);
        dd = fmaf(__uint_as_float(greg[s][w] & 0xffff0000u), __uint_as_float(ov[w] & 0xffff0000u), dd);
      }
    }
    dd += __shfl_xor(dd, 32);
    if (h == 0 && row_ok) a.dd[ridx] = dd;
  }

  const int pos_row = clamp_pos(a, a.q_offset + row);
  const int pos_w_first = clamp_pos(a, a.q_offset + row0);
  const int pos_w_last = clamp_pos(a, a.q_offset + row0 + 31);
  const int lo_row = win_lo(a, row);
  const int lo_w_first = win_lo(a, row0);
  const int lo_w_last = win_lo(a, row0 + 31);

  const int wg_last = clamp_pos(a, a.q_offset + static_cast<int64_t>(qt) * kBr + kBr - 1);
  const int k_end = a.causal ? (wg_last + 1 < a.t_k ? wg_last + 1 : a.t_k) : a.t_k;
  const int n_tiles = k_end > 0 ? (k_end + kBc - 1) / kBc : 0;
  const int t_begin = win_lo(a, static_cast<int64_t>(qt) * kBr) / kBc;
  const int t_w_begin = lo_w_first / kBc;
  const int t_lo_full = (lo_w_last + kBc - 1) / kBc;
  int n_w = n_tiles;
  if (row0 >= a.t_q) {
    n_w = 0;
  } else if (a.causal) {
    const int last = pos_w_last < a.t_k - 1 ? pos_w_last : a.t_k - 1;
    const int tw = last < 0 ? 0 : last / kBc + 1;
    if (tw < n_w) n_w = tw;
  }
  // Tiles every row of the wave sees in full (and every row exists).
  int t_full = a.t_k / kBc;
  if (a.causal) {
    const int tf = (pos_w_first + 1) / kBc;
    if (tf < t_full) t_full = tf;
  }
  if (row0 + kRowsW > a.t_q) t_full = 0;
  if (t_full > n_w) t_full = n_w;

  const uint16_t* kbase = a.k + b * a.ks[0] + kvh * a.ks[1];
  const uint16_t* vbase = a.v + b * a.vs[0] + kvh * a.vs[1];
  const int k_row_bytes = static_cast<int>(a.ks[2]) * 2;
  const int v_row_bytes = static_cast<int>(a.vs[2]) * 2;
  int koff[C::H_DMA], voff[C::V_DMA];
  dma_offsets<C::H_RB, C::H_DMA>(wave, lane, k_row_bytes, koff);
  dma_offsets<C::V_RB, C::V_DMA>(wave, lane, v_row_bytes, voff);
  auto gload = [&](int t) {
    dma_tile<C::H_RB, C::H_DMA>(kbase, static_cast<int64_t>(t) * kBc, a.t_k, k_row_bytes,
                                kring + (t & 1) * C::H_BYTES, wave, koff);
    dma_tile<C::V_RB, C::V_DMA>(vbase, static_cast<int64_t>(t) * kBc, a.t_k, v_row_bytes,
                                vring + (t & 1) * C::V_BYTES, wave, voff);
  };

  f32x16 qacc[C::MQ];
#pragma unroll
  for (int i = 0; i < C::MQ; ++i) qacc[i] = f32x16{};

  // Block q of the tile in `slot`: S^T and dP^T (register r holds key
  // 32 q + 8 (r / 4) + 4 h + (r % 4) of this lane's row).
  auto s_and_dp = [&](int slot, int q, f32x16& sacc, f32x16& dacc) {
    const char* kt = kring + slot * C::H_BYTES;
    const char* vt = vring + slot * C::V_BYTES;
    sacc = f32x16{};
    dacc = f32x16{};
    if constexpr (kDqAhead) {
      // Step i < KS: S with K chunk i; then dP with V chunk i - KS.  The A
      // operand of step i + 1 is read before the product of step i.
      constexpr int kSteps = C::KS + C::MS;
      auto a_op = [&](int i) -> u32x4 {
        const lds_char* p = i < C::KS ? row_chunk<C::H_RB>(kt, 32 * q + lr, i, h)
                                      : row_chunk<C::V_RB>(vt, 32 * q + lr, i - C::KS, h);
        return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(p);
      };
      u32x4 cur = a_op(0);
#pragma unroll
      for (int i = 0; i < kSteps; ++i) {
        u32x4 nxt = cur;
        if (i + 1 < kSteps) nxt = a_op(i + 1);
        if (i < C::KS)
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(cur), as_bf16x8(qreg[i]), sacc, 0, 0, 0);
        else
          dacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(cur), as_bf16x8(greg[i - C::KS]), dacc, 0, 0, 0);
        cur = nxt;
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
      for (int i = 0; i < kSteps; ++i) {
        if (i + 1 < kSteps) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
    } else {
#pragma unroll
      for (int s = 0; s < C::KS; ++s) {
        const u32x4 kop = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
            row_chunk<C::H_RB>(kt, 32 * q + lr, s, h));
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kop), as_bf16x8(qreg[s]), sacc, 0, 0, 0);
      }
#pragma unroll
      for (int s = 0; s < C::MS; ++s) {
        const u32x4 vop = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
            row_chunk<C::V_RB>(vt, 32 * q + lr, s, h));
        dacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vop), as_bf16x8(greg[s]), dacc, 0, 0, 0);
      }
    }
  };
  // dQ^T += K^T dS^T for block q (B operand of step kk2: keys
  // 32 q + 16 kk2 + 4 h + (0..3) and + 8 + (0..3), where the reads fetch K).
  auto dq_acc = [&](int slot, int q, const unsigned* pk) {
    const char* kt = kring + slot * C::H_BYTES;
    if constexpr (kDqAhead) {
      constexpr int kSteps = 2 * C::MQ;
      auto a_op = [&](int i) -> u32x4 {
        const u32x2 lo = tr_read(tr_addr<C::H_RB>(kt, 32 * q, i / C::MQ, i % C::MQ, 0, lane));
        const u32x2 hi = tr_read(tr_addr<C::H_RB>(kt, 32 * q, i / C::MQ, i % C::MQ, 1, lane));
        return u32x4{lo[0], lo[1], hi[0], hi[1]};
      };
      u32x4 cur = a_op(0);
#pragma unroll
      for (int i = 0; i < kSteps; ++i) {
        u32x4 nxt = cur;
        if (i + 1 < kSteps) nxt = a_op(i + 1);
        const int kk2 = i / C::MQ, mo = i % C::MQ;
        const u32x4 bop = {pk[4 * kk2], pk[4 * kk2 + 1], pk[4 * kk2 + 2], pk[4 * kk2 + 3]};
        qacc[mo] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(cur), as_bf16x8(bop), qacc[mo], 0, 0, 0);
        cur = nxt;
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int i = 0; i < kSteps; ++i) {
        if (i + 1 < kSteps) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      return;
    }
#pragma unroll
    for (int kk2 = 0; kk2 < 2; ++kk2) {
      const u32x4 bop = {pk[4 * kk2], pk[4 * kk2 + 1], pk[4 * kk2 + 2], pk[4 * kk2 + 3]};
#pragma unroll
      for (int mo = 0; mo < C::MQ; ++mo) {
        const u32x2 lo = tr_read(tr_addr<C::H_RB>(kt, 32 * q, kk2, mo, 0, lane));
        const u32x2 hi = tr_read(tr_addr<C::H_RB>(kt, 32 * q, kk2, mo, 1, lane));
        const u32x4 aop = {lo[0], lo[1], hi[0], hi[1]};
        qacc[mo] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(aop), as_bf16x8(bop), qacc[mo], 0, 0, 0);
      }
    }
  };
  // dS of a block; MASK: apply causal / window / T_k limits per element.
  auto ds_block = [&](bool mask, int t, int q, const f32x16& sacc, const f32x16& dacc, unsigned* pk) {
    const int kb = t * kBc + 32 * q;
    int lim = a.causal ? pos_row - kb : 32;
    if (a.t_k - 1 - kb < lim) lim = a.t_k - 1 - kb;
    if (!row_ok) lim = -1;
    const int first = lo_row - kb;
    f32x4 mb[4];   // bias of the 16 keys (BIAS only)
    if constexpr (BIAS) {
      const auto rs = make_rsrc(bias_w + t * kBc, bias_w_bytes - static_cast<int64_t>(t) * kBc * 4);
#pragma unroll
      for (int g = 0; g < 4; ++g)
        mb[g] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, bias_off + 128 * q + 32 * g, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float d2[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int r = 2 * i + e;
        const int j = 8 * (r >> 2) + 4 * h + (r & 3);
        const float zb = BIAS ? fmaf(mb[r >> 2][r & 3], kLog2e, -lse2) : -lse2;
        float p = fast_exp2(fmaf(sacc[r], a.scale_log2, zb));
        if (mask) p = (j <= lim && j >= first) ? p : 0.0f;
        d2[e] = p * (dacc[r] - dd);                 // eq 33.7
      }
      pk[i] = pack_bf16(d2[0], d2[1]);
    }
  };

  auto dma_barrier = [&]() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  auto advance = [&](int t) {
    dma_barrier();
    if (t + 2 < n_tiles) gload(t + 2);
  };

  if (t_begin < n_tiles) gload(t_begin);
  if (t_begin + 1 < n_tiles) gload(t_begin + 1);
  dma_barrier();

  auto step = [&](int t, bool fast) {
    if (t < n_w && t >= t_w_begin) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        if (!fast && a.causal && t * kBc + 32 * q > pos_w_last) break;
        if (!fast && t * kBc + 32 * q + 31 < lo_w_first) continue;
        f32x16 sacc, dacc;
        unsigned pk[8];
        s_and_dp(t & 1, q, sacc, dacc);
        ds_block(!fast, t, q, sacc, dacc, pk);
        dq_acc(t & 1, q, pk);
      }
    }
    advance(t);
  };
  int t = t_begin;
  const int f0 = t_lo_full > t_begin ? t_lo_full : t_begin;
  for (; t < f0 && t < n_tiles; ++t) step(t, false);
  for (; t < t_full; ++t) step(t, true);
  for (; t < n_tiles; ++t) step(t, false);

  // dQ = scale dS K (eq 33.8).
  if (!row_ok) return;
  const float sc = a.scale_log2 * kLn2;
  uint16_t* op = a.out + b * a.qs[0] + hq * a.qs[1] + static_cast<int64_t>(row) * a.qs[2];
#pragma unroll
  for (int mo = 0; mo < C::MQ; ++mo) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dcol = 32 * mo + 8 * g + 4 * h;
      u32x2 w;
      w[0] = pack_bf16(qacc[mo][4 * g] * sc, qacc[mo][4 * g + 1] * sc);
      w[1] = pack_bf16(qacc[mo][4 * g + 2] * sc, qacc[mo][4 * g + 3] * sc);
      *reinterpret_cast<u32x2*>(op + dcol) = w;
    }
  }
#endif
}

// ---------------------------------------------------------------------------
// dK (WHICH = 1) or dV (WHICH = 0)
// ---------------------------------------------------------------------------
template <int DH, int DV, int WHICH, class... Extra>
__global__ __launch_bounds__(kThreads, 2) void bwd_kv_mfma_kernel(BArgs a, Extra... ex) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr bool VAR = has_arg<VArgs, Extra...>;
  constexpr bool BIAS = has_arg<BBias, Extra...>;
  using C = BCfg<DH, DV>;
  constexpr bool DK = WHICH == 1;
  constexpr int MOUT = DK ? C::MQ : C::MV;     // 32-wide output slices
  // Q ring, dO ring (two slots each), then per slot 64 LSEs and 64 D values.
  __shared__ __attribute__((aligned(1024))) char smem[2 * C::H_BYTES + 2 * C::V_BYTES + 1024];
  debug_poison_lds(smem, sizeof(smem));
  char* const qring = smem;
  char* const gring = smem + 2 * C::H_BYTES;
  float* const sring = reinterpret_cast<float*>(smem + 2 * C::H_BYTES + 2 * C::V_BYTES);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int lr = lane & 31;

  // Low key tiles first (with causal masking they are seen by more rows).
  const int bid = blockIdx.x;
  int kt = bid / a.n_units;
  int bh = bid % a.n_units;
  if (!VAR && a.batch_major) {
    const int i2 = bid / a.heads_kv;
    kt = i2 % a.n_tiles_grid;
    bh = (i2 / a.n_tiles_grid) * a.heads_kv + bid % a.heads_kv;
  }
  const int b = bh / a.heads_kv;
  const int kvh = bh % a.heads_kv;
  const int32_t t_q_all = a.t_q;   // rows per head of LSE and D
  int32_t row_base = 0;            // packed row of the sequence's row 0
  int32_t key_base = 0;            // packed key of the sequence's key 0
  int32_t t_k_store = a.t_k;       // keys whose gradient this launch writes
  if constexpr (VAR) {
    const VArgs& va = pick<VArgs>(ex...);
    if (va.cu_q != nullptr) {
      const int sq = slot_seq(va.cu_k, va.n_seqs, a.t_k, kt, &kt);
      enter_seq<false>(a, va, sq, DK ? a.ks[2] : a.vs[2], &row_base, &key_base);
      if (kt < 0 || kt * kBr >= a.t_k) return;   // whole workgroup: a slot outside the sequence's tiles
      t_k_store = a.t_k;
    } else {
      const int len = clamp_len(va.kv_lens[b], a.t_k);
      a.q_offset += len - a.t_q;
      a.t_k = len;   // keys [len, T_k) are seen by no row: their gradients are written as 0
    }
  }

  const int key0 = kt * kBr + wave * kRowsW;   // first key of this wave
  const int key = key0 + lr;
  const bool key_ok = key < a.t_k;

  // K^T (and V^T) operands of this lane's key.
  u32x4 kreg[C::KS], vreg[DK ? C::MS : 1];
  {
    const uint16_t* kp = a.k + b * a.ks[0] + kvh * a.ks[1] + static_cast<int64_t>(key) * a.ks[2];
#pragma unroll
    for (int s = 0; s < C::KS; ++s)
      kreg[s] = key_ok ? *reinterpret_cast<const u32x4*>(kp + 16 * s + 8 * h) : u32x4{0, 0, 0, 0};
    if (DK) {
      const uint16_t* vp = a.v + b * a.vs[0] + kvh * a.vs[1] + static_cast<int64_t>(key) * a.vs[2];
#pragma unroll
      for (int s = 0; s < C::MS; ++s)
        vreg[s] = key_ok ? *reinterpret_cast<const u32x4*>(vp + 16 * s + 8 * h) : u32x4{0, 0, 0, 0};
    }
  }

  // Query rows that can see a key of the workgroup: pos_i >= first key
  // (causal) and pos_i - W + 1 <= last key (window).
  const int64_t wk0 = static_cast<int64_t>(kt) * kBr;
  int64_t i_lo = 0, i_hi = a.t_q;
  if (a.causal && wk0 - a.q_offset > i_lo) i_lo = wk0 - a.q_offset;
  if (a.window > 0 && wk0 + kBr - 1 - a.q_offset + a.window < i_hi) i_hi = wk0 + kBr - 1 - a.q_offset + a.window;
  if (VAR && wk0 >= a.t_k) i_hi = 0;   // per-batch lengths: a tile past L_b sees no row
  if (i_lo > i_hi) i_lo = i_hi;
  const int qt_lo = static_cast<int>(i_lo / kBc);
  const int n_qt = i_hi > i_lo ? static_cast<int>((i_hi + kBc - 1) / kBc) - qt_lo : 0;
  const int n_units = n_qt * a.group;          // (query head of the group, query tile)

  const int q_row_bytes = static_cast<int>(a.qs[2]) * 2;
  const int g_row_bytes = static_cast<int>(a.os[2]) * 2;
  int qoff[C::H_DMA], goff[C::V_DMA];
  dma_offsets<C::H_RB, C::H_DMA>(wave, lane, q_row_bytes, qoff);
  dma_offsets<C::V_RB, C::V_DMA>(wave, lane, g_row_bytes, goff);
  auto unit = [&](int u, int& hq, int& i0) {
    hq = kvh * a.group + u / n_qt;
    i0 = (qt_lo + u % n_qt) * kBc;
  };
  auto gload = [&](int u) {
    int hq, i0;
    unit(u, hq, i0);
    const int slot = u & 1;
    dma_tile<C::H_RB, C::H_DMA>(a.q + b * a.qs[0] + hq * a.qs[1], i0, a.t_q, q_row_bytes,
                                qring + slot * C::H_BYTES, wave, qoff);
    dma_tile<C::V_RB, C::V_DMA>(a.d_o + b * a.os[0] + hq * a.os[1], i0, a.t_q, g_row_bytes,
                                gring + slot * C::V_BYTES, wave, goff);
    if (wave == 0) {
      // 64 LSEs and 64 D values of the tile's rows (4 bytes per lane; rows
      // past T_q read as 0 and are masked).
      const int64_t r0 = (static_cast<int64_t>(b) * a.heads_q + hq) * t_q_all + row_base + i0;
      const int64_t n = a.t_q - i0;
      const auto rl = make_rsrc(a.lse + r0, n * 4);
      const auto rd = make_rsrc(a.dd + r0, n * 4);
      lds_copy<4>(rl, (__attribute__((address_space(3))) void*)(sring + slot * 128), lane * 4);
      lds_copy<4>(rd, (__attribute__((address_space(3))) void*)(sring + slot * 128 + 64), lane * 4);
    }
  };

  f32x16 acc[MOUT];
#pragma unroll
  for (int i = 0; i < MOUT; ++i) acc[i] = f32x16{};

  auto dma_barrier = [&]() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  if (n_units > 0) gload(0);
  if (n_units > 1) gload(1);
  dma_barrier();

  const int last_key = key0 + kRowsW - 1;
  // Block q of a unit (rows r0 .. r0 + 31): does it hold a legal (row, key)
  // pair of this wave, and are all its pairs legal?
  auto block_flags = [&](int r0, bool& any, bool& full) {
    const int64_t pf = a.q_offset + r0, pl = a.q_offset + r0 + 31;
    any = key0 < a.t_k && r0 < a.t_q;
    if (a.causal && pl < key0) any = false;
    if (a.window > 0 && pf - a.window + 1 > last_key) any = false;
    full = last_key < a.t_k && r0 + 31 < a.t_q;
    if (a.causal && pf < last_key) full = false;
    if (a.window > 0 && pl - a.window + 1 > key0) full = false;
  };
  // S of block q (register r holds row 32 q + 8 (r / 4) + 4 h + (r % 4) of
  // the tile for this lane's key).
  auto scores = [&](const char* qt_, int q, f32x16& sacc) {
    sacc = f32x16{};
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      const u32x4 qop = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
          row_chunk<C::H_RB>(qt_, 32 * q + lr, s, h));
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(qop), as_bf16x8(kreg[s]), sacc, 0, 0, 0);
    }
  };
  // acc^T += A^T W for block q, A the tile at `at` read transposed, W packed.
  auto accumulate = [&](const char* at, int q, const unsigned* pk) {
#pragma unroll
    for (int kk2 = 0; kk2 < 2; ++kk2) {
      const u32x4 bop = {pk[4 * kk2], pk[4 * kk2 + 1], pk[4 * kk2 + 2], pk[4 * kk2 + 3]};
#pragma unroll
      for (int mo = 0; mo < MOUT; ++mo) {
        u32x2 lo, hi;
        if (DK) {
          lo = tr_read(tr_addr<C::H_RB>(at, 32 * q, kk2, mo, 0, lane));
          hi = tr_read(tr_addr<C::H_RB>(at, 32 * q, kk2, mo, 1, lane));
        } else {
          lo = tr_read(tr_addr<C::V_RB>(at, 32 * q, kk2, mo, 0, lane));
          hi = tr_read(tr_addr<C::V_RB>(at, 32 * q, kk2, mo, 1, lane));
        }
        const u32x4 aop = {lo[0], lo[1], hi[0], hi[1]};
        acc[mo] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(aop), as_bf16x8(bop), acc[mo], 0, 0, 0);
      }
    }
  };
  // P of a fully legal block, packed to bf16 (dV only).
  // Bias of this lane's key for the 16 rows it holds in block q of the unit
  // (hq, i0) (BIAS only): one dword each through a buffer that ends at the
  // unit's last row and key.
  auto load_bias = [&](int hq, int i0, int q, float* mb) {
    if constexpr (BIAS) {
      const BBias& bb = pick<BBias>(ex...);
      const int rows_u = a.t_q - i0 < kBc ? a.t_q - i0 : kBc;
      const auto rs = make_rsrc(bb.bias + b * bb.bs[0] + hq * bb.bs[1] +
                                    static_cast<int64_t>(row_base + i0) * bb.bs[2] + key_base,
                                (static_cast<int64_t>(rows_u - 1) * bb.bs[2] + a.t_k) * 4);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rr = 32 * q + 8 * (r >> 2) + 4 * h + (r & 3);
        mb[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                              rs, (rr * static_cast<int>(bb.bs[2]) + key) * 4, 0, 0));
      }
    }
  };
  // One bias entry: row 32 q + 8 (r / 4) + 4 h + r % 4 of the unit, this
  // lane's key.
  auto bias_at = [&](int hq, int i0, int q, int r) -> float {
    if constexpr (BIAS) {
      const BBias& bb = pick<BBias>(ex...);
      const int rows_u = a.t_q - i0 < kBc ? a.t_q - i0 : kBc;
      const auto rs = make_rsrc(bb.bias + b * bb.bs[0] + hq * bb.bs[1] +
                                    static_cast<int64_t>(row_base + i0) * bb.bs[2] + key_base,
                                (static_cast<int64_t>(rows_u - 1) * bb.bs[2] + a.t_k) * 4);
      const int rr = 32 * q + 8 * (r >> 2) + 4 * h + (r & 3);
      return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                           rs, (rr * static_cast<int>(bb.bs[2]) + key) * 4, 0, 0));
    } else {
      return 0.0f;
    }
  };
  // Exponent offset of a row: -LSE (base 2) plus its bias entry; a row with
  // no legal key (LSE = -inf) gets weight 0 (with a bias a full block can
  // hold one).
  auto zoff = [&](float lse, float mbias) {
    if constexpr (BIAS) {
      const float l2 = lse == -INFINITY ? INFINITY : lse * kLog2e;
      return fmaf(mbias, kLog2e, -l2);
    } else {
      return -lse * kLog2e;
    }
  };
  auto probs_full = [&](const float* st_, int hq, int i0, int q, const f32x16& sacc, unsigned* pk) {
    f32x4 l4[4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
      l4[g] = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
          (const __attribute__((address_space(3))) char*)(st_) + (32 * q + 8 * g + 4 * h) * 4);
    float mb[16];
    load_bias(hq, i0, q, mb);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 2 * i;
      const float p0 = fast_exp2(fmaf(sacc[r], a.scale_log2, zoff(l4[r >> 2][r & 3], BIAS ? mb[r] : 0.0f)));
      const float p1 =
          fast_exp2(fmaf(sacc[r + 1], a.scale_log2, zoff(l4[(r + 1) >> 2][(r + 1) & 3], BIAS ? mb[r + 1] : 0.0f)));
      pk[i] = pack_bf16(p0, p1);
    }
  };
  // One MFMA then BWD_SCHED VALU instructions, n times.
  auto interleave = [&](int n) {
    if (BWD_SCHED > 0) {
      for (int i = 0; i < n; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, BWD_SCHED, 0);
      }
    }
  };
  for (int u = 0; u < n_units; ++u) {
    int hq, i0;
    unit(u, hq, i0);
    const int slot = u & 1;
    const char* qt_ = qring + slot * C::H_BYTES;
    const char* gt_ = gring + slot * C::V_BYTES;
    const float* st_ = sring + slot * 128;
    bool any_b[2], full_b[2];
    block_flags(i0, any_b[0], full_b[0]);
    block_flags(i0 + 32, any_b[1], full_b[1]);
    if (!DK && BWD_PIPE && !BIAS && full_b[0] && full_b[1]) {
      // Both blocks fully legal: S of both blocks first, then block 0's
      // weights under block 1's score MFMAs and block 1's weights under
      // block 0's accumulation MFMAs (no dependence between them).
      f32x16 s0, s1;
      unsigned pk0[8], pk1[8];
      scores(qt_, 0, s0);
      if (BWD_SCHED > 0) __builtin_amdgcn_sched_barrier(0);
      scores(qt_, 1, s1);
      probs_full(st_, hq, i0, 0, s0, pk0);
      interleave(C::KS);
      accumulate(gt_, 0, pk0);
      probs_full(st_, hq, i0, 1, s1, pk1);
      interleave(2 * MOUT);
      accumulate(gt_, 1, pk1);
    } else {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int r0 = i0 + 32 * q;                 // first row of the block
      const bool any = any_b[q], full = full_b[q];
      if (!any) continue;

      // S = Q K^T (and dP = dO V^T): register r holds row
      // r0 + 8 (r / 4) + 4 h + (r % 4) of this lane's key.
      f32x16 sacc = f32x16{}, dacc = f32x16{};
#pragma unroll
      for (int s = 0; s < C::KS; ++s) {
        const u32x4 qop = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
            row_chunk<C::H_RB>(qt_, 32 * q + lr, s, h));
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(qop), as_bf16x8(kreg[s]), sacc, 0, 0, 0);
      }
      if (DK) {
#pragma unroll
        for (int s = 0; s < C::MS; ++s) {
          const u32x4 gop = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
              row_chunk<C::V_RB>(gt_, 32 * q + lr, s, h));
          dacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(gop), as_bf16x8(vreg[s]), dacc, 0, 0, 0);
        }
      }
      // LSE (and D) of the 16 rows this lane holds (with a bias, read per pair
      // where they are used, with the pair's bias entries: fewer live
      // registers).
      f32x4 l4[4], d4[4];
      if constexpr (!BIAS) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          l4[g] = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
              (const __attribute__((address_space(3))) char*)(st_) + (32 * q + 8 * g + 4 * h) * 4);
          if (DK)
            d4[g] = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
                (const __attribute__((address_space(3))) char*)(st_) + 256 + (32 * q + 8 * g + 4 * h) * 4);
        }
      }
      // Straight-line over the 16 pairs (no branch per score); a partly legal
      // block then zeroes its illegal pairs.
      float wv[16];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float mb2[2], lse2p[2], dd2p[2];
        if constexpr (BIAS) {
          const int off = (32 * q + 8 * (i >> 1) + 4 * h + 2 * (i & 1)) * 4;
          const f32x2 lp = *reinterpret_cast<const __attribute__((address_space(3))) f32x2*>(
              (const __attribute__((address_space(3))) char*)(st_) + off);
          lse2p[0] = lp[0];
          lse2p[1] = lp[1];
          if (DK) {
            const f32x2 dp = *reinterpret_cast<const __attribute__((address_space(3))) f32x2*>(
                (const __attribute__((address_space(3))) char*)(st_) + 256 + off);
            dd2p[0] = dp[0];
            dd2p[1] = dp[1];
          }
#pragma unroll
          for (int e = 0; e < 2; ++e) mb2[e] = bias_at(hq, i0, q, 2 * i + e);
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int r = 2 * i + e;
          const float lse_r = BIAS ? lse2p[e] : l4[r >> 2][r & 3];
          const float p = fast_exp2(fmaf(sacc[r], a.scale_log2, zoff(lse_r, BIAS ? mb2[e] : 0.0f)));
          const float dd_r = BIAS ? dd2p[e] : d4[r >> 2][r & 3];
          wv[r] = DK ? p * (dacc[r] - dd_r) : p;   // dS (eq 33.7) or P
        }
      }
      if (!full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = r0 + 8 * (r >> 2) + 4 * h + (r & 3);
          const int64_t pos = a.q_offset + row;
          bool ok = key_ok && row < a.t_q;
          ok = ok && !(a.causal && key > pos);
          ok = ok && !(a.window > 0 && key < pos - a.window + 1);
          wv[r] = ok ? wv[r] : 0.0f;
        }
      }
      unsigned pk[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) pk[i] = pack_bf16(wv[2 * i], wv[2 * i + 1]);
      // dV^T += dO^T P or dK^T += Q^T dS (A = transposed reads of the tile).
      accumulate(DK ? qt_ : gt_, q, pk);
    }
    }
    // End of unit u: this wave's copies of unit u + 1 are done, every wave is
    // done with slot u & 1; copy unit u + 2 into it.
    dma_barrier();
    if (u + 2 < n_units) gload(u + 2);
  }

  // dK = scale dS^T Q (eq 33.8) or dV = P^T dO (eq 33.6); keys no row sees get 0.
  if (!(VAR ? key < t_k_store : key_ok)) return;
  const float sc = DK ? a.scale_log2 * kLn2 : 1.0f;
  uint16_t* op = DK ? a.out + b * a.ks[0] + kvh * a.ks[1] + static_cast<int64_t>(key) * a.ks[2]
                    : a.out + b * a.vs[0] + kvh * a.vs[1] + static_cast<int64_t>(key) * a.vs[2];
#pragma unroll
  for (int mo = 0; mo < MOUT; ++mo) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dcol = 32 * mo + 8 * g + 4 * h;
      u32x2 w;
      w[0] = pack_bf16(acc[mo][4 * g] * sc, acc[mo][4 * g + 1] * sc);
      w[1] = pack_bf16(acc[mo][4 * g + 2] * sc, acc[mo][4 * g + 3] * sc);
      *reinterpret_cast<u32x2*>(op + dcol) = w;
    }
  }
#endif
}

// ---------------------------------------------------------------------------
// dK and dV in one pass (calls without a bias: dense batches, packed
// sequences, per-batch KV lengths)
// ---------------------------------------------------------------------------
// The workgroup's 128 keys as in the dK / dV kernels (wavefront w owns keys
// 32 w .. 32 w + 31, K^T resident as the B operand of S = Q K^T), but each
// streamed block of 32 query rows serves both gradients: S = Q K^T and
// dP = dO V^T are computed once, then dV^T += dO^T P and dK^T += Q^T dS.  So a
// (row, key) pair costs 4 products here and 3 in the dQ kernel, 7 in all
// instead of the 8 of separate dV and dK launches (each of which recomputes
// S).  Two accumulator sets leave no registers for V^T, so the workgroup's
// 128 V rows are copied into LDS once and read as the B operand of dP
// (16-byte row reads); Q / dO stream in 32-row tiles through rings of NS
// slots.  The shape used: W = 4 wavefronts (128 keys) with two slots, which
// keeps the rings and the V rows within 80 KB (two workgroups per CU).  The
// template also builds, for d_h = d_v = 128, W = 8 (256 keys, one workgroup
// per CU) with four slots, each streamed tile serving twice the keys and
// copied three units ahead (BWD_FUSED_W8; measured slower, off).
constexpr int kBf = 32;   // rows per streamed tile

#ifndef BWD_FUSED_VAR
#define BWD_FUSED_VAR 1   // 1: packed sequences and per-batch KV lengths also take the fused launch
#endif
#ifndef BWD_FUSED_W8
#define BWD_FUSED_W8 0    // 1: the fused d 128 kernel as 8 wavefronts with a 4-slot ring (measured slower)
#endif

template <int DH, int DV, int W>
struct FusedCfg {
  static constexpr int KS = DH / 16;
  static constexpr int MS = DV / 16;
  static constexpr int MQ = DH / 32;
  static constexpr int MV = DV / 32;
  static constexpr int H_RB = DH * 2;
  static constexpr int V_RB = DV * 2;
  static constexpr int H_BYTES = kBf * H_RB;
  static constexpr int V_BYTES = kBf * V_RB;
  static constexpr int H_DMA = H_BYTES / 1024 / W;   // 1 KB copies per wavefront per tile
  static constexpr int V_DMA = V_BYTES / 1024 / W;
  static constexpr int KEYS = kRowsW * W;            // keys per workgroup
  static constexpr int VS_BYTES = KEYS * V_RB;       // the workgroup's V rows
  static constexpr int VS_DMA = VS_BYTES / 1024 / W;
  static_assert(H_DMA >= 1 && V_DMA >= 1 && H_BYTES % (1024 * W) == 0 && V_BYTES % (1024 * W) == 0,
                "each wavefront copies whole 1 KB blocks of a tile");
};

template <int DH, int DV, int W, int NS, class... Extra>
__global__ __launch_bounds__(64 * W, 2) void bwd_kvf_mfma_kernel(BArgs a, uint16_t* d_v, Extra... ex) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr bool VAR = has_arg<VArgs, Extra...>;
  using C = FusedCfg<DH, DV, W>;
  static_assert(!VAR || C::KEYS == kBr, "packed slots are counted in 128-key tiles");
  // Q ring, dO ring (NS slots each), the V rows of the workgroup's keys, then
  // per slot 64 LSEs and 64 D values.
  __shared__ __attribute__((aligned(1024))) char smem[NS * (C::H_BYTES + C::V_BYTES) + C::VS_BYTES + NS * 512];
  debug_poison_lds(smem, sizeof(smem));
  char* const qring = smem;
  char* const gring = smem + NS * C::H_BYTES;
  char* const vstage = smem + NS * (C::H_BYTES + C::V_BYTES);
  float* const sring = reinterpret_cast<float*>(smem + NS * (C::H_BYTES + C::V_BYTES) + C::VS_BYTES);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int lr = lane & 31;

  // Low key tiles first (with causal masking they are seen by more rows).
  const int bid = blockIdx.x;
  int kt = bid / a.n_units;
  int bh = bid % a.n_units;
  if (!VAR && a.batch_major) {
    const int i2 = bid / a.heads_kv;
    kt = i2 % a.n_tiles_grid;
    bh = (i2 / a.n_tiles_grid) * a.heads_kv + bid % a.heads_kv;
  }
  const int b = bh / a.heads_kv;
  const int kvh = bh % a.heads_kv;
  // Variable-length batches, as in the separate dK / dV launches: a packed
  // slot enters its sequence (sizes, pointers and q_offset its own; LSE and
  // D keep the packed rows); per-batch KV lengths cut T_k (keys past it see
  // no row and get 0).
  const int32_t t_q_all = a.t_q;   // rows per head of LSE and D
  int32_t row_base = 0;            // packed row of the sequence's row 0
  int32_t t_k_store = a.t_k;       // keys whose gradients this launch writes
  if constexpr (VAR) {
    const VArgs& va = pick<VArgs>(ex...);
    if (va.cu_q != nullptr) {
      int32_t key_base = 0;
      const int sq = slot_seq(va.cu_k, va.n_seqs, a.t_k, kt, &kt);
      enter_seq<false>(a, va, sq, a.ks[2], &row_base, &key_base);
      d_v += static_cast<int64_t>(key_base) * a.vs[2];
      if (kt < 0 || kt * C::KEYS >= a.t_k) return;   // whole workgroup: a slot outside the sequence's tiles
      t_k_store = a.t_k;
    } else {
      const int len = clamp_len(va.kv_lens[b], a.t_k);
      a.q_offset += len - a.t_q;
      a.t_k = len;
    }
  }

  const int key0 = kt * C::KEYS + wave * kRowsW;   // first key of this wave
  const int key = key0 + lr;
  const bool key_ok = key < a.t_k;

  // K^T operand of this lane's key.
  u32x4 kreg[C::KS];
  {
    const uint16_t* kp = a.k + b * a.ks[0] + kvh * a.ks[1] + static_cast<int64_t>(key) * a.ks[2];
#pragma unroll
    for (int s = 0; s < C::KS; ++s)
      kreg[s] = key_ok ? *reinterpret_cast<const u32x4*>(kp + 16 * s + 8 * h) : u32x4{0, 0, 0, 0};
  }

  // Query rows that can see a key of the workgroup.
  const int64_t wk0 = static_cast<int64_t>(kt) * C::KEYS;
  int64_t i_lo = 0, i_hi = a.t_q;
  if (a.causal && wk0 - a.q_offset > i_lo) i_lo = wk0 - a.q_offset;
  if (a.window > 0 && wk0 + C::KEYS - 1 - a.q_offset + a.window < i_hi) i_hi = wk0 + C::KEYS - 1 - a.q_offset + a.window;
  if (VAR && wk0 >= a.t_k) i_hi = 0;   // per-batch lengths: a tile past L_b sees no row
  if (i_lo > i_hi) i_lo = i_hi;
  const int qt_lo = static_cast<int>(i_lo / kBf);
  const int n_qt = i_hi > i_lo ? static_cast<int>((i_hi + kBf - 1) / kBf) - qt_lo : 0;
  const int n_units = n_qt * a.group;          // (query head of the group, 32-row tile)

  const int q_row_bytes = static_cast<int>(a.qs[2]) * 2;
  const int g_row_bytes = static_cast<int>(a.os[2]) * 2;
  const int v_row_bytes = static_cast<int>(a.vs[2]) * 2;
  int qoff[C::H_DMA], goff[C::V_DMA];
  dma_offsets<C::H_RB, C::H_DMA>(wave, lane, q_row_bytes, qoff);
  dma_offsets<C::V_RB, C::V_DMA>(wave, lane, g_row_bytes, goff);
  // Units in order: (head of the group g, row tile qt), qt fastest.  The next
  // unit to copy is tracked incrementally: its Q / dO tile addresses, the
  // bytes left to the end of the head's rows and its first LSE / D index
  // advance by one row tile per unit and move to the next head's first tile
  // when qt wraps (additions only; no 64-bit products per unit).  At
  // d_h = d_v = 128 that scalar state costs the kernel registers it does not
  // have (a further spill, 3 % slower there), so it recomputes each unit's
  // addresses from the head and row tile instead.
  constexpr bool kIncr = DH + DV < 256;
  int l_u = 0, l_g = 0, l_qt = 0;
  const int64_t i_first = static_cast<int64_t>(qt_lo) * kBf;
  const char* q_head = reinterpret_cast<const char*>(a.q + b * a.qs[0] + static_cast<int64_t>(kvh) * a.group * a.qs[1]);
  const char* g_head = reinterpret_cast<const char*>(a.d_o + b * a.os[0] + static_cast<int64_t>(kvh) * a.group * a.os[1]);
  const char* q_next = q_head + i_first * q_row_bytes;
  const char* g_next = g_head + i_first * g_row_bytes;
  int64_t rows_left = a.t_q - i_first;   // rows from the next unit's first row to T_q
  int64_t q_left = rows_left * q_row_bytes, g_left = rows_left * g_row_bytes;
  int64_t r_next = (static_cast<int64_t>(b) * a.heads_q + static_cast<int64_t>(kvh) * a.group) * t_q_all + row_base +
                   i_first;
  auto gload_next = [&]() {
    if constexpr (!kIncr) {
      const int hq = kvh * a.group + l_g;
      const int i0 = (qt_lo + l_qt) * kBf;
      const int slot = l_u % NS;
      ++l_u;
      if (++l_qt == n_qt) {
        l_qt = 0;
        ++l_g;
      }
      dma_tile<C::H_RB, C::H_DMA>(a.q + b * a.qs[0] + hq * a.qs[1], i0, a.t_q, q_row_bytes,
                                  qring + slot * C::H_BYTES, wave, qoff);
      dma_tile<C::V_RB, C::V_DMA>(a.d_o + b * a.os[0] + hq * a.os[1], i0, a.t_q, g_row_bytes,
                                  gring + slot * C::V_BYTES, wave, goff);
      if (wave == 0) {
        const int64_t r0 = (static_cast<int64_t>(b) * a.heads_q + hq) * t_q_all + row_base + i0;
        const int64_t n = a.t_q - i0;
        const auto rl = make_rsrc(a.lse + r0, n * 4);
        const auto rd = make_rsrc(a.dd + r0, n * 4);
        lds_copy<4>(rl, (__attribute__((address_space(3))) void*)(sring + slot * 128), lane * 4);
        lds_copy<4>(rd, (__attribute__((address_space(3))) void*)(sring + slot * 128 + 64), lane * 4);
      }
      return;
    }
    const int slot = l_u % NS;
    ++l_u;
    const auto rq = make_rsrc(q_next, q_left);
    const auto rg = make_rsrc(g_next, g_left);
#pragma unroll
    for (int j = 0; j < C::H_DMA; ++j)
      lds_copy<16>(rq, (__attribute__((address_space(3))) void*)(qring + slot * C::H_BYTES + (wave * C::H_DMA + j) * 1024), qoff[j]);
#pragma unroll
    for (int j = 0; j < C::V_DMA; ++j)
      lds_copy<16>(rg, (__attribute__((address_space(3))) void*)(gring + slot * C::V_BYTES + (wave * C::V_DMA + j) * 1024), goff[j]);
    if (wave == 0) {
      // LSEs and D values of the tile's rows, 4 bytes per lane (rows past
      // T_q read as 0 and are masked; the upper 32 are not used).
      const auto rl = make_rsrc(a.lse + r_next, rows_left * 4);
      const auto rd = make_rsrc(a.dd + r_next, rows_left * 4);
      lds_copy<4>(rl, (__attribute__((address_space(3))) void*)(sring + slot * 128), lane * 4);
      lds_copy<4>(rd, (__attribute__((address_space(3))) void*)(sring + slot * 128 + 64), lane * 4);
    }
    if (++l_qt == n_qt) {   // next head of the group, from its first row tile
      l_qt = 0;
      q_head += a.qs[1] * 2;
      g_head += a.os[1] * 2;
      q_next = q_head + i_first * q_row_bytes;
      g_next = g_head + i_first * g_row_bytes;
      rows_left = a.t_q - i_first;
      q_left = rows_left * q_row_bytes;
      g_left = rows_left * g_row_bytes;
      r_next += t_q_all - static_cast<int64_t>(n_qt - 1) * kBf;
    } else {
      q_next += kBf * q_row_bytes;
      g_next += kBf * g_row_bytes;
      rows_left -= kBf;
      q_left -= kBf * q_row_bytes;
      g_left -= kBf * g_row_bytes;
      r_next += kBf;
    }
  };

  f32x16 acck[C::MQ], accv[C::MV];
#pragma unroll
  for (int i = 0; i < C::MQ; ++i) acck[i] = f32x16{};
#pragma unroll
  for (int i = 0; i < C::MV; ++i) accv[i] = f32x16{};

  // Wait until this wave's copies of unit u have landed (the copies of the
  // units after it, issued later, may still be in flight: in-order
  // completion), then the workgroup barrier; a bare s_barrier, since the
  // fence __syncthreads adds would also wait for those later copies.
  constexpr int kOps = C::H_DMA + C::V_DMA;   // copies per unit and wavefront (+2 on wavefront 0)
  const int ops = kOps + (wave == 0 ? 2 : 0);
  // `last` = the last unit whose copies were issued.
  auto unit_barrier = [&](int u, int last) {
    int later = (last < n_units - 1 ? last : n_units - 1) - u;   // units issued after u
    if (later < 0) later = 0;
    wait_vm_upto<(NS - 1) * (kOps + 2)>(later * ops);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };

  // The workgroup's V rows (rows past T_k arrive as zeros), then the first
  // two units.
  {
    int vsoff[C::VS_DMA];
    dma_offsets<C::V_RB, C::VS_DMA>(wave, lane, v_row_bytes, vsoff);
    dma_tile<C::V_RB, C::VS_DMA>(a.v + b * a.vs[0] + kvh * a.vs[1], wk0, a.t_k, v_row_bytes, vstage, wave,
                                 vsoff);
  }
#pragma unroll
  for (int u = 0; u < NS; ++u)
    if (u < n_units) gload_next();
  unit_barrier(0, NS - 1);

  const int last_key = key0 + kRowsW - 1;
  int c_qt = 0;   // row tile of unit u
  for (int u = 0; u < n_units; ++u) {
    const int i0 = (qt_lo + c_qt) * kBf;
    if (++c_qt == n_qt) c_qt = 0;
    const int slot = u % NS;
    const char* qt_ = qring + slot * C::H_BYTES;
    const char* gt_ = gring + slot * C::V_BYTES;
    const float* st_ = sring + slot * 128;
    // Does the block hold a legal (row, key) pair of this wave, and are all
    // its pairs legal?
    const int64_t pf = a.q_offset + i0, pl = a.q_offset + i0 + 31;
    bool any = key0 < a.t_k && i0 < a.t_q;
    if (a.causal && pl < key0) any = false;
    if (a.window > 0 && pf - a.window + 1 > last_key) any = false;
    bool full = last_key < a.t_k && i0 + 31 < a.t_q;
    if (a.causal && pf < last_key) full = false;
    if (a.window > 0 && pl - a.window + 1 > key0) full = false;
    if (any) {
      // S = Q K^T and dP = dO V^T: register r holds row i0 + 8 (r / 4) +
      // 4 h + (r % 4) for this lane's key.
      f32x16 sacc = f32x16{}, dacc = f32x16{};
#pragma unroll
      for (int s = 0; s < C::KS; ++s) {
        const u32x4 qop = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
            row_chunk<C::H_RB>(qt_, lr, s, h));
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(qop), as_bf16x8(kreg[s]), sacc, 0, 0, 0);
      }
#pragma unroll
      for (int s = 0; s < C::MS; ++s) {
        const u32x4 gop = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
            row_chunk<C::V_RB>(gt_, lr, s, h));
        const u32x4 vop = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
            row_chunk<C::V_RB>(vstage, wave * kRowsW + lr, s, h));
        dacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(gop), as_bf16x8(vop), dacc, 0, 0, 0);
      }
      // P (eq 33.6's weights) and dS = P (dP - D) (eq 33.7), packed to bf16.
      // Straight-line (no branch per score, so the LDS reads of LSE and D are
      // scheduled ahead of their use); a partly legal block then zeroes its
      // illegal pairs.
      __builtin_amdgcn_sched_barrier(0);   // the products above stay above
      float w[16], dsv[16];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int off = (8 * (i >> 1) + 4 * h + 2 * (i & 1)) * 4;
        const f32x2 lp = *reinterpret_cast<const __attribute__((address_space(3))) f32x2*>(
            (const __attribute__((address_space(3))) char*)(st_) + off);
        const f32x2 dp = *reinterpret_cast<const __attribute__((address_space(3))) f32x2*>(
            (const __attribute__((address_space(3))) char*)(st_) + 256 + off);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int r = 2 * i + e;
          w[r] = fast_exp2(fmaf(sacc[r], a.scale_log2, -lp[e] * kLog2e));
          dsv[r] = w[r] * (dacc[r] - dp[e]);
        }
      }
      if (!full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = i0 + 8 * (r >> 2) + 4 * h + (r & 3);
          const int64_t pos = a.q_offset + row;
          bool ok = key_ok && row < a.t_q;
          ok = ok && !(a.causal && key > pos);
          ok = ok && !(a.window > 0 && key < pos - a.window + 1);
          w[r] = ok ? w[r] : 0.0f;
          dsv[r] = ok ? dsv[r] : 0.0f;
        }
      }
      unsigned pk[8], pd[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pk[i] = pack_bf16(w[2 * i], w[2 * i + 1]);
        pd[i] = pack_bf16(dsv[2 * i], dsv[2 * i + 1]);
      }
      __builtin_amdgcn_sched_barrier(0);
      // dV^T += dO^T P and dK^T += Q^T dS (A = transposed reads of the tiles).
      // Step i = (kk2, then the MV dV slices, then the MQ dK slices); with
      // kAhead the A operand of step i + 1 is read before the product of
      // step i, so each product waits only for reads issued a step earlier
      // instead of for its own.  Not at d_h = d_v = 128, which has no
      // registers for it (4 more spilled, 6 % slower).
      constexpr bool kAhead = BWD_READ_AHEAD && DH + DV < 256;
      if constexpr (kAhead) {
        constexpr int kSteps = 2 * (C::MV + C::MQ);
        auto a_op = [&](int i) -> u32x4 {
          const int kk2 = i / (C::MV + C::MQ), j = i % (C::MV + C::MQ);
          const bool dv = j < C::MV;
          const int mo = dv ? j : j - C::MV;
          const lds_char* p0 = dv ? tr_addr<C::V_RB>(gt_, 0, kk2, mo, 0, lane) : tr_addr<C::H_RB>(qt_, 0, kk2, mo, 0, lane);
          const lds_char* p1 = dv ? tr_addr<C::V_RB>(gt_, 0, kk2, mo, 1, lane) : tr_addr<C::H_RB>(qt_, 0, kk2, mo, 1, lane);
          const u32x2 lo = tr_read(p0);
          const u32x2 hi = tr_read(p1);
          return u32x4{lo[0], lo[1], hi[0], hi[1]};
        };
        u32x4 cur = a_op(0);
#pragma unroll
        for (int i = 0; i < kSteps; ++i) {
          u32x4 nxt = cur;
          if (i + 1 < kSteps) nxt = a_op(i + 1);
          const int kk2 = i / (C::MV + C::MQ), j = i % (C::MV + C::MQ);
          if (j < C::MV) {
            const u32x4 bp = {pk[4 * kk2], pk[4 * kk2 + 1], pk[4 * kk2 + 2], pk[4 * kk2 + 3]};
            accv[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(cur), as_bf16x8(bp), accv[j], 0, 0, 0);
          } else {
            const u32x4 bd = {pd[4 * kk2], pd[4 * kk2 + 1], pd[4 * kk2 + 2], pd[4 * kk2 + 3]};
            acck[j - C::MV] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(cur), as_bf16x8(bd), acck[j - C::MV], 0, 0, 0);
          }
          cur = nxt;
        }
        // Keep that order: the first operand's two reads, then per step the
        // next operand's two reads and the step's product.
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int i = 0; i < kSteps; ++i) {
          if (i + 1 < kSteps) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
      } else {
#pragma unroll
        for (int kk2 = 0; kk2 < 2; ++kk2) {
          const u32x4 bp = {pk[4 * kk2], pk[4 * kk2 + 1], pk[4 * kk2 + 2], pk[4 * kk2 + 3]};
          const u32x4 bd = {pd[4 * kk2], pd[4 * kk2 + 1], pd[4 * kk2 + 2], pd[4 * kk2 + 3]};
#pragma unroll
          for (int mo = 0; mo < C::MV; ++mo) {
            const u32x2 lo = tr_read(tr_addr<C::V_RB>(gt_, 0, kk2, mo, 0, lane));
            const u32x2 hi = tr_read(tr_addr<C::V_RB>(gt_, 0, kk2, mo, 1, lane));
            const u32x4 aop = {lo[0], lo[1], hi[0], hi[1]};
            accv[mo] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(aop), as_bf16x8(bp), accv[mo], 0, 0, 0);
          }
#pragma unroll
          for (int mo = 0; mo < C::MQ; ++mo) {
            const u32x2 lo = tr_read(tr_addr<C::H_RB>(qt_, 0, kk2, mo, 0, lane));
            const u32x2 hi = tr_read(tr_addr<C::H_RB>(qt_, 0, kk2, mo, 1, lane));
            const u32x4 aop = {lo[0], lo[1], hi[0], hi[1]};
            acck[mo] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(aop), as_bf16x8(bd), acck[mo], 0, 0, 0);
          }
        }
      }
    }
    // Unit u done: unit u + 1's copies have landed, every wave is done with
    // slot u % NS, which takes unit u + NS.
    if (u + 1 < n_units) unit_barrier(u + 1, u + NS - 1);
    if (u + NS < n_units) gload_next();
  }

  // dK = scale dS^T Q (eq 33.8) and dV = P^T dO (eq 33.6); keys no row sees get 0.
  if (!(VAR ? key < t_k_store : key_ok)) return;
  const float sc = a.scale_log2 * kLn2;
  uint16_t* kp = a.out + b * a.ks[0] + kvh * a.ks[1] + static_cast<int64_t>(key) * a.ks[2];
  uint16_t* vp = d_v + b * a.vs[0] + kvh * a.vs[1] + static_cast<int64_t>(key) * a.vs[2];
#pragma unroll
  for (int mo = 0; mo < C::MQ; ++mo)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 w;
      w[0] = pack_bf16(acck[mo][4 * g] * sc, acck[mo][4 * g + 1] * sc);
      w[1] = pack_bf16(acck[mo][4 * g + 2] * sc, acck[mo][4 * g + 3] * sc);
      *reinterpret_cast<u32x2*>(kp + 32 * mo + 8 * g + 4 * h) = w;
    }
#pragma unroll
  for (int mo = 0; mo < C::MV; ++mo)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 w;
      w[0] = pack_bf16(accv[mo][4 * g], accv[mo][4 * g + 1]);
      w[1] = pack_bf16(accv[mo][4 * g + 2], accv[mo][4 * g + 3]);
      *reinterpret_cast<u32x2*>(vp + 32 * mo + 8 * g + 4 * h) = w;
    }
#endif
}

template <int DH, int DV, int W, int NS, class... X>
hipError_t launch_kvf(const BArgs& a, uint16_t* d_v, int64_t blocks, hipStream_t s, X... x) {
  hipLaunchKernelGGL((bwd_kvf_mfma_kernel<DH, DV, W, NS, X...>), dim3(static_cast<unsigned>(blocks)), dim3(64 * W),
                     0, s, a, d_v, x...);
  return hipGetLastError();
}

// The fused launch without or with variable lengths.
template <int DH, int DV>
hipError_t launch_kvf_var(const BArgs& a, const VArgs& va, bool var, uint16_t* d_v, int64_t blocks, hipStream_t s) {
  return var ? launch_kvf<DH, DV, kW, 2>(a, d_v, blocks, s, va) : launch_kvf<DH, DV, kW, 2>(a, d_v, blocks, s);
}

template <int DH, int DV, int WHICH, class... X>
void launch_kv_x(const BArgs& a, int64_t blocks, hipStream_t s, X... x) {
  hipLaunchKernelGGL((bwd_kv_mfma_kernel<DH, DV, WHICH, X...>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads),
                     0, s, a, x...);
}

// Packed sequences and a bias each add one trailing kernel argument; the
// instances without them keep the plain argument block.
template <int DH, int DV, int WHICH>
hipError_t launch_kv(const BArgs& a, const VArgs& va, const BBias& bb, int64_t blocks, hipStream_t s) {
  const bool var = va.cu_q != nullptr || va.kv_lens != nullptr;
  if (var && bb.bias != nullptr) launch_kv_x<DH, DV, WHICH>(a, blocks, s, va, bb);
  else if (var) launch_kv_x<DH, DV, WHICH>(a, blocks, s, va);
  else if (bb.bias != nullptr) launch_kv_x<DH, DV, WHICH>(a, blocks, s, bb);
  else launch_kv_x<DH, DV, WHICH>(a, blocks, s);
  return hipGetLastError();
}

template <int DH, int DV, class... X>
void launch_dq_x(const BArgs& a, int64_t blocks, hipStream_t s, X... x) {
  hipLaunchKernelGGL((bwd_dq_mfma_kernel<DH, DV, X...>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, s,
                     a, x...);
}

template <int DH, int DV>
hipError_t launch_dq(const BArgs& a, const VArgs& va, const BBias& bb, int64_t blocks, hipStream_t s) {
  const bool var = va.cu_q != nullptr || va.kv_lens != nullptr;
  if (var && bb.bias != nullptr) launch_dq_x<DH, DV>(a, blocks, s, va, bb);
  else if (var) launch_dq_x<DH, DV>(a, blocks, s, va);
  else if (bb.bias != nullptr) launch_dq_x<DH, DV>(a, blocks, s, bb);
  else launch_dq_x<DH, DV>(a, blocks, s);
  return hipGetLastError();
}

// The bias the MFMA kernels take: keys contiguous, row offsets of a unit
// (64 rows) and key offsets within 32 bits.
bool bias_ok(const Problem& pb) {
  if (pb.bias == nullptr) return true;
  return pb.bs[3] == 1 && pb.bs[2] < (int64_t(1) << 22) && pb.t_k < (int64_t(1) << 28);
}

BBias make_bias(const Problem& pb) {
  BBias bb{};
  bb.bias = pb.bias;
  for (int i = 0; i < 3; ++i) bb.bs[i] = pb.bs[i];
  return bb;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Dense batches whose K/V (all batches and KV heads) outgrows the 256 MB
// Infinity Cache run batch after batch, as in the prefill (measured on the
// backward: +2 to +18 % on three such shapes; at 134 MB and below the
// default order was as fast or up to 19 % faster).
int32_t batch_major(const Problem& pb) {
  const int64_t kv_bytes = pb.batch * pb.heads_kv * pb.t_k * (pb.d_h + pb.d_v) * 2;
  return pb.cu_q == nullptr && pb.batch > 1 && kv_bytes > (int64_t(256) << 20);
}

}  // namespace

// Takes bf16 problems with d_h, d_v in {64, 128}, positive scale, 16-byte
// aligned rows, sizes that fit 32-bit indices and no bias or a bias the
// kernels take (bias_ok); launches the
// dQ kernel, which also computes D from o and d_o into dd (for the dK / dV
// launches that follow).  Returns false when it does not apply.
bool launch_bwd_dq_mfma(const Problem& pb, int dtype, const void* q, const void* k, const void* v,
                        const void* o, const float* lse, const void* d_o, float* dd, void* d_q,
                        hipStream_t stream, hipError_t* err) {
  if (dtype != ATTN_BF16 || !bias_ok(pb)) return false;
  if (!((pb.d_h == 64 || pb.d_h == 128) && (pb.d_v == 64 || pb.d_v == 128))) return false;
  if (!(pb.scale_log2 > 0.0f)) return false;
  if (pb.t_q >= (int64_t(1) << 30) || pb.t_k >= (int64_t(1) << 30)) return false;
  if (pb.ks[2] >= (int64_t(1) << 24) || pb.vs[2] >= (int64_t(1) << 24)) return false;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(d_o) || !aligned16(d_q))
    return false;
  for (int i = 0; i < 3; ++i)
    if ((pb.qs[i] | pb.ks[i] | pb.vs[i] | pb.os[i]) & 7) return false;
  const bool packed = pb.cu_q != nullptr;
  const int64_t n_qtiles = packed ? pb.t_q / kBr + pb.n_seqs : (pb.t_q + kBr - 1) / kBr;
  const int64_t blocks = n_qtiles * pb.batch * pb.heads_q;
  if (blocks >= (int64_t(1) << 31) || pb.batch * pb.heads_q >= (int64_t(1) << 30)) return false;
  BArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.d_o = static_cast<const uint16_t*>(d_o);
  a.lse = lse;
  a.dd = dd;
  a.o = static_cast<const uint16_t*>(o);
  a.out = static_cast<uint16_t*>(d_q);
  for (int i = 0; i < 3; ++i) {
    a.qs[i] = pb.qs[i]; a.ks[i] = pb.ks[i]; a.vs[i] = pb.vs[i]; a.os[i] = pb.os[i];
  }
  a.q_offset = pb.q_offset;
  a.window = pb.window;
  a.t_q = static_cast<int32_t>(pb.t_q);
  a.t_k = static_cast<int32_t>(pb.t_k);
  a.heads_q = static_cast<int32_t>(pb.heads_q);
  a.heads_kv = static_cast<int32_t>(pb.heads_kv);
  a.group = pb.group;
  a.n_tiles_grid = static_cast<int32_t>(n_qtiles);
  const VArgs va{pb.cu_q, pb.cu_k, static_cast<int32_t>(pb.n_seqs), static_cast<int32_t>(n_qtiles), pb.kv_lens};
  const BBias bb = make_bias(pb);
  a.n_units = static_cast<int32_t>(pb.batch * pb.heads_q);
  a.scale_log2 = pb.scale_log2;
  a.causal = pb.causal;
  a.batch_major = batch_major(pb);
  if (blocks == 0) {
    *err = hipSuccess;
    return true;
  }
  if (pb.d_h == 128 && pb.d_v == 128) *err = launch_dq<128, 128>(a, va, bb, blocks, stream);
  else if (pb.d_h == 64 && pb.d_v == 128) *err = launch_dq<64, 128>(a, va, bb, blocks, stream);
  else if (pb.d_h == 128 && pb.d_v == 64) *err = launch_dq<128, 64>(a, va, bb, blocks, stream);
  else *err = launch_dq<64, 64>(a, va, bb, blocks, stream);
  return true;
}

// dK and dV with the MFMA kernels (same conditions as launch_bwd_dq_mfma).
bool launch_bwd_dkdv_mfma(const Problem& pb, int dtype, const void* q, const void* k, const void* v,
                          const float* lse, const void* d_o, const float* dd, void* d_k, void* d_v,
                          hipStream_t stream, hipError_t* err) {
  if (dtype != ATTN_BF16 || !bias_ok(pb)) return false;
  if (!((pb.d_h == 64 || pb.d_h == 128) && (pb.d_v == 64 || pb.d_v == 128))) return false;
  if (!(pb.scale_log2 > 0.0f)) return false;
  if (pb.t_q >= (int64_t(1) << 30) || pb.t_k >= (int64_t(1) << 30)) return false;
  if (pb.qs[2] >= (int64_t(1) << 24) || pb.os[2] >= (int64_t(1) << 24)) return false;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(d_o) || !aligned16(d_k) ||
      !aligned16(d_v))
    return false;
  for (int i = 0; i < 3; ++i)
    if ((pb.qs[i] | pb.ks[i] | pb.vs[i] | pb.os[i]) & 7) return false;
  const bool packed = pb.cu_q != nullptr;
  const int64_t n_ktiles = packed ? pb.t_k / kBr + pb.n_seqs : (pb.t_k + kBr - 1) / kBr;
  const int64_t blocks = n_ktiles * pb.batch * pb.heads_kv;
  if (blocks >= (int64_t(1) << 31) || pb.batch * pb.heads_kv >= (int64_t(1) << 30)) return false;
  BArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.d_o = static_cast<const uint16_t*>(d_o);
  a.lse = lse;
  a.dd = const_cast<float*>(dd);   // read only by the dK / dV kernels
  for (int i = 0; i < 3; ++i) {
    a.qs[i] = pb.qs[i]; a.ks[i] = pb.ks[i]; a.vs[i] = pb.vs[i]; a.os[i] = pb.os[i];
  }
  a.q_offset = pb.q_offset;
  a.window = pb.window;
  a.t_q = static_cast<int32_t>(pb.t_q);
  a.t_k = static_cast<int32_t>(pb.t_k);
  a.heads_q = static_cast<int32_t>(pb.heads_q);
  a.heads_kv = static_cast<int32_t>(pb.heads_kv);
  a.group = pb.group;
  a.n_tiles_grid = static_cast<int32_t>(n_ktiles);
  const VArgs va{pb.cu_q, pb.cu_k, static_cast<int32_t>(pb.n_seqs), static_cast<int32_t>(n_ktiles), pb.kv_lens};
  const BBias bb = make_bias(pb);
  a.n_units = static_cast<int32_t>(pb.batch * pb.heads_kv);
  a.scale_log2 = pb.scale_log2;
  a.causal = pb.causal;
  a.batch_major = batch_major(pb);
  *err = hipSuccess;
  if (blocks == 0) return true;
  // Without a bias: one launch for both gradients (dense batches, packed
  // sequences and per-batch KV lengths).
  const bool var = packed || pb.kv_lens != nullptr;
  if (BWD_FUSED && pb.bias == nullptr && (BWD_FUSED_VAR || !var)) {
    a.out = static_cast<uint16_t*>(d_k);
    uint16_t* dv = static_cast<uint16_t*>(d_v);
    if (BWD_FUSED_W8 && !var && pb.d_h == 128 && pb.d_v == 128) {
      // 256 keys per workgroup.
      const int64_t n8 = (pb.t_k + 2 * kBr - 1) / (2 * kBr);
      a.n_tiles_grid = static_cast<int32_t>(n8);
      *err = launch_kvf<128, 128, 8, 4>(a, dv, n8 * pb.batch * pb.heads_kv, stream);
    } else if (pb.d_h == 128 && pb.d_v == 128) {
      *err = launch_kvf_var<128, 128>(a, va, var, dv, blocks, stream);
    } else if (pb.d_h == 64 && pb.d_v == 128) {
      *err = launch_kvf_var<64, 128>(a, va, var, dv, blocks, stream);
    } else if (pb.d_h == 128 && pb.d_v == 64) {
      *err = launch_kvf_var<128, 64>(a, va, var, dv, blocks, stream);
    } else {
      *err = launch_kvf_var<64, 64>(a, va, var, dv, blocks, stream);
    }
    return true;
  }
  for (int which = 0; which < 2 && *err == hipSuccess; ++which) {
    a.out = static_cast<uint16_t*>(which ? d_k : d_v);
    if (pb.d_h == 128 && pb.d_v == 128) *err = which ? launch_kv<128, 128, 1>(a, va, bb, blocks, stream) : launch_kv<128, 128, 0>(a, va, bb, blocks, stream);
    else if (pb.d_h == 64 && pb.d_v == 128) *err = which ? launch_kv<64, 128, 1>(a, va, bb, blocks, stream) : launch_kv<64, 128, 0>(a, va, bb, blocks, stream);
    else if (pb.d_h == 128 && pb.d_v == 64) *err = which ? launch_kv<128, 64, 1>(a, va, bb, blocks, stream) : launch_kv<128, 64, 0>(a, va, bb, blocks, stream);
    else *err = which ? launch_kv<64, 64, 1>(a, va, bb, blocks, stream) : launch_kv<64, 64, 0>(a, va, bb, blocks, stream);
  }
  return true;
}

}  // namespace attn
