// MFMA prefill kernel for bf16 Q/K/V/O, d_h and d_v in {64, 128}.
//
// What it computes: for every query row, Algorithm 33.1 of "Chapter 33
// 推理计算优化" §33.2 over key tiles of 64 (128 in the large shape), i.e. exact softmax attention
// (eq 33.2) with the running statistics (m, l, u) of eq 33.3 merged tile by
// tile (eqs 33.4-33.5).  Tiles that no row of a wave can see are skipped and
// tiles that every row sees in full need no mask (§33.3, causal block
// skipping); every legal key of every row is processed.
//
// Mapping onto CDNA4 (gfx950):
// * A workgroup of 4 wavefronts owns 128 consecutive query rows of one
//   (batch, head); wavefront w owns rows 32w..32w+31.  A large shape (8
//   wavefronts, 256 rows, 128-key tiles) serves long problems without bias,
//   window or variable lengths (see the launcher for the rule).
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
// * K/V tiles are double-buffered in LDS and filled by buffer_load ... lds
//   (HBM -> LDS without registers); tile t + 2 is in flight while tile t is
//   computed.  16-byte chunks are XOR-swizzled per row so that the 16-byte K
//   reads and the transposed V reads are free of bank conflicts.
// * Within a tile the 32-key blocks are software-pipelined: block q's
//   softmax (VALU) runs while the score MFMAs of block q + 1 and the P V
//   MFMAs of block q - 1 execute.
// * Rescaling is lazy: the reference maximum m of a row only moves when a
//   tile's maximum exceeds it by more than 8 (base-2 units); the merge rule
//   holds for any reference value, so o = u / l is unchanged, and the weights
//   stay below 2^8.
// * Scores live in the base-2 domain: p = exp2(dot * scale * log2(e) - m2) on
//   v_exp_f32; LSE is converted back to natural-log units at the end.
#include <type_traits>

#include "attn_internal.h"
#include "kernels.h"
#include "prefill_common.h"

namespace attn {
namespace {

using namespace pf;

#ifndef PREFILL_BLOCKS
#define PREFILL_BLOCKS 2               // 32-key blocks per key tile (one barrier per tile)
#endif
#ifndef PREFILL_BIAS_XCD
#define PREFILL_BIAS_XCD 1             // head-shared bias: heads of a query tile on one XCD (see the work order)
#endif
#ifndef PREFILL_XCD_MAP
#define PREFILL_XCD_MAP 0              // 1: keep one head per XCD at a time (see the work order)
#endif
#ifndef PREFILL_WAVES
#define PREFILL_WAVES 4                // wavefronts (32 query rows each) per workgroup
#endif
#ifndef PREFILL_SCHED
#define PREFILL_SCHED 8                // VALU instructions placed after each MFMA of a full tile (0: compiler's order)
#endif
#ifndef PREFILL_PIN
#define PREFILL_PIN 1                  // 1: full-tile weights computed before the rescale branch
#endif
#ifndef PREFILL_FIRST_FAST
#define PREFILL_FIRST_FAST 1           // 1: a wave's first tile, if fully visible, on the pipelined path
#endif
#ifndef PREFILL_BIG
#define PREFILL_BIG 1                  // 0: the standard shape for every problem
#endif
#ifndef PREFILL_BIG_D64
#define PREFILL_BIG_D64 1              // 1: the large shape also for d_h = 64, d_v = 128 (small grids)
#endif
#ifndef PREFILL_BIAS_NAT
#define PREFILL_BIAS_NAT 1             // 1: bias scores formed in natural-log units (one VALU op fewer each)
#endif
#ifndef PREFILL_BIAS_PF
#define PREFILL_BIAS_PF 1              // 1: bias of a full tile loaded at the previous tile's barrier (no counts)
#endif
#ifndef PREFILL_BIAS_LDS
#define PREFILL_BIAS_LDS 1             // 1: full tiles' bias staged through LDS where it fits
#endif
#ifndef PREFILL_BIAS_SKIP
#define PREFILL_BIAS_SKIP 1            // 1: a full tile whose staged bias is all -inf for the wave is skipped
#endif
#ifndef PREFILL_BIAS_EARLY
#define PREFILL_BIAS_EARLY 1           // 1: a staged block's next-tile bias copied as soon as it is read
#endif
#ifndef PREFILL_HILO_KEYS
#define PREFILL_HILO_KEYS 256          // general tiles use hi + lo weights unless every row has this many legal keys
#endif
#ifndef PREFILL_WAVES_PER_SIMD
#define PREFILL_WAVES_PER_SIMD 2       // resident waves per SIMD the kernel is built for
#endif

// Workgroup shapes: wavefronts (32 query rows each), 32-key blocks per key
// tile (one barrier per tile), VALU instructions placed after each MFMA of
// a full tile.  Both keep two wavefronts per SIMD.  The standard shape (4
// wavefronts, 64-key tiles, two workgroups per CU) serves every problem; the
// large one (8 wavefronts, 128-key tiles, 128 KB of LDS, one workgroup per
// CU) halves the HBM -> LDS copies and the barriers per key, which pays on
// long d = 128 sequences with enough query tiles to give every CU one.
struct ShapeStd {
  static constexpr int kWaves = PREFILL_WAVES, kNQ = PREFILL_BLOCKS, kSched = PREFILL_SCHED;
};
#ifndef PREFILL_BIG_BLOCKS
#define PREFILL_BIG_BLOCKS 4
#endif
#ifndef PREFILL_BIG_SCHED
#define PREFILL_BIG_SCHED 3
#endif
struct ShapeBig {
  static constexpr int kWaves = 8, kNQ = PREFILL_BIG_BLOCKS, kSched = PREFILL_BIG_SCHED;
};

template <int DH, int DV, class S>
struct Cfg {
  static constexpr int kBc = 32 * S::kNQ;        // keys per tile
  static constexpr int KS = DH / 16;             // k-steps of K Q^T
  static constexpr int MO = DV / 32;             // 32-row slices of O^T
  static constexpr int K_RB = DH * 2;            // bytes per K row (LDS, unpadded)
  static constexpr int V_RB = DV * 2;            // bytes per V row
  static constexpr int K_BYTES = kBc * K_RB;
  static constexpr int V_BYTES = kBc * V_RB;
  static constexpr int K_DMA = K_BYTES / 1024 / S::kWaves;   // 1 KB DMA writes per wave per tile
  static constexpr int V_DMA = V_BYTES / 1024 / S::kWaves;
};

template <int DH, int DV, bool BIAS, bool COUNT, bool VAR, class S>
__global__ __launch_bounds__(64 * S::kWaves, PREFILL_WAVES_PER_SIMD) void prefill_kernel(Args a) {
  // The host pass only needs this kernel's signature (its launch stub); the
  // body is device code (it otherwise drops the stub of this template).
#if defined(__HIP_DEVICE_COMPILE__)
  using C = Cfg<DH, DV, S>;
  constexpr int kNQ = S::kNQ;
  constexpr int kBc = C::kBc;            // keys per tile
  constexpr int kBr = 32 * S::kWaves;    // query rows per workgroup
  constexpr int kSched = S::kSched;
  // Two K slots then two V slots; tile t lives in slot t & 1.  Instances with
  // a bias (no counts) whose rings leave room for two workgroups per CU add a
  // 4 KB bias block per wave and 32-key block (staged bias, below).
  constexpr int kRing = 2 * C::K_BYTES + 2 * C::V_BYTES;
  constexpr int kBiasStage = S::kWaves * kNQ * 4096;
  constexpr int kLdsShare = 163840 * S::kWaves / (4 * PREFILL_WAVES_PER_SIMD);   // LDS per workgroup
  constexpr bool kBiasLds = BIAS && !COUNT && PREFILL_BIAS_LDS && kRing + kBiasStage <= kLdsShare;
  constexpr bool kBiasEarly = kBiasLds && PREFILL_BIAS_EARLY;
  __shared__ __attribute__((aligned(1024))) char smem[kRing + (kBiasLds ? kBiasStage : 0)];
  debug_poison_lds(smem, sizeof(smem));
  char* const kring = smem;
  char* const vring = smem + 2 * C::K_BYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, kept in an SGPR
  const int h = lane >> 5;        // which half of the wave
  const int lr = lane & 31;       // this lane's query row within the wave

  // Work order.  Consecutive workgroup ids go round-robin to the 8 XCDs
  // (each with its own L2).  Default: query tiles outermost, heaviest first
  // (with causal masking, later tiles see more keys), every (batch, head) of
  // a tile together.  batch_major: batches one after the other, each in that
  // order (for K/V larger than the Infinity Cache).  PREFILL_XCD_MAP (a
  // measured alternative, off): XCD x works through heads x, x + 8, ... one
  // at a time.
  const int bid = blockIdx.x;
  int idx, bh;   // idx = 0 for the first-dispatched (heaviest) query tile
  if (PREFILL_XCD_MAP && a.batch_heads % 8 == 0) {
    const int xcd = bid & 7, local = bid >> 3;
    idx = local % a.n_qtiles;
    bh = xcd + 8 * (local / a.n_qtiles);
  } else if (!VAR && a.batch_major) {
    const int i2 = bid / a.heads_q;
    idx = i2 % a.n_qtiles;
    bh = (i2 / a.n_qtiles) * a.heads_q + bid % a.heads_q;
  } else if (!VAR && a.xcd_heads) {
    // The default order in groups g = (tile, batch) of heads_q workgroups.
    // XCD x (= bid mod 8) receives ids x, x + 8, ...: here it runs groups x,
    // x + 8, ... one after the other, so the heads that read the same bias
    // rows run at the same time behind one L2, and every XCD still sees the
    // tiles heaviest first.  Ids past the last whole round of 8 groups keep
    // the default order.
    const int rounds8 = a.n_qtiles * (a.batch_heads / a.heads_q) / 8;
    if (bid < rounds8 * 8 * a.heads_q) {
      const int local = bid >> 3;
      const int g = (local / a.heads_q) * 8 + (bid & 7);
      const int nb = a.batch_heads / a.heads_q;
      idx = g / nb;
      bh = (g % nb) * a.heads_q + local % a.heads_q;
    } else {
      idx = bid / a.batch_heads;
      bh = bid % a.batch_heads;
    }
  } else {
    idx = bid / a.batch_heads;
    bh = bid % a.batch_heads;
  }
  const int b = bh / a.heads_q;
  const int hq = bh % a.heads_q;
  const int kvh = hq / a.group;
  int qt = a.n_qtiles - 1 - idx;

  // Variable-length batches.  Packed sequences: grid slot idx is sequence
  // idx / rounds, round r = idx % rounds, i.e. one sequence after the other
  // (all heads of a tile together), each from its last (most keys, when
  // causal) tile; the workgroup then computes tiles n_tiles - 1 - r, that
  // minus rounds, ... so any sequence length is covered.  Sequence by
  // sequence keeps the K/V an XCD is reading to a few sequences' worth, which
  // its L2 holds (all sequences' last tiles first measured 5 % slower on 8
  // sequences of up to 4065 rows).  Pointers are moved to the sequence's first row and key and the
  // sizes become the sequence's own, with its rows at the end of its keys.
  // Per-batch KV lengths: the batch's keys are [0, L_b) and its rows sit at
  // q_offset + L_b - T_q + i.
  const int32_t t_q_all = a.t_q;   // rows per head in LSE / n_legal
  int32_t row_base = 0;            // packed row of this sequence's row 0
  if (VAR) {
    if (a.cu_q != nullptr) {
      const int sq = idx / a.rounds, r = idx % a.rounds;
      const int q0 = clamp_len(a.cu_q[sq], a.t_q);
      const int q1 = max(q0, clamp_len(a.cu_q[sq + 1], a.t_q));
      const int k0 = clamp_len(a.cu_k[sq], a.t_k);
      const int k1 = max(k0, clamp_len(a.cu_k[sq + 1], a.t_k));
      qt = (q1 - q0 + kBr - 1) / kBr - 1 - r;
      if (qt < 0) return;   // whole workgroup: nothing of this sequence is left for it
      a.q += static_cast<int64_t>(q0) * a.qs[2];
      a.o += static_cast<int64_t>(q0) * a.os[2];
      a.k += static_cast<int64_t>(k0) * a.ks[2];
      a.v += static_cast<int64_t>(k0) * a.vs[2];
      if (BIAS) a.bias += static_cast<int64_t>(q0) * a.bs[2] + static_cast<int64_t>(k0) * a.bs[3];
      row_base = q0;
      a.q_offset += (k1 - k0) - (q1 - q0);
      a.t_q = q1 - q0;
      a.t_k = k1 - k0;
    } else {
      const int lk = clamp_len(a.kv_lens[b], a.t_k);
      a.q_offset += lk - a.t_q;
      a.t_k = lk;
    }
  }

  // One query tile (128 rows of one head); a packed-sequence workgroup runs
  // it for several tiles in turn.
  auto tile_body = [&](const int qt) __attribute__((always_inline)) {
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
  // First key inside the sliding window of a row at logical row r (0 without a
  // window), clamped to [0, T_k]; keys below it are not legal.
  auto win_lo = [&](int64_t r) -> int {
    if (a.window <= 0) return 0;
    const int64_t lo = a.q_offset + r - a.window + 1;
    return lo < 0 ? 0 : (lo > a.t_k ? a.t_k : static_cast<int>(lo));
  };
  const int lo_row = win_lo(row);
  const int lo_w_first = win_lo(row0);
  const int lo_w_last = win_lo(row0 + 31);

  // Tiles the workgroup streams: keys [0, k_end).  Tiles the wave computes:
  // the first n_w of them (every later one is above the wave's diagonal).
  // Tiles t < t_full need no mask for any row of the wave.
  const int wg_last = clamp_pos(a.q_offset + static_cast<int64_t>(qt) * kBr + kBr - 1);
  const int k_end = a.causal ? (wg_last + 1 < a.t_k ? wg_last + 1 : a.t_k) : a.t_k;
  const int n_tiles = k_end > 0 ? (k_end + kBc - 1) / kBc : 0;
  // The workgroup streams tiles [t_begin, n_tiles): below t_begin every key is
  // outside the window of its first row (and so of every row).
  const int t_begin = win_lo(static_cast<int64_t>(qt) * kBr) / kBc;
  // Tiles below t_w_begin hold no key inside the window of any row of the wave.
  const int t_w_begin = lo_w_first / kBc;
  // Tiles from t_lo_full on lie inside the window of every row of the wave.
  const int t_lo_full = (lo_w_last + kBc - 1) / kBc;
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
  if (t_full > n_w) t_full = n_w;

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

  // ---- tile movement: HBM -> LDS by buffer_load ... lds ----
  // DMA instruction j of this wave fills LDS bytes [1024 (wave * n + j), +1024)
  // of the slot; lane l writes the 16 bytes at l * 16 of that block, i.e. one
  // row and chunk slot of the swizzled layout, so it loads the row's chunk
  // slot ^ swz(row).  The descriptor starts at the tile's first key and ends
  // at T_k, so rows past T_k are filled with zeros.
  int koff[C::K_DMA], voff[C::V_DMA];
#pragma unroll
  for (int j = 0; j < C::K_DMA; ++j) {
    const int byte = (wave * C::K_DMA + j) * 1024 + lane * 16;
    const int r = byte / C::K_RB, sl = (byte % C::K_RB) / 16;
    koff[j] = r * k_row_bytes + (sl ^ swz_k<C::K_RB>(r)) * 16;
  }
#pragma unroll
  for (int j = 0; j < C::V_DMA; ++j) {
    const int byte = (wave * C::V_DMA + j) * 1024 + lane * 16;
    const int r = byte / C::V_RB, sl = (byte % C::V_RB) / 16;
    voff[j] = r * v_row_bytes + (sl ^ swz_v<C::V_RB>(r)) * 16;
  }
  auto gload = [&](int t) {
    const int kb = t * kBc;
    const int slot = t & 1;
    const auto krs = make_rsrc(reinterpret_cast<const char*>(kbase) + static_cast<int64_t>(kb) * k_row_bytes,
                               static_cast<int64_t>(a.t_k - kb) * k_row_bytes);
    const auto vrs = make_rsrc(reinterpret_cast<const char*>(vbase) + static_cast<int64_t>(kb) * v_row_bytes,
                               static_cast<int64_t>(a.t_k - kb) * v_row_bytes);
#pragma unroll
    for (int j = 0; j < C::K_DMA; ++j)
      lds_copy<16>(krs, (__attribute__((address_space(3))) void*)(kring + slot * C::K_BYTES + (wave * C::K_DMA + j) * 1024), koff[j]);
#pragma unroll
    for (int j = 0; j < C::V_DMA; ++j)
      lds_copy<16>(vrs, (__attribute__((address_space(3))) void*)(vring + slot * C::V_BYTES + (wave * C::V_DMA + j) * 1024), voff[j]);
  };
  // Wait for this wave's DMA writes, then the workgroup barrier.
  auto dma_barrier = [&]() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  // LDS read addresses, fixed per lane; the slot and block enter as
  // immediate offsets where they are compile-time constants.
  // K operand of k-step s: row lr (+ 32 q) of the tile, chunk (2 s + h) ^ swz,
  // where the swizzle of rows lr and 32 q + lr is the same.
  const lds_char* kp[C::KS];
  {
    const int kx = swz_k<C::K_RB>(lr);
#pragma unroll
    for (int s2 = 0; s2 < C::KS; ++s2)
      kp[s2] = (const lds_char*)kring + lr * C::K_RB + (((2 * s2 + h) ^ kx) << 4);
  }
  // V^T operand of output slice mo: the transposed read of rows src + 8 e
  // (e = 0, 1) with src = 32 q + 16 kk2 + 4 h + (lane % 16) / 4; the swizzle
  // depends only on src % 16, so q and kk2 are immediate offsets.
  const lds_char* vp[2][C::MO];
  {
    const int src = 4 * h + ((lane & 15) >> 2);
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int mo = 0; mo < C::MO; ++mo) {
        const int cb = 64 * mo + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);   // byte column
        const int c = cb >> 4, hb = cb & 15;
        vp[e][mo] = (const lds_char*)vring + (src + 8 * e) * C::V_RB +
                    ((c ^ swz_v<C::V_RB>(src + 8 * e)) << 4) + hb;
      }
  }

  // S^T of 32-key block q of the K tile in `slot`.  Register r of the result
  // holds key 32 q + 8 (r / 4) + 4 h + (r % 4) (tile-relative) of this
  // lane's row.
  auto scores_q = [&](int slot, int q, f32x16& sacc) {
    const int off = slot * C::K_BYTES + 32 * q * C::K_RB;
    sacc = f32x16{};
#pragma unroll
    for (int s2 = 0; s2 < C::KS; ++s2) {
      const u32x4 kop = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(kp[s2] + off);
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kop), as_bf16x8(qreg[s2]), sacc, 0, 0, 0);
    }
  };

  // O^T += V^T P^T for 32-key block q (two 16-key MFMA steps).  The B
  // operand of step kk2 is pk[4 kk2 .. 4 kk2 + 3]: keys base + (0..3) and
  // base + 8 + (0..3) with base = 32 q + 16 kk2 + 4 h, which is where the
  // transposed reads fetch V from.
  auto pv_q = [&](int slot, int q, const unsigned* pk) {
#pragma unroll
    for (int kk2 = 0; kk2 < 2; ++kk2) {
      const u32x4 bop = {pk[4 * kk2], pk[4 * kk2 + 1], pk[4 * kk2 + 2], pk[4 * kk2 + 3]};
      const int off = slot * C::V_BYTES + (32 * q + 16 * kk2) * C::V_RB;
#pragma unroll
      for (int mo = 0; mo < C::MO; ++mo) {
        const u32x2 lo = tr_read(vp[0][mo] + off);
        const u32x2 hi = tr_read(vp[1][mo] + off);
        const u32x4 aop = {lo[0], lo[1], hi[0], hi[1]};
        oacc[mo] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(aop), as_bf16x8(bop), oacc[mo], 0, 0, 0);
      }
    }
  };

  // The same product with each weight carried as two bf16 terms, hi + lo
  // (hi = the weight rounded to bf16, lo = the rounded remainder, so hi + lo
  // is within 2^-16 of the fp32 weight): both share each V^T operand read.
  // General blocks use it: they hold every key of the rows with only a few
  // keys, whose output is close to a single value row, where a weight
  // rounded once to bf16 (2^-8) would add to the output's own bf16 rounding.
  auto pv2_q = [&](int slot, int q, const unsigned* pk, const unsigned* pl) {
#pragma unroll
    for (int kk2 = 0; kk2 < 2; ++kk2) {
      const u32x4 bop = {pk[4 * kk2], pk[4 * kk2 + 1], pk[4 * kk2 + 2], pk[4 * kk2 + 3]};
      const u32x4 bol = {pl[4 * kk2], pl[4 * kk2 + 1], pl[4 * kk2 + 2], pl[4 * kk2 + 3]};
      const int off = slot * C::V_BYTES + (32 * q + 16 * kk2) * C::V_RB;
#pragma unroll
      for (int mo = 0; mo < C::MO; ++mo) {
        const u32x2 lo = tr_read(vp[0][mo] + off);
        const u32x2 hi = tr_read(vp[1][mo] + off);
        const u32x4 aop = {lo[0], lo[1], hi[0], hi[1]};
        oacc[mo] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(aop), as_bf16x8(bop), oacc[mo], 0, 0, 0);
        oacc[mo] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(aop), as_bf16x8(bol), oacc[mo], 0, 0, 0);
      }
    }
  };

  // Rescale O and l when a row's reference maximum moved (wave-uniform test).
  auto rescale = [&](float m_new, float alpha) {
    if (__ballot(m_new != m2) != 0) {
#pragma unroll
      for (int i = 0; i < C::MO; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
    }
    m2 = m_new;
  };

  // The 16 bias values of block q of tile t this lane's row meets (16-byte
  // loads of the 4 consecutive keys each register group holds).
  auto load_bias = [&](int t, int q, float* mb) {
    const auto rs = make_rsrc(bias_w + t * kBc, bias_w_bytes - static_cast<int64_t>(t) * kBc * 4);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 x = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, bias_off + 128 * q + 32 * g, 0, 0));
#pragma unroll
      for (int e = 0; e < 4; ++e) mb[4 * g + e] = x[e];
    }
  };

  // Bias values of the next full tile, loaded right after the barrier that
  // ends the tile before it and ahead of that barrier's K/V copies, so they
  // have the score MFMAs of the tile's first blocks to arrive and the next
  // barrier (which waits for every load) never waits for them.  Counting
  // instances keep per-block loads: they have no registers to spare.
  constexpr bool kBiasPf = BIAS && !COUNT && PREFILL_BIAS_PF && !kBiasLds;
  float mbp[kBiasPf ? kNQ : 1][16];
  // Staged bias (kBiasLds): a lane's own 16-byte loads touch 32 rows, i.e. 32
  // cache lines, per instruction, and that line rate bounds a biased tile.
  // Instead each wave copies its 32 rows x 32 keys (4 KB per block) with
  // buffer_load ... lds, 8 whole rows per instruction, into its own LDS
  // block, 16-byte chunk c of row r at chunk slot c ^ bswz(r); lane l of
  // copy i carries row 8 i + l / 8, chunk slot l % 8.  A 16-byte read serves
  // 16 lanes (16 rows of one chunk) per cycle, and with 128-byte rows rows r
  // and r + 8 share banks unless their slots differ: with bswz(r) =
  // (r >> 1) & 7 the 16 rows of a read cover all 64 banks once (r & 7 left
  // two-way conflicts).
  auto bswz = [](int r) { return (r >> 1) & 7; };
  char* const bstage = smem + kRing + wave * (kNQ * 4096);
  int bdma[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = 8 * i + (lane >> 3);
    bdma[i] = kBiasLds ? static_cast<int>(rr * a.bs[2] * 4) + 16 * ((lane & 7) ^ bswz(rr)) : 0;
  }
  // Copies of block q of tile t's bias into the wave's staging block q (four
  // instructions).
  auto stage_block = [&](int t, int q) {
    const auto rs = make_rsrc(bias_w + t * kBc, bias_w_bytes - static_cast<int64_t>(t) * kBc * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      lds_copy<16>(rs, (__attribute__((address_space(3))) void*)(bstage + q * 4096 + i * 1024), bdma[i] + 128 * q);
  };
  auto prefetch_bias = [&](int t) {
    if (kBiasLds) {
#pragma unroll
      for (int q = 0; q < kNQ; ++q) stage_block(t, q);
    } else {
#pragma unroll
      for (int q = 0; q < (kBiasPf ? kNQ : 1); ++q) load_bias(t, q, mbp[q]);
    }
  };
  // Block q's staged values of tile t: the copies issued after them are the
  // 4 (kNQ - 1 - q) of the later blocks, unless tile t is the last the K/V
  // copies of tile t + 1, and (kBiasEarly, tile t + 1 full) the 4 q copies of
  // tile t + 1's blocks before q, so waiting until at most that many are in
  // flight waits for block q's copies alone; then the 4 chunks 2 g + h of
  // this lane's row.  Byte offsets in a staging block of this lane's row and
  // chunks 2 g + h:
  int bread[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) bread[g] = lr * 128 + (((2 * g + h) ^ bswz(lr)) << 4);
  auto staged_wait = [&](int t, int q) {
    constexpr int kKV = C::K_DMA + C::V_DMA, kMax = 4 * (kNQ - 1) + kKV;
    const bool kv = t + 1 < n_tiles, nb = kBiasEarly && t + 1 < t_full;
    if (kv && nb) wait_vm_upto<kMax>(4 * (kNQ - 1 - q) + kKV + 4 * q);
    else if (kv) wait_vm_upto<kMax>(4 * (kNQ - 1 - q) + kKV);
    else if (nb) wait_vm_upto<kMax>(4 * (kNQ - 1 - q) + 4 * q);
    else wait_vm_upto<kMax>(4 * (kNQ - 1 - q));
  };
  auto staged_bias = [&](int t, int q, float* mb) {
    staged_wait(t, q);
    const lds_char* blk = (const lds_char*)bstage + q * 4096;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 x = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(blk + bread[g]);
#pragma unroll
      for (int e = 0; e < 4; ++e) mb[4 * g + e] = x[e];
    }
  };

  // A full tile whose staged bias is -inf for every row and key of the wave
  // (keys past a padded sequence's end, say) gives every weight 0 and
  // changes no statistic (the valid-flag rule), so the wave may skip its
  // products and softmax.  The test costs a live tile one read and compare:
  // only when every lane's first entry is -inf are all entries read (compared
  // as bits, so a NaN counts as live and reaches the output as it would).
  auto dead_tile = [&](int t) -> bool {
    staged_wait(t, 0);
    const lds_char* b0 = (const lds_char*)bstage;
    const unsigned f = *reinterpret_cast<const __attribute__((address_space(3))) unsigned*>(b0 + bread[0]);
    if (__ballot(f != 0xff800000u) != 0) return false;
    staged_wait(t, kNQ - 1);
    bool live = false;
#pragma unroll
    for (int q = 0; q < kNQ; ++q)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x4 x = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(b0 + q * 4096 + bread[g]);
#pragma unroll
        for (int e = 0; e < 4; ++e) live |= x[e] != 0xff800000u;
      }
    return __ballot(live) == 0;
  };

  // Softmax of a block whose keys are all causally visible (and inside the
  // window) for every row, every row already holding statistics.  The
  // weights are taken against the row's current reference m2 without
  // forming the block maximum: the merge rule holds for any reference, so
  // only their size matters.  A lane whose 16 weights sum past kSumMax (a
  // weight above 2^16, or an overflow to inf) flags the block; the caller
  // then runs redo_q (rare: the reference only lags behind scores more than
  // 16 base-2 units above it).  Branch-free otherwise (weights, sums, bf16
  // packing), so it runs under independent MFMAs.  With a bias, z = scale dot
  // + M in natural-log units (one fma), the base-2 factor riding in the
  // exponent's fma; a -inf entry gives weight 0 by arithmetic alone, and a
  // block whose keys are all -inf for a row adds nothing (the valid-flag
  // rule).  l_prev receives l before the block.
  auto block_bias = [&](int t, int q, float* mb) {
    if constexpr (kBiasLds) {
      staged_bias(t, q, mb);
    } else if (kBiasPf) {
#pragma unroll
      for (int r = 0; r < 16; ++r) mb[r] = mbp[q][r];
    } else {
      load_bias(t, q, mb);
    }
  };
  // Weights of block q against reference m2 into pk; returns this lane's sum
  // (and, with `counting`, adds the block's legal keys to count).
  auto block_weights = [&](int t, int q, const f32x16& sv, unsigned* pk, bool counting) -> float {
    float ps0 = 0.0f, ps1 = 0.0f;
    const float nm = -m2;
    if (BIAS) {
      float mb[16], z[16];
      block_bias(t, q, mb);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
#if PREFILL_BIAS_NAT
        z[r] = fmaf(sv[r], a.scale, mb[r]);
#else
        z[r] = fmaf(mb[r], kLog2e, sv[r] * a.scale_log2);
#endif
        if (COUNT && counting) count += static_cast<int>(mb[r] != -INFINITY);
      }
#if PREFILL_BIAS_NAT
      const float zc = kLog2e;
#else
      const float zc = 1.0f;
#endif
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p0 = fast_exp2(fmaf(z[2 * i], zc, nm));
        const float p1 = fast_exp2(fmaf(z[2 * i + 1], zc, nm));
        pk[i] = pack_bf16(p0, p1);
        ps0 += p0;
        ps1 += p1;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p0 = fast_exp2(fmaf(sv[2 * i], a.scale_log2, nm));
        const float p1 = fast_exp2(fmaf(sv[2 * i + 1], a.scale_log2, nm));
        pk[i] = pack_bf16(p0, p1);
        ps0 += p0;
        ps1 += p1;
      }
      if (COUNT && counting) count += 16;
    }
    return ps0 + ps1;
  };
  auto fast_q = [&](int t, int q, const f32x16& sv, unsigned* pk, bool& need, float& l_prev) {
    const float blk = block_weights(t, q, sv, pk, true);
    need = !(blk <= kSumMax);
    l_prev = l_lane;
    l_lane += blk;
  };
  // The rare path of a flagged block (wave-uniform): the block maximum of
  // every row, the reference moved up where it is exceeded, O and l rescaled
  // by e^(m_old - m_new) (eqs 33.4-33.5), the block's weights recomputed.
  auto redo_q = [&](int t, int q, const f32x16& sv, unsigned* pk, float l_prev) {
    float mx = -INFINITY;
    if (BIAS) {
      float mb[16];
      block_bias(t, q, mb);
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaf(sv[r], a.scale, mb[r]));
      mx = max_xor32(mx) * kLog2e;
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sv[r]);
      mx = max_xor32(mx) * a.scale_log2;
    }
    const float m_new = mx > m2 ? mx : m2;
    const float alpha = fast_exp2(m2 - m_new);
#pragma unroll
    for (int i = 0; i < C::MO; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
    m2 = m_new;
    l_lane = fmaf(l_prev, alpha, block_weights(t, q, sv, pk, false));
  };

  // General softmax of a block (masks, bias, first statistics of a row).
  // Legal iff key < T_k, causally visible, and bias != -inf; illegal scores
  // become -inf and give weight 0; a block with no legal key changes nothing.
  auto general_q = [&](int t, int q, f32x16& sv, unsigned* pk, unsigned* pl) {
    const int kb = t * kBc + 32 * q;
    int lim = a.causal ? pos_row - kb : 32;
    if (a.t_k - 1 - kb < lim) lim = a.t_k - 1 - kb;   // keys past T_k do not exist
    if (lim < -1) lim = -1;
    if (!row_ok) lim = -1;   // rows past T_q: nothing legal, no bias read
    const int first = lo_row - kb;   // keys below the window are not legal
    float mb[16];
    if (BIAS) load_bias(t, q, mb);
    // Legal scores are kept as u with z = c u in base-2 units: u = dot and
    // c = scale log2 e, or with a bias u = scale dot + M and c = log2 e (c > 0,
    // so the maximum commutes with c); the weights take c in their fma.
    float mx = -INFINITY;
#if PREFILL_BIAS_NAT
    const float c = BIAS ? kLog2e : a.scale_log2;
#else
    const float c = 1.0f;
#endif
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = 8 * (r >> 2) + 4 * h + (r & 3);
#if PREFILL_BIAS_NAT
      float z = BIAS ? fmaf(sv[r], a.scale, mb[r]) : sv[r];
#else
      float z = sv[r] * a.scale_log2;
      if (BIAS) z = fmaf(mb[r], kLog2e, z);
#endif
      bool ok = j <= lim && j >= first;
      if (BIAS) ok = ok && mb[r] != -INFINITY;
      if (COUNT) count += static_cast<int>(ok);
      sv[r] = ok ? z : -INFINITY;
      mx = fmaxf(mx, sv[r]);
    }
    const float tmax = max_xor32(mx) * c;
    // First legal key of a row: store; later: lazy reference update.
    float m_new = m2;
    if (tmax != -INFINITY) {
      if (!has) {
        has = true;
        m2 = tmax;
        m_new = tmax;
      } else if (tmax > m2 + kRescale) {
        m_new = tmax;
      }
    }
    const float alpha = fast_exp2(m2 - m_new);
    rescale(m_new, alpha);
    l_lane *= alpha;
    float ps0 = 0.0f, ps1 = 0.0f;
    const float nm2 = -m2;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p0 = fast_exp2(fmaf(sv[2 * i], c, nm2));
      const float p1 = fast_exp2(fmaf(sv[2 * i + 1], c, nm2));
      pk[i] = pack_bf16(p0, p1);
      // Remainders p - bf16(p): exact in fp32 (bf16(p) shares p's leading bits).
      pl[i] = pack_bf16(p0 - __uint_as_float(pk[i] << 16), p1 - __uint_as_float(pk[i] & 0xffff0000u));
      ps0 += p0;
      ps1 += p1;
    }
    l_lane += ps0 + ps1;
  };

  // End of step t: wait for the DMA of tile t + 1 (issued one step ago),
  // barrier (every wave is done with slot t & 1), then DMA tile t + 2 into it.
  // The first full tile always follows a general one, so every full tile's
  // bias was prefetched here at the end of the tile before it.
  // A full tile with kBiasEarly has already issued the copies of tile
  // t + 1's bias (the newest 4 kNQ), so it waits for the older K/V copies
  // only: the barrier then leaves them in flight (this wave's own LDS blocks,
  // which no other wave touches).
  auto advance = [&](int t, bool fast) {
    if (kBiasEarly && fast && t + 1 < t_full) {
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(4 * kNQ) : "memory");
    } else {
      dma_barrier();
      if ((kBiasPf || kBiasLds) && t + 1 < t_full) prefetch_bias(t + 1);
    }
    if (t + 2 < n_tiles) gload(t + 2);
  };

  // Prologue: the first two streamed tiles in flight.
  if (t_begin < n_tiles) gload(t_begin);
  if (t_begin + 1 < n_tiles) gload(t_begin + 1);
  dma_barrier();

  // Tile 0 (first statistics), then the run of full tiles on the fast path,
  // then the rest (diagonal / masked / skipped tiles).  On a general tile the
  // blocks past the wave's last visible key are skipped.
  auto general_step = [&](int t) {
    if (t < n_w && t >= t_w_begin) {
      // Weights as hi + lo terms where some row of the wave may have few
      // legal keys (its output then rests on a few weights, each of which a
      // single bf16 rounding would shift by up to 2^-9); when every row has at
      // least PREFILL_HILO_KEYS legal keys in all (no bias, which can mask any
      // of them), a single product per block, as on full tiles.  The fewest
      // keys of any row of the wave: at least from the last row's window
      // start to the first row's position.
      const int fewest = (a.t_k < pos_w_first + 1 ? a.t_k : pos_w_first + 1) - lo_w_last;
      const bool hilo = BIAS || PREFILL_HILO_KEYS <= 0 || fewest < PREFILL_HILO_KEYS;
      // Two straight-line copies of the block loop (a branch per block
      // between the two products costs the register allocation dearly).
      auto blocks = [&](auto hilo_c) __attribute__((always_inline)) {
        constexpr bool HILO = decltype(hilo_c)::value;
#pragma unroll
        for (int q = 0; q < kNQ; ++q) {
          if (a.causal && t * kBc + 32 * q > pos_w_last) break;
          if (t * kBc + 32 * q + 31 < lo_w_first) continue;   // below every row's window
          f32x16 sv;
          unsigned pk[8], pl[8];
          scores_q(t & 1, q, sv);
          general_q(t, q, sv, pk, pl);
          if constexpr (HILO) pv2_q(t & 1, q, pk, pl);
          else pv_q(t & 1, q, pk);
        }
      };
      if (hilo) blocks(std::true_type{});
      else blocks(std::false_type{});
    }
    advance(t, false);
  };
  // General tiles up to the wave's first tile inside every row's window, then
  // one more (it gives every row its first statistics), the run of full
  // tiles on the fast path, the rest general (diagonal / masked / skipped).
  int t = t_begin;
  while (t < t_lo_full && t < n_tiles) general_step(t++);
  // Software pipeline over the 32-key blocks of a full tile: block q's
  // softmax (VALU) runs under the score MFMAs of block q + 1 and the P V
  // MFMAs of block q - 1, which are independent of it.
  // Block 0 of a wave's first tile when that tile is fully visible and no row
  // has statistics yet (no bias, so every score is legal and finite): the
  // block maximum is the reference, nothing to rescale.
  auto fast_q_first = [&](const f32x16& sv, unsigned* pk, float& m_new) {
    float mx = fmaxf(sv[0], sv[1]);
#pragma unroll
    for (int r = 2; r < 16; ++r) mx = fmaxf(mx, sv[r]);
    m_new = max_xor32(mx) * a.scale_log2;
    const float nm = -m_new;
    float ps0 = 0.0f, ps1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p0 = fast_exp2(fmaf(sv[2 * i], a.scale_log2, nm));
      const float p1 = fast_exp2(fmaf(sv[2 * i + 1], a.scale_log2, nm));
      pk[i] = pack_bf16(p0, p1);
      ps0 += p0;
      ps1 += p1;
    }
    l_lane = ps0 + ps1;
    if (COUNT) count += 16;
  };
  // FIRST: the wave's first statistics come from block 0 of this tile.
  auto fast_step = [&](int t, int slot, auto first) {
    constexpr bool FIRST = decltype(first)::value;
    f32x16 sv[2];
    unsigned pk[2][8];
    float mn = 0.0f, lp = 0.0f;
    bool need = false;
    // Dead tiles skip the products and the softmax but keep the copies.
    const bool dead = kBiasLds && PREFILL_BIAS_SKIP && dead_tile(t);
    if (!dead) {
      scores_q(slot, 0, sv[0]);
      // Nothing of this tile can overlap block 0's score MFMAs.
      if (kSched > 0) __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int q = 0; q < kNQ; ++q) {
      if (!dead) {
        if (q + 1 < kNQ) scores_q(slot, q + 1, sv[(q + 1) & 1]);
        if (q > 0) pv_q(slot, q - 1, pk[(q - 1) & 1]);
        if (FIRST && q == 0) fast_q_first(sv[q & 1], pk[q & 1], mn);
        else fast_q(t, q, sv[q & 1], pk[q & 1], need, lp);
        if (PREFILL_PIN) {
          // Keep the block's weights ahead of the rescale branch, so they are
          // scheduled under the MFMAs issued before it rather than sunk past it.
          const unsigned* w = pk[q & 1];
          asm volatile("" ::"v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]), "v"(w[4]), "v"(w[5]), "v"(w[6]),
                       "v"(w[7]), "v"(l_lane));
        }
        if (kSched > 0) {
          // One MFMA, then kSched VALU instructions of the softmax, so
          // the in-order issue never waits on the matrix pipe with VALU work
          // behind it.
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, kSched, 0);
          }
        }
        if (FIRST && q == 0) {
          m2 = mn;
          has = true;
        } else if (__ballot(need) != 0) {
          redo_q(t, q, sv[q & 1], pk[q & 1], lp);
        }
      }
      // Block q's staged bias is read (the redo included): its LDS block
      // takes tile t + 1's block q now, a tile ahead of its use.
      if (kBiasEarly && t + 1 < t_full) stage_block(t + 1, q);
    }
    if (!dead) pv_q(slot, kNQ - 1, pk[(kNQ - 1) & 1]);
    advance(t, true);
  };
  const std::false_type later{};
  // The first tile: pipelined when it is fully visible and no row has
  // statistics yet (no bias); otherwise general (first statistics, masks).
  if (!BIAS && PREFILL_FIRST_FAST && t < t_full && __ballot(has) == 0) {
    if ((t & 1) == 0) fast_step(t, 0, std::true_type{});
    else fast_step(t, 1, std::true_type{});
    ++t;
  } else if (t < n_tiles) {
    general_step(t++);
  }
  // Tile t lives in slot t & 1; the slot is an immediate in each copy.
  if (t < t_full && __ballot(!has) == 0) {
    if ((t & 1) == 0) fast_step(t++, 0, later);
    for (; t + 1 < t_full; t += 2) {
      fast_step(t, 1, later);
      fast_step(t + 1, 0, later);
    }
    if (t < t_full) fast_step(t++, 1, later);
  }
  for (; t < n_tiles; ++t) general_step(t);

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
    const int64_t ridx = (static_cast<int64_t>(b) * a.heads_q + hq) * t_q_all + row_base + row;
    a.lse[ridx] = has ? (m2 + fast_log2(l_row)) * kLn2 : -INFINITY;
    if (COUNT) a.n_legal[ridx] = count;
  }
  };   // tile_body

  if (VAR && a.cu_q != nullptr) {
    for (; qt >= 0; qt -= a.rounds) {
      tile_body(qt);
      __syncthreads();   // LDS rings are refilled by the next tile's prologue
    }
  } else {
    tile_body(qt);
  }
#endif
}

template <int DH, int DV, bool BIAS, bool COUNT, bool VAR, class S = ShapeStd>
hipError_t launch_cfg(const Args& a, int64_t blocks, hipStream_t stream) {
  hipLaunchKernelGGL((prefill_kernel<DH, DV, BIAS, COUNT, VAR, S>), dim3(static_cast<unsigned>(blocks)),
                     dim3(64 * S::kWaves), 0, stream, a);
  return hipGetLastError();
}

template <int DH, int DV, bool VAR>
hipError_t launch_var(const Args& a, int64_t blocks, bool bias, bool count, hipStream_t s) {
  if (bias)
    return count ? launch_cfg<DH, DV, true, true, VAR>(a, blocks, s) : launch_cfg<DH, DV, true, false, VAR>(a, blocks, s);
  return count ? launch_cfg<DH, DV, false, true, VAR>(a, blocks, s) : launch_cfg<DH, DV, false, false, VAR>(a, blocks, s);
}

template <int DH, int DV>
hipError_t launch_dims(const Args& a, int64_t blocks, bool bias, bool count, bool var, hipStream_t s) {
  return var ? launch_var<DH, DV, true>(a, blocks, bias, count, s) : launch_var<DH, DV, false>(a, blocks, bias, count, s);
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
  // The large shape: no bias, window or variable lengths, and at least one
  // of its 256-row query tiles per CU; d = 128 (measured: 3-10 % faster on
  // long causal and non-causal problems, 2 % slower with a window, much
  // slower on small grids), or d_h = 64, d_v = 128 with at most two tiles per
  // CU (2-10 % faster there; with 1024 or more tiles -7 to +3 %).
  const bool packed = pb.cu_q != nullptr;
  const int64_t big_tiles = (pb.t_q + 255) / 256 * pb.batch * pb.heads_q;
  const bool big_dims = (pb.d_h == 128 && pb.d_v == 128) ||
                        (PREFILL_BIG_D64 && pb.d_h == 64 && pb.d_v == 128 && big_tiles <= 512);
  const bool big = PREFILL_BIG && big_dims && pb.bias == nullptr && pb.window == 0 && !packed &&
                   pb.kv_lens == nullptr && big_tiles >= 256;
  const int64_t kBr = big ? 32 * ShapeBig::kWaves : 32 * ShapeStd::kWaves;   // query rows per workgroup
  // Packed sequences: `rounds` query tiles per sequence in the grid (from the
  // caller's longest-sequence bound; longer sequences loop).
  int64_t rounds = 1;
  if (packed) {
    rounds = (pb.max_seqlen_q + kBr - 1) / kBr;
    if (rounds < 1) rounds = 1;
    const int64_t cap = (pb.t_q + kBr - 1) / kBr;   // no sequence has more tiles than this
    if (rounds > cap) rounds = cap > 0 ? cap : 1;
  }
  const int64_t n_qtiles = packed ? pb.n_seqs * rounds : (pb.t_q + kBr - 1) / kBr;
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
  a.window = pb.window;
  a.t_q = static_cast<int32_t>(pb.t_q);
  a.t_k = static_cast<int32_t>(pb.t_k);
  a.heads_q = static_cast<int32_t>(pb.heads_q);
  a.group = pb.group;
  a.n_qtiles = static_cast<int32_t>(n_qtiles);
  a.batch_heads = static_cast<int32_t>(pb.batch * pb.heads_q);
  a.scale_log2 = pb.scale_log2;
  a.scale = pb.scale_log2 * kLn2;
  a.causal = pb.causal;
  a.cu_q = pb.cu_q;
  a.cu_k = pb.cu_k;
  a.kv_lens = pb.kv_lens;
  a.n_seqs = static_cast<int32_t>(pb.n_seqs);
  a.rounds = static_cast<int32_t>(rounds);
  // Dense batches whose K/V (all batches and KV heads) outgrow the 256 MB
  // Infinity Cache: batches one after the other, so the K/V in flight is a
  // few batches' worth and its re-reads by later query tiles hit the caches
  // (measured +6 to +18 % on nine such shapes from 384 to 512 MB; at 256 MB
  // and below -9 to +6 %, so those keep the default order).
  const int64_t kv_bytes = pb.batch * pb.heads_kv * pb.t_k * (pb.d_h + pb.d_v) * 2;
  a.batch_major = !packed && pb.kv_lens == nullptr && pb.bias == nullptr && pb.batch > 1 &&
                  kv_bytes > (int64_t(256) << 20);
  // A bias shared by the heads is read by every head of a query tile: in the
  // default order those heads sit on all 8 XCDs and each XCD fetches the same
  // bias rows past its L2; grouped by XCD they run together on one.  Measured
  // on d_h = 64, d_v = 128 causal batches of 2048-4096 rows: 4 to 16 batches
  // of 8-32 heads 2-19 % faster, 2 batches of 32 heads 0-5 % slower (there
  // the default order's fixed heads per XCD keep more K/V in its caches).
  a.xcd_heads = PREFILL_BIAS_XCD && !packed && pb.kv_lens == nullptr && pb.bias != nullptr &&
                pb.bs[1] == 0 && pb.bs[2] != 0 && pb.heads_q > 1 && pb.batch >= 4;

  const bool bias = pb.bias != nullptr;
  const bool count = n_legal != nullptr;
  const bool var = packed || pb.kv_lens != nullptr;
  hipError_t e;
  if (big && pb.d_h == 128)
    e = count ? launch_cfg<128, 128, false, true, false, ShapeBig>(a, blocks, stream)
              : launch_cfg<128, 128, false, false, false, ShapeBig>(a, blocks, stream);
#if PREFILL_BIG_D64
  else if (big)
    e = count ? launch_cfg<64, 128, false, true, false, ShapeBig>(a, blocks, stream)
              : launch_cfg<64, 128, false, false, false, ShapeBig>(a, blocks, stream);
#endif
  else if (pb.d_h == 128 && pb.d_v == 128) e = launch_dims<128, 128>(a, blocks, bias, count, var, stream);
  else if (pb.d_h == 64 && pb.d_v == 128) e = launch_dims<64, 128>(a, blocks, bias, count, var, stream);
  else if (pb.d_h == 128 && pb.d_v == 64) e = launch_dims<128, 64>(a, blocks, bias, count, var, stream);
  else e = launch_dims<64, 64>(a, blocks, bias, count, var, stream);
  *status = e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
  return true;
}

}  // namespace attn
