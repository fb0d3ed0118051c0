// Few-query-row kernel for bf16 problems with d_h, d_v in {64, 128}: split-KV
// decode partials (attn_decode_splitkv) and attn_fwd when H_q/H_kv * T_q is
// small (cached decode, multi-query verification).
//
// What it computes: for one (batch, KV head, group of up to 32 query rows,
// key range), the exact attention of every row over the legal keys of the
// range (eq 33.2 of "Chapter 33 推理计算优化" §33.2), either as the final
// output or as the partial (o_s, lse_s) of that range; partials are later
// merged by eqs 33.4-33.5.  The rows of a workgroup are the T_q query rows of
// every query head that shares the KV head, so each K/V byte of the range is
// read from HBM exactly once for all of them.
//
// Mapping onto CDNA4 (gfx950): decode is bound by HBM bandwidth (each step
// reads the whole cache), so the kernel is built to stream K and V once with
// deep prefetch and keep the arithmetic off the critical path:
// * The four wavefronts of a workgroup split the key range into four
//   contiguous parts and each keeps its own statistics (m, l, u) per row.
// * Per 32-key tile: S^T = K Q^T with v_mfma_f32_32x32x16_bf16; the K operand
//   is loaded from HBM straight into registers in the MFMA layout (no LDS),
//   Q^T stays in registers.  V goes through a wave-private LDS buffer and is
//   read back transposed (ds_read_b64_tr_b16) as the A operand of
//   O^T = V^T P^T.  The loads of tile t + 1 are issued before tile t is
//   computed.
// * At the end the four per-wave states are merged in LDS with eqs 33.4-33.5
//   (a wave with no legal key for a row contributes nothing).
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

constexpr int kTile = 32;         // keys per tile
#ifndef FEWROW_INTERLEAVE
#define FEWROW_INTERLEAVE 1       // 1: a long range's tiles go round-robin to the waves
#endif
#ifndef FEWROW_PAIR
#define FEWROW_PAIR 1             // 1: split mode takes two consecutive splits per workgroup
#endif
#ifndef FEWROW_PAIR_RR
#define FEWROW_PAIR_RR 1          // 1: a pair's split deals its tiles round-robin to its two waves
#endif
#ifndef FEWROW_NT
#define FEWROW_NT 1               // 1: K/V loads marked non-temporal
#endif
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32;         // query rows per workgroup
constexpr float kRescale = 8.0f;  // lazy-rescale threshold, base-2 units

template <int DH, int DV>
struct FCfg {
  static constexpr int KS = DH / 16;
  static constexpr int MO = DV / 32;
  static constexpr int V_STRIDE = DV * 2 + 64;         // bytes per V row in LDS
  static constexpr int VBUF = kTile * V_STRIDE;        // one wave's V tile
  static constexpr int V_PER_LANE = kTile * DV / 8 / 64;
  // Wave states in LDS for the end-of-range merge: rows DV + 8 floats apart,
  // so row r starts 8 r banks on and a 16-byte store of up to 8 rows (both
  // lane halves) touches every bank at most once.
  static constexpr int MO_STRIDE = DV + 8;
  static constexpr int MERGE_O = kWaves * kRows * MO_STRIDE * 4;
  static constexpr int MERGE = MERGE_O + 2 * kWaves * kRows * 4;
  static constexpr int SMEM = MERGE > kWaves * VBUF ? MERGE : kWaves * VBUF;
  // Bias instances: two 4 KB staging blocks per wave after the V buffers.
  static constexpr int BSTAGE = kWaves * VBUF;
  static constexpr int SMEM_B = MERGE > BSTAGE + kWaves * 8192 ? MERGE : BSTAGE + kWaves * 8192;
};

struct FArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  float* ws_o;
  float* ws_lse;
  int64_t qs[3], ks[3], vs[3], os[3];
  int64_t q_offset;
  int64_t window;           // sliding window, 0 = none
  int64_t split_size;       // keys per work item
  int32_t t_q, t_k, heads_q, heads_kv, group, rows, n_rg, n_splits;
  int32_t split0, n_active;   // the grid covers splits [split0, split0 + n_active)
  int32_t pair;               // split mode: each workgroup takes two consecutive splits, two waves each
  int32_t batch;
  float scale_log2;
  int32_t causal;
  const int32_t* kv_lens;     // per-batch KV lengths (device), NULL = T_k for every batch
};

// The bias of the bias instances: fp32, contiguous along keys, strides over
// (b, hq, i) in elements.  A separate argument, so the kernels without a
// bias keep their own (smaller) argument block.
struct FBias {
  const float* bias;
  int64_t bs[3];
  int64_t extent;   // elements from `bias` to one past its last element
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ u32x2 tr_read(const lds_char* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

template <class T>
__device__ __forceinline__ const T& first_of(const T& t) { return t; }

// Bias instances take one more argument (an FBias); the others keep the
// argument block of the kernel without a bias.
template <int DH, int DV, bool SPLIT, bool VAR, bool PAIR, class... Bias>
__global__ __launch_bounds__(kThreads, 2) void fewrow_kernel(FArgs a, Bias... bias_arg) {
  constexpr bool BIAS = sizeof...(Bias) > 0;
  static_assert(!PAIR || (SPLIT && !BIAS), "pairs of splits: split mode without a bias");
  using C = FCfg<DH, DV>;
  __shared__ __attribute__((aligned(16))) char smem[BIAS ? C::SMEM_B : C::SMEM];
  debug_poison_lds(smem, sizeof(smem));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int lr = lane & 31;

  // blockIdx -> work item (group g = (b, row group, kvh), split s), split
  // fastest.  Consecutive workgroups go round-robin to the 8 XCDs, so XCD x
  // gets the splits s = x mod 8: balanced when every split holds keys.  With
  // per-batch KV lengths only a prefix of each batch's splits does, so there
  // (group count a multiple of 8) XCD x takes the groups g = x mod 8 (with 8
  // KV heads: KV head x of every batch) with all their splits, split fastest:
  // the same work on every XCD whatever the lengths, and the workgroups on
  // one XCD stream different offsets of their K/V rows.
  // PAIR (split mode, no bias): a work item is two consecutive splits, waves
  // 0-1 on the first and 2-3 on the second: half the workgroups, so half the
  // per-workgroup start and end latency per key.
  const int64_t n_groups = static_cast<int64_t>(a.n_rg) * a.heads_kv * a.batch;
  constexpr bool pair = PAIR;
  const int n_items = pair ? (a.n_active + 1) / 2 : a.n_active;
  int64_t g;
  int item;
  if (VAR && n_groups % 8 == 0) {
    const int64_t x = blockIdx.x % 8, j = blockIdx.x / 8;
    g = (j / n_items) * 8 + x;
    item = static_cast<int>(j % n_items);
  } else {
    g = blockIdx.x / n_items;
    item = static_cast<int>(blockIdx.x % n_items);
  }
  const int s_first = a.split0 + (pair ? 2 * item : item);
  constexpr int kW = pair ? 2 : kWaves;             // waves per split
  const int half = pair ? wave >> 1 : 0;            // which split of the item this wave takes
  const int wi = pair ? wave & 1 : wave;            // the wave's index within its split
  const int s = s_first + half;
  // A split past the grid's range (the second of an odd count) computes and
  // writes nothing.
  bool s_live = !pair || s < a.split0 + a.n_active;
  const int kvh = static_cast<int>(g % a.heads_kv);
  const int rg = static_cast<int>((g / a.heads_kv) % a.n_rg);
  const int b = static_cast<int>(g / a.heads_kv / a.n_rg);
  // Per-batch KV length L_b (clamped to [0, T_k]): keys [0, L_b), rows at
  // q_offset + L_b - T_q + i.
  if (VAR) {
    const int raw = a.kv_lens[b];
    const int lk = raw < 0 ? 0 : (raw > a.t_k ? a.t_k : raw);
    // A range at or past L_b holds no key of this batch: nothing to write
    // (the merge reads only the first ceil(L_b / split_size) partials).
    if (SPLIT && static_cast<int64_t>(s_first) * a.split_size >= lk) return;
    if (pair && static_cast<int64_t>(s) * a.split_size >= lk) s_live = false;
    a.q_offset += lk - a.t_q;
    a.t_k = lk;
  }

  // This lane's row: n = 32 rg + lr -> query head kvh * group + n / T_q, row n % T_q.
  const int n = rg * kRows + lr;
  const bool row_ok = n < a.rows;
  const int gq = row_ok ? n / a.t_q : 0;
  const int qi = row_ok ? n % a.t_q : 0;
  const int hq = kvh * a.group + gq;
  const int64_t pos = a.q_offset + qi;

  // Key range of the work item, cut at the last position any row can see.
  int64_t lo = static_cast<int64_t>(s) * a.split_size;
  int64_t hi = a.split_size < a.t_k - lo ? lo + a.split_size : a.t_k;
  if (a.causal) {
    const int64_t last = a.q_offset + a.t_q - 1;   // largest position of any row
    if (last + 1 < hi) hi = last + 1;
  }
  if (a.window > 0) {
    const int64_t first = a.q_offset - a.window + 1;   // smallest window start of any row
    if (first > lo) lo = first;
  }
  if (pair && !s_live) hi = lo;
  // A work item with no key any of its rows may see (a split wholly past the
  // last position or before the first window, or T_k = 0) only writes its
  // empty result: O = +0 and LSE = -inf (the valid-flag rule of §33.2).  A
  // pair goes on (its waves of an empty split compute nothing, and the merge
  // writes that split's empty result).
  if (hi <= lo && !pair) {
    const int rows_here = a.rows - rg * kRows < kRows ? a.rows - rg * kRows : kRows;
    for (int e = tid; e < rows_here * DV; e += kThreads) {
      const int rr = e / DV, d = e % DV;
      const int nn = rg * kRows + rr;
      const int ghq = kvh * a.group + nn / a.t_q;
      const int gi = nn % a.t_q;
      const int64_t ridx = (static_cast<int64_t>(b) * a.heads_q + ghq) * a.t_q + gi;
      if (SPLIT) {
        a.ws_o[(ridx * a.n_splits + s) * DV + d] = 0.0f;
        if (d == 0) a.ws_lse[ridx * a.n_splits + s] = -INFINITY;
      } else {
        a.o[b * a.os[0] + ghq * a.os[1] + static_cast<int64_t>(gi) * a.os[2] + d] = 0;
        if (d == 0) a.lse[ridx] = -INFINITY;
      }
    }
    return;
  }

  u32x4 qreg[C::KS];
  {
    const uint16_t* qp = a.q + b * a.qs[0] + hq * a.qs[1] + static_cast<int64_t>(qi) * a.qs[2];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      qreg[ks] = row_ok ? *reinterpret_cast<const u32x4*>(qp + 16 * ks + 8 * h) : u32x4{0, 0, 0, 0};
  }

  // The range's 32-key tiles go to the 4 waves as four contiguous parts or,
  // for ranges of more than 16 tiles (FEWROW_INTERLEAVE), round-robin: wave w
  // takes tiles w, w + 4, ..., so the workgroup streams one contiguous 4-tile
  // block after another (measured: multi-query verify over 4096 keys 5 %
  // faster; 512-key decode splits 3 % slower, so they keep the parts).  Tile
  // t of this wave starts at key tile_kb(t); keys at or past whi do not exist.
  const int64_t len = hi > lo ? hi - lo : 0;
  const int64_t all_tiles = (len + kTile - 1) / kTile;
  int64_t wlo, whi, tstep;
  int n_tiles;
  if (FEWROW_INTERLEAVE && (all_tiles > 4 * kWaves || (pair && FEWROW_PAIR_RR))) {
    wlo = lo + static_cast<int64_t>(wi) * kTile;
    whi = hi;
    tstep = kW * kTile;
    n_tiles = all_tiles > wi ? static_cast<int>((all_tiles - wi + kW - 1) / kW) : 0;
  } else {
    const int64_t part = ((len + kW - 1) / kW + kTile - 1) / kTile * kTile;
    wlo = lo + wi * part;
    whi = wlo + part < hi ? wlo + part : hi;
    if (whi < wlo) whi = wlo;
    tstep = kTile;
    n_tiles = static_cast<int>((whi - wlo + kTile - 1) / kTile);
  }
  auto tile_kb = [&](int t) { return wlo + static_cast<int64_t>(t) * tstep; };

  const uint16_t* kbase = a.k + b * a.ks[0] + kvh * a.ks[1];
  const uint16_t* vbase = a.v + b * a.vs[0] + kvh * a.vs[1];
  char* vl_w = smem + wave * C::VBUF;
  const lds_char* vl = (const lds_char*)vl_w;

  bool has = false;
  float m2 = 0.0f;
  float l_lane = 0.0f;
  f32x16 oacc[C::MO];
#pragma unroll
  for (int i = 0; i < C::MO; ++i) oacc[i] = f32x16{};

  // Plain global loads (measured faster here than buffer loads); rows past
  // the wave's range end give zeros.  Bias instances issue every load (rows
  // past the end read key 0 and are then zeroed): the wait for the staged
  // bias below counts the loads issued after it.
  u32x4 kreg[C::KS], vreg[C::V_PER_LANE];
  auto ld = [](const uint16_t* p) -> u32x4 { return *reinterpret_cast<const u32x4*>(p); };
  // V rows are read whole by each instruction (4 rows of 256 bytes): marked
  // non-temporal (FEWROW_NT).  A K instruction reads 32 bytes of each of 32
  // rows and relies on the caches to serve the rest of each line to the next
  // instructions, so K loads stay ordinary.
  auto ld_v = [](const uint16_t* p) -> u32x4 {
    if (FEWROW_NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return *reinterpret_cast<const u32x4*>(p);
  };
  auto load = [&](int t, u32x4* kr, u32x4* vr) {
    const int64_t kb = tile_kb(t);
    const int64_t key = kb + lr;
    const bool kok = key < whi;
    const uint16_t* kp = kbase + (BIAS && !kok ? 0 : key) * a.ks[2] + 8 * h;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      if (BIAS) {
        const u32x4 x = ld(kp + 16 * ks);
        kr[ks] = kok ? x : u32x4{0, 0, 0, 0};
      } else {
        kr[ks] = kok ? ld(kp + 16 * ks) : u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int i = 0; i < C::V_PER_LANE; ++i) {
      const int c = lane + 64 * i;
      const int r = c / (DV / 8), col = c % (DV / 8);
      const bool vok = kb + r < whi;
      if (BIAS) {
        const u32x4 x = ld_v(vbase + (vok ? kb + r : 0) * a.vs[2] + col * 8);
        vr[i] = vok ? x : u32x4{0, 0, 0, 0};
      } else {
        vr[i] = vok ? ld_v(vbase + (kb + r) * a.vs[2] + col * 8) : u32x4{0, 0, 0, 0};
      }
    }
  };

  // Bias (BIAS): each wave copies its 32 rows x 32 keys of tile t (4 KB)
  // into staging block t & 1 with buffer_load ... lds, 8 rows (128 bytes
  // each) per instruction, one tile ahead, from the base of the workgroup's
  // first row (b, kvh * group, row 0) plus the tile's first key; lane l of
  // copy i carries row 8 i + l / 8, chunk slot l % 8, which holds the row's
  // chunk (l % 8) ^ bswz(row), so a 16-byte read of 16 rows' same chunk
  // covers all 64 banks.  Rows past the group's rows copy row 0 (never
  // legal).  The descriptor's size ends at the bias's last element, so keys
  // past it read zeros.
  const float* bias_w = nullptr;
  int64_t bias_left = 0;   // elements from bias_w to the end of the bias
  int bdma[4];
  char* const bstage = smem + C::BSTAGE + wave * 8192;
  auto bswz = [](int r) { return (r >> 1) & 7; };
  if constexpr (BIAS) {
    const FBias& fb = first_of(bias_arg...);
    const int64_t off0 = b * fb.bs[0] + static_cast<int64_t>(kvh) * a.group * fb.bs[1];
    bias_w = fb.bias + off0;
    bias_left = fb.extent - off0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 8 * i + (lane >> 3);
      const int nn = rg * kRows + row;
      const int64_t roff = nn < a.rows ? (nn / a.t_q) * fb.bs[1] + static_cast<int64_t>(nn % a.t_q) * fb.bs[2] : 0;
      bdma[i] = static_cast<int>(roff * 4) + 16 * ((lane & 7) ^ bswz(row));
    }
  }
  auto stage_bias = [&](int t) {
    const int64_t kb = tile_kb(t);
    const auto rs = make_rsrc(bias_w + kb, (bias_left - kb) * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      lds_copy<16>(rs, (__attribute__((address_space(3))) void*)(bstage + (t & 1) * 4096 + i * 1024), bdma[i]);
  };
  int bread[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) bread[g] = lr * 128 + (((2 * g + h) ^ bswz(lr)) << 4);

  if (n_tiles > 0) {
    load(0, kreg, vreg);
    if (BIAS) stage_bias(0);
  }

  for (int t = 0; t < n_tiles; ++t) {
    const int64_t kb = tile_kb(t);
    // V tile -> this wave's LDS buffer (read back transposed below).
#pragma unroll
    for (int i = 0; i < C::V_PER_LANE; ++i) {
      const int c = lane + 64 * i;
      const int r = c / (DV / 8), col = c % (DV / 8);
      *reinterpret_cast<u32x4*>(vl_w + r * C::V_STRIDE + col * 16) = vreg[i];
    }
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kreg[ks]), as_bf16x8(qreg[ks]), sacc, 0, 0, 0);
    if (t + 1 < n_tiles) {
      load(t + 1, kreg, vreg);
      if (BIAS) stage_bias(t + 1);
    }
    f32x4 mb[BIAS ? 4 : 1];
    if (BIAS) {
      // Tile t's copies are older than the KS + V_PER_LANE loads and 4
      // copies of tile t + 1 issued above (all of them unconditional), so at
      // most that many in flight means they have landed.
      asm volatile("" ::: "memory");
      if (t + 1 < n_tiles) {
        constexpr int kYounger = C::KS + C::V_PER_LANE + 4;
        static_assert(kYounger < 64, "vmcnt holds 6 bits");
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kYounger) : "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      const lds_char* blk = (const lds_char*)bstage + (t & 1) * 4096;
#pragma unroll
      for (int g = 0; g < 4; ++g) mb[g] = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(blk + bread[g]);
    }

    // Register r holds key kb + 8 (r / 4) + 4 h + (r % 4) of this lane's row.
    int64_t lim64 = whi - 1 - kb;
    if (a.causal && pos - kb < lim64) lim64 = pos - kb;
    int lim = lim64 < -1 ? -1 : (lim64 > kTile ? kTile : static_cast<int>(lim64));
    if (!row_ok) lim = -1;
    // Window: keys below pos - window + 1 are not legal.
    int64_t first64 = a.window > 0 ? pos - a.window + 1 - kb : 0;
    const int first = first64 < 0 ? 0 : (first64 > kTile ? kTile : static_cast<int>(first64));
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = 8 * (r >> 2) + 4 * h + (r & 3);
      float z;
      if (BIAS)   // -inf entries mask their key
        z = (j <= lim && j >= first) ? fmaf(mb[r >> 2][r & 3], kLog2e, sacc[r] * a.scale_log2) : -INFINITY;
      else
        z = (j <= lim && j >= first) ? sacc[r] * a.scale_log2 : -INFINITY;
      sacc[r] = z;
      mx = fmaxf(mx, z);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));

    bool need = false;
    if (mx != -INFINITY) {
      if (!has) {
        has = true;
        m2 = mx;
      } else if (mx > m2 + kRescale) {
        need = true;
      }
    }
    if (__ballot(need) != 0) {
      const float alpha = need ? fast_exp2(m2 - mx) : 1.0f;
      if (need) m2 = mx;
      l_lane *= alpha;
#pragma unroll
      for (int i = 0; i < C::MO; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
    }

    // Weights as two bf16 terms each, hi = bf16(p) and lo = bf16(p - hi)
    // (p - hi is exact in fp32), so hi + lo is within 2^-16 of p and a row
    // with only a few keys, whose output is nearly one value row, does not
    // add a 2^-8 weight rounding to the output's own bf16 rounding.  The
    // second product costs matrix-pipe time, which this HBM-bound kernel has
    // to spare.
    unsigned pk[8], pl[8];
    {
      float p[16];
      float ls = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = fast_exp2(sacc[r] - m2);
        ls += p[r];
      }
      l_lane += ls;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pk[i] = pack_bf16(p[2 * i], p[2 * i + 1]);
        pl[i] = pack_bf16(p[2 * i] - __uint_as_float(pk[i] << 16),
                          p[2 * i + 1] - __uint_as_float(pk[i] & 0xffff0000u));
      }
    }

    asm volatile("" ::: "memory");   // keep the V stores above the transposed reads
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const u32x4 bop = {pk[4 * kk], pk[4 * kk + 1], pk[4 * kk + 2], pk[4 * kk + 3]};
      const u32x4 bol = {pl[4 * kk], pl[4 * kk + 1], pl[4 * kk + 2], pl[4 * kk + 3]};
      const int src_row = 16 * kk + 4 * h + ((lane & 15) >> 2);
#pragma unroll
      for (int mo = 0; mo < C::MO; ++mo) {
        const int col = 32 * mo + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        const lds_char* p0 = vl + src_row * C::V_STRIDE + col * 2;
        const u32x2 x0 = tr_read(p0);
        const u32x2 x1 = tr_read(p0 + 8 * C::V_STRIDE);
        const u32x4 aop = {x0[0], x0[1], x1[0], x1[1]};
        oacc[mo] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(aop), as_bf16x8(bop), oacc[mo], 0, 0, 0);
        oacc[mo] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(aop), as_bf16x8(bol), oacc[mo], 0, 0, 0);
      }
    }
    asm volatile("" ::: "memory");   // the next tile's V stores come after these reads
  }

  // ---- merge the four wave states (eqs 33.4-33.5) ----
  const float l_row = l_lane + __shfl_xor(l_lane, 32, 64);
  __syncthreads();                         // V buffers are free now
  debug_poison_lds(smem, C::MERGE);        // the merge area: only stored states are read
  float* mo_area = reinterpret_cast<float*>(smem);
  float* m_area = mo_area + kWaves * kRows * C::MO_STRIDE;
  float* l_area = m_area + kWaves * kRows;
  // Only the group's rows are stored (decode: G of the 32 lanes' rows).
  const int rows_here = a.rows - rg * kRows < kRows ? a.rows - rg * kRows : kRows;
  if (lr < rows_here) {
    float* dst = mo_area + (wave * kRows + lr) * C::MO_STRIDE;
#pragma unroll
    for (int mo = 0; mo < C::MO; ++mo)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 x = {oacc[mo][4 * g], oacc[mo][4 * g + 1], oacc[mo][4 * g + 2], oacc[mo][4 * g + 3]};
        *reinterpret_cast<f32x4*>(dst + 32 * mo + 8 * g + 4 * h) = x;
      }
    if (h == 0) {
      m_area[wave * kRows + lr] = has ? m2 : -INFINITY;
      l_area[wave * kRows + lr] = l_row;
    }
  }
  __syncthreads();
  // Each split's kW wave states merge into its partial; with a pair the
  // second split is written only if it lies in the grid's range and (per-batch
  // lengths) before L_b.
  constexpr int n_half = pair ? 2 : 1;
#pragma unroll
  for (int hf = 0; hf < n_half; ++hf)
  for (int e = tid; e < rows_here * DV; e += kThreads) {
    const int rr = e / DV, d = e % DV;
    const int w0 = hf * kW;
    const int sp = s_first + hf;
    if (pair && !(sp < a.split0 + a.n_active && static_cast<int64_t>(sp) * a.split_size < a.t_k)) continue;
    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < kW; ++i) M = fmaxf(M, m_area[(w0 + i) * kRows + rr]);
    float num = 0.0f, den = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int i = 0; i < kW; ++i) {
        const int w = w0 + i;
        const float mw = m_area[w * kRows + rr];
        if (mw == -INFINITY) continue;       // this wave saw no legal key
        const float c = fast_exp2(mw - M);
        num = fmaf(c, mo_area[(w * kRows + rr) * C::MO_STRIDE + d], num);
        den = fmaf(c, l_area[w * kRows + rr], den);
      }
    }
    const int nn = rg * kRows + rr;
    const int ghq = kvh * a.group + nn / a.t_q;
    const int gi = nn % a.t_q;
    const int64_t ridx = (static_cast<int64_t>(b) * a.heads_q + ghq) * a.t_q + gi;
    const bool live = M != -INFINITY;
    const float val = live ? num / den : 0.0f;
    if (SPLIT) {
      a.ws_o[(ridx * a.n_splits + sp) * DV + d] = val;
      if (d == 0) a.ws_lse[ridx * a.n_splits + sp] = live ? (M + fast_log2(den)) * kLn2 : -INFINITY;
    } else {
      uint16_t* op = a.o + b * a.os[0] + ghq * a.os[1] + static_cast<int64_t>(gi) * a.os[2];
      op[d] = f32_to_bf16(val);
      if (d == 0) a.lse[ridx] = live ? (M + fast_log2(den)) * kLn2 : -INFINITY;
    }
  }
}

template <int DH, int DV, bool SPLIT, bool VAR>
hipError_t launch_fb(const FArgs& a, const FBias& fb, int64_t blocks, hipStream_t stream) {
  if (fb.bias != nullptr)
    hipLaunchKernelGGL((fewrow_kernel<DH, DV, SPLIT, VAR, false, FBias>), dim3(static_cast<unsigned>(blocks)),
                       dim3(kThreads), 0, stream, a, fb);
  else if (SPLIT && a.pair)
    hipLaunchKernelGGL((fewrow_kernel<DH, DV, SPLIT, VAR, SPLIT>), dim3(static_cast<unsigned>(blocks)),
                       dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((fewrow_kernel<DH, DV, SPLIT, VAR, false>), dim3(static_cast<unsigned>(blocks)),
                       dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int DH, int DV, bool SPLIT>
hipError_t launch_f(const FArgs& a, const FBias& fb, int64_t blocks, hipStream_t stream) {
  return a.kv_lens != nullptr ? launch_fb<DH, DV, SPLIT, true>(a, fb, blocks, stream)
                              : launch_fb<DH, DV, SPLIT, false>(a, fb, blocks, stream);
}

template <bool SPLIT>
hipError_t launch_split(const FArgs& a, const FBias& fb, int64_t blocks, int d_h, int d_v, hipStream_t s) {
  if (d_h == 128 && d_v == 128) return launch_f<128, 128, SPLIT>(a, fb, blocks, s);
  if (d_h == 64 && d_v == 128) return launch_f<64, 128, SPLIT>(a, fb, blocks, s);
  if (d_h == 128 && d_v == 64) return launch_f<128, 64, SPLIT>(a, fb, blocks, s);
  return launch_f<64, 64, SPLIT>(a, fb, blocks, s);
}

FBias make_bias(const Problem& pb) {
  FBias fb{};
  fb.bias = pb.bias;
  for (int i = 0; i < 3; ++i) fb.bs[i] = pb.bs[i];
  fb.extent = (pb.batch - 1) * pb.bs[0] + (pb.heads_q - 1) * pb.bs[1] + (pb.t_q - 1) * pb.bs[2] + pb.t_k;
  return fb;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

bool eligible(const Problem& pb, int dtype, const void* q, const void* k, const void* v,
              const void* o) {
  if (dtype != ATTN_BF16 || pb.cu_q != nullptr) return false;
  // A bias must be contiguous along keys with 16-byte aligned rows, and a
  // row group's rows must start within 2^29 - 32 elements of its first row
  // (the staging copies address them with 31-bit byte offsets).
  if (pb.bias != nullptr &&
      (pb.bs[3] != 1 || ((pb.bs[0] | pb.bs[1] | pb.bs[2]) & 3) != 0 ||
       (reinterpret_cast<uintptr_t>(pb.bias) & 15) != 0 ||
       (pb.group - 1) * pb.bs[1] + (pb.t_q - 1) * pb.bs[2] >= (int64_t(1) << 29) - 32))
    return false;
  if (!((pb.d_h == 64 || pb.d_h == 128) && (pb.d_v == 64 || pb.d_v == 128))) return false;
  if (!(pb.scale_log2 > 0.0f)) return false;
  if (pb.t_q >= (int64_t(1) << 30) || pb.t_k >= (int64_t(1) << 30)) return false;
  if (pb.batch * pb.heads_kv >= (int64_t(1) << 30)) return false;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || (o && !aligned16(o))) return false;
  for (int i = 0; i < 3; ++i)
    if ((pb.qs[i] | pb.ks[i] | pb.vs[i]) & 7) return false;
  return true;
}

FArgs make_args(const Problem& pb, const void* q, const void* k, const void* v) {
  FArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
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
  a.rows = static_cast<int32_t>(pb.group * pb.t_q);
  a.n_rg = (a.rows + kRows - 1) / kRows;
  a.scale_log2 = pb.scale_log2;
  a.causal = pb.causal;
  a.kv_lens = pb.kv_lens;
  a.batch = static_cast<int32_t>(pb.batch);
  return a;
}

}  // namespace

bool launch_fewrow_fwd(const Problem& pb, int dtype, const void* q, const void* k,
                       const void* v, void* o, float* lse, int32_t* n_legal,
                       hipStream_t stream, int* status) {
  if (n_legal != nullptr) return false;
  if (!eligible(pb, dtype, q, k, v, o)) return false;
  if (pb.group * pb.t_q > kRows) return false;   // many rows: the prefill kernel
  for (int i = 0; i < 3; ++i)
    if (pb.os[i] & 7) return false;
  FArgs a = make_args(pb, q, k, v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.split_size = pb.t_k > 0 ? pb.t_k : 1;
  a.n_splits = 1;
  a.split0 = 0;
  a.n_active = 1;
  const int64_t blocks = pb.batch * pb.heads_kv * a.n_rg;
  const hipError_t e = launch_split<false>(a, make_bias(pb), blocks, static_cast<int>(pb.d_h),
                                           static_cast<int>(pb.d_v), stream);
  *status = e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
  return true;
}

bool launch_fewrow_partials(const Problem& pb, int dtype, const void* q, const void* k,
                            const void* v, const SplitLayout& L, float* ws_o, float* ws_lse,
                            hipStream_t stream, hipError_t* err) {
  if (!eligible(pb, dtype, q, k, v, nullptr)) return false;
  if (L.n_splits >= (int64_t(1) << 30)) return false;
  FArgs a = make_args(pb, q, k, v);
  a.ws_o = ws_o;
  a.ws_lse = ws_lse;
  a.split_size = L.split_size;
  a.n_splits = static_cast<int32_t>(L.n_splits);
  // Only the splits some row may see run (L.s0, L.s1); the merge reads no
  // other.  With per-batch lengths every split is launched, and one at or
  // past its batch's length returns at once.
  a.split0 = static_cast<int32_t>(L.s0);
  a.n_active = static_cast<int32_t>(L.s1 - L.s0);
  // Two splits per workgroup (two waves each; no bias) when the grid holds at
  // most 8 work items per CU (2048): there the per-workgroup start and end
  // latency is what the split costs (windowed decode, 1024 items: 56.8 ->
  // 49.4 us; 32-row decode groups, 2048 items: 121 -> 116 us).  The decode
  // workload's grid (8192 items of 4 rows) streams better one split per
  // workgroup (343 -> 353 us with pairs).
  const int64_t singles = pb.batch * pb.heads_kv * a.n_rg * a.n_active;
  a.pair = FEWROW_PAIR && a.n_active >= 2 && pb.bias == nullptr && singles <= 2048;
  const int64_t items = a.pair ? (a.n_active + 1) / 2 : a.n_active;
  const int64_t blocks = pb.batch * pb.heads_kv * a.n_rg * items;
  if (blocks >= (int64_t(1) << 31)) return false;
  *err = hipSuccess;
  if (blocks > 0)
    *err = launch_split<true>(a, make_bias(pb), blocks, static_cast<int>(pb.d_h), static_cast<int>(pb.d_v),
                              stream);
  return true;
}

}  // namespace attn
