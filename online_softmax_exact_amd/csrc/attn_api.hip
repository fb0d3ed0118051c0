// Host side of the C ABI: argument validation (before any launch, without
// touching device memory), kernel choice and launches on the caller's stream.
// Validation mirrors the interface conditions of §33.3 of "Chapter 33
// 推理计算优化" (mask polarity, non-square causal alignment, head grouping,
// scale, strides must be consistent) and rejects input it cannot honour
// instead of proceeding, as the cached forward of "Generation and Caching
// with the Same Model" does for inconsistent caches.
#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "attn_internal.h"
#include "kernels.h"

// Decode workspace of attn_decode_splitkv_noalloc, for callers that cannot
// allocate device memory: one array per GPU, held until the process ends.
// Host code never passes its name to a kernel (on the host the name is only
// a stand-in for the device variable); it uses the per-device address that
// hipGetSymbolAddress returns.
static __device__ __align__(256) char scratch[ATTN_DECODE_SCRATCH_BYTES];

namespace attn {

SplitLayout split_layout(const Problem& pb, int64_t split_size) {
  SplitLayout L{};
  L.split_size = split_size;
  L.rows = pb.batch * pb.heads_q * pb.t_q;
  L.n_splits = pb.t_k > 0 ? pb.t_k / split_size + (pb.t_k % split_size != 0) : 1;
  const size_t o_bytes = static_cast<size_t>(L.rows) * L.n_splits * pb.d_v * sizeof(float);
  L.o_bytes = o_bytes;
  L.lse_offset = (o_bytes + 255) & ~static_cast<size_t>(255);
  L.total = L.lse_offset + ((static_cast<size_t>(L.rows) * L.n_splits * sizeof(float) + 255) &
                            ~static_cast<size_t>(255));
  L.s0 = 0;
  L.s1 = L.n_splits;
  if (pb.kv_lens == nullptr) {
    int64_t k_lo = 0, k_hi = pb.t_k;
    if (pb.causal && pb.q_offset + pb.t_q < k_hi) k_hi = pb.q_offset + pb.t_q;
    if (pb.window > 0 && pb.q_offset - pb.window + 1 > k_lo) k_lo = pb.q_offset - pb.window + 1;
    if (k_hi > k_lo) {
      L.s0 = k_lo / split_size;
      L.s1 = (k_hi - 1) / split_size + 1;
      if (L.s1 > L.n_splits) L.s1 = L.n_splits;
      if (L.s0 > L.s1) L.s0 = L.s1;
    } else {
      L.s0 = L.s1 = 0;
    }
  }
  return L;
}

namespace {

constexpr int64_t kMaxHead = 256;
constexpr int64_t kMaxDim = int64_t(1) << 40;     // any size or row count
constexpr int64_t kMaxOffset = int64_t(1) << 60;  // |q_offset|

bool product_ok(int64_t a, int64_t b, int64_t c) {
  const __int128 x = static_cast<__int128>(a) * b * c;
  return x <= kMaxDim;
}

bool numel_nonzero(int64_t a, int64_t b, int64_t c, int64_t d) {
  return a > 0 && b > 0 && c > 0 && d > 0;
}

int validate(const attn_params_t* p, Problem* pb) {
  if (p == nullptr) return ATTN_E_NULL;
  if (p->dtype != ATTN_F32 && p->dtype != ATTN_BF16) return ATTN_E_DTYPE;
  if (p->batch < 0 || p->t_q < 0 || p->t_k < 0 || p->heads_q < 1 || p->heads_kv < 1)
    return ATTN_E_SHAPE;
  if (p->batch > kMaxDim || p->t_q > kMaxDim || p->t_k > kMaxDim || p->heads_q > kMaxDim)
    return ATTN_E_SHAPE;
  if (p->heads_q % p->heads_kv != 0) return ATTN_E_SHAPE;
  // Row counts must stay far from int64 overflow in the index math.
  if (!product_ok(p->batch, p->heads_q, p->t_q) || !product_ok(p->batch, p->heads_kv, p->t_k))
    return ATTN_E_SHAPE;
  if (p->causal != 0 && p->causal != 1) return ATTN_E_SHAPE;
  if (p->window < 0) return ATTN_E_SHAPE;
  if (p->q_offset > kMaxOffset || p->q_offset < -kMaxOffset) return ATTN_E_SHAPE;
  if (p->d_h < 1 || p->d_h > kMaxHead || p->d_v < 1 || p->d_v > kMaxHead) return ATTN_E_UNSUPPORTED;
  if (!isfinite(p->scale)) return ATTN_E_UNSUPPORTED;
  for (int i = 0; i < 3; ++i)
    if (p->q_stride[i] < 0 || p->k_stride[i] < 0 || p->v_stride[i] < 0 || p->o_stride[i] < 0)
      return ATTN_E_STRIDE;
  for (int i = 0; i < 4; ++i)
    if (p->bias_stride[i] < 0) return ATTN_E_STRIDE;
  // Variable-length fields: cu_seqlens entries and KV lengths are int32.
  if (p->cu_seqlens_q != nullptr) {
    if (p->cu_seqlens_k == nullptr) return ATTN_E_NULL;
    if (p->batch != 1 || p->seqlens_k != nullptr) return ATTN_E_SHAPE;
    if (p->n_seqs < 0 || p->n_seqs >= (int64_t(1) << 30)) return ATTN_E_SHAPE;
    if (p->max_seqlen_q < 0 || p->max_seqlen_q > kMaxDim) return ATTN_E_SHAPE;
    if (p->t_q >= (int64_t(1) << 31) || p->t_k >= (int64_t(1) << 31)) return ATTN_E_SHAPE;
  } else if (p->cu_seqlens_k != nullptr) {
    return ATTN_E_SHAPE;   // key offsets without row offsets
  }
  if (p->seqlens_k != nullptr && p->t_k >= (int64_t(1) << 31)) return ATTN_E_SHAPE;

  pb->batch = p->batch; pb->heads_q = p->heads_q; pb->heads_kv = p->heads_kv;
  pb->t_q = p->t_q; pb->t_k = p->t_k; pb->d_h = p->d_h; pb->d_v = p->d_v;
  pb->q_offset = p->q_offset;
  memcpy(pb->qs, p->q_stride, sizeof(pb->qs));
  memcpy(pb->ks, p->k_stride, sizeof(pb->ks));
  memcpy(pb->vs, p->v_stride, sizeof(pb->vs));
  memcpy(pb->os, p->o_stride, sizeof(pb->os));
  memcpy(pb->bs, p->bias_stride, sizeof(pb->bs));
  pb->bias = p->bias;
  pb->scale_log2 = p->scale * kLog2e;
  pb->causal = p->causal;
  pb->group = static_cast<int32_t>(p->heads_q / p->heads_kv);
  pb->window = p->window;
  pb->cu_q = p->cu_seqlens_q;
  pb->cu_k = p->cu_seqlens_q != nullptr ? p->cu_seqlens_k : nullptr;
  pb->n_seqs = p->cu_seqlens_q != nullptr ? p->n_seqs : 0;
  pb->max_seqlen_q = p->cu_seqlens_q != nullptr ? p->max_seqlen_q : 0;
  pb->kv_lens = p->seqlens_k;
  return ATTN_OK;
}

// Pointers of tensors with elements must be non-NULL.
int check_pointers(const Problem& pb, const void* q, const void* k, const void* v,
                   const void* o, const void* lse) {
  const bool rows = numel_nonzero(pb.batch, pb.heads_q, pb.t_q, 1);
  const bool keys = numel_nonzero(pb.batch, pb.heads_kv, pb.t_k, 1);
  if (rows && (q == nullptr || o == nullptr || lse == nullptr)) return ATTN_E_NULL;
  if (rows && keys && (k == nullptr || v == nullptr)) return ATTN_E_NULL;
  return ATTN_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_E_HIP; }

// Device address of `scratch` on the current device, looked up on the first
// call on that device (with it current) and kept: each GPU holds its own
// copy of the array at its own address.
constexpr int kMaxDevices = 64;
std::atomic<char*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_of_current_device(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_E_HIP;
  char* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch[dev].load(std::memory_order_relaxed);
    if (ptr == nullptr) {
      void* addr = nullptr;
      if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr)
        return ATTN_E_HIP;
      ptr = static_cast<char*>(addr);
      g_scratch[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return ATTN_OK;
}

// Split-KV partials into the workspace `ws` (layout L), then their merge
// into o / lse.  Shared by both decode entry points.
int decode_into(const Problem& pb, int dtype, int64_t split_size, const void* q,
                const void* k_cache, const void* v_cache, void* o, float* lse, char* ws,
                const SplitLayout& L, hipStream_t s) {
  float* ws_o = reinterpret_cast<float*>(ws);
  float* ws_l = reinterpret_cast<float*>(ws + L.lse_offset);
  hipError_t e = hipSuccess;
  if (!launch_fast_decode_partials(pb, dtype, q, k_cache, v_cache, L, ws_o, ws_l, s, &e))
    e = launch_generic(pb, dtype, q, k_cache, v_cache, nullptr, nullptr, nullptr,
                       split_size, ws_o, ws_l, s);
  if (e != hipSuccess) return ATTN_E_HIP;
  // The merge reads the splits some row can see (a row with none gets the
  // defined (+0, -inf)).
  const int64_t out_strides[3] = {pb.os[0], pb.os[1], pb.os[2]};
  return hip_status(launch_merge(L.rows, L.s1 - L.s0, pb.d_v, ws_o + L.s0 * pb.d_v, L.n_splits * pb.d_v,
                                 pb.d_v, ws_l + L.s0, L.n_splits, 1, dtype, o, pb.heads_q, pb.t_q,
                                 out_strides, lse, s, pb.kv_lens, split_size, pb.t_k));
}

}  // namespace
}  // namespace attn

using namespace attn;

extern "C" {

size_t attn_params_sizeof(void) { return sizeof(attn_params_t); }

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

const char* attn_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_E_NULL: return "a required pointer is NULL";
    case ATTN_E_SHAPE: return "invalid shape (negative size or window, heads_q not a multiple of heads_kv, bad flag or split size)";
    case ATTN_E_DTYPE: return "unknown element type";
    case ATTN_E_UNSUPPORTED: return "unsupported head size (d_h and d_v must be 1..256), non-finite scale, or a variable-length field this entry point does not take";
    case ATTN_E_STRIDE: return "negative stride";
    case ATTN_E_WORKSPACE: return "decode workspace missing or too small";
    case ATTN_E_HIP: return "HIP runtime error at launch";
    case ATTN_E_SCRATCH: return "decode needs more workspace than the no-allocation entry point holds (ATTN_DECODE_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int attn_fwd(const attn_params_t* p, const void* q, const void* k, const void* v,
             void* o, float* lse, int32_t* n_legal, void* stream) {
  Problem pb;
  int st = validate(p, &pb);
  if (st != ATTN_OK) return st;
  if ((st = check_pointers(pb, q, k, v, o, lse)) != ATTN_OK) return st;
  if (pb.batch == 0 || pb.t_q == 0) return ATTN_OK;
  if (pb.cu_q != nullptr && pb.n_seqs == 0) return ATTN_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (launch_fast_fwd(pb, p->dtype, q, k, v, o, lse, n_legal, s, &st)) return st;
  return hip_status(launch_generic(pb, p->dtype, q, k, v, o, lse, n_legal, 0, nullptr, nullptr, s));
}

size_t attn_bwd_workspace_bytes(const attn_params_t* p) {
  Problem pb;
  if (validate(p, &pb) != ATTN_OK) return 0;
  const size_t rows = static_cast<size_t>(pb.batch * pb.heads_q * pb.t_q);
  return ((rows > 0 ? rows : 1) * sizeof(float) + 255) & ~static_cast<size_t>(255);
}

int attn_bwd(const attn_params_t* p, const void* q, const void* k, const void* v, const void* o,
             const float* lse, const void* d_o, void* d_q, void* d_k, void* d_v, void* workspace,
             size_t workspace_bytes, void* stream) {
  Problem pb;
  int st = validate(p, &pb);
  if (st != ATTN_OK) return st;
  if ((st = check_pointers(pb, q, k, v, o, lse)) != ATTN_OK) return st;
  if (pb.cu_q != nullptr && pb.n_seqs == 0) return ATTN_OK;
  const bool rows = numel_nonzero(pb.batch, pb.heads_q, pb.t_q, 1);
  const bool keys = numel_nonzero(pb.batch, pb.heads_kv, pb.t_k, 1);
  if (rows && (d_o == nullptr || d_q == nullptr)) return ATTN_E_NULL;
  if (keys && (k == nullptr || v == nullptr || d_k == nullptr || d_v == nullptr)) return ATTN_E_NULL;
  if (!rows && !keys) return ATTN_OK;
  if (workspace == nullptr || workspace_bytes < attn_bwd_workspace_bytes(p)) return ATTN_E_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return ATTN_E_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* ws_d = static_cast<float*>(workspace);
  // D = <dO, O> per row: computed by the MFMA dQ kernel for its rows, else
  // by the row-dot kernel ahead of the generic dQ kernel.  dK / dV run after
  // dQ on the same stream and read it.
  hipError_t e = hipSuccess;
  if (!launch_bwd_dq_mfma(pb, p->dtype, q, k, v, o, lse, d_o, ws_d, d_q, s, &e)) {
    e = launch_bwd_rowdot(pb, p->dtype, o, d_o, ws_d, s);
    if (e == hipSuccess) e = launch_bwd_dq_generic(pb, p->dtype, q, k, v, lse, d_o, ws_d, d_q, s);
  }
  if (e == hipSuccess && !launch_bwd_dkdv_mfma(pb, p->dtype, q, k, v, lse, d_o, ws_d, d_k, d_v, s, &e))
    e = launch_bwd_dkdv_generic(pb, p->dtype, q, k, v, lse, d_o, ws_d, d_k, d_v, s);
  return hip_status(e);
}

size_t attn_decode_workspace_bytes(const attn_params_t* p, int64_t split_size) {
  Problem pb;
  if (validate(p, &pb) != ATTN_OK || split_size < 1) return 0;
  return split_layout(pb, split_size).total;
}

int attn_decode_splitkv(const attn_params_t* p, int64_t split_size, const void* q,
                        const void* k_cache, const void* v_cache, void* o, float* lse,
                        void* workspace, size_t workspace_bytes, void* stream) {
  Problem pb;
  int st = validate(p, &pb);
  if (st != ATTN_OK) return st;
  if (split_size < 1) return ATTN_E_SHAPE;
  if ((st = check_pointers(pb, q, k_cache, v_cache, o, lse)) != ATTN_OK) return st;
  if (pb.cu_q != nullptr) return ATTN_E_UNSUPPORTED;
  if (pb.batch == 0 || pb.t_q == 0) return ATTN_OK;
  const SplitLayout L = split_layout(pb, split_size);
  if (workspace == nullptr || workspace_bytes < L.total) return ATTN_E_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return ATTN_E_WORKSPACE;
  return decode_into(pb, p->dtype, split_size, q, k_cache, v_cache, o, lse,
                     static_cast<char*>(workspace), L, static_cast<hipStream_t>(stream));
}

int attn_decode_splitkv_noalloc(const attn_params_t* p, int64_t split_size, const void* q,
                                const void* k_cache, const void* v_cache, void* o, float* lse,
                                void* stream) {
  Problem pb;
  int st = validate(p, &pb);
  if (st != ATTN_OK) return st;
  if (split_size < 1) return ATTN_E_SHAPE;
  if ((st = check_pointers(pb, q, k_cache, v_cache, o, lse)) != ATTN_OK) return st;
  if (pb.cu_q != nullptr) return ATTN_E_UNSUPPORTED;
  if (pb.batch == 0 || pb.t_q == 0) return ATTN_OK;
  const SplitLayout L = split_layout(pb, split_size);
  if (L.total > static_cast<size_t>(ATTN_DECODE_SCRATCH_BYTES)) return ATTN_E_SCRATCH;
  // Every partial the merge reads is written by this call's partial kernels
  // first, so nothing left in the array by an earlier call is read.
  char* ws = nullptr;
  if ((st = scratch_of_current_device(&ws)) != ATTN_OK) return st;
  return decode_into(pb, p->dtype, split_size, q, k_cache, v_cache, o, lse, ws, L,
                     static_cast<hipStream_t>(stream));
}

int attn_merge_states(int64_t n_rows, int64_t n_states, int64_t d_v, const float* o_states,
                      int64_t o_row_stride, int64_t o_state_stride, const float* lse_states,
                      int64_t lse_row_stride, int64_t lse_state_stride, int32_t out_dtype,
                      void* o_out, int64_t o_out_row_stride, float* lse_out, void* stream) {
  if (out_dtype != ATTN_F32 && out_dtype != ATTN_BF16) return ATTN_E_DTYPE;
  if (n_rows < 0 || n_states < 0 || n_rows > (int64_t(1) << 32)) return ATTN_E_SHAPE;
  if (d_v < 1 || d_v > kMaxHead) return ATTN_E_UNSUPPORTED;
  if (o_row_stride < 0 || o_state_stride < 0 || lse_row_stride < 0 || lse_state_stride < 0 ||
      o_out_row_stride < 0)
    return ATTN_E_STRIDE;
  if (n_rows == 0) return ATTN_OK;
  if (n_states < 1) return ATTN_E_SHAPE;
  if (o_states == nullptr || lse_states == nullptr || o_out == nullptr || lse_out == nullptr)
    return ATTN_E_NULL;
  const int64_t out_strides[3] = {o_out_row_stride, 0, 0};
  return hip_status(launch_merge(n_rows, n_states, d_v, o_states, o_row_stride, o_state_stride,
                                 lse_states, lse_row_stride, lse_state_stride, out_dtype, o_out,
                                 1, 1, out_strides, lse_out, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
