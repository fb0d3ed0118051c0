/*
 * attn_mi355x.h - C ABI of an exact blocked attention library for AMD
 * Instinct MI355X (gfx950).
 *
 * The library computes scaled-dot-product attention exactly, key block by key
 * block, carrying per query row the online-softmax statistics of the keys seen
 * so far: the maximum score m, the scaled exponential sum l and the scaled
 * value sum u.  Two disjoint key sets merge by m = max(m_A, m_B),
 * l = e^{m_A-m} l_A + e^{m_B-m} l_B, u = e^{m_A-m} u_A + e^{m_B-m} u_B, and a
 * row's output is o = u / l.  Sources: "Chapter 33 推理计算优化"
 * (faketrader.github.io, llm-from-scratch), §33.2 eq 33.2 (the operation),
 * eq 33.3 (statistics), eqs 33.4-33.5 (merge), the valid-flag rule and
 * Algorithm 33.1; §33.3 (blocking, causal block skipping, interface
 * consistency: mask polarity, non-square causal alignment, head grouping,
 * scale, strides).  Query positions follow the KV-cache section of
 * "Generation and Caching with the Same Model" (aihero.club): query row i is
 * at logical position q_offset + i and, when causal, sees keys j <= q_offset + i.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *   allocates no device memory and keeps no mutable global state, so calls on
 *   different streams may run concurrently; the one exception is the fixed
 *   per-GPU workspace of attn_decode_splitkv_noalloc (see there).
 * - Layout is [B, H, T, D] with the innermost (D) dimension contiguous; the
 *   three outer strides are given in ELEMENTS, must be >= 0, and may be 0 to
 *   broadcast.  LSE and n_legal are contiguous [B, H_q, T_q].
 * - Every call is asynchronous on the given stream (a hipStream_t passed as
 *   void*; NULL = the null stream).  The library never synchronises and
 *   never reads device memory on the host.
 * - Arguments are validated before anything is launched; on an error nothing
 *   is written and a negative attn_status_t is returned.  ATTN_E_HIP reports a
 *   failed launch; faults inside a kernel surface at the caller's next
 *   synchronisation.
 * - A row with no legal key (every key causally invisible or masked by a
 *   -inf bias, or T_k = 0) is NOT an error: its output row is +0.0 (all bits
 *   zero) and its LSE is -inf (0xFF800000), its n_legal 0.  No NaN is formed.
 * - A pointer may be NULL only when the tensor it stands for has no elements.
 */
#ifndef ATTN_MI355X_H
#define ATTN_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 4

/* Size of the per-GPU decode workspace that attn_decode_splitkv_noalloc uses
 * (32 MiB: the GQA decode of batch 16, 32 query heads, 64 ranges and d_v 128
 * needs 16.9 MB). */
#define ATTN_DECODE_SCRATCH_BYTES (32u << 20)

typedef enum {
  ATTN_OK = 0,
  ATTN_E_NULL = -1,        /* a required pointer is NULL */
  ATTN_E_SHAPE = -2,       /* negative size or window, H_q % H_kv != 0, bad split size */
  ATTN_E_DTYPE = -3,       /* unknown element type */
  ATTN_E_UNSUPPORTED = -4, /* d_h or d_v outside [1, 256], non-finite scale, or a
                              variable-length field the entry point does not take */
  ATTN_E_STRIDE = -5,      /* a negative stride */
  ATTN_E_WORKSPACE = -6,   /* decode workspace missing or too small */
  ATTN_E_HIP = -7,         /* the HIP runtime refused a launch */
  ATTN_E_SCRATCH = -8      /* attn_decode_splitkv_noalloc: the problem needs more than
                              ATTN_DECODE_SCRATCH_BYTES of workspace */
} attn_status_t;

typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype_t;

/* Problem description (eq 33.2 of §33.2 with the symbols of Table 33.1).
 * z_ij = scale * <q_i, k_j> + M_ij, where M is the optional additive bias
 * (never scaled).  Key j is LEGAL for row i iff it is causally visible
 * (causal == 0, or j <= q_offset + i), inside the sliding window when one is
 * set (window W >= 1: j >= q_offset + i - W + 1, the W positions ending at
 * the row's own; §33.7, the sliding-window paragraph with eq 33.16) and
 * M_ij != -inf.  Query head hq reads KV head hq / (heads_q / heads_kv)
 * (contiguous head groups). */
typedef struct {
  int64_t batch;          /* B >= 0 */
  int64_t heads_q;        /* H_q >= 1, a multiple of heads_kv */
  int64_t heads_kv;       /* H_kv >= 1 */
  int64_t t_q;            /* T_q >= 0 query rows */
  int64_t t_k;            /* T_k >= 0 keys */
  int64_t d_h;            /* key/query head size, 1..256 */
  int64_t d_v;            /* value head size, 1..256 */
  int64_t q_offset;       /* logical position of query row 0; any value */
  int64_t q_stride[3];    /* Q [B, H_q, T_q, d_h]: strides of b, h, t */
  int64_t k_stride[3];    /* K [B, H_kv, T_k, d_h] */
  int64_t v_stride[3];    /* V [B, H_kv, T_k, d_v] */
  int64_t o_stride[3];    /* O [B, H_q, T_q, d_v] */
  int64_t bias_stride[4]; /* bias over [b, hq, i, j]; 0 broadcasts */
  const float* bias;      /* fp32 additive bias/mask, NULL = none; -inf masks;
                             +inf and NaN are outside the contract */
  float scale;            /* finite; usually 1/sqrt(d_h) */
  int32_t dtype;          /* attn_dtype_t of Q, K, V and O */
  int32_t causal;         /* 0 or 1 */
  int32_t window;         /* sliding window W >= 1 keys, 0 = none; < 0 is an error */
  /* Unpadded variable-length batches (§33.4, shape bucketing: padding every
   * sequence to a bucket length b(T) costs dense attention about
   * E[b(T)^2 - T^2] extra score work; these fields remove the padding).
   *
   * Packed sequences (attn_fwd and attn_bwd): with cu_seqlens_q != NULL, batch must
   * be 1 and Q, O (rows) and K, V (keys) hold n_seqs sequences one after the
   * other along T.  Sequence s owns query rows [cu_seqlens_q[s],
   * cu_seqlens_q[s+1]) and keys [cu_seqlens_k[s], cu_seqlens_k[s+1]); with
   * L_q and L_k its lengths, its row i sits at logical position
   * q_offset + (L_k - L_q) + i (its rows are the last L_q positions of its
   * keys) and sees only its own keys.  The bias, if any, is indexed by packed
   * row and packed key (sequence s reads its diagonal block; stride 0
   * broadcasts as usual, so bias_stride[2] = 0 gives one M_j per packed key).
   * Both arrays are DEVICE int32 arrays of n_seqs + 1 entries, non-decreasing,
   * from 0 up to T_q and T_k.  The library never reads them on the host; in a
   * kernel each entry is clamped to [0, T] and a decreasing pair is an empty
   * sequence, so no access leaves the tensors; rows outside every sequence are
   * not written.  max_seqlen_q sizes the grid (one pass covers that many rows
   * per sequence); any value >= 0 gives the same result, a smaller one than
   * the longest L_q only costs time.  lse and n_legal are [1, H_q, T_q]. */
  const int32_t* cu_seqlens_q; /* NULL = one dense batch */
  const int32_t* cu_seqlens_k; /* required with cu_seqlens_q */
  int64_t n_seqs;              /* >= 0 with cu_seqlens_q, else ignored */
  int64_t max_seqlen_q;        /* >= 0 with cu_seqlens_q, else ignored */
  /* Per-batch KV lengths (attn_fwd, attn_bwd and attn_decode_splitkv, not with
   * cu_seqlens_q): batch b uses keys [0, L_b) of K and V, L_b =
   * seqlens_k[b] clamped to [0, T_k] in the kernel, and its row i sits at
   * q_offset + L_b - T_q + i.  DEVICE int32 array of B entries; NULL = every
   * batch uses all T_k keys at positions q_offset + i. */
  const int32_t* seqlens_k;
} attn_params_t;

/* sizeof(attn_params_t), so that bindings can check their mirror of it.
 * (Binding plumbing: no passage of the pages defines it.) */
size_t attn_params_sizeof(void);
/* ATTN_ABI_VERSION as built into the library, for the same check. */
int attn_abi_version(void);
/* A one-line description of an attn_status_t.  Every entry point reports
 * input it cannot honour with one of these codes instead of proceeding: the
 * consistency conditions of §33.3 ("interface, backends and correctness
 * conditions": mask polarity, causal alignment, head grouping, scale,
 * strides) and the rejection of inconsistent caches by the cached forward of
 * "Generation and Caching with the Same Model".  Unknown codes give
 * "unknown status"; the string is static. */
const char* attn_strerror(int status);

/* Exact attention over all query rows (prefill, non-square causal, verify).
 * Implements Algorithm 33.1 of §33.2 for every (b, hq, i) with the keys read
 * in tiles; tiles that no row of a query tile can see are skipped (§33.3).
 * Outputs: o [B, H_q, T_q, d_v] in p->dtype (bf16 rounded to nearest even),
 * lse [B, H_q, T_q] fp32 = ln sum_{legal j} e^{z_ij} (natural log), and
 * optionally n_legal [B, H_q, T_q] int32 = number of legal keys (NULL to
 * skip).  Returns ATTN_OK or a negative attn_status_t. */
int attn_fwd(const attn_params_t* p, const void* q, const void* k,
             const void* v, void* o, float* lse, int32_t* n_legal,
             void* stream);

/* Bytes of device workspace that attn_decode_splitkv needs for this problem
 * and split size: one stored partial per query row and key range, the
 * range's (o_s, lse_s), which stands for its statistics (m, l, u) =
 * (lse_s, 1, o_s) in the merge of eqs 33.4-33.5 (§33.2; the merge holds for
 * any reference maximum).  Layout: fp32 partial outputs [B, H_q, T_q, S, d_v]
 * followed by fp32 partial LSEs [B, H_q, T_q, S] (each array 256-byte
 * aligned), where S = ceil(T_k / split_size) (at least 1).  Returns 0 on
 * invalid arguments. */
size_t attn_decode_workspace_bytes(const attn_params_t* p, int64_t split_size);

/* Split-KV attention for few query rows over a long KV cache (decode).
 * Keys are cut into contiguous ranges [s*S, min((s+1)*S, T_k)); for each
 * (b, kv head, range) one partial (o_s, lse_s) per query row is written to
 * the workspace (the range's own exact attention; o_s = 0 and lse_s = -inf if
 * the range holds no legal key), then the partials of every row are merged by
 * eqs 33.4-33.5 of §33.2 taking (lse_s, 1, o_s) as each range's statistics.
 * Same outputs and conventions as attn_fwd (no n_legal).  split_size >= 1.
 * workspace must hold attn_decode_workspace_bytes(p, split_size) bytes
 * (256-byte aligned); its contents after the call are the partials in the
 * layout above for the ranges some row may see; the others hold no legal key
 * of any row and are neither written nor read: without seqlens_k, ranges at
 * or past the last causal position q_offset + T_q (causal) and ranges wholly
 * before the first window start q_offset - window + 1 (window > 0); with
 * seqlens_k, ranges at or past L_b (the merge reads only the first
 * ceil(L_b / split_size) partials of a row of batch b).  cu_seqlens_q is not
 * taken (ATTN_E_UNSUPPORTED). */
int attn_decode_splitkv(const attn_params_t* p, int64_t split_size,
                        const void* q, const void* k_cache,
                        const void* v_cache, void* o, float* lse,
                        void* workspace, size_t workspace_bytes,
                        void* stream);

/* attn_decode_splitkv without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that
 * forbid allocation).  Same problem, split size, inputs, outputs and results
 * (the same kernels) as attn_decode_splitkv; the partials go to a fixed
 * array of ATTN_DECODE_SCRATCH_BYTES in device memory that the library holds
 * on every GPU it runs on until the process ends (its address on the current
 * device is looked up on the first call there).  The call runs on the
 * current device, which must be the device of the tensors and the stream.
 * Returns ATTN_E_SCRATCH, before touching the device, when
 * attn_decode_workspace_bytes(p, split_size) exceeds
 * ATTN_DECODE_SCRATCH_BYTES.  Allocates nothing.  Every call on a GPU shares
 * that GPU's array: calls that overlap on one GPU (on different streams, or
 * from several threads) race and their results are undefined; calls ordered
 * on one stream are safe, since each call writes every partial it reads. */
int attn_decode_splitkv_noalloc(const attn_params_t* p, int64_t split_size,
                                const void* q, const void* k_cache,
                                const void* v_cache, void* o, float* lse,
                                void* stream);

/* Merge n_states partial results per row (eqs 33.4-33.5 of §33.2).
 * Row r, state s: o_states[r*o_row_stride + s*o_state_stride + d] (fp32, d <
 * d_v) and lse_states[r*lse_row_stride + s*lse_state_stride] (fp32, natural
 * log; -inf marks an empty state, which is skipped).  Each valid state stands
 * for the triple (m, l, u) = (lse_s, 1, o_s).  Output row r:
 * o_out[r*o_out_row_stride + d] in out_dtype and lse_out[r] (contiguous);
 * a row with no valid state gets (+0.0, -inf).  n_states >= 1 unless
 * n_rows == 0; 1 <= d_v <= 256; strides >= 0. */
int attn_merge_states(int64_t n_rows, int64_t n_states, int64_t d_v,
                      const float* o_states, int64_t o_row_stride,
                      int64_t o_state_stride, const float* lse_states,
                      int64_t lse_row_stride, int64_t lse_state_stride,
                      int32_t out_dtype, void* o_out,
                      int64_t o_out_row_stride, float* lse_out, void* stream);

/* Bytes of device workspace that attn_bwd needs: fp32 D_i = <dO_i, O_i> for
 * every query row [B, H_q, T_q] (256-byte aligned).  Returns 0 on invalid
 * arguments. */
size_t attn_bwd_workspace_bytes(const attn_params_t* p);

/* Gradients of attn_fwd's attention with respect to Q, K and V by
 * recomputation from the saved LSE (eqs 33.6-33.8 of §33.3 and Exercise
 * 33.4): with P_ij = e^{z_ij - LSE_i} on legal keys (0 elsewhere),
 * dV = P^T dO, dP = dO V^T, dS_ij = P_ij (dP_ij - <dO_i, O_i>),
 * dQ = scale dS K, dK = scale dS^T Q.  Inputs: q, k, v as for attn_fwd, the
 * forward outputs o and lse of the same call, and the upstream gradient d_o
 * [B, H_q, T_q, d_v].  Outputs (overwritten, never accumulated): d_q
 * [B, H_q, T_q, d_h], d_k [B, H_kv, T_k, d_h], d_v [B, H_kv, T_k, d_v]; dK and
 * dV of a KV head sum over the query heads of its group.  Each gradient and
 * d_o use the element type and the strides of their forward tensor (d_o and o
 * share o_stride, d_q q_stride, d_k k_stride, d_v v_stride).  The bias (if
 * any) is a constant input and gets no gradient; rows with no legal key (LSE
 * = -inf) contribute nothing.  workspace: attn_bwd_workspace_bytes(p) bytes,
 * 256-byte aligned.  Packed sequences (cu_seqlens_q) are taken as in
 * attn_fwd, each sequence's gradients from its own rows and keys; rows and
 * keys outside every sequence are not written, and n_seqs = 0 writes nothing.
 * Per-batch KV lengths (seqlens_k) are taken as in attn_fwd; the keys of
 * batch b at or past L_b get zero gradients. */
int attn_bwd(const attn_params_t* p, const void* q, const void* k, const void* v,
             const void* o, const float* lse, const void* d_o, void* d_q, void* d_k,
             void* d_v, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MI355X_H */
