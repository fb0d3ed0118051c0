"""Plain fp64 CPU oracle for exact softmax attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check of the graft entry
module and the CPU-baseline leg of the benchmark may import this module.  The
product path (the HIP library and its Python binding) never calls it and shares
no code with it.

Sources (the pages this follows; cited by page title and section / equation):

* "Chapter 33 推理计算优化" (faketrader.github.io, llm-from-scratch), §33.2:
  eq 33.2 (single-query attention with additive bias/mask M_j), eq 33.3 (the
  sufficient statistics m, ℓ, u of a non-empty legal key set), eqs 33.4-33.5
  (the merge of two disjoint sets), the valid-flag rule for empty blocks and
  fully masked rows, Algorithm 33.1 (single-query blocked exact attention) and
  Example 25.1; §33.3 (the explicit T_q x T_k implementation, causal block
  skipping, non-square causal alignment by logical position); §33.7, the
  sliding-window paragraph (only keys in a prescribed range stay visible) and
  eq 33.16 (the error bound against full attention); §33.3, "block size,
  parallelism and backward recomputation": eqs 33.6-33.8 (gradients from the
  recomputed probabilities) and Exercise 33.4 (the row-mean term from the
  softmax Jacobian); §33.4, shape bucketing (the padding cost E[b(T)^2 - T^2]
  that unpadded variable-length batches avoid).
* "Generation and Caching with the Same Model" (aihero.club), the KV-cache
  section and its `causal_attention` listing: the [B, H, T, D] layout and the
  rule that query row i sits at logical position q_offset + i and sees the
  keys j <= q_offset + i.

Two independent formulations live here:

1. ``attention`` / ``attention_rows``: the definition written out.  The whole
   T_q x T_k score matrix of one (batch, head) is materialised in fp64, the
   illegal entries are set to -inf, and each row with at least one legal key
   is normalised by its own maximum.  This is the explicit implementation of
   §33.3, with the fully masked row defined as (O = +0, LSE = -inf) instead of
   the NaN that a plain softmax of an all -inf row would give.
2. ``block_stats`` / ``merge_stats`` / ``finalize`` / ``blocked_single_query``:
   the pages' statistics and merge (eqs 33.3-33.5) and Algorithm 33.1 step by
   step, generic over the arithmetic so that tests can run them in exact
   rational arithmetic as well as in fp64.

Readings taken where the pages leave a step open (each is listed in the design
notes of the repository):

* LSE of a row is ln sum_{legal j} e^{z_j} = m + ln ℓ (natural log, scale and
  bias included).
* A key is legal for row i iff it is causally visible (j <= q_offset + i, or
  always when not causal), inside the sliding window when there is one
  (j >= q_offset + i - W + 1: the W positions ending at the row's own; the
  window is a lower bound only, also without causal masking) and its bias is
  not -inf.
* A row with no legal key returns O = +0.0 and LSE = -inf (and a legal-key
  count of 0); it is not an error.
* Grouped heads: query head hq reads KV head hq // (H_q / H_kv).
* A stored partial (o_s, lse_s) stands for the triple (lse_s, 1, o_s); a
  partial with lse_s = -inf is empty and is skipped, never subtracted.
* Split-KV partials cover contiguous key ranges [s*S, min((s+1)*S, T_k)).
* Unpadded variable-length batches: row i of packed sequence s sits at
  q_offset + (L_k,s - L_q,s) + i, i.e. a sequence's rows are the last L_q
  positions of its keys (the pages name the padding cost, not the layout).
* Backward (eqs 33.6-33.8): the score scale replaces 1/sqrt(d_h) in eq 33.8
  (its trailing "." is a garble); the bias gets no gradient; illegal keys and
  fully masked rows have P = 0 and so contribute no gradient; the K and V
  gradients of a KV head sum over the query heads that read it.

Nothing here is pinned by itself: the ``-m "not gpu"`` tests pin it against
the printed example, closed forms, invariants, brute force over block
partitions and an independent library softmax.
"""

from __future__ import annotations

import functools
import math
from fractions import Fraction
from typing import Callable, List, Optional, Sequence, Tuple

import numpy as np

NEG_INF = float("-inf")


# ---------------------------------------------------------------------------
# 1. The definition, materialised (eq 33.2, §33.3 explicit implementation)
# ---------------------------------------------------------------------------

def legal_keys(t_q: int, t_k: int, causal: bool, q_offset: int,
               bias_rows: Optional[np.ndarray] = None,
               window: int = 0) -> np.ndarray:
    """Boolean [t_q, t_k]: key j is legal for query row i.

    Row i sits at logical position q_offset + i (KV-cache section of
    "Generation and Caching with the Same Model"); with causal masking it sees
    key j iff j <= q_offset + i (§33.3, interface and correctness conditions:
    alignment is by logical position, not by the top-left corner).  A bias of
    -inf masks a key (eq 33.2: M_j is an additive bias or mask).  A sliding
    window of W >= 1 keys (§33.7, the sliding-window paragraph with eq 33.16:
    only keys inside the prescribed range stay visible) keeps the W positions
    ending at the row's own, j >= q_offset + i - W + 1; window 0 means no
    window.
    """
    i = np.arange(t_q, dtype=np.int64)[:, None]
    j = np.arange(t_k, dtype=np.int64)[None, :]
    if causal:
        legal = j <= (q_offset + i)
    else:
        legal = np.ones((t_q, t_k), dtype=bool)
    if window > 0:
        legal = legal & (j >= q_offset + i - window + 1)
    if bias_rows is not None:
        legal = legal & (bias_rows != NEG_INF)
    return legal


def softmax_rows(scores: np.ndarray, legal: np.ndarray,
                 values: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Exact softmax-weighted average of ``values`` for each score row.

    scores [R, T_k] fp64, legal [R, T_k] bool, values [T_k, d_v] fp64.
    Returns (o [R, d_v], lse [R], n_legal [R] int64).  For a row with legal
    keys: m = max legal score, w_j = e^{z_j - m} on legal keys and 0 elsewhere,
    ℓ = sum w, o = sum w_j v_j / ℓ, lse = m + ln ℓ (eq 33.2).  A row with no
    legal key gets o = +0.0, lse = -inf (§33.2 valid-flag rule).
    """
    r = scores.shape[0]
    d_v = values.shape[1]
    n_legal = legal.sum(axis=1).astype(np.int64)
    o = np.zeros((r, d_v), dtype=np.float64)
    lse = np.full(r, NEG_INF, dtype=np.float64)
    live = n_legal > 0
    if not live.any():
        return o, lse, n_legal
    s = np.where(legal[live], scores[live], NEG_INF)
    m = s.max(axis=1)
    w = np.exp(s - m[:, None])            # e^{-inf} = 0 on illegal keys
    ell = w.sum(axis=1)
    o[live] = (w @ values) / ell[:, None]
    lse[live] = m + np.log(ell)
    return o, lse, n_legal


def _check_shapes(q, k, v, bias):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, T, D]")
    b, hq, _, d_h = q.shape
    bk, hkv, t_k, d_hk = k.shape
    if bk != b or v.shape[0] != b or v.shape[1] != hkv or v.shape[2] != t_k:
        raise ValueError("k and v must be [B, H_kv, T_k, *] with q's batch")
    if d_hk != d_h:
        raise ValueError("q and k must share d_h")
    if hkv == 0 or hq % hkv != 0:
        raise ValueError("H_q must be a multiple of H_kv")
    if bias is not None and bias.ndim != 4:
        raise ValueError("bias must broadcast as [B, H_q, T_q, T_k]")


def _bias_rows(bias: Optional[np.ndarray], b: int, hq: int, t_q: int,
               t_k: int, rows=slice(None)) -> Optional[np.ndarray]:
    if bias is None:
        return None
    bb = bias[b if bias.shape[0] > 1 else 0, hq if bias.shape[1] > 1 else 0]
    return np.broadcast_to(bb, (t_q, t_k))[rows]


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, *, scale: float,
              causal: bool, q_offset: int = 0,
              bias: Optional[np.ndarray] = None,
              key_range: Optional[Tuple[int, int]] = None,
              window: int = 0):
    """Materialised exact attention over every (batch, query head).

    q [B, H_q, T_q, d_h], k [B, H_kv, T_k, d_h], v [B, H_kv, T_k, d_v] (any
    real dtype; converted exactly to fp64), bias broadcastable to
    [B, H_q, T_q, T_k] or None.  z_ij = scale * <q_i, k_j> + M_ij (eq 33.2;
    the bias is added after scaling and is never scaled).  ``key_range``
    restricts the legal set to keys [lo, hi) (used for split partials);
    ``window`` is the sliding window of ``legal_keys``.

    Returns (o [B, H_q, T_q, d_v], lse [B, H_q, T_q], n_legal [B, H_q, T_q]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if bias is not None:
        bias = np.asarray(bias, dtype=np.float64)
    _check_shapes(q, k, v, bias)
    bsz, h_q, t_q, _ = q.shape
    h_kv, t_k, d_v = k.shape[1], k.shape[2], v.shape[3]
    group = h_q // h_kv
    o = np.zeros((bsz, h_q, t_q, d_v))
    lse = np.full((bsz, h_q, t_q), NEG_INF)
    n = np.zeros((bsz, h_q, t_q), dtype=np.int64)
    for b in range(bsz):
        for hq in range(h_q):
            kvh = hq // group
            m_rows = _bias_rows(bias, b, hq, t_q, t_k)
            s = scale * (q[b, hq] @ k[b, kvh].T)
            if m_rows is not None:
                s = s + np.where(m_rows == NEG_INF, 0.0, m_rows)
            legal = legal_keys(t_q, t_k, causal, q_offset, m_rows, window)
            if key_range is not None:
                lo, hi = key_range
                j = np.arange(t_k)[None, :]
                legal = legal & (j >= lo) & (j < hi)
            o[b, hq], lse[b, hq], n[b, hq] = softmax_rows(s, legal, v[b, kvh])
    return o, lse, n


def attention_rows(q, k, v, rows: Sequence[Tuple[int, int, int]], *,
                   scale: float, causal: bool, q_offset: int = 0,
                   bias=None, window: int = 0):
    """The same definition evaluated for selected rows (b, hq, i) only.

    Each row is computed on its own from its query vector and every key of its
    KV head, so full-size workloads can be checked on a sample of rows.  Inputs
    may be torch CPU tensors or numpy arrays; only the needed slices are
    converted to fp64.  Returns (o [R, d_v], lse [R], n_legal [R]).
    """
    def f64(x):
        if hasattr(x, "detach"):
            import torch  # only for the exact dtype conversion of a slice
            return x.detach().to(torch.float64).numpy()
        return np.asarray(x, dtype=np.float64)

    h_q = q.shape[1]
    h_kv = k.shape[1]
    t_k = k.shape[2]
    group = h_q // h_kv
    outs_o, outs_l, outs_n = [], [], []
    cache = {}
    for (b, hq, i) in rows:
        kvh = hq // group
        key = (b, kvh)
        if key not in cache:
            cache.clear()
            cache[key] = (f64(k[b, kvh]), f64(v[b, kvh]))
        kk, vv = cache[key]
        qi = f64(q[b, hq, i])
        s = scale * (kk @ qi)
        m_row = None
        if bias is not None:
            bb = bias[b if bias.shape[0] > 1 else 0, hq if bias.shape[1] > 1 else 0]
            bi = bb[i if bb.shape[0] > 1 else 0]
            m_row = np.broadcast_to(f64(bi), (t_k,))
            s = s + np.where(m_row == NEG_INF, 0.0, m_row)
        pos = q_offset + i
        j = np.arange(t_k)
        legal = (j <= pos) if causal else np.ones(t_k, dtype=bool)
        if window > 0:
            legal = legal & (j >= pos - window + 1)
        if m_row is not None:
            legal = legal & (m_row != NEG_INF)
        o1, l1, n1 = softmax_rows(s[None, :], legal[None, :], vv)
        outs_o.append(o1[0]); outs_l.append(l1[0]); outs_n.append(n1[0])
    return np.array(outs_o), np.array(outs_l), np.array(outs_n, dtype=np.int64)


def split_partials(q, k, v, *, scale: float, causal: bool, q_offset: int,
                   split_size: int, bias=None, window: int = 0):
    """Per-split partial results for split-KV decode.

    Split s covers keys [s*S, min((s+1)*S, T_k)); its partial is the
    definition applied to that key range alone, stored as (o_s, lse_s), with
    (0, -inf) for a split that holds no legal key.  Returns
    (o_parts [B, H_q, T_q, n_splits, d_v], lse_parts [B, H_q, T_q, n_splits]).
    """
    t_k = np.asarray(k).shape[2]
    n_splits = max(1, -(-t_k // split_size))
    o_parts, l_parts = [], []
    for s in range(n_splits):
        o_s, l_s, _ = attention(q, k, v, scale=scale, causal=causal,
                                q_offset=q_offset, bias=bias,
                                key_range=(s * split_size,
                                           min((s + 1) * split_size, t_k)),
                                window=window)
        o_parts.append(o_s); l_parts.append(l_s)
    return np.stack(o_parts, axis=3), np.stack(l_parts, axis=3)


def attention_varlen(q, k, v, cu_q, cu_k, *, scale: float, causal: bool,
                     q_offset: int = 0, bias=None, window: int = 0):
    """Unpadded variable-length batch (§33.4, shape bucketing: padding every
    sequence to a bucket b(T) costs about E[b(T)^2 - T^2] extra score work for
    dense attention; this is the result without that padding).

    q [1, H_q, sum L_q, d_h], k and v [1, H_kv, sum L_k, *]: sequences packed
    along the token axis; sequence s has query rows [cu_q[s], cu_q[s+1]) and
    keys [cu_k[s], cu_k[s+1]).  Each sequence is exact attention on its own
    rows and keys (``attention``), its rows being the last L_q positions of its
    keys: row i of sequence s sits at q_offset + (L_k - L_q) + i.  The bias
    (optional, [1, H_q or 1, sum L_q, sum L_k]) is indexed by packed row and
    packed key, so sequence s reads its diagonal block.  Returns
    (o [1, H_q, sum L_q, d_v], lse [1, H_q, sum L_q], n_legal likewise);
    rows outside every sequence stay (0, -inf, 0).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    cu_q = [int(x) for x in cu_q]
    cu_k = [int(x) for x in cu_k]
    h_q, t_q, d_v = q.shape[1], q.shape[2], v.shape[3]
    o = np.zeros((1, h_q, t_q, d_v))
    lse = np.full((1, h_q, t_q), NEG_INF)
    n = np.zeros((1, h_q, t_q), dtype=np.int64)
    for s in range(len(cu_q) - 1):
        q0, q1, k0, k1 = cu_q[s], cu_q[s + 1], cu_k[s], cu_k[s + 1]
        if q1 == q0:
            continue
        b_s = None
        if bias is not None:   # size-1 (broadcast) row or key dims are kept whole
            bb = np.asarray(bias, dtype=np.float64)
            b_s = bb[:, :, (slice(q0, q1) if bb.shape[2] != 1 else slice(None)),
                     (slice(k0, k1) if bb.shape[3] != 1 else slice(None))]
        o_s, l_s, n_s = attention(q[:, :, q0:q1], k[:, :, k0:k1], v[:, :, k0:k1], scale=scale,
                                  causal=causal, q_offset=q_offset + (k1 - k0) - (q1 - q0),
                                  bias=b_s, window=window)
        o[:, :, q0:q1], lse[:, :, q0:q1], n[:, :, q0:q1] = o_s, l_s, n_s
    return o, lse, n


def attention_kvlens(q, k, v, kv_lens, *, scale: float, causal: bool,
                     q_offset: int = 0, bias=None, window: int = 0):
    """Per-batch KV lengths (the unpadded form of a batch of caches of
    different lengths, §33.4 shape bucketing): batch b uses keys
    [0, kv_lens[b]) of k and v [B, H_kv, T_k, *], and its row i sits at
    q_offset + kv_lens[b] - T_q + i (the rows are the last T_q positions of
    its keys).  Each batch is ``attention`` on its own keys; the bias, if any,
    is [B, *, T_q, T_k] and only its first kv_lens[b] keys are read.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    b_n, h_q, t_q, d_v = q.shape[0], q.shape[1], q.shape[2], v.shape[3]
    o = np.zeros((b_n, h_q, t_q, d_v))
    lse = np.full((b_n, h_q, t_q), NEG_INF)
    n = np.zeros((b_n, h_q, t_q), dtype=np.int64)
    for b in range(b_n):
        n_k = int(kv_lens[b])
        b_s = None
        if bias is not None:   # a size-1 (broadcast) batch or key dim is kept whole
            bb = np.asarray(bias, dtype=np.float64)
            b_s = bb[(slice(b, b + 1) if bb.shape[0] != 1 else slice(None)), :, :,
                     (slice(0, n_k) if bb.shape[3] != 1 else slice(None))]
        o[b:b + 1], lse[b:b + 1], n[b:b + 1] = attention(
            q[b:b + 1], k[b:b + 1, :, :n_k], v[b:b + 1, :, :n_k], scale=scale, causal=causal,
            q_offset=q_offset + n_k - t_q, bias=b_s, window=window)
    return o, lse, n


def attention_backward(q, k, v, d_o, *, scale: float, causal: bool,
                       q_offset: int = 0, bias=None, window: int = 0):
    """Gradients of O = softmax(S) V with respect to Q, K and V for an upstream
    gradient G_O (§33.3, "block size, parallelism and backward recomputation":
    eqs 33.6-33.8).

    Per (batch, query head) the probabilities are rebuilt from the definition
    (eq 33.2, the legal set of ``legal_keys``): P_ij = e^{z_ij - m_i} / ℓ_i on
    legal keys, 0 on illegal keys and on rows with no legal key.  Then

        G_V = P^T G_O,  G_P = G_O V^T                       (eq 33.6)
        (G_S)_ij = P_ij [(G_P)_ij - sum_k P_ik (G_P)_ik]    (eq 33.7)
        G_Q = scale * G_S K,  G_K = scale * G_S^T Q         (eq 33.8)

    with the score scale in place of 1/sqrt(d_h) (z = scale <q, k> + M).  The
    bias M is a constant input (mask or additive bias) and gets no gradient.
    G_K and G_V of a KV head sum the contributions of every query head of its
    group.  Returns (dq [B, H_q, T_q, d_h], dk [B, H_kv, T_k, d_h],
    dv [B, H_kv, T_k, d_v]).
    """
    def f64(x):
        if hasattr(x, "detach"):
            import torch  # exact dtype conversion of torch CPU inputs only
            return x.detach().to(torch.float64).numpy()
        return np.asarray(x, dtype=np.float64)

    q, k, v, d_o = f64(q), f64(k), f64(v), f64(d_o)
    if bias is not None:
        bias = f64(bias)
    _check_shapes(q, k, v, bias)
    bsz, h_q, t_q, _ = q.shape
    h_kv, t_k = k.shape[1], k.shape[2]
    group = h_q // h_kv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(bsz):
        for hq in range(h_q):
            kvh = hq // group
            m_rows = _bias_rows(bias, b, hq, t_q, t_k)
            s = scale * (q[b, hq] @ k[b, kvh].T)
            if m_rows is not None:
                s = s + np.where(m_rows == NEG_INF, 0.0, m_rows)
            legal = legal_keys(t_q, t_k, causal, q_offset, m_rows, window)
            p = np.zeros((t_q, t_k))
            live = legal.any(axis=1)
            if live.any():
                z = np.where(legal[live], s[live], NEG_INF)
                w = np.exp(z - z.max(axis=1, keepdims=True))
                p[live] = w / w.sum(axis=1, keepdims=True)
            g_o = d_o[b, hq]
            dv[b, kvh] += p.T @ g_o                                   # eq 33.6
            g_p = g_o @ v[b, kvh].T                                   # eq 33.6
            g_s = p * (g_p - (p * g_p).sum(axis=1, keepdims=True))    # eq 33.7
            dq[b, hq] = scale * (g_s @ k[b, kvh])                     # eq 33.8
            dk[b, kvh] += scale * (g_s.T @ q[b, hq])                  # eq 33.8
    return dq, dk, dv


def attention_varlen_backward(q, k, v, d_o, cu_q, cu_k, *, scale: float, causal: bool,
                              q_offset: int = 0, bias=None, window: int = 0):
    """Gradients of ``attention_varlen`` (packed sequences, §33.4 shape
    bucketing; backward of §33.3, eqs 33.6-33.8): each sequence's gradients
    are ``attention_backward`` of its own rows and keys, with its rows at
    q_offset + (L_k - L_q) + i and the bias (packed row x packed key) cut to
    its diagonal block.  Rows and keys outside every sequence get zero.
    Returns (dq, dk, dv) in the packed layout of q, k, v."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d_o = np.asarray(d_o, dtype=np.float64)
    cu_q = [int(x) for x in cu_q]
    cu_k = [int(x) for x in cu_k]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for s in range(len(cu_q) - 1):
        q0, q1, k0, k1 = cu_q[s], cu_q[s + 1], cu_k[s], cu_k[s + 1]
        if q1 == q0 and k1 == k0:
            continue
        b_s = None
        if bias is not None:   # size-1 (broadcast) row or key dims are kept whole
            bb = np.asarray(bias, dtype=np.float64)
            b_s = bb[:, :, (slice(q0, q1) if bb.shape[2] != 1 else slice(None)),
                     (slice(k0, k1) if bb.shape[3] != 1 else slice(None))]
        g = attention_backward(q[:, :, q0:q1], k[:, :, k0:k1], v[:, :, k0:k1], d_o[:, :, q0:q1],
                               scale=scale, causal=causal, q_offset=q_offset + (k1 - k0) - (q1 - q0),
                               bias=b_s, window=window)
        dq[:, :, q0:q1], dk[:, :, k0:k1], dv[:, :, k0:k1] = g
    return dq, dk, dv


def attention_kvlens_backward(q, k, v, d_o, kv_lens, *, scale: float, causal: bool,
                              q_offset: int = 0, bias=None, window: int = 0):
    """Gradients of ``attention_kvlens`` (per-batch KV lengths, §33.4 shape
    bucketing; backward of §33.3, eqs 33.6-33.8): batch b's gradients are
    ``attention_backward`` of its rows over keys [0, kv_lens[b]), with its
    rows at q_offset + kv_lens[b] - T_q + i; keys at or past kv_lens[b] get
    zero.  Returns (dq, dk, dv) in the layout of q, k, v."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d_o = np.asarray(d_o, dtype=np.float64)
    t_q = q.shape[2]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(q.shape[0]):
        n_k = int(kv_lens[b])
        b_s = None
        if bias is not None:   # a size-1 (broadcast) batch or key dim is kept whole
            bb = np.asarray(bias, dtype=np.float64)
            b_s = bb[(slice(b, b + 1) if bb.shape[0] != 1 else slice(None)), :, :,
                     (slice(0, n_k) if bb.shape[3] != 1 else slice(None))]
        g = attention_backward(q[b:b + 1], k[b:b + 1, :, :n_k], v[b:b + 1, :, :n_k], d_o[b:b + 1],
                               scale=scale, causal=causal, q_offset=q_offset + n_k - t_q, bias=b_s,
                               window=window)
        dq[b:b + 1], dk[b:b + 1, :, :n_k], dv[b:b + 1, :, :n_k] = g
    return dq, dk, dv


def attention_backward_sampled(q, k, v, d_o, *, rows=(), keys=(), scale: float,
                               causal: bool, q_offset: int = 0, window: int = 0):
    """The gradients of ``attention_backward`` (eqs 33.6-33.8) at selected
    places only, for full-size problems: G_Q of query rows (b, hq, i) and
    G_K, G_V of keys (b, kv head, j).  A row needs its own probability row;
    a key needs the probability column of every query head of its group, so
    those heads' P and G_P are materialised one head at a time.  No bias.
    Inputs may be torch CPU tensors or numpy arrays.  Returns
    (dq [R, d_h], dk [K, d_h], dv [K, d_v])."""
    def f64(x):
        if hasattr(x, "detach"):
            import torch  # exact dtype conversion of torch CPU inputs only
            return x.detach().to(torch.float64).numpy()
        return np.asarray(x, dtype=np.float64)

    h_q, h_kv, t_q, t_k = q.shape[1], k.shape[1], q.shape[2], k.shape[2]
    group = h_q // h_kv

    def head(b, hq, row_sel):
        kvh = hq // group
        qq, kk, vv, gg = f64(q[b, hq][row_sel]), f64(k[b, kvh]), f64(v[b, kvh]), f64(d_o[b, hq][row_sel])
        ii = np.arange(t_q)[row_sel]
        s_ = scale * (qq @ kk.T)
        j = np.arange(t_k)[None, :]
        pos = (q_offset + ii)[:, None]
        legal = (j <= pos) if causal else np.ones(s_.shape, dtype=bool)
        if window > 0:
            legal = legal & (j >= pos - window + 1)
        p = np.zeros_like(s_)
        live = legal.any(axis=1)
        if live.any():
            z = np.where(legal[live], s_[live], NEG_INF)
            w = np.exp(z - z.max(axis=1, keepdims=True))
            p[live] = w / w.sum(axis=1, keepdims=True)
        g_p = gg @ vv.T                                               # eq 33.6
        g_s = p * (g_p - (p * g_p).sum(axis=1, keepdims=True))        # eq 33.7
        return qq, kk, gg, p, g_s

    dq = []
    for (b, hq, i) in rows:
        _, kk, _, _, g_s = head(b, hq, slice(i, i + 1))
        dq.append(scale * (g_s @ kk)[0])                              # eq 33.8
    dk = {key: 0.0 for key in keys}
    dv = {key: 0.0 for key in keys}
    by_head = {}
    for (b, kvh, j) in keys:
        by_head.setdefault((b, kvh), []).append(j)
    for (b, kvh), js in by_head.items():
        for hq in range(kvh * group, (kvh + 1) * group):
            qq, _, gg, p, g_s = head(b, hq, slice(None))
            for j in js:
                dv[(b, kvh, j)] = dv[(b, kvh, j)] + p[:, j] @ gg        # eq 33.6
                dk[(b, kvh, j)] = dk[(b, kvh, j)] + scale * (g_s[:, j] @ qq)   # eq 33.8
    d_h, d_v = q.shape[3], v.shape[3]
    return (np.array(dq).reshape(len(rows), d_h),
            np.array([dk[key] for key in keys]).reshape(len(keys), d_h),
            np.array([dv[key] for key in keys]).reshape(len(keys), d_v))


# ---------------------------------------------------------------------------
# 2. Statistics, merge and Algorithm 33.1 (eqs 33.3-33.5), arithmetic-generic
# ---------------------------------------------------------------------------

class Arith:
    """The three scalar operations the statistics need.

    ``exp_diff(a, b)`` = e^{a - b} for scores a <= b or any pair, ``log(x)`` the
    natural log, ``gt(a, b)`` score comparison.  ``to_log`` maps an LSE-type
    value back to the score domain of this arithmetic.
    """

    def __init__(self, exp_diff: Callable, log_plus: Callable, gt: Callable):
        self.exp_diff = exp_diff
        self.log_plus = log_plus      # (m, ell) -> m + ln(ell)
        self.gt = gt


FP64 = Arith(exp_diff=lambda a, b: math.exp(a - b),
             log_plus=lambda m, ell: m + math.log(ell),
             gt=lambda a, b: a > b)


class LogOf:
    """The score ln(a) of a positive rational a, kept exact as a Fraction.

    e^{ln a - ln b} = a / b is then an exact rational, so the statistics and
    the merge can be checked with no rounding at all.
    """

    __slots__ = ("a",)

    def __init__(self, a):
        self.a = Fraction(a)
        if self.a <= 0:
            raise ValueError("LogOf needs a positive rational")

    def __repr__(self):
        return f"ln({self.a})"

    def __eq__(self, other):
        return isinstance(other, LogOf) and self.a == other.a

    def __hash__(self):
        return hash(self.a)


EXACT = Arith(exp_diff=lambda x, y: x.a / y.a,
              log_plus=lambda m, ell: LogOf(m.a * ell),
              gt=lambda x, y: x.a > y.a)


def block_stats(z: Sequence, values: Sequence[Sequence], legal: Sequence[bool],
                arith: Arith = FP64):
    """(m, ℓ, u) of the legal keys of one block (eq 33.3), or None if empty.

    m = max legal z_j, ℓ = sum e^{z_j - m}, u = sum e^{z_j - m} v_j.  An empty
    block has no statistics at all (§33.2 valid-flag rule); no arithmetic is
    done on the maximum of an empty set.
    """
    idx = [j for j, ok in enumerate(legal) if ok]
    if not idx:
        return None
    m = z[idx[0]]
    for j in idx[1:]:
        if arith.gt(z[j], m):
            m = z[j]
    d_v = len(values[idx[0]])
    ell = 0
    u = [0] * d_v
    for j in idx:
        w = arith.exp_diff(z[j], m)
        ell = ell + w
        u = [u[d] + w * values[j][d] for d in range(d_v)]
    return (m, ell, u)


def merge_stats(a, b, arith: Arith = FP64):
    """Merge two statistics of disjoint key sets (eqs 33.4-33.5).

    m = max(m_A, m_B); ℓ = e^{m_A - m} ℓ_A + e^{m_B - m} ℓ_B;
    u = e^{m_A - m} u_A + e^{m_B - m} u_B.  An empty side (None) contributes
    nothing: the other side is returned as is (§33.2 valid flags, Exercise 33.3).
    """
    if a is None:
        return b
    if b is None:
        return a
    m_a, l_a, u_a = a
    m_b, l_b, u_b = b
    m = m_a if not arith.gt(m_b, m_a) else m_b
    ca = arith.exp_diff(m_a, m)
    cb = arith.exp_diff(m_b, m)
    ell = ca * l_a + cb * l_b
    u = [ca * x + cb * y for x, y in zip(u_a, u_b)]
    return (m, ell, u)


def finalize(state, d_v: int, arith: Arith = FP64):
    """Output of a row: (u / ℓ, m + ln ℓ) or, with no legal key, (0, -inf)."""
    if state is None:
        return [0.0] * d_v, NEG_INF
    m, ell, u = state
    return [x / ell for x in u], arith.log_plus(m, ell)


def blocked_single_query(z: Sequence, values: Sequence[Sequence],
                         legal: Sequence[bool], blocks: Sequence[Sequence[int]],
                         arith: Arith = FP64):
    """One query's result computed from per-block statistics (eqs 33.3-33.5).

    ``blocks`` lists key indices and must partition the keys.  Each block is
    summarised by its statistics (m, ℓ, u) over its legal keys (eq 33.3), or
    by "empty" when it has none; the summaries are folded left to right with
    the merge rule (eqs 33.4-33.5), where an empty summary is the identity
    (§33.2 valid flags); the folded state gives u/ℓ and m + ln ℓ, or the
    defined output of a row with no legal key.  The merge is associative and
    commutative in exact arithmetic, so any partition and order must give the
    same result as the materialised definition.
    """
    d_v = len(values[0]) if len(values) else 0
    summaries = (block_stats([z[j] for j in blk], [values[j] for j in blk],
                             [legal[j] for j in blk], arith) for blk in blocks)
    state = functools.reduce(lambda acc, st: merge_stats(acc, st, arith), summaries, None)
    return finalize(state, d_v, arith)


def merge_partials(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Merge stored partials (o_s, lse_s) along the last state axis.

    o_parts [..., S, d_v], lse_parts [..., S].  Each valid partial is the
    triple (lse_s, 1, o_s) and the triples are folded with ``merge_stats``
    (eqs 33.4-33.5); partials with lse_s = -inf are skipped.  Returns
    (o [..., d_v], lse [...]).
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    lead = lse_parts.shape[:-1]
    n_states = lse_parts.shape[-1]
    d_v = o_parts.shape[-1]
    o_flat = o_parts.reshape(-1, n_states, d_v)
    l_flat = lse_parts.reshape(-1, n_states)
    o_out = np.zeros((o_flat.shape[0], d_v))
    l_out = np.full(o_flat.shape[0], NEG_INF)
    for r in range(o_flat.shape[0]):
        state = None
        for s in range(n_states):
            if l_flat[r, s] == NEG_INF:
                continue
            st = (float(l_flat[r, s]), 1.0, list(o_flat[r, s]))
            state = st if state is None else merge_stats(state, st, FP64)
        o_r, l_r = finalize(state, d_v, FP64)
        o_out[r] = o_r
        l_out[r] = l_r
    return o_out.reshape(lead + (d_v,)), l_out.reshape(lead)


def set_partitions(items: List[int]):
    """Every set partition of ``items`` exactly once, as lists of blocks.

    A partition of [x] + rest is a partition of rest with x either added to
    one of its blocks or put in a block of its own; distinct choices give
    distinct partitions, so there are Bell(n) of them.
    """
    if not items:
        yield []
        return
    first, rest = items[0], items[1:]
    for part in set_partitions(rest):
        for i in range(len(part)):
            yield part[:i] + [[first] + part[i]] + part[i + 1:]
        yield [[first]] + part
