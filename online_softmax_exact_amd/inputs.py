"""Seeded synthetic inputs for the attention workloads.

This module draws random tensors and fixes shapes; it holds none of the
attention arithmetic, so both the HIP path's tests and the CPU oracle can take
their inputs from it.  Every draw uses its own local ``torch.Generator`` on the
CPU (as the KV-cache page of "Generation and Caching with the Same Model"
recommends).  Tensor number t of a workload (Q = 0, K = 1, V = 2, bias = 3)
is drawn in chunks along its two outer dimensions; chunk c comes from a
generator seeded with ``derive_seed(seed, t, c)``, so the values do not depend
on how many threads draw them.  bf16 tensors are fp32 N(0, 1) draws rounded to
nearest-even by ``Tensor.to(torch.bfloat16)``.

Workloads (the shapes of the pages' sizing example and of the cached-decode,
speculative-verify and padded-batch uses the pages describe):

1. fp32 causal, batch 1, 1 head, T_q = T_k = 128, d_h = d_v = 64.
2. bf16 causal prefill, batch 1, 32 heads, T = 8192, d = 128 (the 8192 x 8192,
   32-head score-matrix sizing example of §33.3 of "Chapter 33 推理计算优化").
3. bf16 cached decode with grouped heads: batch 16, 32 query heads on 8 KV
   heads, one query at position T_k - 1, T_k = 32768, d = 128, split into
   blocks of 512 keys.
4. bf16 multi-query verify: batch 32, 32 heads, 5 queries at positions
   T_k - 5 .. T_k - 1, T_k = 4096, d = 128.
5. bf16 padded variable-length batch with an additive fp32 bias: batch 8,
   16 heads, T = 4096, d_h = 64, d_v = 128; per-sequence length L_b uniform in
   [1, 4096]; bias N(0, 1) with -inf on padded keys j >= L_b and on every key
   of two seeded rows per sequence.
"""

from __future__ import annotations

import concurrent.futures as cf
import math
import os
from dataclasses import dataclass, field
from typing import Optional

import torch

NEG_INF = float("-inf")


@dataclass
class Workload:
    """One synthetic attention problem on the CPU (tensors in [B, H, T, D])."""
    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    scale: float
    causal: bool
    q_offset: int
    bias: Optional[torch.Tensor] = None
    split_size: Optional[int] = None
    extras: dict = field(default_factory=dict)

    @property
    def dims(self):
        b, hq, tq, dh = self.q.shape
        return dict(batch=b, heads_q=hq, heads_kv=self.k.shape[1], t_q=tq,
                    t_k=self.k.shape[2], d_h=dh, d_v=self.v.shape[3])


SPECS = {
    1: dict(name="fp32 causal 1x1x128 d64", dtype=torch.float32, batch=1,
            heads_q=1, heads_kv=1, t_q=128, t_k=128, d_h=64, d_v=64,
            q_offset=0, causal=True),
    2: dict(name="bf16 causal prefill 1x32x8192 d128", dtype=torch.bfloat16,
            batch=1, heads_q=32, heads_kv=32, t_q=8192, t_k=8192, d_h=128,
            d_v=128, q_offset=0, causal=True),
    3: dict(name="bf16 GQA decode 16x32/8 Tk32768 d128 split512",
            dtype=torch.bfloat16, batch=16, heads_q=32, heads_kv=8, t_q=1,
            t_k=32768, d_h=128, d_v=128, q_offset=32767, causal=True,
            split_size=512),
    4: dict(name="bf16 verify 32x32 Tq5 Tk4096 d128", dtype=torch.bfloat16,
            batch=32, heads_q=32, heads_kv=32, t_q=5, t_k=4096, d_h=128,
            d_v=128, q_offset=4091, causal=True),
    5: dict(name="bf16 padded varlen + fp32 bias 8x16x4096 d64/128",
            dtype=torch.bfloat16, batch=8, heads_q=16, heads_kv=16, t_q=4096,
            t_k=4096, d_h=64, d_v=128, q_offset=0, causal=True, bias=True),
}


def default_scale(d_h: int) -> float:
    """1/sqrt(d_h) rounded to fp32 (the value both sides receive)."""
    return float(torch.tensor(1.0 / math.sqrt(d_h), dtype=torch.float32))


def derive_seed(seed: int, tensor: int, chunk: int) -> int:
    return (seed * 1_000_003 + tensor * 7_919 + chunk * 104_729 + 1) % (1 << 62)


def _draw(shape, seed: int, tensor: int, dtype) -> torch.Tensor:
    """N(0, 1) tensor of ``shape``; chunk c = (i0, i1) of the two outer dims."""
    shape = tuple(int(x) for x in shape)
    out = torch.empty(shape, dtype=dtype)
    n0, n1 = shape[0], shape[1]
    inner = shape[2:]

    def one(c):
        i0, i1 = divmod(c, n1)
        g = torch.Generator("cpu").manual_seed(derive_seed(seed, tensor, c))
        x = torch.randn(inner, generator=g, dtype=torch.float32)
        out[i0, i1] = x if dtype == torch.float32 else x.to(dtype)

    chunks = n0 * n1
    workers = min(16, os.cpu_count() or 1, max(1, chunks))
    if workers == 1 or out.numel() < (1 << 20):
        for c in range(chunks):
            one(c)
    else:
        with cf.ThreadPoolExecutor(workers) as ex:
            list(ex.map(one, range(chunks)))
    return out


def make_config(k: int, seed: Optional[int] = None) -> Workload:
    """Workload k (1..5) at its full size, drawn from seed 1000 + k."""
    spec = SPECS[k]
    seed = 1000 + k if seed is None else seed
    b, hq, hkv = spec["batch"], spec["heads_q"], spec["heads_kv"]
    tq, tk, dh, dv = spec["t_q"], spec["t_k"], spec["d_h"], spec["d_v"]
    dt = spec["dtype"]
    q = _draw((b, hq, tq, dh), seed, 0, dt)
    kk = _draw((b, hkv, tk, dh), seed, 1, dt)
    v = _draw((b, hkv, tk, dv), seed, 2, dt)
    wl = Workload(name=spec["name"], q=q, k=kk, v=v, scale=default_scale(dh),
                  causal=spec["causal"], q_offset=spec["q_offset"],
                  split_size=spec.get("split_size"))
    if spec.get("bias"):
        bias, lengths, rows = padded_bias(b, tq, tk, seed)
        wl.bias = bias
        wl.extras = dict(lengths=lengths, masked_rows=rows)
    return wl


def padded_bias(batch: int, t_q: int, t_k: int, seed: int):
    """fp32 bias [batch, 1, t_q, t_k] for a padded variable-length batch.

    bias ~ N(0, 1) (tensor number 3 of the workload); then, from one generator
    seeded with ``derive_seed(seed, 4, 0)``: lengths L_b ~ U{1..t_k} and, per
    sequence, two distinct rows among the first max(L_b, 2).  Keys j >= L_b
    get -inf (padding masks keys only) and the two chosen rows get -inf on
    every key, so each sequence has exactly two rows with no legal key.
    """
    bias = _draw((batch, 1, t_q, t_k), seed, 3, torch.float32)
    gen = torch.Generator("cpu").manual_seed(derive_seed(seed, 4, 0))
    lengths = torch.randint(1, t_k + 1, (batch,), generator=gen)
    rows = []
    for b in range(batch):
        L = int(lengths[b])
        bias[b, 0, :, L:] = NEG_INF
        r = torch.randperm(max(L, 2), generator=gen)[:2]
        r = [int(x) for x in r]
        for x in r:
            bias[b, 0, x, :] = NEG_INF
        rows.append(r)
    return bias, [int(x) for x in lengths], rows


def make_random(batch: int, heads_q: int, heads_kv: int, t_q: int, t_k: int,
                d_h: int, d_v: int, *, dtype=torch.bfloat16, seed: int = 0,
                causal: bool = True, q_offset: int = 0, bias: str = "none",
                scale: Optional[float] = None, split_size: Optional[int] = None,
                masked_frac: float = 0.0) -> Workload:
    """A small seeded problem of any shape, for parity cases.

    ``bias``: "none"; "dense" (fp32 N(0,1) [B, H_q, T_q, T_k]); "shared"
    ([B, 1, T_q, T_k], broadcast over heads); "keys" ([B, 1, 1, T_k], one row
    broadcast over queries and heads); "rows" ([B, 1, T_q, 1], broadcast over
    keys).  ``masked_frac`` sets that fraction of bias entries to -inf.
    """
    q = _draw((batch, heads_q, t_q, d_h), seed, 0, dtype)
    k = _draw((batch, heads_kv, t_k, d_h), seed, 1, dtype)
    v = _draw((batch, heads_kv, t_k, d_v), seed, 2, dtype)
    gen = torch.Generator("cpu").manual_seed(derive_seed(seed, 3, 0))
    shapes = {"dense": (batch, heads_q, t_q, t_k), "shared": (batch, 1, t_q, t_k),
              "keys": (batch, 1, 1, t_k), "rows": (batch, 1, t_q, 1)}
    m = None
    if bias != "none":
        m = torch.randn(shapes[bias], generator=gen, dtype=torch.float32)
        if masked_frac > 0:
            drop = torch.rand(shapes[bias], generator=gen) < masked_frac
            m[drop] = NEG_INF
    return Workload(name=f"random seed {seed}", q=q, k=k, v=v,
                    scale=default_scale(d_h) if scale is None else scale,
                    causal=causal, q_offset=q_offset, bias=m,
                    split_size=split_size)


def varlen_lengths(n: int, max_len: int, seed: int):
    """n sequence lengths uniform in [1, max_len]: the first draw of
    ``padded_bias``'s generator, so the padded variable-length batch's seed gives
    its own lengths."""
    gen = torch.Generator("cpu").manual_seed(derive_seed(seed, 4, 0))
    return [int(x) for x in torch.randint(1, max_len + 1, (n,), generator=gen)]


def offsets(lengths):
    """Packed offsets [0, L_0, L_0 + L_1, ...] as an int32 tensor."""
    out = [0]
    for n in lengths:
        out.append(out[-1] + int(n))
    return torch.tensor(out, dtype=torch.int32)


def make_packed(lengths_q, lengths_k, heads_q: int, heads_kv: int, d_h: int, d_v: int, *,
                dtype=torch.bfloat16, seed: int = 0, bias: str = "none",
                masked_frac: float = 0.0):
    """Packed variable-length batch: q [1, H_q, sum L_q, d_h], k [1, H_kv,
    sum L_k, d_h], v [1, H_kv, sum L_k, d_v] (N(0, 1), drawn like
    ``make_random``) with int32 offsets cu_q, cu_k.  ``bias``: "none";
    "packed" (fp32 N(0, 1) [1, H_q, sum L_q, sum L_k], indexed by packed row
    and key); "keys" ([1, 1, 1, sum L_k], one value per packed key).
    ``masked_frac`` of the bias entries are -inf.  Returns
    (q, k, v, bias, cu_q, cu_k)."""
    cu_q, cu_k = offsets(lengths_q), offsets(lengths_k)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    q = _draw((1, heads_q, tq, d_h), seed, 0, dtype)
    k = _draw((1, heads_kv, tk, d_h), seed, 1, dtype)
    v = _draw((1, heads_kv, tk, d_v), seed, 2, dtype)
    m = None
    if bias != "none":
        gen = torch.Generator("cpu").manual_seed(derive_seed(seed, 3, 0))
        shape = {"packed": (1, heads_q, tq, tk), "keys": (1, 1, 1, tk)}[bias]
        m = torch.randn(shape, generator=gen, dtype=torch.float32)
        if masked_frac > 0:
            m[torch.rand(shape, generator=gen) < masked_frac] = NEG_INF
    return q, k, v, m, cu_q, cu_k
