"""Calls of every kernel family on small seeded problems, for the LDS-poison
comparison: ``run(path)`` computes them with whatever build of the library
this process loaded (``ATTN_MI355X_LIBRARY`` names the poisoning build in the
child process of tests/test_poison_gpu.py) and saves the outputs; ``compute()``
returns them as a dict of CPU tensors.  Covered: the prefill kernel (standard
and large workgroup shapes, a dense bias staged through LDS, n_legal counts,
a sliding window, packed sequences), the few-row kernel (few-row attn_fwd,
split-KV decode with split pairs, a bias, per-batch KV lengths, a grid of
more than 2048 splits), the merge kernel, both fp32 kernels, the generic
kernels (d = 96) and the backward kernels (fused dK/dV at d 128 and d 64/128,
separate dV/dK with a bias, packed sequences, the generic backward)."""

import sys

import torch

import online_softmax_exact_amd as attn
from online_softmax_exact_amd import inputs


def _dev(*ts):
    d = torch.device("cuda:0")
    return tuple(None if t is None else t.to(d) for t in ts)


def compute():
    out = {}

    def fwd(name, wl, **kw):
        q, k, v, m = _dev(wl.q, wl.k, wl.v, wl.bias)
        res = attn.attn_fwd(q, k, v, scale=wl.scale, causal=wl.causal, q_offset=wl.q_offset, bias=m, **kw)
        for i, t in enumerate(res):
            out[f"{name}.{i}"] = t
        return q, k, v, m, res

    def bwd(name, wl, **kw):
        q, k, v, m, (o, lse) = fwd(name + ".fwd", wl, **{x: y for x, y in kw.items() if x != "max_seqlen_q"})
        g = torch.Generator().manual_seed(7)
        d_o = torch.randn(o.shape, generator=g).to(o.dtype).to(o.device)
        grads = attn.attn_bwd(q, k, v, o, lse, d_o, scale=wl.scale, causal=wl.causal, q_offset=wl.q_offset,
                              bias=m, **kw)
        for i, t in enumerate(grads):
            out[f"{name}.d{i}"] = t

    r = inputs.make_random
    fwd("std", r(2, 4, 2, 300, 300, 128, 128, seed=1, causal=True))
    fwd("big", r(1, 32, 32, 2048, 2048, 128, 128, seed=2, causal=True))
    fwd("bias", r(2, 4, 4, 600, 600, 64, 128, seed=3, causal=True, bias="dense", masked_frac=0.1))
    fwd("bias_count", r(2, 4, 4, 300, 300, 64, 128, seed=4, causal=True, bias="shared", masked_frac=0.1),
        return_n_legal=True)
    fwd("window", r(1, 8, 8, 700, 700, 128, 128, seed=5, causal=True), window=200)
    fwd("fewrow", r(2, 8, 2, 4, 1000, 128, 128, seed=6, causal=True, q_offset=996))
    fwd("fp32_split", r(1, 2, 1, 150, 300, 64, 64, dtype=torch.float32, seed=8, causal=True, q_offset=150),
        return_n_legal=True)
    fwd("fp32_std", r(8, 8, 8, 150, 150, 64, 128, dtype=torch.float32, seed=9, causal=True))
    fwd("generic", r(1, 2, 2, 100, 130, 96, 96, seed=10, causal=True))

    # Packed sequences (prefill kernel VAR instances).
    lens = [90, 300, 1, 257]
    tq = sum(lens)
    wl = r(1, 4, 4, tq, tq, 64, 128, seed=11, causal=False)
    cu = torch.tensor([0] + list(torch.tensor(lens).cumsum(0)), dtype=torch.int32)
    q, k, v = _dev(wl.q, wl.k, wl.v)
    cud, = _dev(cu)
    o, lse = attn.attn_fwd(q, k, v, scale=wl.scale, causal=True, cu_seqlens_q=cud, cu_seqlens_k=cud,
                           max_seqlen_q=max(lens))
    out["packed.0"], out["packed.1"] = o, lse
    g = torch.Generator().manual_seed(12)
    d_o = torch.randn(o.shape, generator=g).to(o.dtype).to(o.device)
    for i, t in enumerate(attn.attn_bwd(q, k, v, o, lse, d_o, scale=wl.scale, causal=True, cu_seqlens_q=cud,
                                        cu_seqlens_k=cud, max_seqlen_q=max(lens))):
        out[f"packed_bwd.d{i}"] = t

    # Split-KV decode: split pairs (small grid), a bias, per-batch KV lengths,
    # more than 2048 splits.
    for name, wl, split, kw in (
            ("dec_pairs", r(2, 8, 2, 1, 3000, 128, 128, seed=13, causal=True, q_offset=2999), 256, {}),
            ("dec_bias", r(2, 8, 2, 2, 1500, 128, 128, seed=14, causal=True, q_offset=1498, bias="dense",
                           masked_frac=0.1), 128, {}),
            ("dec_big", r(4, 32, 8, 1, 8300, 128, 128, seed=15, causal=True, q_offset=8299), 128, {})):
        q, k, v, m = _dev(wl.q, wl.k, wl.v, wl.bias)
        o, lse, ws = attn.attn_decode_splitkv(q, k, v, split_size=split, scale=wl.scale, causal=True,
                                              q_offset=wl.q_offset, bias=m)
        out[f"{name}.0"], out[f"{name}.1"] = o, lse
    wl = r(4, 16, 4, 1, 5000, 128, 128, seed=16, causal=True)
    q, k, v = _dev(wl.q, wl.k, wl.v)
    sl, = _dev(torch.tensor([5000, 1, 0, 3333], dtype=torch.int32))
    o, lse, _ = attn.attn_decode_splitkv(q, k, v, split_size=512, scale=wl.scale, seqlens_k=sl)
    out["dec_kvlens.0"], out["dec_kvlens.1"] = o, lse

    # Merge kernel on partials with empty states.
    g = torch.Generator().manual_seed(17)
    os_ = torch.randn(64, 9, 128, generator=g)
    ls_ = torch.randn(64, 9, generator=g)
    ls_[::5, 2] = float("-inf")
    ls_[3, :] = float("-inf")
    o, lse = attn.attn_merge_states(*_dev(os_, ls_), out_dtype=torch.bfloat16)
    out["merge.0"], out["merge.1"] = o, lse

    # Backward: fused dK/dV (d 128: 8-wavefront form; d 64/128), separate
    # launches with a bias, the generic kernels.
    bwd("bwd128", r(1, 4, 2, 600, 600, 128, 128, seed=18, causal=True))
    bwd("bwd64", r(2, 4, 4, 300, 300, 64, 128, seed=19, causal=True))
    bwd("bwd_bias", r(1, 4, 4, 300, 300, 128, 128, seed=20, causal=True, bias="keys", masked_frac=0.2))
    bwd("bwd_generic", r(1, 2, 2, 100, 100, 96, 96, seed=21, causal=True))
    torch.cuda.synchronize()
    return {name: t.detach().cpu() for name, t in out.items()}


def run(path):
    torch.save(compute(), path)


if __name__ == "__main__":
    import os
    from online_softmax_exact_amd import _lib
    _lib.load_library()
    want = os.environ.get("ATTN_MI355X_LIBRARY")
    if want and want not in open("/proc/self/maps").read():
        raise SystemExit(f"{want} is not the library this process loaded")
    run(sys.argv[1])
