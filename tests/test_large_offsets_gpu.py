"""Largest offsets: tensors whose batch stride exceeds 2^31 elements (byte
offsets above 4 GiB for bf16, 8 GiB for fp32), so every kernel family's
address arithmetic must be 64-bit.  Each batch's rows live more than 2^31
elements apart inside one device allocation (a strided view), and the results
are compared element by element with the oracle on the same values in an
ordinary CPU layout."""

import numpy as np
import pytest
import torch

import oracle
import online_softmax_exact_amd as attn
from online_softmax_exact_amd import inputs
from gpu_util import assert_close, dev, ensure_built, f64

pytestmark = pytest.mark.gpu

GAP = (1 << 31) + 4096   # batch stride in elements


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def far_apart(t, gap=GAP):
    """A device view of the CPU tensor t [B, H, T, D] whose batch b starts
    b * gap elements into one allocation (heads, rows, columns packed)."""
    b, h, n, d = t.shape
    buf = torch.empty((b - 1) * gap + h * n * d, dtype=t.dtype, device=dev())
    view = buf.as_strided(t.shape, (gap, n * d, d, 1))
    view.copy_(t.to(dev()))
    return view


def far_empty(shape, dtype, gap=GAP):
    b, h, n, d = shape
    buf = torch.zeros((b - 1) * gap + h * n * d, dtype=dtype, device=dev())
    return buf.as_strided(shape, (gap, n * d, d, 1))


@pytest.mark.parametrize("dtype,d,t", [(torch.bfloat16, 128, 300), (torch.float32, 64, 200), (torch.float32, 40, 70)])
def test_fwd_batch_stride_over_2_31(dtype, d, t):
    """attn_fwd (bf16 and fp32 MFMA prefills, the generic kernel for fp32 with
    d = 40) with Q, K, V and O batches more than 2^31 elements apart."""
    wl = inputs.make_random(2, 2, 1, t, t, d, d, dtype=dtype, seed=31 + d, causal=True)
    q, k, v = far_apart(wl.q), far_apart(wl.k), far_apart(wl.v)
    o = far_empty((2, 2, t, d), dtype)
    _, lse, n = attn.attn_fwd(q, k, v, scale=wl.scale, causal=True, out=o, return_n_legal=True)
    torch.cuda.synchronize()
    o_ref, l_ref, n_ref = oracle.attention(f64(wl.q), f64(wl.k), f64(wl.v), scale=wl.scale, causal=True)
    assert_close(o, lse, o_ref, l_ref, dtype, what="far-apart batches")
    assert np.array_equal(n.cpu().numpy(), n_ref)


def test_decode_batch_stride_over_2_31():
    """Split-KV decode (few-row partials + merge) over a K/V cache whose
    batches are more than 2^31 elements apart, with per-batch KV lengths."""
    wl = inputs.make_random(2, 8, 2, 1, 3000, 128, 128, seed=77, causal=True, q_offset=2999)
    k, v = far_apart(wl.k), far_apart(wl.v)
    q = wl.q.to(dev())
    o, lse, _ = attn.attn_decode_splitkv(q, k, v, split_size=512, scale=wl.scale)
    lens = [3000, 1234]
    o2, lse2, _ = attn.attn_decode_splitkv(q, k, v, split_size=512, scale=wl.scale,
                                           seqlens_k=torch.tensor(lens, dtype=torch.int32, device=dev()))
    torch.cuda.synchronize()
    o_ref, l_ref, _ = oracle.attention(f64(wl.q), f64(wl.k), f64(wl.v), scale=wl.scale, causal=True,
                                       q_offset=2999)
    assert_close(o, lse, o_ref, l_ref, torch.bfloat16, what="far-apart cache")
    o_ref2, l_ref2, _ = oracle.attention_kvlens(f64(wl.q), f64(wl.k), f64(wl.v), lens, scale=wl.scale,
                                                causal=True)
    assert_close(o2, lse2, o_ref2, l_ref2, torch.bfloat16, what="far-apart cache, per-batch lengths")


def test_backward_batch_stride_over_2_31():
    """attn_bwd (MFMA dQ, dV, dK kernels) with every input and gradient batch
    more than 2^31 elements apart."""
    b, h, t, d = 2, 2, 200, 128
    wl = inputs.make_random(b, h, h, t, t, d, d, seed=99, causal=True)
    g = torch.Generator().manual_seed(5)
    d_o = torch.randn(b, h, t, d, generator=g).to(torch.bfloat16)
    q, k, v = far_apart(wl.q), far_apart(wl.k), far_apart(wl.v)
    o = far_empty((b, h, t, d), torch.bfloat16)
    _, lse = attn.attn_fwd(q, k, v, scale=wl.scale, causal=True, out=o)
    go = far_empty((b, h, t, d), torch.bfloat16)
    go.copy_(d_o.to(dev()))
    dq, dk, dv = attn.attn_bwd(q, k, v, o, lse, go, scale=wl.scale, causal=True)
    torch.cuda.synchronize()
    assert dq.stride(0) == GAP
    ref = oracle.attention_backward(f64(wl.q), f64(wl.k), f64(wl.v), f64(d_o), scale=wl.scale, causal=True)
    for name, got, want in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        g64 = f64(got)
        scale = max(np.abs(want).max(), 1e-30)
        err = np.abs(g64 - want) / scale
        assert err.max() <= 2e-2 and err.mean() <= 2e-3, f"{name}: {err.max():.3e} / {err.mean():.3e}"
