"""GPU parity of attn_bwd on packed sequences (§33.4 of "Chapter 33
推理计算优化", shape bucketing; gradients by recomputation, eqs 33.6-33.8 of
§33.3): the MFMA dQ / dK / dV kernels for bf16 with d in {64, 128} (with or
without a bias), the generic kernels otherwise.  Each case is compared element by element with
the oracle's attention_varlen_backward, relative to each gradient's largest
entry, with exact zeros where nothing contributes; rows and keys outside every
sequence keep what the caller's buffers held.  At the packed workload's size
(8 sequences of up to 4065 rows, 16 heads, d_h 64, d_v 128) every sequence's
gradients equal a dense call on that sequence alone bit for bit, and sampled
rows and keys match the oracle's sampled gradients."""

import zlib

import numpy as np
import pytest
import torch

import oracle
import online_softmax_exact_amd as attn
from online_softmax_exact_amd import inputs
from gpu_util import dev, ensure_built, f64

pytestmark = pytest.mark.gpu

BWD_TOL = {torch.float32: dict(max=1e-5, mean=1e-6), torch.bfloat16: dict(max=2e-2, mean=2e-3)}


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _seed(case):
    return zlib.crc32(repr(case).encode()) % 10_000


def _grad_out(shape, dtype, seed):
    return torch.randn(shape, generator=torch.Generator().manual_seed(seed)).to(dtype)


def _check(name, got, want, tol):
    g64 = got if isinstance(got, np.ndarray) else f64(got)
    assert not np.isnan(g64).any(), name
    scale = max(float(np.abs(want).max()), 1e-30)
    err = np.abs(g64 - want) / scale
    print(name, "relative errors", float(err.max()), float(err.mean()), flush=True)
    assert err.max() <= tol["max"] and err.mean() <= tol["mean"], f"{name}: {err.max():.2e} / {err.mean():.2e}"


BWD_CASES = [
    # (dtype, Hq, Hkv, L_q per sequence, L_k per sequence, dh, dv, causal, bias, masked_frac,
    #  window, q_offset)
    (torch.bfloat16, 2, 2, [1, 128, 129, 300, 7], [1, 128, 129, 300, 7], 128, 128, True, "none", 0.0, 0, 0),
    (torch.bfloat16, 8, 2, [50, 200, 0, 129], [300, 200, 10, 400], 64, 128, True, "none", 0.0, 0, 0),
    # rows before every key of their sequence (L_q > L_k), an empty key set
    (torch.bfloat16, 4, 4, [100, 40, 1], [30, 40, 0], 128, 64, True, "none", 0.0, 0, 0),
    (torch.bfloat16, 2, 1, [600, 300, 5], [600, 700, 5], 128, 128, True, "none", 0.0, 0, 0),
    (torch.bfloat16, 2, 2, [260, 33], [260, 90], 64, 64, True, "none", 0.0, 0, 0),
    (torch.bfloat16, 4, 2, [130, 257], [500, 257], 128, 128, False, "none", 0.0, 0, 0),
    (torch.bfloat16, 2, 2, [500, 140], [500, 400], 128, 128, True, "none", 0.0, 100, 0),
    (torch.bfloat16, 4, 1, [90, 200], [150, 200], 64, 64, True, "none", 0.0, 0, -7),
    (torch.bfloat16, 2, 2, [0, 0, 64], [0, 30, 64], 128, 128, True, "none", 0.0, 0, 0),
    # a bias (MFMA kernels); fp32 and odd head sizes (generic kernels)
    (torch.bfloat16, 4, 2, [200, 77, 129], [200, 300, 129], 64, 128, True, "packed", 0.1, 0, 0),
    (torch.bfloat16, 2, 2, [300, 64], [300, 100], 128, 128, True, "keys", 0.05, 0, 0),
    (torch.float32, 2, 1, [70, 1, 33], [70, 5, 100], 64, 64, True, "none", 0.0, 0, 0),
    (torch.float32, 4, 2, [20, 50], [90, 50], 40, 24, True, "packed", 0.1, 7, 0),
    (torch.bfloat16, 2, 2, [65, 130], [65, 140], 96, 80, False, "none", 0.0, 0, 3),
]


@pytest.mark.parametrize("case", BWD_CASES,
                         ids=[f"c{i}" for i in range(len(BWD_CASES))])
def test_packed_backward_parity(case):
    dtype, hq, hkv, lq, lk, dh, dv, causal, bias, mf, window, q_offset = case
    print("case", case, flush=True)
    q, k, v, m, cu_q, cu_k = inputs.make_packed(lq, lk, hq, hkv, dh, dv, dtype=dtype, seed=_seed(case),
                                                bias=bias, masked_frac=mf)
    g = _grad_out((1, hq, q.shape[2], dv), dtype, _seed(case) + 1)
    d = dev()
    scale = inputs.default_scale(dh)
    kw = dict(scale=scale, causal=causal, q_offset=q_offset, bias=None if m is None else m.to(d), window=window,
              cu_seqlens_q=cu_q.to(d), cu_seqlens_k=cu_k.to(d), max_seqlen_q=max(lq))
    qd, kd, vd = q.to(d), k.to(d), v.to(d)
    o, lse = attn.attn_fwd(qd, kd, vd, **kw)
    dq, dk, dv_ = attn.attn_bwd(qd, kd, vd, o, lse, g.to(d), **kw)
    torch.cuda.synchronize()
    ref = oracle.attention_varlen_backward(f64(q), f64(k), f64(v), f64(g), cu_q.tolist(), cu_k.tolist(),
                                           scale=scale, causal=causal, q_offset=q_offset,
                                           bias=None if m is None else f64(m), window=window)
    _, l_ref, _ = oracle.attention_varlen(f64(q), f64(k), f64(v), cu_q.tolist(), cu_k.tolist(), scale=scale,
                                          causal=causal, q_offset=q_offset, bias=None if m is None else f64(m),
                                          window=window)
    assert np.all(f64(dq)[np.isneginf(l_ref)] == 0), "dQ of a row without a legal key"
    dead = np.all(ref[2] == 0, axis=-1)
    assert np.all(f64(dk)[dead] == 0) and np.all(f64(dv_)[dead] == 0), "gradient of an unseen key"
    for name, got, want in zip(("dQ", "dK", "dV"), (dq, dk, dv_), ref):
        _check(name, got, want, BWD_TOL[dtype])


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_packed_backward_outside_untouched(dtype, d):
    """Rows and keys past the last sequence keep the caller's values (a
    sentinel), and an empty sequence list writes nothing."""
    lq, lk = [40, 150], [60, 150]
    q, k, v, _, cu_q, cu_k = inputs.make_packed(lq + [30], lk + [20], 4, 2, d, d, dtype=dtype, seed=3)
    cu_q, cu_k = cu_q[:3], cu_k[:3]         # the third sequence's rows and keys are outside every sequence
    dd = dev()
    qd, kd, vd = q.to(dd), k.to(dd), v.to(dd)
    kw = dict(scale=inputs.default_scale(d), causal=True, cu_seqlens_q=cu_q.to(dd), cu_seqlens_k=cu_k.to(dd),
              max_seqlen_q=150)
    o, lse = attn.attn_fwd(qd, kd, vd, **kw)
    g = _grad_out(o.shape, dtype, 9).to(dd)
    sentinel = -12345.0
    gq, gk, gv = (torch.full(t.shape, sentinel, dtype=dtype, device=dd) for t in (qd, kd, vd))
    attn.attn_bwd(qd, kd, vd, o, lse, g, d_q=gq, d_k=gk, d_v=gv, **kw)
    torch.cuda.synchronize()
    assert torch.all(gq[:, :, 190:] == sentinel) and torch.all(gk[:, :, 210:] == sentinel)
    assert torch.all(gv[:, :, 210:] == sentinel)
    assert not torch.any(gq[:, :, :190] == sentinel) and not torch.any(gk[:, :, :210] == sentinel)
    ref = oracle.attention_varlen_backward(f64(q), f64(k), f64(v), f64(g.cpu()), cu_q.tolist(), cu_k.tolist(),
                                           scale=inputs.default_scale(d), causal=True)
    for name, got, want in zip(("dQ", "dK", "dV"), (gq[:, :, :190], gk[:, :, :210], gv[:, :, :210]),
                               (ref[0][:, :, :190], ref[1][:, :, :210], ref[2][:, :, :210])):
        _check(name, got, want, BWD_TOL[dtype])
    none = torch.zeros(1, dtype=torch.int32, device=dd)
    attn.attn_bwd(qd, kd, vd, o, lse, g, d_q=gq.fill_(sentinel), d_k=gk.fill_(sentinel), d_v=gv.fill_(sentinel),
                  scale=inputs.default_scale(d), causal=True, cu_seqlens_q=none, cu_seqlens_k=none,
                  max_seqlen_q=0)
    torch.cuda.synchronize()
    assert torch.all(gq == sentinel) and torch.all(gk == sentinel) and torch.all(gv == sentinel)


@pytest.mark.parametrize("lq,lk,dh,dv", [(300, 300, 128, 128), (200, 457, 64, 128), (129, 64, 128, 64)])
def test_single_sequence_backward_is_the_dense_call_bitwise(lq, lk, dh, dv):
    """One packed sequence runs the same tiles in the same order as the dense
    call with q_offset = L_k - L_q: identical bits."""
    q, k, v, _, cu_q, cu_k = inputs.make_packed([lq], [lk], 4, 2, dh, dv, seed=lq + lk)
    d = dev()
    qd, kd, vd = q.to(d), k.to(d), v.to(d)
    scale = inputs.default_scale(dh)
    o, lse = attn.attn_fwd(qd, kd, vd, scale=scale, causal=True, q_offset=lk - lq)
    g = _grad_out(o.shape, torch.bfloat16, 4).to(d)
    dense = attn.attn_bwd(qd, kd, vd, o, lse, g, scale=scale, causal=True, q_offset=lk - lq)
    packed = attn.attn_bwd(qd, kd, vd, o, lse, g, scale=scale, causal=True, cu_seqlens_q=cu_q.to(d),
                           cu_seqlens_k=cu_k.to(d), max_seqlen_q=lq)
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV"), dense, packed):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name


def test_packed_backward_workload_size():
    """The packed workload (8 causal sequences, lengths drawn as for the
    padded-batch workload, 16 heads, d_h 64, d_v 128): each sequence's
    gradients equal a dense attn_bwd call on that sequence alone, given the
    same forward outputs, bit for bit (the dense forward of the longest
    sequence may pick another workgroup shape, so O and LSE come from the
    packed call), and rows and keys sampled across sequences and heads match
    the oracle's sampled gradients of that sequence."""
    lengths = inputs.varlen_lengths(8, 4096, 1005)
    hq, dh, dv = 16, 64, 128
    q, k, v, _, cu_q, cu_k = inputs.make_packed(lengths, lengths, hq, hq, dh, dv, seed=1005)
    d = dev()
    scale = inputs.default_scale(dh)
    qd, kd, vd = q.to(d), k.to(d), v.to(d)
    kw = dict(scale=scale, causal=True, cu_seqlens_q=cu_q.to(d), cu_seqlens_k=cu_k.to(d),
              max_seqlen_q=max(lengths))
    o, lse = attn.attn_fwd(qd, kd, vd, **kw)
    g = _grad_out(o.shape, torch.bfloat16, 77)
    gd = g.to(d)
    dq, dk, dv_ = attn.attn_bwd(qd, kd, vd, o, lse, gd, **kw)
    torch.cuda.synchronize()
    offs = cu_q.tolist()
    for s in range(len(lengths)):
        a, b = offs[s], offs[s + 1]
        sl = lambda t: t[:, :, a:b].contiguous()
        ref = attn.attn_bwd(sl(qd), sl(kd), sl(vd), sl(o), lse[:, :, a:b].contiguous(), sl(gd), scale=scale,
                            causal=True)
        torch.cuda.synchronize()
        for name, got, want in zip(("dQ", "dK", "dV"), (dq, dk, dv_), ref):
            assert torch.equal(sl(got).view(torch.int16), want.view(torch.int16)), f"sequence {s}: {name}"
    r = np.random.default_rng(8)
    for s in (0, 3, 7):
        a, b = offs[s], offs[s + 1]
        n = b - a
        rows = [(0, int(h), int(i)) for h, i in zip(r.integers(0, hq, 6), list(r.integers(0, n, 4)) + [0, n - 1])]
        keys = [(0, int(h), int(j)) for h, j in zip(r.integers(0, hq, 6), list(r.integers(0, n, 4)) + [0, n - 1])]
        rq, rk, rv = oracle.attention_backward_sampled(q[:, :, a:b], k[:, :, a:b], v[:, :, a:b], g[:, :, a:b],
                                                       rows=rows, keys=keys, scale=scale, causal=True)
        got_q = np.stack([f64(dq[0, h, a + i]) for _, h, i in rows])
        got_k = np.stack([f64(dk[0, h, a + j]) for _, h, j in keys])
        got_v = np.stack([f64(dv_[0, h, a + j]) for _, h, j in keys])
        for name, got, want in (("dq", got_q, rq), ("dk", got_k, rk), ("dv", got_v, rv)):
            _check(f"sequence {s} {name}", got, want, BWD_TOL[torch.bfloat16])


KV_BWD_CASES = [
    # (dtype, B, Hq, Hkv, Tq, Tk, lens, dh, dv, causal, bias, masked_frac, window)
    (torch.bfloat16, 3, 4, 2, 200, 700, [700, 333, 0], 128, 128, True, "none", 0.0, 0),
    (torch.bfloat16, 2, 8, 2, 64, 1000, [129, 1000], 64, 128, True, "none", 0.0, 0),
    (torch.bfloat16, 2, 2, 2, 300, 300, [300, 170], 128, 64, False, "none", 0.0, 0),
    (torch.bfloat16, 2, 4, 4, 150, 500, [500, 260], 128, 128, True, "keys", 0.2, 90),
    (torch.float32, 2, 2, 1, 40, 120, [120, 33], 64, 64, True, "dense", 0.1, 0),
    (torch.bfloat16, 2, 2, 2, 50, 90, [90, 7], 96, 80, True, "none", 0.0, 0),
]


@pytest.mark.parametrize("case", KV_BWD_CASES, ids=[f"k{i}" for i in range(len(KV_BWD_CASES))])
def test_kvlens_backward_parity(case):
    """attn_bwd with per-batch KV lengths (MFMA kernels for bf16 with d in
    {64, 128}, generic otherwise) against the oracle's gradients; keys past a
    batch's length are written as zero (the gradient buffers start as a
    sentinel)."""
    dtype, b, hq, hkv, tq, tk, lens, dh, dv, causal, bias, mf, w = case
    print("case", case, flush=True)
    wl = inputs.make_random(b, hq, hkv, tq, tk, dh, dv, dtype=dtype, seed=_seed(case), causal=causal,
                            bias=bias, masked_frac=mf)
    d = dev()
    q, k, v = wl.q.to(d), wl.k.to(d), wl.v.to(d)
    m = None if wl.bias is None else wl.bias.to(d)
    lens_t = torch.tensor(lens, dtype=torch.int32, device=d)
    kw = dict(scale=wl.scale, causal=causal, bias=m, window=w, seqlens_k=lens_t)
    o, lse = attn.attn_fwd(q, k, v, **kw)
    g = _grad_out(o.shape, dtype, _seed(case) + 1)
    gq, gk, gv = (torch.full(t.shape, -777.0, dtype=dtype, device=d) for t in (q, k, v))
    attn.attn_bwd(q, k, v, o, lse, g.to(d), d_q=gq, d_k=gk, d_v=gv, **kw)
    torch.cuda.synchronize()
    ref = oracle.attention_kvlens_backward(f64(wl.q), f64(wl.k), f64(wl.v), f64(g), lens, scale=wl.scale,
                                           causal=causal, bias=None if wl.bias is None else f64(wl.bias),
                                           window=w)
    for bb, n in enumerate(lens):
        assert torch.all(gk[bb, :, n:] == 0) and torch.all(gv[bb, :, n:] == 0), f"batch {bb}: keys past {n}"
    for name, got, want in zip(("dQ", "dK", "dV"), (gq, gk, gv), ref):
        _check(name, got, want, BWD_TOL[dtype])
