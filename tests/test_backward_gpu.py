"""GPU parity of the backward pass (eqs 33.6-33.8 of "Chapter 33 推理计算优化"
§33.3, recomputation from the saved LSE): attn_bwd through the C ABI against
the fp64 oracle's gradients on the same inputs, element by element."""

import zlib

import numpy as np
import pytest
import torch

import oracle
import online_softmax_exact_amd as attn
from online_softmax_exact_amd import inputs
from gpu_util import ensure_built, f64, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


BWD_CASES = [
    # (dtype, B, Hq, Hkv, Tq, Tk, dh, dv, causal, offset, bias, masked_frac, window)
    (torch.float32, 1, 2, 1, 70, 70, 64, 64, True, 0, "none", 0.0, 0),
    (torch.float32, 2, 4, 2, 33, 101, 40, 24, True, 68, "dense", 0.2, 0),
    (torch.bfloat16, 1, 2, 2, 200, 200, 128, 128, True, 0, "none", 0.0, 0),
    (torch.bfloat16, 2, 8, 2, 130, 300, 128, 128, True, 170, "none", 0.0, 0),
    (torch.bfloat16, 1, 4, 4, 150, 150, 64, 128, True, 0, "shared", 0.1, 0),
    (torch.bfloat16, 1, 4, 2, 120, 180, 128, 64, False, 0, "none", 0.0, 0),
    (torch.bfloat16, 1, 2, 2, 260, 260, 128, 128, True, 0, "none", 0.0, 50),
    (torch.bfloat16, 1, 2, 1, 64, 90, 64, 64, True, -20, "rows", 0.3, 0),
    # MFMA kernels: several 128-row / 128-key workgroup tiles, ragged tails
    (torch.bfloat16, 1, 4, 1, 300, 450, 64, 64, True, 150, "none", 0.0, 0),
    (torch.bfloat16, 2, 2, 2, 257, 257, 128, 128, True, 0, "none", 0.0, 130),
    (torch.bfloat16, 1, 4, 4, 2048, 2048, 128, 128, True, 0, "none", 0.0, 0),
    (torch.bfloat16, 1, 2, 2, 5, 700, 128, 128, True, 695, "none", 0.0, 0),
    # MFMA kernels with a bias: rows 301 floats apart (unaligned 16-byte
    # loads), -inf entries and wholly masked rows inside fully visible blocks,
    # a per-key bias with a window, grouped heads
    (torch.bfloat16, 1, 4, 2, 257, 301, 128, 128, True, 44, "dense", 0.1, 0),
    (torch.bfloat16, 2, 4, 4, 200, 200, 128, 128, True, 0, "keys", 0.3, 60),
    (torch.bfloat16, 1, 8, 2, 300, 300, 64, 128, False, 0, "rows", 0.2, 0),
    (torch.bfloat16, 2, 2, 1, 190, 190, 128, 64, True, 0, "shared", 0.05, 0),
]


# Error bounds relative to the largest |gradient| of each tensor.  bf16: the
# outputs alone are rounded to 2^-9 of their size, and the MFMA path also
# rounds P, dS and the operands to bf16 (fp32 accumulation), so 2e-2 of the
# largest gradient (1e-2 is the bar on O, whose entries are O(1)) and a mean
# of 2e-3; fp32 matches the forward's 1e-5.
BWD_TOL = {torch.float32: dict(max=1e-5, mean=1e-6), torch.bfloat16: dict(max=2e-2, mean=2e-3)}


def _rel(g, ref):
    scale = max(float(np.abs(ref).max()), 1e-30)
    err = np.abs(g - ref)
    return float(err.max() / scale), float(err.mean() / scale)


@pytest.mark.parametrize("case", BWD_CASES,
                         ids=lambda c: f"{str(c[0])[6:]}-B{c[1]}H{c[2]}/{c[3]}-T{c[4]}x{c[5]}-d{c[6]}/{c[7]}-c{int(c[8])}-off{c[9]}-{c[10]}-W{c[12]}")
def test_backward_parity(case):
    dt, b, hq, hkv, tq, tk, dh, dv, causal, off, bias, frac, w = case
    print("case:", case, flush=True)
    seed = zlib.crc32(repr(case).encode()) % 10_000
    wl = inputs.make_random(b, hq, hkv, tq, tk, dh, dv, dtype=dt, seed=seed, causal=causal,
                            q_offset=off, bias=bias, masked_frac=frac)
    g = torch.randn((b, hq, tq, dv), generator=torch.Generator().manual_seed(seed + 7)).to(dt)
    q, k, v, m = to_dev(wl)
    d_o = g.to(q.device)
    o, lse = attn.attn_fwd(q, k, v, scale=wl.scale, causal=causal, q_offset=off, bias=m, window=w)
    dq, dk, dvv = attn.attn_bwd(q, k, v, o, lse, d_o, scale=wl.scale, causal=causal, q_offset=off,
                                bias=m, window=w)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_backward(wl.q, wl.k, wl.v, g, scale=wl.scale, causal=causal,
                                           q_offset=off, bias=None if wl.bias is None else f64(wl.bias),
                                           window=w)
    errs = {n: _rel(f64(x), r) for n, x, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dvv, rv))}
    print("relative errors (max, mean):", errs, flush=True)
    for n, x in (("dq", dq), ("dk", dk), ("dv", dvv)):
        assert not torch.isnan(x).any(), n
    # Exact zeros where nothing contributes: dQ of rows without a legal key,
    # dK and dV of keys that no row sees (dV_j = sum_i P_ij dO_i is zero only
    # then).
    _, l_ref, _ = oracle.attention(f64(wl.q), f64(wl.k), f64(wl.v), scale=wl.scale, causal=causal,
                                   q_offset=off, bias=None if wl.bias is None else f64(wl.bias),
                                   window=w)
    dead_rows = np.isneginf(l_ref)
    dead_keys = np.all(rv == 0, axis=-1)
    assert np.all(f64(dq)[dead_rows] == 0)
    assert np.all(f64(dk)[dead_keys] == 0) and np.all(f64(dvv)[dead_keys] == 0)
    tol = BWD_TOL[dt]
    for n, (mx, mean) in errs.items():
        assert mx <= tol["max"] and mean <= tol["mean"], f"{n}: {mx:.2e} / {mean:.2e} > {tol}"


def test_backward_full_size_sampled():
    """The causal prefill of the benchmark (B = 1, 32 heads, T = 8192,
    d = 128) through the GPU forward and backward; dQ of sampled rows and
    dK, dV of sampled keys against the oracle evaluated at those places."""
    wl = inputs.make_config(2)
    q, k, v, _ = to_dev(wl)
    g = torch.randn(q.shape, generator=torch.Generator().manual_seed(4242)).to(torch.bfloat16)
    d_o = g.to(q.device)
    o, lse = attn.attn_fwd(q, k, v, scale=wl.scale, causal=True)
    dq, dk, dv = attn.attn_bwd(q, k, v, o, lse, d_o, scale=wl.scale, causal=True)
    torch.cuda.synchronize()
    t = q.shape[2]
    rows = [(0, h, i) for h in (0, 17) for i in (0, 1, 127, 128, 4095, 5000, t - 2, t - 1)]
    keys = [(0, h, j) for h in (3, 31) for j in (0, 1, 64, 2047, 6000, t - 64, t - 1)]
    rq, rk, rv = oracle.attention_backward_sampled(wl.q, wl.k, wl.v, g, rows=rows, keys=keys,
                                                   scale=wl.scale, causal=True)
    got_q = np.stack([f64(dq[r]) for r in rows])
    got_k = np.stack([f64(dk[x]) for x in keys])
    got_v = np.stack([f64(dv[x]) for x in keys])
    for n, x, r in (("dq", got_q, rq), ("dk", got_k, rk), ("dv", got_v, rv)):
        mx, mean = _rel(x, r)
        print(n, "relative errors", mx, mean, flush=True)
        assert mx <= BWD_TOL[torch.bfloat16]["max"] and mean <= BWD_TOL[torch.bfloat16]["mean"], n


def test_backward_batch_major_sampled():
    """Dense batches whose K/V exceeds 256 MB (B = 3, 32 heads, T = 6000,
    d = 128: 295 MB) run batch after batch in all three MFMA kernels; sampled
    rows and keys of every batch against the oracle's gradients at those
    places."""
    b, h, t = 3, 32, 6000
    assert b * h * t * 256 * 2 > 256 << 20   # the order this test covers
    wl = inputs.make_random(b, h, h, t, t, 128, 128, seed=606, causal=True)
    q, k, v, _ = to_dev(wl)
    g = torch.randn(q.shape, generator=torch.Generator().manual_seed(607)).to(torch.bfloat16)
    o, lse = attn.attn_fwd(q, k, v, scale=wl.scale, causal=True)
    dq, dk, dv = attn.attn_bwd(q, k, v, o, lse, g.to(q.device), scale=wl.scale, causal=True)
    torch.cuda.synchronize()
    r = np.random.default_rng(5)
    rows = [(bb, int(hh), int(i)) for bb in range(b) for hh, i in zip(r.integers(0, h, 4), [0, 128, t - 1, int(r.integers(0, t))])]
    keys = [(bb, int(hh), int(j)) for bb in range(b) for hh, j in zip(r.integers(0, h, 4), [0, 127, t - 1, int(r.integers(0, t))])]
    rq, rk, rv = oracle.attention_backward_sampled(wl.q, wl.k, wl.v, g, rows=rows, keys=keys, scale=wl.scale,
                                                   causal=True)
    dqc, dkc, dvc = dq.cpu(), dk.cpu(), dv.cpu()
    got = (np.stack([f64(dqc[x]) for x in rows]), np.stack([f64(dkc[x]) for x in keys]),
           np.stack([f64(dvc[x]) for x in keys]))
    for n, x, ref in zip(("dq", "dk", "dv"), got, (rq, rk, rv)):
        mx, mean = _rel(x, ref)
        print(n, "relative errors", mx, mean, flush=True)
        assert mx <= BWD_TOL[torch.bfloat16]["max"] and mean <= BWD_TOL[torch.bfloat16]["mean"], n
