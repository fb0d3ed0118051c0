"""Seeded random problems across every option of the entry points, each
compared element by element with the oracle: dtype, head sizes on the fast
kernels (64, 128) and on the generic one, head grouping, causal or not, any
query offset (negative, inside, past the keys), sliding windows, every bias
broadcast with -inf entries, T_k = 0, split-KV decode with any split size,
packed sequences and per-batch KV lengths, and the backward on dense and
packed batches.  Sizes stay small so the oracle finishes in well under a
second per case."""

import numpy as np
import pytest
import torch

import oracle
import online_softmax_exact_amd as attn
from online_softmax_exact_amd import inputs
from gpu_util import assert_close, dev, ensure_built, f64

pytestmark = pytest.mark.gpu

N_CASES = 64


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def draw_case(i):
    """Case i: a dict of everything the call needs, from its own generator."""
    r = np.random.default_rng(5000 + i)
    c = {}
    c["mode"] = r.choice(["fwd", "fwd", "decode", "packed", "kvlens"])
    c["dtype"] = torch.float32 if r.random() < 0.2 else torch.bfloat16
    fast = r.random() < 0.75
    c["d_h"] = int(r.choice([64, 128])) if fast else int(r.choice([8, 32, 40, 96, 256]))
    c["d_v"] = int(r.choice([64, 128])) if fast else int(r.choice([16, 24, 64, 200]))
    c["h_kv"] = int(r.choice([1, 2, 4]))
    c["h_q"] = c["h_kv"] * int(r.choice([1, 2, 4, 8]))
    c["causal"] = bool(r.random() < 0.7)
    c["window"] = 0 if r.random() < 0.6 else int(r.integers(1, 400))
    c["bias"] = str(r.choice(["none", "none", "keys", "rows", "dense", "shared"]))
    c["masked_frac"] = float(r.choice([0.0, 0.05, 0.3]))
    if c["mode"] == "fwd":
        c["b"] = int(r.integers(1, 4))
        c["t_q"] = int(r.integers(1, 300))
        c["t_k"] = int(r.choice([0, int(r.integers(1, 700))]) if r.random() < 0.1 else r.integers(1, 700))
        c["q_offset"] = int(r.integers(-60, c["t_k"] + 60))
    elif c["mode"] == "decode":
        c["b"] = int(r.integers(1, 5))
        c["t_q"] = int(r.integers(1, 6))
        c["t_k"] = int(r.integers(1, 3000))
        c["q_offset"] = c["t_k"] - c["t_q"] if r.random() < 0.7 else int(r.integers(-10, c["t_k"] + 10))
        c["split"] = int(r.choice([1, 7, 64, 256, 512, 1000, 5000]))
    elif c["mode"] == "packed":
        n = int(r.integers(1, 6))
        c["lq"] = [int(x) for x in r.integers(0, 260, n)]
        c["lk"] = [max(0, int(x)) for x in (np.array(c["lq"]) + r.integers(-40, 300, n))]
        c["bias"] = str(r.choice(["none", "packed", "keys"]))
        c["q_offset"] = int(r.choice([0, 0, 0, 5, -3]))
        c["max_q"] = int(r.choice([max(c["lq"]), 0, 100]))
    else:  # kvlens
        c["b"] = int(r.integers(1, 5))
        c["t_q"] = int(r.integers(1, 200)) if r.random() < 0.5 else int(r.integers(1, 6))
        c["t_k"] = int(r.integers(1, 2000))
        c["lens"] = [int(x) for x in r.integers(0, c["t_k"] + 1, c["b"])]
        c["q_offset"] = 0
        c["decode"] = bool(r.random() < 0.5)
        c["split"] = int(r.choice([64, 333, 512]))
    if c["mode"] == "decode" and c["dtype"] == torch.bfloat16 and c["bias"] != "none":
        c["bias"] = "none" if r.random() < 0.5 else c["bias"]   # half of them on the fast kernel
    return c


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_parity(i):
    c = draw_case(i)
    print("case", i, c, flush=True)
    dd = dev()
    if c["mode"] == "packed":
        q, k, v, m, cu_q, cu_k = inputs.make_packed(c["lq"], c["lk"], c["h_q"], c["h_kv"], c["d_h"], c["d_v"],
                                                    dtype=c["dtype"], seed=i, bias=c["bias"],
                                                    masked_frac=c["masked_frac"])
        scale = inputs.default_scale(c["d_h"])
        if q.shape[2] == 0:
            pytest.skip("no rows drawn")
        o, lse, n = attn.attn_fwd(q.to(dd), k.to(dd), v.to(dd), scale=scale, causal=c["causal"],
                                  q_offset=c["q_offset"], bias=None if m is None else m.to(dd),
                                  window=c["window"], return_n_legal=True, cu_seqlens_q=cu_q.to(dd),
                                  cu_seqlens_k=cu_k.to(dd), max_seqlen_q=c["max_q"])
        torch.cuda.synchronize()
        o_ref, l_ref, n_ref = oracle.attention_varlen(
            f64(q), f64(k), f64(v), cu_q.tolist(), cu_k.tolist(), scale=scale, causal=c["causal"],
            q_offset=c["q_offset"], bias=None if m is None else f64(m), window=c["window"])
        assert_close(o, lse, o_ref, l_ref, c["dtype"], what=str(c))
        assert np.array_equal(n.cpu().numpy(), n_ref), "n_legal differs"
        return

    wl = inputs.make_random(c["b"], c["h_q"], c["h_kv"], c["t_q"], c["t_k"], c["d_h"], c["d_v"],
                            dtype=c["dtype"], seed=i, causal=c["causal"], q_offset=c["q_offset"],
                            bias=c["bias"], masked_frac=c["masked_frac"])
    q, k, v = wl.q.to(dd), wl.k.to(dd), wl.v.to(dd)
    m = None if wl.bias is None else wl.bias.to(dd)
    b64 = None if wl.bias is None else f64(wl.bias)
    if c["mode"] == "kvlens":
        lens_t = torch.tensor(c["lens"], dtype=torch.int32, device=dd)
        if c["decode"]:
            o, lse, _ = attn.attn_decode_splitkv(q, k, v, split_size=c["split"], scale=wl.scale,
                                                 causal=c["causal"], q_offset=0, window=c["window"],
                                                 seqlens_k=lens_t, bias=m)
            n = None
        else:
            o, lse, n = attn.attn_fwd(q, k, v, scale=wl.scale, causal=c["causal"], window=c["window"], bias=m,
                                      seqlens_k=lens_t, return_n_legal=True)
        torch.cuda.synchronize()
        o_ref, l_ref, n_ref = oracle.attention_kvlens(f64(wl.q), f64(wl.k), f64(wl.v), c["lens"], scale=wl.scale,
                                                      causal=c["causal"], bias=b64, window=c["window"])
    elif c["mode"] == "decode":
        o, lse, _ = attn.attn_decode_splitkv(q, k, v, split_size=c["split"], scale=wl.scale, causal=c["causal"],
                                             q_offset=c["q_offset"], bias=m, window=c["window"])
        n = None
        torch.cuda.synchronize()
        o_ref, l_ref, n_ref = oracle.attention(f64(wl.q), f64(wl.k), f64(wl.v), scale=wl.scale, causal=c["causal"],
                                               q_offset=c["q_offset"], bias=b64, window=c["window"])
    else:
        o, lse, n = attn.attn_fwd(q, k, v, scale=wl.scale, causal=c["causal"], q_offset=c["q_offset"], bias=m,
                                  window=c["window"], return_n_legal=True)
        o2, lse2 = attn.attn_fwd(q, k, v, scale=wl.scale, causal=c["causal"], q_offset=c["q_offset"], bias=m,
                                 window=c["window"])
        torch.cuda.synchronize()
        o_ref, l_ref, n_ref = oracle.attention(f64(wl.q), f64(wl.k), f64(wl.v), scale=wl.scale, causal=c["causal"],
                                               q_offset=c["q_offset"], bias=b64, window=c["window"])
        assert_close(o2, lse2, o_ref, l_ref, c["dtype"], what=str(c) + " (no counts)")
    assert_close(o, lse, o_ref, l_ref, c["dtype"], what=str(c))
    if n is not None:
        assert np.array_equal(n.cpu().numpy(), n_ref), "n_legal differs"


N_BWD = 24
BWD_TOL = {torch.float32: dict(max=1e-5, mean=1e-6), torch.bfloat16: dict(max=2e-2, mean=2e-3)}


def draw_bwd_case(i):
    r = np.random.default_rng(7000 + i)
    fast = r.random() < 0.7
    c = dict(dtype=torch.float32 if r.random() < 0.25 else torch.bfloat16,
             d_h=int(r.choice([64, 128])) if fast else int(r.choice([16, 40, 96])),
             d_v=int(r.choice([64, 128])) if fast else int(r.choice([24, 64, 80])),
             h_kv=int(r.choice([1, 2])), b=int(r.integers(1, 3)),
             t_q=int(r.integers(1, 260)), t_k=int(r.integers(1, 400)),
             causal=bool(r.random() < 0.7), window=0 if r.random() < 0.6 else int(r.integers(1, 300)),
             bias=str(r.choice(["none", "none", "none", "keys", "dense"])),
             masked_frac=float(r.choice([0.0, 0.1])))
    c["h_q"] = c["h_kv"] * int(r.choice([1, 2, 4]))
    c["q_offset"] = int(r.integers(-30, c["t_k"] + 30))
    return c


@pytest.mark.parametrize("i", range(N_BWD))
def test_random_backward_parity(i):
    """attn_bwd on random problems (MFMA kernels for bf16 with d in {64, 128},
    with or without a bias, the generic ones otherwise), relative to each gradient's
    largest entry, with exact zeros where nothing contributes."""
    c = draw_bwd_case(i)
    print("case", i, c, flush=True)
    wl = inputs.make_random(c["b"], c["h_q"], c["h_kv"], c["t_q"], c["t_k"], c["d_h"], c["d_v"],
                            dtype=c["dtype"], seed=100 + i, causal=c["causal"], q_offset=c["q_offset"],
                            bias=c["bias"], masked_frac=c["masked_frac"])
    g = torch.randn((c["b"], c["h_q"], c["t_q"], c["d_v"]), generator=torch.Generator().manual_seed(i)).to(c["dtype"])
    dd = dev()
    q, k, v = wl.q.to(dd), wl.k.to(dd), wl.v.to(dd)
    m = None if wl.bias is None else wl.bias.to(dd)
    kw = dict(scale=wl.scale, causal=c["causal"], q_offset=c["q_offset"], bias=m, window=c["window"])
    o, lse = attn.attn_fwd(q, k, v, **kw)
    dq, dk, dv = attn.attn_bwd(q, k, v, o, lse, g.to(dd), **kw)
    torch.cuda.synchronize()
    b64 = None if wl.bias is None else f64(wl.bias)
    ref = oracle.attention_backward(f64(wl.q), f64(wl.k), f64(wl.v), f64(g), scale=wl.scale, causal=c["causal"],
                                    q_offset=c["q_offset"], bias=b64, window=c["window"])
    _, l_ref, _ = oracle.attention(f64(wl.q), f64(wl.k), f64(wl.v), scale=wl.scale, causal=c["causal"],
                                   q_offset=c["q_offset"], bias=b64, window=c["window"])
    assert np.all(f64(dq)[np.isneginf(l_ref)] == 0), "dQ of a row without a legal key"
    dead_keys = np.all(ref[2] == 0, axis=-1)
    assert np.all(f64(dk)[dead_keys] == 0) and np.all(f64(dv)[dead_keys] == 0), "gradient of an unseen key"
    tol = BWD_TOL[c["dtype"]]
    for name, got, want in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        g64 = f64(got)
        assert not np.isnan(g64).any(), name
        scale = max(float(np.abs(want).max()), 1e-30)
        err = np.abs(g64 - want) / scale
        assert err.max() <= tol["max"] and err.mean() <= tol["mean"], f"{name}: {err.max():.2e} / {err.mean():.2e}"


N_BWD_PACKED = 16


def draw_packed_bwd_case(i):
    r = np.random.default_rng(9000 + i)
    fast = r.random() < 0.7
    n = int(r.integers(1, 6))
    lq = [int(x) for x in r.integers(0, 300, n)]
    c = dict(dtype=torch.float32 if r.random() < 0.2 else torch.bfloat16,
             d_h=int(r.choice([64, 128])) if fast else int(r.choice([16, 40, 96])),
             d_v=int(r.choice([64, 128])) if fast else int(r.choice([24, 64, 80])),
             h_kv=int(r.choice([1, 2])), lq=lq,
             lk=[max(0, int(x)) for x in (np.array(lq) + r.integers(-40, 300, n))],
             causal=bool(r.random() < 0.7), window=0 if r.random() < 0.6 else int(r.integers(1, 300)),
             bias=str(r.choice(["none", "none", "none", "packed", "keys"])),
             masked_frac=float(r.choice([0.0, 0.1])), q_offset=int(r.choice([0, 0, 0, 5, -3])))
    c["h_q"] = c["h_kv"] * int(r.choice([1, 2, 4]))
    return c


@pytest.mark.parametrize("i", range(N_BWD_PACKED))
def test_random_packed_backward_parity(i):
    """attn_bwd on random packed batches (empty sequences, L_q above or below
    L_k, windows, biases, query offsets) against the oracle's packed
    gradients, relative to each gradient's largest entry."""
    c = draw_packed_bwd_case(i)
    print("case", i, c, flush=True)
    q, k, v, m, cu_q, cu_k = inputs.make_packed(c["lq"], c["lk"], c["h_q"], c["h_kv"], c["d_h"], c["d_v"],
                                                dtype=c["dtype"], seed=200 + i, bias=c["bias"],
                                                masked_frac=c["masked_frac"])
    if q.shape[2] == 0:
        pytest.skip("no rows drawn")
    g = torch.randn((1, c["h_q"], q.shape[2], c["d_v"]), generator=torch.Generator().manual_seed(i)).to(c["dtype"])
    dd = dev()
    scale = inputs.default_scale(c["d_h"])
    kw = dict(scale=scale, causal=c["causal"], q_offset=c["q_offset"], bias=None if m is None else m.to(dd),
              window=c["window"], cu_seqlens_q=cu_q.to(dd), cu_seqlens_k=cu_k.to(dd), max_seqlen_q=max(c["lq"]))
    qd, kd, vd = q.to(dd), k.to(dd), v.to(dd)
    o, lse = attn.attn_fwd(qd, kd, vd, **kw)
    dq, dk, dv = attn.attn_bwd(qd, kd, vd, o, lse, g.to(dd), **kw)
    torch.cuda.synchronize()
    b64 = None if m is None else f64(m)
    ref = oracle.attention_varlen_backward(f64(q), f64(k), f64(v), f64(g), cu_q.tolist(), cu_k.tolist(),
                                           scale=scale, causal=c["causal"], q_offset=c["q_offset"], bias=b64,
                                           window=c["window"])
    _, l_ref, _ = oracle.attention_varlen(f64(q), f64(k), f64(v), cu_q.tolist(), cu_k.tolist(), scale=scale,
                                          causal=c["causal"], q_offset=c["q_offset"], bias=b64, window=c["window"])
    # Exact zeros: rows without a legal key, and keys no row sees (dV's
    # zeros; a row with a single legal key has dQ = 0 only up to rounding).
    assert np.all(f64(dq)[np.isneginf(l_ref)] == 0), "dQ of a row without a legal key"
    dead = np.all(ref[2] == 0, axis=-1)
    assert np.all(f64(dk)[dead] == 0) and np.all(f64(dv)[dead] == 0), "gradient of an unseen key"
    tol = BWD_TOL[c["dtype"]]
    for name, got, want in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        g64 = f64(got)
        assert not np.isnan(g64).any(), name
        s = max(float(np.abs(want).max()), 1e-30)
        err = np.abs(g64 - want) / s
        assert err.max() <= tol["max"] and err.mean() <= tol["mean"], f"{name}: {err.max():.2e} / {err.mean():.2e}"


N_BWD_KVLENS = 12


@pytest.mark.parametrize("i", range(N_BWD_KVLENS))
def test_random_kvlens_backward_parity(i):
    """attn_bwd on random batches with per-batch KV lengths (zero lengths,
    lengths below T_q, windows, biases) against the oracle's gradients; keys
    past each length are written as zero."""
    r = np.random.default_rng(11000 + i)
    fast = r.random() < 0.7
    dtype = torch.float32 if r.random() < 0.2 else torch.bfloat16
    d_h = int(r.choice([64, 128])) if fast else int(r.choice([16, 40, 96]))
    d_v = int(r.choice([64, 128])) if fast else int(r.choice([24, 64, 80]))
    h_kv = int(r.choice([1, 2]))
    h_q = h_kv * int(r.choice([1, 2, 4]))
    b = int(r.integers(1, 4))
    t_q = int(r.integers(1, 200))
    t_k = int(r.integers(1, 600))
    lens = [int(x) for x in r.integers(0, t_k + 1, b)]
    causal = bool(r.random() < 0.7)
    window = 0 if r.random() < 0.6 else int(r.integers(1, 300))
    bias = str(r.choice(["none", "none", "keys", "dense"]))
    print("case", i, dict(dtype=dtype, d_h=d_h, d_v=d_v, h=(h_q, h_kv), b=b, t_q=t_q, t_k=t_k, lens=lens,
                          causal=causal, window=window, bias=bias), flush=True)
    wl = inputs.make_random(b, h_q, h_kv, t_q, t_k, d_h, d_v, dtype=dtype, seed=300 + i, causal=causal,
                            bias=bias, masked_frac=0.1 if bias != "none" else 0.0)
    g = torch.randn((b, h_q, t_q, d_v), generator=torch.Generator().manual_seed(i)).to(dtype)
    dd = dev()
    q, k, v = wl.q.to(dd), wl.k.to(dd), wl.v.to(dd)
    m = None if wl.bias is None else wl.bias.to(dd)
    kw = dict(scale=wl.scale, causal=causal, bias=m, window=window,
              seqlens_k=torch.tensor(lens, dtype=torch.int32, device=dd))
    o, lse = attn.attn_fwd(q, k, v, **kw)
    dq, dk, dv = attn.attn_bwd(q, k, v, o, lse, g.to(dd), **kw)
    torch.cuda.synchronize()
    b64 = None if wl.bias is None else f64(wl.bias)
    ref = oracle.attention_kvlens_backward(f64(wl.q), f64(wl.k), f64(wl.v), f64(g), lens, scale=wl.scale,
                                           causal=causal, bias=b64, window=window)
    _, l_ref, _ = oracle.attention_kvlens(f64(wl.q), f64(wl.k), f64(wl.v), lens, scale=wl.scale, causal=causal,
                                          bias=b64, window=window)
    assert np.all(f64(dq)[np.isneginf(l_ref)] == 0), "dQ of a row without a legal key"
    dead = np.all(ref[2] == 0, axis=-1)
    assert np.all(f64(dk)[dead] == 0) and np.all(f64(dv)[dead] == 0), "gradient of an unseen key"
    tol = BWD_TOL[dtype]
    for name, got, want in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        g64 = f64(got)
        assert not np.isnan(g64).any(), name
        s = max(float(np.abs(want).max()), 1e-30)
        err = np.abs(g64 - want) / s
        assert err.max() <= tol["max"] and err.mean() <= tol["mean"], f"{name}: {err.max():.2e} / {err.mean():.2e}"
