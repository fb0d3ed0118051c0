"""Long contexts, compared with the oracle on sampled rows (each row computed
from its own query and every key of its KV head): split-KV decode over a
cache of 2^20 keys (2048 splits of 512 merged per row), the same with
per-batch KV lengths near that size, and a causal prefill of 65536 rows on
the large workgroup shape.  Positions, split indices and tile counts reach
sizes no other test does; every index the kernels form stays far below 2^31,
and the test shows the results stay exact there."""

import numpy as np
import pytest
import torch

import oracle
import online_softmax_exact_amd as attn
from online_softmax_exact_amd import inputs
from gpu_util import TOL, dev, ensure_built, f64, o_max_allowed

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _check_rows(o, lse, rows, ro, rl, what):
    got_o = np.stack([f64(o[r]) for r in rows])
    got_l = np.array([float(lse[r]) for r in rows])
    err = np.abs(got_o - ro)
    tol = TOL[torch.bfloat16]
    print(what, "max", float(err.max()), "mean", float(err.mean()), flush=True)
    assert np.all(err <= o_max_allowed(ro, torch.bfloat16)) and err.mean() <= tol["o_mean"], what
    dead = np.isneginf(rl)
    assert np.array_equal(np.isneginf(got_l), dead), what + ": masked-row flags"
    assert np.all(got_o[dead] == 0), what + ": masked row not zero"
    if (~dead).any():
        assert np.abs(got_l[~dead] - rl[~dead]).max() <= tol["lse"], what


def test_decode_one_million_keys():
    """GQA decode, 8 query heads over 2 KV heads, T_k = 2^20, every row
    checked."""
    t_k = 1 << 20
    wl = inputs.make_random(1, 8, 2, 1, t_k, 128, 128, seed=2020, causal=True, q_offset=t_k - 1)
    q, k, v = wl.q.to(dev()), wl.k.to(dev()), wl.v.to(dev())
    o, lse, _ = attn.attn_decode_splitkv(q, k, v, split_size=512, scale=wl.scale)
    torch.cuda.synchronize()
    rows = [(0, h, 0) for h in range(8)]
    ro, rl, _ = oracle.attention_rows(wl.q, wl.k, wl.v, rows, scale=wl.scale, causal=True, q_offset=t_k - 1)
    _check_rows(o.cpu(), lse.cpu(), rows, ro, rl, "decode 2^20 keys")


def test_decode_kvlens_near_one_million():
    """Per-batch KV lengths 2^20, 777777 and 1 in a cache of 2^20 keys."""
    t_k = 1 << 20
    lens = [t_k, 777_777, 1]
    wl = inputs.make_random(3, 4, 1, 2, t_k, 128, 128, seed=2021, causal=True)
    q, k, v = wl.q.to(dev()), wl.k.to(dev()), wl.v.to(dev())
    o, lse, _ = attn.attn_decode_splitkv(q, k, v, split_size=512, scale=wl.scale,
                                         seqlens_k=torch.tensor(lens, dtype=torch.int32, device=dev()))
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    for b, n in enumerate(lens):
        rows = [(0, h, i) for h in range(4) for i in range(2)]
        ro, rl, _ = oracle.attention_rows(wl.q[b:b + 1], wl.k[b:b + 1, :, :n], wl.v[b:b + 1, :, :n], rows,
                                          scale=wl.scale, causal=True, q_offset=n - 2)
        _check_rows(o[b:b + 1], lse[b:b + 1], rows, ro, rl, f"batch {b}, {n} keys")


def test_prefill_64k_rows():
    """Causal prefill, 2 heads of 65536 rows (the large workgroup shape),
    rows sampled at tile edges and across the range."""
    t = 1 << 16
    wl = inputs.make_random(1, 2, 2, t, t, 128, 128, seed=2022, causal=True)
    q, k, v = wl.q.to(dev()), wl.k.to(dev()), wl.v.to(dev())
    o, lse, n = attn.attn_fwd(q, k, v, scale=wl.scale, causal=True, return_n_legal=True)
    torch.cuda.synchronize()
    r = np.random.default_rng(3)
    picks = [0, 1, 31, 127, 128, 255, 256, 4095, 32767, 32768, t - 129, t - 2, t - 1] + \
        [int(x) for x in r.integers(0, t, 8)]
    rows = [(0, h, i) for h in range(2) for i in picks]
    ro, rl, rn = oracle.attention_rows(wl.q, wl.k, wl.v, rows, scale=wl.scale, causal=True)
    _check_rows(o.cpu(), lse.cpu(), rows, ro, rl, "prefill 65536 rows")
    n = n.cpu()
    assert [int(n[x]) for x in rows] == [int(x) for x in rn]
