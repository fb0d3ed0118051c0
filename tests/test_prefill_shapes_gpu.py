"""GPU parity of the MFMA prefill's large workgroup shape (8 wavefronts of 32
query rows, 128-key tiles), which attn_fwd picks without bias, window or
variable lengths for d_h = d_v = 128 when the problem has at least 256 query
tiles of 256 rows, and for d_h = 64, d_v = 128 when it has 256 to 512 of
them.  Sizes here are just large enough to select it and small enough for the
whole oracle: ragged T_q, grouped heads, non-square causal alignment
(negative and positive offsets, and causal rows from position 0 on, whose
few keys leave the output close to one value row), non-causal calls and the
n_legal counts; a windowed case of the same size (the standard shape) rides
along."""

import zlib

import numpy as np
import pytest
import torch

import oracle
import online_softmax_exact_amd as attn
from online_softmax_exact_amd import inputs
from gpu_util import assert_close, ensure_built, o_max_allowed, oracle_full, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


CASES = [
    # (B, Hq, Hkv, Tq, Tk, causal, q_offset, window, d_h)
    (2, 32, 32, 1000, 1000, True, 0, 0, 128),
    (1, 64, 8, 1024, 1024, True, 0, 0, 128),
    (2, 32, 16, 777, 1500, True, 723, 0, 128),
    (2, 32, 32, 900, 900, False, 0, 0, 128),
    (1, 64, 64, 1100, 1100, True, 0, 300, 128),
    (4, 16, 4, 1000, 1000, True, -40, 0, 128),
    (1, 128, 32, 520, 2000, False, 0, 0, 128),
    # d_h = 64 on the large shape, causal cases from position 0 on (rows
    # with one to a few keys, whose output is nearly one value row) and past
    # the first keys.
    (1, 256, 64, 500, 500, True, 0, 0, 64),
    (2, 128, 32, 300, 700, True, 0, 0, 64),
    (2, 64, 16, 700, 700, True, 0, 0, 64),
    (1, 256, 64, 500, 500, True, 40, 0, 64),
    (2, 64, 16, 700, 900, True, 200, 0, 64),
    (1, 128, 128, 1000, 1000, False, 0, 0, 64),
    (2, 128, 32, 300, 700, True, 380, 0, 64),
]


@pytest.mark.parametrize("case", CASES,
                         ids=lambda c: f"B{c[0]}H{c[1]}/{c[2]}-T{c[3]}x{c[4]}-c{int(c[5])}-off{c[6]}-W{c[7]}-d{c[8]}")
def test_large_shape_parity(case):
    b, hq, hkv, tq, tk, causal, off, w, dh = case
    tiles = (tq + 255) // 256 * b * hq
    assert tiles >= 256 and (dh == 128 or tiles <= 512)   # the shape this file covers
    print("case:", case, flush=True)
    wl = inputs.make_random(b, hq, hkv, tq, tk, dh, 128, seed=zlib.crc32(repr(case).encode()) % 10_000,
                            causal=causal, q_offset=off)
    q, k, v, _ = to_dev(wl)
    o, lse, n = attn.attn_fwd(q, k, v, scale=wl.scale, causal=causal, q_offset=off, window=w, return_n_legal=True)
    o2, lse2 = attn.attn_fwd(q, k, v, scale=wl.scale, causal=causal, q_offset=off, window=w)
    torch.cuda.synchronize()
    o_ref, l_ref, n_ref = oracle_full(wl, window=w)
    assert_close(o, lse, o_ref, l_ref, torch.bfloat16, what=str(case))
    assert_close(o2, lse2, o_ref, l_ref, torch.bfloat16, what=str(case) + " (no counts)")
    assert np.array_equal(n.cpu().numpy(), n_ref), "n_legal differs"


@pytest.mark.parametrize("case", [(9, 32, 32, 4000, 128, True), (40, 16, 8, 3000, 64, False)],
                         ids=["B9H32-T4000-d128-c1", "B40H16/8-T3000-d64-c0"])
def test_batch_major_order_sampled(case):
    """Dense batches whose K/V exceeds 256 MB run batch after batch (the large
    and the standard shape); rows sampled in every batch, at tile edges and
    the ragged end, against the oracle row by row."""
    b, hq, hkv, t, dh, causal = case
    assert b * hkv * t * (dh + 128) * 2 > 256 << 20   # the order this test covers
    print("case:", case, flush=True)
    wl = inputs.make_random(b, hq, hkv, t, t, dh, 128, seed=zlib.crc32(repr(case).encode()) % 10_000,
                            causal=causal)
    q, k, v, _ = to_dev(wl)
    o, lse, n = attn.attn_fwd(q, k, v, scale=wl.scale, causal=causal, return_n_legal=True)
    o2, lse2 = attn.attn_fwd(q, k, v, scale=wl.scale, causal=causal)   # the instance without counts
    torch.cuda.synchronize()
    # Both instances run the same arithmetic in the same order: the same bits.
    assert torch.equal(o2.view(torch.int16), o.view(torch.int16)), "O without counts differs"
    assert torch.equal(lse2, lse), "LSE without counts differs"
    r = np.random.default_rng(b)
    rows = [(bb, int(h), int(i)) for bb in range(b)
            for h, i in zip(r.integers(0, hq, 6), [0, 127, 128, 255, t - 1, int(r.integers(0, t))])]
    ro, rl, rn = oracle.attention_rows(wl.q, wl.k, wl.v, rows, scale=wl.scale, causal=causal)
    oc, lc, nc = o.cpu(), lse.cpu(), n.cpu()
    got_o = np.stack([oc[x].double().numpy() for x in rows])
    got_l = np.array([float(lc[x]) for x in rows])
    err = np.abs(got_o - ro)
    assert np.all(err <= o_max_allowed(ro, torch.bfloat16)) and err.mean() <= 1e-3, (err.max(), err.mean())
    assert np.abs(got_l - rl).max() <= 1e-3
    assert [int(nc[x]) for x in rows] == [int(x) for x in rn]
