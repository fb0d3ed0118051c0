"""GPU parity of sliding-window visibility (§33.7 of "Chapter 33 推理计算优化",
the sliding-window paragraph with eq 33.16): row i keeps only the keys
j >= q_offset + i - W + 1 (and j <= q_offset + i when causal).  Every kernel
the entry points dispatch to is covered: the fp32 / odd-size generic kernel,
the MFMA prefill (window edges inside and across 64-key tiles, first streamed
tile > 0, full-tile runs starting on either LDS slot), the few-row kernel and
the split-KV decode (splits wholly outside the window give empty partials)."""

import zlib

import numpy as np
import pytest
import torch

import oracle
import online_softmax_exact_amd as attn
from online_softmax_exact_amd import inputs
from gpu_util import assert_close, ensure_built, f64, oracle_full, to_dev, visible_splits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


WINDOW_FWD_CASES = [
    # (dtype, B, Hq, Hkv, Tq, Tk, dh, dv, causal, offset, bias, masked_frac, window)
    (torch.float32, 1, 2, 1, 100, 100, 64, 64, True, 0, "none", 0.0, 17),
    (torch.float32, 2, 4, 2, 70, 201, 40, 24, True, 131, "dense", 0.1, 64),
    (torch.bfloat16, 1, 2, 2, 600, 600, 128, 128, True, 0, "none", 0.0, 100),
    (torch.bfloat16, 1, 4, 2, 700, 700, 128, 128, True, 0, "none", 0.0, 256),
    (torch.bfloat16, 2, 8, 2, 300, 900, 128, 128, True, 600, "none", 0.0, 129),
    (torch.bfloat16, 1, 4, 4, 500, 500, 128, 64, True, 0, "none", 0.0, 1),
    (torch.bfloat16, 1, 4, 4, 400, 400, 64, 128, True, 0, "shared", 0.05, 200),
    (torch.bfloat16, 1, 2, 2, 333, 333, 64, 64, False, 0, "none", 0.0, 150),
    (torch.bfloat16, 1, 2, 1, 200, 300, 128, 128, True, -50, "none", 0.0, 90),
    (torch.bfloat16, 1, 2, 2, 300, 300, 128, 128, True, 0, "none", 0.0, 5000),
    # few query rows per KV head (the few-row kernel)
    (torch.bfloat16, 2, 8, 2, 4, 1000, 128, 128, True, 996, "none", 0.0, 300),
    (torch.bfloat16, 1, 32, 1, 1, 2000, 64, 64, True, 1999, "none", 0.0, 1),
    (torch.bfloat16, 2, 4, 4, 3, 500, 128, 64, False, 200, "none", 0.0, 77),
]


@pytest.mark.parametrize("case", WINDOW_FWD_CASES,
                         ids=lambda c: f"{str(c[0])[6:]}-B{c[1]}H{c[2]}/{c[3]}-T{c[4]}x{c[5]}-d{c[6]}/{c[7]}-c{int(c[8])}-off{c[9]}-{c[10]}-W{c[12]}")
def test_window_fwd_parity(case):
    dt, b, hq, hkv, tq, tk, dh, dv, causal, off, bias, frac, w = case
    print("case:", case, flush=True)
    wl = inputs.make_random(b, hq, hkv, tq, tk, dh, dv, dtype=dt, seed=zlib.crc32(repr(case).encode()) % 10_000,
                            causal=causal, q_offset=off, bias=bias, masked_frac=frac)
    q, k, v, m = to_dev(wl)
    o, lse, n = attn.attn_fwd(q, k, v, scale=wl.scale, causal=causal, q_offset=off, bias=m,
                              window=w, return_n_legal=True)
    torch.cuda.synchronize()
    o2, lse2 = attn.attn_fwd(q, k, v, scale=wl.scale, causal=causal, q_offset=off, bias=m, window=w)
    torch.cuda.synchronize()
    o_ref, l_ref, n_ref = oracle_full(wl, window=w)
    assert_close(o, lse, o_ref, l_ref, dt, what=str(case))
    assert_close(o2, lse2, o_ref, l_ref, dt, what=str(case) + " (no counts)")
    assert np.array_equal(n.cpu().numpy(), n_ref), "n_legal differs"


def test_window_long_causal_sampled():
    """A long causal prefill with a window: the first streamed tile of late
    query tiles is far from 0 and full-tile runs start on both slots.  Rows are
    sampled across the whole range (each row computed on its own by the
    oracle), n_legal is checked exactly for every row."""
    b, hq, t, d, w = 1, 8, 4096, 128, 1000
    wl = inputs.make_random(b, hq, hq, t, t, d, d, seed=77, causal=True)
    q, k, v, _ = to_dev(wl)
    o, lse, n = attn.attn_fwd(q, k, v, scale=wl.scale, causal=True, window=w, return_n_legal=True)
    torch.cuda.synchronize()
    pos = np.arange(t)
    want = np.minimum(pos + 1, w)
    assert np.array_equal(n.cpu().numpy()[0], np.broadcast_to(want, (hq, t)))
    rng = np.random.default_rng(5)
    rows = [(0, int(h), int(i)) for h in range(hq)
            for i in sorted(set(rng.integers(0, t, 12).tolist()) | {0, w - 1, w, t - 1})]
    o_ref, l_ref, _ = oracle.attention_rows(wl.q, wl.k, wl.v, rows, scale=wl.scale, causal=True, window=w)
    og = np.stack([f64(o[r[0], r[1], r[2]]) for r in rows])
    lg = np.array([float(lse[r[0], r[1], r[2]]) for r in rows])
    assert_close(og, lg, o_ref, l_ref, torch.bfloat16, what="sampled window rows")


WINDOW_DECODE_CASES = [
    # (dtype, B, Hq, Hkv, Tq, Tk, dh, dv, split, window)
    (torch.bfloat16, 2, 8, 2, 1, 3000, 128, 128, 256, 700),
    (torch.bfloat16, 1, 4, 4, 5, 1000, 128, 128, 100, 33),
    (torch.bfloat16, 1, 8, 1, 3, 600, 64, 128, 64, 1),
    (torch.float32, 1, 2, 1, 1, 900, 64, 64, 96, 250),
]


@pytest.mark.parametrize("case", WINDOW_DECODE_CASES,
                         ids=lambda c: f"{str(c[0])[6:]}-B{c[1]}H{c[2]}/{c[3]}-T{c[4]}x{c[5]}-S{c[8]}-W{c[9]}")
def test_window_decode_parity(case):
    dt, b, hq, hkv, tq, tk, dh, dv, split, w = case
    off = tk - tq
    print("case:", case, flush=True)
    wl = inputs.make_random(b, hq, hkv, tq, tk, dh, dv, dtype=dt, seed=zlib.crc32(repr(case).encode()) % 10_000,
                            causal=True, q_offset=off)
    q, k, v, _ = to_dev(wl)
    o, lse, ws = attn.attn_decode_splitkv(q, k, v, split_size=split, scale=wl.scale, causal=True,
                                          q_offset=off, window=w)
    torch.cuda.synchronize()
    o_ref, l_ref, _ = oracle_full(wl, window=w)
    assert_close(o, lse, o_ref, l_ref, dt, what=str(case))
    op_ref, lp_ref = oracle.split_partials(f64(wl.q), f64(wl.k), f64(wl.v), scale=wl.scale, causal=True,
                                           q_offset=off, split_size=split, window=w)
    o_parts, l_parts = attn.split_workspace_views(ws, q, v, split)
    assert bool(np.isneginf(lp_ref).any())
    # Ranges no row can see are neither written nor merged: the oracle's
    # partials there are all empty.
    s0, s1 = visible_splits(tq, tk, off, split, window=w)
    assert s1 - s0 < o_parts.shape[3]
    assert bool(np.isneginf(lp_ref[..., :s0]).all()) and bool(np.isneginf(lp_ref[..., s1:]).all())
    assert_close(f64(o_parts[..., s0:s1, :]), f64(l_parts[..., s0:s1]), op_ref[..., s0:s1, :],
                 lp_ref[..., s0:s1], torch.float32 if dt == torch.float32 else torch.bfloat16,
                 what="window partials")


def test_window_negative_rejected():
    wl = inputs.make_random(1, 1, 1, 4, 8, 64, 64, seed=3)
    q, k, v, _ = to_dev(wl)
    with pytest.raises(ValueError):
        attn.attn_fwd(q, k, v, window=-1)
