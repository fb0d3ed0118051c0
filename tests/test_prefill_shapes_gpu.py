"""GPU parity of the MFMA prefill's large workgroup shape (8 wavefronts of 32
query rows, 128-key tiles), which attn_fwd picks for d_h = d_v = 128 without
bias, window or variable lengths when the problem has at least 256 query
tiles of 256 rows.  Sizes here are just large enough to select it and small
enough for the whole oracle: ragged T_q, grouped heads, non-square causal
alignment (negative and positive offsets), non-causal calls and the n_legal
counts; a windowed case of the same size (the standard shape) rides along."""

import zlib

import numpy as np
import pytest
import torch

import online_softmax_exact_amd as attn
from online_softmax_exact_amd import inputs
from gpu_util import assert_close, ensure_built, oracle_full, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


CASES = [
    # (B, Hq, Hkv, Tq, Tk, causal, q_offset, window)
    (2, 32, 32, 1000, 1000, True, 0, 0),
    (1, 64, 8, 1024, 1024, True, 0, 0),
    (2, 32, 16, 777, 1500, True, 723, 0),
    (2, 32, 32, 900, 900, False, 0, 0),
    (1, 64, 64, 1100, 1100, True, 0, 300),
    (4, 16, 4, 1000, 1000, True, -40, 0),
    (1, 128, 32, 520, 2000, False, 0, 0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}H{c[1]}/{c[2]}-T{c[3]}x{c[4]}-c{int(c[5])}-off{c[6]}-W{c[7]}")
def test_large_shape_parity(case):
    b, hq, hkv, tq, tk, causal, off, w = case
    assert (tq + 255) // 256 * b * hq >= 256   # the shape this file covers
    print("case:", case, flush=True)
    wl = inputs.make_random(b, hq, hkv, tq, tk, 128, 128, seed=zlib.crc32(repr(case).encode()) % 10_000,
                            causal=causal, q_offset=off)
    q, k, v, _ = to_dev(wl)
    o, lse, n = attn.attn_fwd(q, k, v, scale=wl.scale, causal=causal, q_offset=off, window=w, return_n_legal=True)
    o2, lse2 = attn.attn_fwd(q, k, v, scale=wl.scale, causal=causal, q_offset=off, window=w)
    torch.cuda.synchronize()
    o_ref, l_ref, n_ref = oracle_full(wl, window=w)
    assert_close(o, lse, o_ref, l_ref, torch.bfloat16, what=str(case))
    assert_close(o2, lse2, o_ref, l_ref, torch.bfloat16, what=str(case) + " (no counts)")
    assert np.array_equal(n.cpu().numpy(), n_ref), "n_legal differs"
