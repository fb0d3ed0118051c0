"""GPU parity of the fp32 MFMA prefill (fp32 with d_h, d_v in {64, 128}, any
bias and window, no variable lengths), element by element against the oracle at
the fp32 tolerances (max |dO| 1e-5, mean 1e-6, LSE 1e-5): several 128-row
workgroup tiles and 32-key tiles with ragged ends, causal and not, square and
non-square alignment (offsets before, inside and past the keys), grouped
heads, T_k = 0 and wholly masked rows, n_legal counts, and a strided output
view.  Grids of fewer than 64 128-row workgroups run the key-split kernel
(one workgroup per 32 rows, keys split over its wavefronts, states merged in
LDS): CASES and BIAS_CASES take it; GRID_CASES are sized to take the 128-row
kernel with the same options."""

import zlib

import numpy as np
import pytest
import torch

import online_softmax_exact_amd as attn
from online_softmax_exact_amd import inputs
from gpu_util import assert_close, dev, ensure_built, f64, oracle_full, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


CASES = [
    # (B, Hq, Hkv, Tq, Tk, dh, dv, causal, q_offset)
    (1, 1, 1, 128, 128, 64, 64, True, 0),        # the single-head fp32 workload's shape
    (2, 4, 2, 300, 300, 128, 128, True, 0),
    (1, 8, 2, 257, 700, 64, 128, True, 443),
    (2, 2, 2, 200, 200, 128, 64, False, 0),
    (1, 4, 1, 150, 90, 64, 64, True, -70),       # leading rows see no key
    (1, 2, 2, 33, 1000, 128, 128, True, 2000),   # every row sees every key
    (3, 2, 1, 129, 31, 64, 128, True, 0),
    (1, 2, 2, 1, 513, 64, 64, False, 0),
    (1, 3, 3, 64, 0, 64, 64, True, 0),           # no keys at all
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_fp32_mfma_parity(case):
    b, hq, hkv, tq, tk, dh, dv, causal, off = case
    print("case", case, flush=True)
    wl = inputs.make_random(b, hq, hkv, tq, tk, dh, dv, dtype=torch.float32,
                            seed=zlib.crc32(repr(case).encode()) % 10_000, causal=causal, q_offset=off)
    q, k, v, _ = to_dev(wl)
    o, lse, n = attn.attn_fwd(q, k, v, scale=wl.scale, causal=causal, q_offset=off, return_n_legal=True)
    o2, lse2 = attn.attn_fwd(q, k, v, scale=wl.scale, causal=causal, q_offset=off)
    torch.cuda.synchronize()
    o_ref, l_ref, n_ref = oracle_full(wl)
    assert_close(o, lse, o_ref, l_ref, torch.float32, what=str(case))
    assert_close(o2, lse2, o_ref, l_ref, torch.float32, what=str(case) + " (no counts)")
    assert np.array_equal(n.cpu().numpy(), n_ref), "n_legal differs"


def test_fp32_mfma_strided_output_and_larger():
    """B=1, 8 heads, T=1024 causal, d=64 into an output view whose rows are
    80 floats apart (16-byte aligned: the MFMA kernel), and the same into an
    output with rows 66 floats apart (not a multiple of 4: the generic kernel);
    both match the oracle and each other within the fp32 tolerance."""
    wl = inputs.make_random(1, 8, 8, 1024, 1024, 64, 64, dtype=torch.float32, seed=41, causal=True)
    q, k, v, _ = to_dev(wl)
    o_ref, l_ref, _ = oracle_full(wl)
    for width in (80, 66):
        buf = torch.full((1, 8, 1024, width), 7.0, device=dev())
        out = buf[..., :64]
        _, lse = attn.attn_fwd(q, k, v, scale=wl.scale, causal=True, out=out)
        torch.cuda.synchronize()
        assert_close(out, lse, o_ref, l_ref, torch.float32, what=f"row stride {width}")
        assert torch.all(buf[..., 64:] == 7.0), "wrote past the output view"


BIAS_CASES = [
    # (B, Hq, Hkv, Tq, Tk, dh, dv, causal, q_offset, bias, masked_frac, window)
    (2, 4, 2, 200, 300, 64, 64, True, 100, "dense", 0.1, 0),
    (1, 4, 4, 257, 257, 128, 128, True, 0, "keys", 0.3, 0),
    (1, 2, 1, 150, 150, 64, 128, False, 0, "rows", 0.3, 0),   # wholly masked rows
    (2, 2, 2, 300, 300, 128, 64, True, 0, "shared", 0.05, 40),
    (1, 4, 2, 400, 400, 64, 64, True, 0, "none", 0.0, 1),
    (1, 2, 2, 130, 600, 64, 64, True, 470, "none", 0.0, 200),
]


@pytest.mark.parametrize("case", BIAS_CASES, ids=[f"b{i}" for i in range(len(BIAS_CASES))])
def test_fp32_mfma_bias_and_window(case):
    """The fp32 MFMA prefill with every bias broadcast (-inf entries, wholly
    masked rows) and sliding windows, against the oracle at fp32 tolerances."""
    b, hq, hkv, tq, tk, dh, dv, causal, off, bias, mf, w = case
    print("case", case, flush=True)
    wl = inputs.make_random(b, hq, hkv, tq, tk, dh, dv, dtype=torch.float32,
                            seed=zlib.crc32(repr(case).encode()) % 10_000, causal=causal, q_offset=off,
                            bias=bias, masked_frac=mf)
    q, k, v, m = to_dev(wl)
    o, lse, n = attn.attn_fwd(q, k, v, scale=wl.scale, causal=causal, q_offset=off, bias=m, window=w,
                              return_n_legal=True)
    torch.cuda.synchronize()
    o_ref, l_ref, n_ref = oracle_full(wl, window=w)
    assert_close(o, lse, o_ref, l_ref, torch.float32, what=str(case))
    assert np.array_equal(n.cpu().numpy(), n_ref), "n_legal differs"


def _standard_grid(b, hq, tq):
    return b * hq * -(-tq // 128) >= 64


GRID_CASES = [
    # (B, Hq, Hkv, Tq, Tk, dh, dv, causal, q_offset, bias, masked_frac, window)
    (4, 8, 2, 300, 300, 128, 128, True, 0, "none", 0.0, 0),
    (8, 8, 8, 150, 90, 64, 64, True, -70, "none", 0.0, 0),
    (16, 4, 4, 129, 31, 64, 128, True, 0, "none", 0.0, 0),
    (64, 1, 1, 64, 0, 64, 64, True, 0, "none", 0.0, 0),
    (8, 8, 2, 100, 700, 128, 64, False, 0, "none", 0.0, 0),
    (8, 8, 4, 200, 300, 64, 64, True, 100, "dense", 0.1, 0),
    (8, 8, 8, 130, 130, 128, 128, True, 0, "shared", 0.05, 40),
]


def test_case_lists_take_their_kernels():
    """CASES and BIAS_CASES are small grids (key-split kernel), GRID_CASES
    large ones (128-row kernel)."""
    for c in CASES + BIAS_CASES:
        assert not _standard_grid(c[0], c[1], c[3]), c
    for c in GRID_CASES:
        assert _standard_grid(c[0], c[1], c[3]), c


@pytest.mark.parametrize("case", GRID_CASES, ids=[f"g{i}" for i in range(len(GRID_CASES))])
def test_fp32_mfma_standard_grid(case):
    """The 128-row fp32 kernel (grids of 64 workgroups or more) on the options
    the small-grid cases above give the key-split kernel."""
    b, hq, hkv, tq, tk, dh, dv, causal, off, bias, mf, w = case
    print("case", case, flush=True)
    wl = inputs.make_random(b, hq, hkv, tq, tk, dh, dv, dtype=torch.float32,
                            seed=zlib.crc32(repr(case).encode()) % 10_000, causal=causal, q_offset=off,
                            bias=bias, masked_frac=mf)
    q, k, v, m = to_dev(wl)
    o, lse, n = attn.attn_fwd(q, k, v, scale=wl.scale, causal=causal, q_offset=off, bias=m, window=w,
                              return_n_legal=True)
    o2, lse2 = attn.attn_fwd(q, k, v, scale=wl.scale, causal=causal, q_offset=off, bias=m, window=w)
    torch.cuda.synchronize()
    o_ref, l_ref, n_ref = oracle_full(wl, window=w)
    assert_close(o, lse, o_ref, l_ref, torch.float32, what=str(case))
    assert_close(o2, lse2, o_ref, l_ref, torch.float32, what=str(case) + " (no counts)")
    assert np.array_equal(n.cpu().numpy(), n_ref), "n_legal differs"


def test_fp32_split_kernel_strided_output():
    """The key-split kernel (a small grid) writing into an output view whose
    rows are 80 floats apart: matches the oracle and leaves the rest of each
    row untouched."""
    wl = inputs.make_random(1, 2, 1, 100, 300, 64, 64, dtype=torch.float32, seed=43, causal=True,
                            q_offset=150)
    assert not _standard_grid(1, 2, 100)
    q, k, v, _ = to_dev(wl)
    o_ref, l_ref, _ = oracle_full(wl)
    buf = torch.full((1, 2, 100, 80), 7.0, device=dev())
    out = buf[..., :64]
    _, lse = attn.attn_fwd(q, k, v, scale=wl.scale, causal=True, q_offset=150, out=out)
    torch.cuda.synchronize()
    assert_close(out, lse, o_ref, l_ref, torch.float32, what="split kernel, row stride 80")
    assert torch.all(buf[..., 64:] == 7.0), "wrote past the output view"
