"""GPU parity of the bf16 prefill with a bias on the path that stages each
full tile's bias through LDS (calls without legal-key counts, d_h/d_v of
64/128, 64/64 and 128/64).  Each case runs the call with counts too (bias
loaded per block straight into registers): the two must give the same bits,
and both must match the oracle element by element.  Cases: grouped heads,
query rows ending inside a wavefront, several full key tiles with a ragged
tail, causal and not, offsets, biases per head, shared by heads (also over
4 or more batches, whose workgroups run in the XCD-grouped order) and shared
by rows, a strided bias view (rows wider than T_k), -inf entries, a sliding
window (also a three-key window from position 0, so that every row's output
is nearly one value row), and packed sequences with a packed or per-key
bias."""

import zlib

import numpy as np
import pytest
import torch

import oracle
import online_softmax_exact_amd as attn
from online_softmax_exact_amd import inputs
from gpu_util import assert_close, dev, ensure_built, f64, oracle_full, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


CASES = [
    # (B, Hq, Hkv, Tq, Tk, dh, dv, causal, q_offset, bias, masked_frac, window, row_pad)
    (2, 4, 2, 300, 700, 64, 128, True, 0, "shared", 0.1, 0, 0),
    (1, 4, 4, 200, 513, 64, 64, False, 0, "dense", 0.2, 0, 0),
    (2, 2, 1, 257, 400, 128, 64, True, 143, "shared", 0.3, 0, 0),
    (1, 2, 2, 100, 1000, 64, 128, True, 900, "keys", 0.1, 0, 0),
    (1, 2, 2, 190, 333, 64, 128, True, 143, "shared", 0.05, 0, 40),   # bias rows 373 floats apart
    (2, 4, 4, 385, 435, 64, 128, True, 50, "shared", 0.1, 100, 0),
    (2, 4, 4, 385, 435, 64, 128, True, 0, "shared", 0.1, 3, 0),
    (1, 8, 2, 31, 600, 128, 64, False, 0, "dense", 0.0, 0, 0),          # one partial wavefront of rows
    # Head-shared bias over 4 or more batches: workgroups grouped by XCD,
    # 15 (tile, batch) groups (one whole round of 8, the rest in the default
    # order) and 24 (three whole rounds).
    (5, 3, 3, 300, 420, 64, 128, True, 0, "shared", 0.1, 0, 0),
    (4, 2, 1, 700, 700, 64, 128, True, 0, "shared", 0.05, 0, 0),
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{i}" for i in range(len(CASES))])
def test_staged_bias_parity(case):
    b, hq, hkv, tq, tk, dh, dv, causal, off, bias, mf, w, pad = case
    print("case", case, flush=True)
    wl = inputs.make_random(b, hq, hkv, tq, tk, dh, dv, dtype=torch.bfloat16,
                            seed=zlib.crc32(repr(case).encode()) % 10_000, causal=causal, q_offset=off,
                            bias=bias, masked_frac=mf)
    q, k, v, m = to_dev(wl)
    if pad:
        wide = torch.full(m.shape[:-1] + (tk + pad,), 3.0, dtype=torch.float32, device=dev())
        wide[..., :tk] = m
        m = wide[..., :tk]
        assert m.stride(2) == tk + pad
    o, lse = attn.attn_fwd(q, k, v, scale=wl.scale, causal=causal, q_offset=off, bias=m, window=w)
    o_c, lse_c, n = attn.attn_fwd(q, k, v, scale=wl.scale, causal=causal, q_offset=off, bias=m, window=w,
                                  return_n_legal=True)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_c.view(torch.int16)), "staged and per-block bias give other bits"
    assert torch.equal(lse, lse_c), "staged and per-block bias give another LSE"
    o_ref, l_ref, n_ref = oracle_full(wl, window=w)
    assert np.array_equal(n.cpu().numpy(), n_ref), "n_legal differs"
    assert_close(o, lse, o_ref, l_ref, torch.bfloat16, what=str(case))


PADDED_CASES = [
    # (B, Hq, Hkv, Tq, Tk, dh, dv, causal, q_offset)
    (4, 4, 4, 700, 700, 64, 128, True, 0),
    (2, 4, 2, 600, 900, 64, 64, True, 300),
    (3, 2, 2, 500, 800, 128, 64, False, 0),
]


@pytest.mark.parametrize("case", PADDED_CASES, ids=[f"pad{i}" for i in range(len(PADDED_CASES))])
def test_staged_bias_padded_keys(case):
    """Head-shared bias of a padded batch (keys past each sequence's length
    -inf, two rows -inf throughout): full tiles whose staged bias is -inf for
    every row of a wavefront are skipped, which adds exactly nothing, so the
    call gives the bits of the per-block instance (which computes them) and
    matches the oracle."""
    b, hq, hkv, tq, tk, dh, dv, causal, off = case
    print("case", case, flush=True)
    seed = zlib.crc32(repr(case).encode()) % 10_000
    wl = inputs.make_random(b, hq, hkv, tq, tk, dh, dv, dtype=torch.bfloat16, seed=seed, causal=causal,
                            q_offset=off)
    wl.bias, lengths, _ = inputs.padded_bias(b, tq, tk, seed)
    assert min(lengths) + 64 < tk   # at least one whole tile of padded keys
    q, k, v, m = to_dev(wl)
    o, lse = attn.attn_fwd(q, k, v, scale=wl.scale, causal=causal, q_offset=off, bias=m)
    o_c, lse_c, n = attn.attn_fwd(q, k, v, scale=wl.scale, causal=causal, q_offset=off, bias=m,
                                  return_n_legal=True)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_c.view(torch.int16)), "skipping dead tiles changed bits"
    assert torch.equal(lse, lse_c), "skipping dead tiles changed the LSE"
    o_ref, l_ref, n_ref = oracle_full(wl)
    assert np.array_equal(n.cpu().numpy(), n_ref), "n_legal differs"
    assert_close(o, lse, o_ref, l_ref, torch.bfloat16, what=str(case))


PACKED_CASES = [
    # (Hq, Hkv, L_q per sequence, L_k per sequence, dh, dv, causal, bias, masked_frac, max_seqlen_q)
    (4, 4, [200, 77, 129, 300], [200, 300, 129, 500], 64, 128, True, "packed", 0.1, 300),
    (4, 2, [130, 257], [500, 257], 128, 64, False, "packed", 0.05, 128),   # workgroups loop over tiles
    (2, 2, [300, 64], [300, 100], 64, 64, True, "keys", 0.05, 300),
]


@pytest.mark.parametrize("case", PACKED_CASES, ids=[f"p{i}" for i in range(len(PACKED_CASES))])
def test_staged_bias_packed(case):
    """Packed sequences with a packed (or per-key) bias through the staged
    path, against the per-block path (bitwise) and the oracle."""
    hq, hkv, lq, lk, dh, dv, causal, bias, mf, max_q = case
    print("case", case, flush=True)
    q, k, v, m, cu_q, cu_k = inputs.make_packed(lq, lk, hq, hkv, dh, dv, dtype=torch.bfloat16,
                                                seed=zlib.crc32(repr(case).encode()) % 10_000,
                                                bias=bias, masked_frac=mf)
    d = dev()
    scale = inputs.default_scale(dh)
    kw = dict(scale=scale, causal=causal, bias=m.to(d), cu_seqlens_q=cu_q.to(d), cu_seqlens_k=cu_k.to(d),
              max_seqlen_q=max_q)
    o, lse = attn.attn_fwd(q.to(d), k.to(d), v.to(d), **kw)
    o_c, lse_c, _ = attn.attn_fwd(q.to(d), k.to(d), v.to(d), return_n_legal=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_c.view(torch.int16)), "staged and per-block bias give other bits"
    assert torch.equal(lse, lse_c), "staged and per-block bias give another LSE"
    o_ref, l_ref, _ = oracle.attention_varlen(f64(q), f64(k), f64(v), cu_q.tolist(), cu_k.tolist(),
                                              scale=scale, causal=causal, bias=f64(m))
    assert_close(o, lse, o_ref, l_ref, torch.bfloat16, what=str(case))
