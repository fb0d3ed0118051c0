"""GPU parity on small seeded problems: the HIP path (through the C ABI)
against the fp64 oracle, element by element, at sizes that span several key
and query tiles plus a ragged tail, with the pages' edge cases."""

import math
import zlib

import numpy as np
import pytest
import torch

import oracle
import online_softmax_exact_amd as attn
from online_softmax_exact_amd import inputs
from gpu_util import assert_close, dev, ensure_built, f64, oracle_full, to_dev, visible_splits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _print_case(**kw):
    print("case:", kw, flush=True)


FWD_CASES = [
    # (dtype, B, Hq, Hkv, Tq, Tk, dh, dv, causal, offset, bias, masked_frac)
    (torch.float32, 1, 1, 1, 128, 128, 64, 64, True, 0, "none", 0.0),
    (torch.float32, 2, 4, 2, 70, 201, 64, 128, True, 131, "dense", 0.1),
    (torch.bfloat16, 1, 2, 2, 300, 300, 128, 128, True, 0, "none", 0.0),
    (torch.bfloat16, 2, 8, 2, 200, 333, 128, 128, True, 133, "none", 0.0),
    (torch.bfloat16, 1, 8, 1, 5, 517, 128, 128, True, 512, "none", 0.0),
    (torch.bfloat16, 2, 4, 4, 257, 257, 64, 128, True, 0, "shared", 0.05),
    (torch.bfloat16, 2, 4, 4, 190, 190, 64, 64, False, 0, "keys", 0.2),
    (torch.bfloat16, 1, 4, 2, 129, 300, 128, 64, True, -40, "rows", 0.3),
    (torch.bfloat16, 1, 2, 1, 64, 100, 128, 128, True, 10_000, "none", 0.0),
    (torch.bfloat16, 1, 3, 3, 33, 47, 40, 24, True, 14, "dense", 0.5),
    (torch.bfloat16, 3, 16, 2, 17, 1000, 128, 128, True, 983, "none", 0.0),
    # few query rows per KV head (H_q/H_kv * T_q <= 32)
    (torch.bfloat16, 2, 8, 2, 4, 300, 128, 128, True, 296, "none", 0.0),
    (torch.bfloat16, 1, 32, 1, 1, 1000, 64, 64, True, 999, "none", 0.0),
    (torch.bfloat16, 2, 4, 4, 3, 200, 128, 64, True, -1, "none", 0.0),
    (torch.bfloat16, 2, 2, 2, 7, 70, 64, 128, False, 0, "none", 0.0),
    # few rows with a bias (the call without n_legal takes the few-row kernel)
    (torch.bfloat16, 2, 8, 2, 4, 300, 128, 128, True, 296, "keys", 0.1),
    (torch.bfloat16, 1, 16, 4, 2, 516, 64, 64, True, 514, "dense", 0.2),
    (torch.bfloat16, 2, 4, 4, 3, 200, 128, 64, False, 0, "shared", 0.3),
]


@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: f"{str(c[0])[6:]}-B{c[1]}H{c[2]}/{c[3]}-T{c[4]}x{c[5]}-d{c[6]}/{c[7]}-c{int(c[8])}-off{c[9]}-{c[10]}")
def test_fwd_parity(case):
    dt, b, hq, hkv, tq, tk, dh, dv, causal, off, bias, frac = case
    _print_case(case=case)
    wl = inputs.make_random(b, hq, hkv, tq, tk, dh, dv, dtype=dt, seed=zlib.crc32(repr(case).encode()) % 10_000,
                            causal=causal, q_offset=off, bias=bias, masked_frac=frac)
    q, k, v, m = to_dev(wl)
    o, lse, n = attn.attn_fwd(q, k, v, scale=wl.scale, causal=causal, q_offset=off, bias=m,
                              return_n_legal=True)
    torch.cuda.synchronize()
    # Without the legal-key counts the entry point may take another kernel.
    o2, lse2 = attn.attn_fwd(q, k, v, scale=wl.scale, causal=causal, q_offset=off, bias=m)
    torch.cuda.synchronize()
    o_ref, l_ref, n_ref = oracle_full(wl)
    assert_close(o, lse, o_ref, l_ref, dt, what=str(case))
    assert_close(o2, lse2, o_ref, l_ref, dt, what=str(case) + " (no counts)")
    assert np.array_equal(n.cpu().numpy(), n_ref), "n_legal differs"


def test_masked_rows_bit_exact_and_empty_keys():
    wl = inputs.make_random(1, 2, 2, 9, 40, 64, 64, seed=11, bias="dense", q_offset=31)
    wl.bias[0, 1, 4, :] = float("-inf")
    wl.bias[0, 0, :, 16:32] = float("-inf")   # a masked block inside every row
    q, k, v, m = to_dev(wl)
    o, lse, n = attn.attn_fwd(q, k, v, scale=wl.scale, causal=True, q_offset=31, bias=m,
                              return_n_legal=True)
    torch.cuda.synchronize()
    o_ref, l_ref, n_ref = oracle_full(wl)
    assert_close(o, lse, o_ref, l_ref, torch.bfloat16)
    assert torch.equal(o[0, 1, 4].view(torch.int16).cpu(), torch.zeros(64, dtype=torch.int16))
    assert lse[0, 1, 4].item() == -math.inf and n[0, 1, 4].item() == 0
    # T_k = 0: every row is masked.
    o2, l2 = attn.attn_fwd(q, k[:, :, :0], v[:, :, :0], scale=wl.scale, causal=True)
    torch.cuda.synchronize()
    assert torch.all(o2.view(torch.int16) == 0) and torch.all(torch.isneginf(l2))
    # T_q = 0: nothing to do.
    o3, l3 = attn.attn_fwd(q[:, :, :0], k, v, scale=wl.scale)
    assert o3.numel() == 0 and l3.numel() == 0


def _pinned_example(dtype):
    """Example 25.1 of §33.2 embedded in d_h = 64: q = 0 so z_j = M_j =
    (ln 2, ln 1, ln 6); value column 0 = (1, 4, 5), other columns 0."""
    d = dev()
    q = torch.zeros(1, 1, 1, 64, dtype=dtype, device=d)
    k = torch.randn(1, 1, 3, 64, generator=torch.Generator().manual_seed(3)).to(dtype).to(d)
    v = torch.zeros(1, 1, 3, 64, dtype=dtype)
    v[0, 0, :, 0] = torch.tensor([1.0, 4.0, 5.0])
    bias = torch.tensor([math.log(2), 0.0, math.log(6)], dtype=torch.float32).view(1, 1, 1, 3)
    return q, k, v.to(d), bias.to(d)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_example_25_1_on_gpu(dtype):
    q, k, v, bias = _pinned_example(dtype)
    o, lse = attn.attn_fwd(q, k, v, scale=0.125, causal=False, bias=bias)
    od, ld, ws = attn.attn_decode_splitkv(q, k, v, split_size=2, scale=0.125, causal=False,
                                          q_offset=0, bias=bias)
    torch.cuda.synchronize()
    for oo, ll in ((o, lse), (od, ld)):
        assert abs(oo[0, 0, 0, 0].item() - 4.0) <= 2e-6 * 4
        assert torch.all(oo[0, 0, 0, 1:] == 0)
        assert abs(ll.item() - math.log(9)) <= 2e-6
    o_parts, l_parts = attn.split_workspace_views(ws, q, v, 2)
    assert abs(o_parts[0, 0, 0, 0, 0].item() - 2.0) <= 2e-6 * 2
    assert abs(o_parts[0, 0, 0, 1, 0].item() - 5.0) <= 2e-6 * 5
    assert abs(l_parts[0, 0, 0, 0].item() - math.log(3)) <= 2e-6
    assert abs(l_parts[0, 0, 0, 1].item() - math.log(6)) <= 2e-6
    # The naive answers 7 (sum) and 3.5 (mean of local outputs) do not come out.
    assert abs(o[0, 0, 0, 0].item() - 7.0) > 1 and abs(o[0, 0, 0, 0].item() - 3.5) > 0.25


def test_merge_states_kernel():
    d = dev()
    # Exercise 33.2 of the workbook: masses 1 and 3, values 0 and 4 -> 3.
    o_s = torch.tensor([[[0.0], [4.0]]], device=d)
    l_s = torch.tensor([[0.0, math.log(3)]], device=d)
    om, lm = attn.attn_merge_states(o_s, l_s)
    torch.cuda.synchronize()
    assert abs(om.item() - 3.0) <= 1e-6 * 3 and abs(lm.item() - math.log(4)) <= 1e-6
    # Random partials with empty states, including a row with none valid.
    g = torch.Generator().manual_seed(21)
    rows, states, dv = 37, 70, 96
    o_parts = torch.randn(rows, states, dv, generator=g, dtype=torch.float64)
    l_parts = torch.randn(rows, states, generator=g, dtype=torch.float64) * 4
    l_parts[torch.rand(rows, states, generator=g) < 0.3] = -math.inf
    l_parts[5] = -math.inf
    want_o, want_l = oracle.merge_partials(o_parts.numpy(), l_parts.numpy())
    for out_dtype, tol in ((torch.float32, 1e-5), (torch.bfloat16, 1e-2)):
        om, lm = attn.attn_merge_states(o_parts.float().to(d), l_parts.float().to(d),
                                        out_dtype=out_dtype)
        torch.cuda.synchronize()
        og = f64(om)
        assert np.array_equal(np.isneginf(f64(lm)), np.isneginf(want_l))
        assert np.all(og[5] == 0)
        assert np.abs(og - want_o).max() <= tol
        fin = np.isfinite(want_l)
        assert np.abs(f64(lm)[fin] - want_l[fin]).max() <= 1e-5


DECODE_CASES = [
    # (dtype, B, Hq, Hkv, Tq, Tk, dh, dv, split, offset(None = Tk - Tq), bias)
    (torch.bfloat16, 2, 8, 2, 1, 2000, 128, 128, 512, None, "none"),
    (torch.bfloat16, 2, 4, 4, 5, 777, 128, 128, 100, None, "none"),
    (torch.bfloat16, 1, 8, 1, 3, 300, 64, 128, 1, None, "none"),
    (torch.bfloat16, 1, 4, 2, 2, 513, 128, 128, 4096, None, "none"),
    (torch.bfloat16, 2, 4, 2, 4, 640, 128, 128, 64, 100, "none"),   # many splits beyond pos
    (torch.bfloat16, 1, 4, 2, 3, 300, 128, 128, 64, -8, "none"),    # no key visible: no split runs
    (torch.float32, 1, 2, 1, 1, 1000, 64, 64, 96, None, "keys"),
    (torch.bfloat16, 1, 4, 4, 2, 400, 64, 128, 128, None, "dense"),
    (torch.bfloat16, 1, 8, 1, 5, 700, 128, 128, 128, None, "none"),   # 40 rows: 2 row groups
    (torch.bfloat16, 2, 16, 2, 1, 3000, 128, 64, 1000, None, "none"),
    (torch.bfloat16, 1, 2, 1, 2, 5, 64, 64, 3, None, "none"),
    # a bias contiguous along keys with 16-byte aligned rows: the few-row kernel
    (torch.bfloat16, 2, 8, 2, 1, 2000, 128, 128, 512, None, "keys"),
    (torch.bfloat16, 2, 4, 4, 5, 780, 128, 128, 100, None, "dense"),
    (torch.bfloat16, 1, 8, 2, 3, 1024, 64, 128, 256, None, "shared"),
    (torch.bfloat16, 2, 16, 4, 1, 4096, 128, 64, 512, None, "keys"),
    (torch.bfloat16, 1, 4, 2, 2, 301, 64, 64, 64, None, "keys"),      # rows not 16-byte aligned: generic
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: f"{str(c[0])[6:]}-B{c[1]}H{c[2]}/{c[3]}-T{c[4]}x{c[5]}-S{c[8]}-off{c[9]}-{c[10]}")
def test_decode_parity(case):
    dt, b, hq, hkv, tq, tk, dh, dv, split, off, bias = case
    off = tk - tq if off is None else off
    _print_case(case=case)
    wl = inputs.make_random(b, hq, hkv, tq, tk, dh, dv, dtype=dt, seed=zlib.crc32(repr(case).encode()) % 10_000,
                            causal=True, q_offset=off, bias=bias, masked_frac=0.1)
    q, k, v, m = to_dev(wl)
    o, lse, ws = attn.attn_decode_splitkv(q, k, v, split_size=split, scale=wl.scale,
                                          causal=True, q_offset=off, bias=m)
    torch.cuda.synchronize()
    o_ref, l_ref, _ = oracle_full(wl)
    assert_close(o, lse, o_ref, l_ref, dt, what=str(case))
    # The workspace holds the per-split partials of the documented layout.
    op_ref, lp_ref = oracle.split_partials(f64(wl.q), f64(wl.k), f64(wl.v), scale=wl.scale,
                                           causal=True, q_offset=off, split_size=split,
                                           bias=None if wl.bias is None else f64(wl.bias))
    # Ranges past every row's last position are neither written nor merged:
    # the oracle's partials there are all empty.
    o_parts, l_parts = attn.split_workspace_views(ws, q, v, split)
    s0, s1 = visible_splits(tq, tk, off, split)
    assert bool(np.isneginf(lp_ref[..., :s0]).all()) and bool(np.isneginf(lp_ref[..., s1:]).all())
    assert_close(f64(o_parts[..., s0:s1, :]), f64(l_parts[..., s0:s1]), op_ref[..., s0:s1, :],
                 lp_ref[..., s0:s1], torch.float32 if dt == torch.float32 else torch.bfloat16, what="partials")


def test_incremental_equals_full():
    """Row t of a causal prefill equals decode of q_t at offset t over the
    first t + 1 keys (the KV-cache check of "Generation and Caching with the
    Same Model"), on the GPU path."""
    wl = inputs.make_random(1, 4, 2, 96, 96, 128, 128, seed=31)
    q, k, v, _ = to_dev(wl)
    o, lse = attn.attn_fwd(q, k, v, scale=wl.scale, causal=True)
    for t in (0, 1, 63, 64, 95):
        od, ld, _ = attn.attn_decode_splitkv(q[:, :, t:t + 1], k[:, :, :t + 1], v[:, :, :t + 1],
                                             split_size=32, scale=wl.scale, q_offset=t)
        torch.cuda.synchronize()
        assert (od.float() - o[:, :, t:t + 1].float()).abs().max().item() <= 1e-2
        assert (ld - lse[:, :, t:t + 1]).abs().max().item() <= 1e-3


def test_alignment_negative_control():
    """Decode aligned at the newest position equals non-causal attention; the
    wrong alignment (offset 0) sees key 0 only and must differ."""
    wl = inputs.make_random(1, 2, 2, 1, 300, 128, 128, seed=41)
    q, k, v, _ = to_dev(wl)
    o_right, _ = attn.attn_fwd(q, k, v, scale=wl.scale, causal=True, q_offset=299)
    o_full, _ = attn.attn_fwd(q, k, v, scale=wl.scale, causal=False)
    o_wrong, _, n = attn.attn_fwd(q, k, v, scale=wl.scale, causal=True, q_offset=0,
                                  return_n_legal=True)
    torch.cuda.synchronize()
    assert torch.equal(o_right, o_full)
    assert torch.all(n == 1)
    assert torch.equal(o_wrong[:, :, 0], v[:, :, 0])
    assert (o_wrong.float() - o_right.float()).abs().max().item() > 0.1


def test_deterministic():
    wl = inputs.make_random(1, 8, 8, 200, 200, 128, 128, seed=51)
    q, k, v, _ = to_dev(wl)
    o1, l1 = attn.attn_fwd(q, k, v, scale=wl.scale)
    o2, l2 = attn.attn_fwd(q, k, v, scale=wl.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_strided_views():
    """Non-contiguous Q/K/V/O views (a packed [B, T, H, D] buffer) give the
    same result as contiguous copies."""
    g = torch.Generator().manual_seed(61)
    b, t, h, d = 2, 150, 4, 128
    qkv = torch.randn(b, t, 3, h, d, generator=g).to(torch.bfloat16).to(dev())
    q = qkv[:, :, 0].permute(0, 2, 1, 3)
    k = qkv[:, :, 1].permute(0, 2, 1, 3)
    v = qkv[:, :, 2].permute(0, 2, 1, 3)
    out = torch.empty(b, t, h, d, dtype=torch.bfloat16, device=dev()).permute(0, 2, 1, 3)
    o1, l1 = attn.attn_fwd(q, k, v, out=out)
    o2, l2 = attn.attn_fwd(q.contiguous(), k.contiguous(), v.contiguous())
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_bad_arguments_raise():
    wl = inputs.make_random(1, 3, 2, 4, 8, 64, 64, seed=1)
    q, k, v, _ = to_dev(wl)
    with pytest.raises(ValueError):
        attn.attn_fwd(q, k, v)
    k2 = k[:, :1]
    with pytest.raises(ValueError):
        attn.attn_decode_splitkv(q, k2, v[:, :1], split_size=0)
