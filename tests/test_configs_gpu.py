"""GPU parity on the five full-size workloads, through the same entry points
and launch configuration the benchmark times.  Every element of every output
is compared with the fp64 oracle (run over the workload's (batch, KV head)
groups on the host's cores), for the call the benchmark times and, where it
takes another kernel instance, for the call that also returns the legal-key
counts, which must match bit for bit."""

import numpy as np
import pytest
import torch

import oracle
import online_softmax_exact_amd as attn
from online_softmax_exact_amd import inputs
from gpu_util import assert_close, assert_close_full, ensure_built, oracle_by_group, oracle_full, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def test_fp32_causal_1x1x128_d64():
    wl = inputs.make_config(1)
    print("workload", wl.name, flush=True)
    q, k, v, _ = to_dev(wl)
    o, lse, n = attn.attn_fwd(q, k, v, scale=wl.scale, causal=True, q_offset=0,
                              return_n_legal=True)
    torch.cuda.synchronize()
    o_ref, l_ref, n_ref = oracle_full(wl)
    assert_close(o, lse, o_ref, l_ref, torch.float32)
    assert np.array_equal(n.cpu().numpy(), n_ref)


def test_causal_prefill_1x32x8192_d128():
    wl = inputs.make_config(2)
    print("workload", wl.name, flush=True)
    q, k, v, _ = to_dev(wl)
    # The benchmarked call (no counts), then the counting instance.
    o2, lse2 = attn.attn_fwd(q, k, v, scale=wl.scale, causal=True, q_offset=0)
    o, lse, n = attn.attn_fwd(q, k, v, scale=wl.scale, causal=True, q_offset=0,
                              return_n_legal=True)
    torch.cuda.synchronize()
    want_n = torch.arange(1, 8193, dtype=torch.int32, device=n.device).expand_as(n)
    assert torch.equal(n, want_n)
    o_ref, l_ref, n_ref = oracle_by_group(wl)
    assert np.array_equal(n.cpu().numpy(), n_ref)
    assert_close_full(o2, lse2, o_ref, l_ref, torch.bfloat16, what="prefill (timed call)")
    assert_close_full(o, lse, o_ref, l_ref, torch.bfloat16, what="prefill (with counts)")


def test_gqa_decode_16x32x8_tk32768_split512():
    wl = inputs.make_config(3)
    print("workload", wl.name, flush=True)
    q, k, v, _ = to_dev(wl)
    o, lse, ws = attn.attn_decode_splitkv(q, k, v, split_size=wl.split_size, scale=wl.scale,
                                          causal=True, q_offset=wl.q_offset)
    torch.cuda.synchronize()
    o_ref, l_ref, _ = oracle_by_group(wl)
    assert_close_full(o, lse, o_ref, l_ref, torch.bfloat16, what="decode")
    # Every partial of the workspace: split s of row (b, h) is the exact
    # attention over keys [512 s, 512 s + 512).
    o_parts, l_parts = attn.split_workspace_views(ws, q, v, wl.split_size)
    po_ref, pl_ref = oracle_by_group(wl, fn=oracle.split_partials, split_size=wl.split_size)
    assert po_ref.shape == tuple(o_parts.shape) and pl_ref.shape == tuple(l_parts.shape)
    # [B, H, T_q, S, d] -> one "row" per split for the comparator.
    assert_close_full(o_parts.reshape(16, 32, 64, 128), l_parts.reshape(16, 32, 64),
                      po_ref.reshape(16, 32, 64, 128), pl_ref.reshape(16, 32, 64),
                      torch.bfloat16, what="decode partials")


def test_verify_32x32_tq5_tk4096():
    wl = inputs.make_config(4)
    print("workload", wl.name, flush=True)
    q, k, v, _ = to_dev(wl)
    # The benchmarked call (no counts) takes the few-row kernel; the counting
    # call the MFMA prefill kernel.
    o2, lse2 = attn.attn_fwd(q, k, v, scale=wl.scale, causal=True, q_offset=wl.q_offset)
    o, lse, n = attn.attn_fwd(q, k, v, scale=wl.scale, causal=True, q_offset=wl.q_offset,
                              return_n_legal=True)
    torch.cuda.synchronize()
    want_n = torch.arange(4092, 4097, dtype=torch.int32, device=n.device).expand_as(n)
    assert torch.equal(n, want_n)
    o_ref, l_ref, n_ref = oracle_by_group(wl)
    assert np.array_equal(n.cpu().numpy(), n_ref)
    assert_close_full(o2, lse2, o_ref, l_ref, torch.bfloat16, what="verify (timed call)")
    assert_close_full(o, lse, o_ref, l_ref, torch.bfloat16, what="verify (with counts)")


def test_padded_varlen_bias_8x16x4096_d64x128():
    wl = inputs.make_config(5)
    print("workload", wl.name, "lengths", wl.extras["lengths"], flush=True)
    q, k, v, m = to_dev(wl)
    # The benchmarked call (no counts: full tiles stage the bias through
    # LDS), then the counting instance.
    o2, lse2 = attn.attn_fwd(q, k, v, scale=wl.scale, causal=True, q_offset=0, bias=m)
    o, lse, n = attn.attn_fwd(q, k, v, scale=wl.scale, causal=True, q_offset=0, bias=m,
                              return_n_legal=True)
    torch.cuda.synchronize()
    # Exactly the two seeded rows per sequence are masked: +0.0 and -inf.
    dead = torch.isneginf(lse2).cpu()
    assert int(dead.sum()) == 8 * 2 * 16
    for b, rows in enumerate(wl.extras["masked_rows"]):
        for r in rows:
            assert bool(dead[b, :, r].all())
            assert bool((o2[b, :, r].view(torch.int16) == 0).all())
    o_ref, l_ref, n_ref = oracle_by_group(wl)
    # Exact legal-key counts for every row.
    assert np.array_equal(n.cpu().numpy(), n_ref)
    assert_close_full(o2, lse2, o_ref, l_ref, torch.bfloat16, what="padded bias (timed call)")
    assert_close_full(o, lse, o_ref, l_ref, torch.bfloat16, what="padded bias (with counts)")
    # Both instances run the same arithmetic: the same bits.
    assert torch.equal(o2.view(torch.int16), o.view(torch.int16)), "O without counts differs"
    assert torch.equal(lse2, lse), "LSE without counts differs"
