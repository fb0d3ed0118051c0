"""GPU parity of unpadded variable-length batches (§33.4 of "Chapter 33
推理计算优化", shape bucketing: padding every sequence to a bucket length b(T)
costs dense attention about E[b(T)^2 - T^2] extra score work).

Packed sequences go through attn_fwd (the MFMA prefill for bf16 with d in
{64, 128}, the generic kernel otherwise); per-batch KV lengths go through
attn_fwd (MFMA prefill, few-row kernel, generic kernel) and
attn_decode_splitkv.  Each case is compared element by element with the
oracle's attention_varlen / attention_kvlens.  At the padded workload's size
the packed result equals the padded path on legal rows, bit-for-bit in the
masked-row flags and n_legal, and a single sequence equals the dense call bit
for bit."""

import zlib

import numpy as np
import pytest
import torch

import oracle
import online_softmax_exact_amd as attn
from online_softmax_exact_amd import inputs
from gpu_util import TOL, assert_close, dev, ensure_built, f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _seed(case):
    return zlib.crc32(repr(case).encode()) % 10_000


def run_packed(q, k, v, m, cu_q, cu_k, *, scale, causal, window=0, max_q=None, q_offset=0):
    d = dev()
    return attn.attn_fwd(q.to(d), k.to(d), v.to(d), scale=scale, causal=causal, q_offset=q_offset,
                         bias=None if m is None else m.to(d), window=window, return_n_legal=True,
                         cu_seqlens_q=cu_q.to(d), cu_seqlens_k=cu_k.to(d), max_seqlen_q=max_q)


PACKED_CASES = [
    # (dtype, Hq, Hkv, L_q per sequence, L_k per sequence, dh, dv, causal, bias, masked_frac,
    #  window, max_seqlen_q)
    (torch.bfloat16, 2, 2, [1, 128, 129, 300, 7], [1, 128, 129, 300, 7], 128, 128, True, "none", 0.0, 0, None),
    (torch.bfloat16, 8, 2, [50, 200, 0, 129], [300, 200, 10, 400], 64, 128, True, "none", 0.0, 0, 200),
    # rows before every key of their sequence (L_q > L_k), an empty key set
    (torch.bfloat16, 4, 4, [100, 40, 1], [30, 40, 0], 128, 64, True, "none", 0.0, 0, 100),
    # max_seqlen_q below the longest sequence: workgroups loop over its tiles
    (torch.bfloat16, 2, 1, [600, 300, 5], [600, 700, 5], 128, 128, True, "none", 0.0, 0, 128),
    (torch.bfloat16, 2, 2, [260, 33], [260, 90], 64, 64, True, "none", 0.0, 0, 0),
    (torch.bfloat16, 4, 2, [130, 257], [500, 257], 128, 128, False, "none", 0.0, 0, 257),
    (torch.bfloat16, 4, 4, [200, 77, 129], [200, 300, 129], 64, 128, True, "packed", 0.1, 0, 200),
    (torch.bfloat16, 4, 2, [300, 64], [300, 100], 128, 128, True, "keys", 0.05, 0, 300),
    (torch.bfloat16, 2, 2, [500, 140], [500, 400], 128, 128, True, "none", 0.0, 100, 500),
    # generic kernel: fp32, odd head sizes, bf16 with d = 96
    (torch.float32, 2, 1, [70, 1, 33], [70, 5, 100], 64, 64, True, "none", 0.0, 0, 70),
    (torch.float32, 4, 2, [20, 50], [90, 50], 40, 24, True, "packed", 0.1, 7, 50),
    (torch.bfloat16, 2, 2, [45, 3], [45, 60], 96, 96, True, "none", 0.0, 0, 45),
]


@pytest.mark.parametrize("case", PACKED_CASES,
                         ids=lambda c: f"{str(c[0])[6:]}-H{c[1]}/{c[2]}-n{len(c[3])}-d{c[5]}/{c[6]}-c{int(c[7])}-{c[8]}-W{c[10]}-mq{c[11]}")
def test_packed_parity(case):
    dt, hq, hkv, lq, lk, dh, dv, causal, bias, frac, w, max_q = case
    print("case:", case, flush=True)
    q, k, v, m, cu_q, cu_k = inputs.make_packed(lq, lk, hq, hkv, dh, dv, dtype=dt, seed=_seed(case),
                                                bias=bias, masked_frac=frac)
    scale = inputs.default_scale(dh)
    o, lse, n = run_packed(q, k, v, m, cu_q, cu_k, scale=scale, causal=causal, window=w, max_q=max_q)
    torch.cuda.synchronize()
    o_ref, l_ref, n_ref = oracle.attention_varlen(f64(q), f64(k), f64(v), cu_q.tolist(), cu_k.tolist(),
                                                  scale=scale, causal=causal, window=w,
                                                  bias=None if m is None else f64(m))
    assert_close(o, lse, o_ref, l_ref, dt, what=str(case))
    assert np.array_equal(n.cpu().numpy(), n_ref), "n_legal differs"


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_packed_rows_outside_sequences_untouched(dtype, d):
    """Rows past the last offset belong to no sequence and are not written;
    offsets outside [0, T] are clamped (here to the same sequences as
    [0, 40, 40, 90] rows and [0, 60, 60, 150] keys)."""
    lq, lk = [40, 0, 50], [60, 0, 90]
    q, k, v, _, cu_q, cu_k = inputs.make_packed(lq, lk, 2, 2, d, d, dtype=dtype, seed=8)
    qx = torch.cat([q, torch.randn(1, 2, 30, d).to(dtype)], dim=2)      # T_q = 120, rows 90.. outside
    raw_q = torch.tensor([-7, 40, 40, 90], dtype=torch.int32)
    raw_k = torch.tensor([-3, 60, 60, 1 << 30], dtype=torch.int32)   # clamps to T_k = 150
    dd = dev()
    out = torch.full((1, 2, 120, d), 7.0, dtype=dtype, device=dd)
    lse = torch.full((1, 2, 120), 123.0, device=dd)
    o, l = attn.attn_fwd(qx.to(dd), k.to(dd), v.to(dd), scale=inputs.default_scale(d), causal=True,
                         out=out, lse=lse, cu_seqlens_q=raw_q.to(dd), cu_seqlens_k=raw_k.to(dd),
                         max_seqlen_q=50)
    torch.cuda.synchronize()
    assert bool((o[:, :, 90:] == 7.0).all()) and bool((l[:, :, 90:] == 123.0).all())
    o_ref, l_ref, _ = oracle.attention_varlen(f64(q), f64(k), f64(v), cu_q.tolist(), cu_k.tolist(),
                                              scale=inputs.default_scale(d), causal=True)
    assert_close(o[:, :, :90], l[:, :, :90], o_ref, l_ref, dtype, what="clamped offsets")


@pytest.mark.parametrize("lq,lk", [(300, 300), (200, 457), (129, 64)])
def test_single_sequence_is_the_dense_call_bitwise(lq, lk):
    """One packed sequence runs the same arithmetic as the dense call with the
    rows at the end of the keys (q_offset = L_k - L_q): identical bits."""
    q, k, v, _, cu_q, cu_k = inputs.make_packed([lq], [lk], 4, 2, 128, 128, seed=lq + lk)
    scale = inputs.default_scale(128)
    o, lse, n = run_packed(q, k, v, None, cu_q, cu_k, scale=scale, causal=True, max_q=lq)
    dd = dev()
    o2, lse2, n2 = attn.attn_fwd(q.to(dd), k.to(dd), v.to(dd), scale=scale, causal=True, q_offset=lk - lq,
                                 return_n_legal=True)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))
    assert torch.equal(n, n2)


def test_packed_equals_padded_workload_size():
    """The padded workload's eight lengths (uniform in [1, 4096]), 16 heads,
    d_h = 64, d_v = 128, causal: packed vs the padded batch with a -inf bias on
    the padded keys.  On every legal row the masked-row flags and n_legal agree
    bit for bit and O agrees within twice the bf16 tolerance; sampled rows of
    the packed result match the oracle (each row computed on its own)."""
    lengths = inputs.varlen_lengths(8, 4096, 1005)
    hq, dh, dv, t = 16, 64, 128, 4096
    print("lengths:", lengths, flush=True)
    q, k, v, _, cu_q, cu_k = inputs.make_packed(lengths, lengths, hq, hq, dh, dv, seed=1005)
    scale = inputs.default_scale(dh)
    o, lse, n = run_packed(q, k, v, None, cu_q, cu_k, scale=scale, causal=True, max_q=max(lengths))
    dd = dev()
    qp = torch.zeros(8, hq, t, dh, dtype=torch.bfloat16, device=dd)
    kp = torch.zeros(8, hq, t, dh, dtype=torch.bfloat16, device=dd)
    vp = torch.zeros(8, hq, t, dv, dtype=torch.bfloat16, device=dd)
    bias = torch.zeros(8, 1, 1, t, device=dd)
    for b, L in enumerate(lengths):
        s0 = int(cu_q[b])
        qp[b, :, :L] = q[0, :, s0:s0 + L].to(dd)
        kp[b, :, :L] = k[0, :, s0:s0 + L].to(dd)
        vp[b, :, :L] = v[0, :, s0:s0 + L].to(dd)
        bias[b, 0, 0, L:] = float("-inf")
    op, lp, npad = attn.attn_fwd(qp, kp, vp, scale=scale, causal=True, bias=bias, return_n_legal=True)
    torch.cuda.synchronize()
    worst = 0.0
    for b, L in enumerate(lengths):
        s0 = int(cu_q[b])
        a_l, p_l = lse[0, :, s0:s0 + L].cpu(), lp[b, :, :L].cpu()
        assert torch.equal(torch.isneginf(a_l), torch.isneginf(p_l)), f"flags differ, sequence {b}"
        assert torch.equal(n[0, :, s0:s0 + L].cpu(), npad[b, :, :L].cpu()), f"n_legal differs, sequence {b}"
        assert torch.equal(n[0, 0, s0:s0 + L].cpu(), torch.arange(1, L + 1, dtype=torch.int32))
        diff = (o[0, :, s0:s0 + L].float() - op[b, :, :L].float()).abs()
        worst = max(worst, float(diff.max()))
        assert float(diff.max()) <= 2 * TOL[torch.bfloat16]["o_max"]
        assert float(diff.mean()) <= 2 * TOL[torch.bfloat16]["o_mean"]
    print("max |packed - padded|:", worst, flush=True)
    # Sampled rows against the oracle: each sequence's first, last and random rows.
    rng = np.random.default_rng(3)
    got_o, got_l, ref_o, ref_l = [], [], [], []
    for b, L in enumerate(lengths):
        s0 = int(cu_q[b])
        sub = (q[:, :, s0:s0 + L], k[:, :, s0:s0 + L], v[:, :, s0:s0 + L])
        rows = [(0, int(rng.integers(hq)), i) for i in sorted({0, L - 1, int(rng.integers(L))})]
        ro, rl, _ = oracle.attention_rows(*sub, rows, scale=scale, causal=True, q_offset=0)
        ref_o.append(ro); ref_l.append(rl)
        got_o.append(np.stack([f64(o[0, h, s0 + i]) for _, h, i in rows]))
        got_l.append(np.array([float(lse[0, h, s0 + i]) for _, h, i in rows]))
    assert_close(np.concatenate(got_o), np.concatenate(got_l), np.concatenate(ref_o), np.concatenate(ref_l),
                 torch.bfloat16, what="packed sampled rows")


KV_CASES = [
    # (entry, dtype, B, Hq, Hkv, Tq, Tk, dh, dv, causal, lengths, window, bias, split_size)
    ("decode", torch.bfloat16, 6, 32, 8, 1, 5000, 128, 128, True, [5000, 0, 1, 4097, 512, 2500], 0, "none", 512),
    ("decode", torch.bfloat16, 4, 8, 8, 1, 3000, 64, 64, True, [3000, 1500, 7, 0], 600, "none", 256),
    ("decode", torch.bfloat16, 3, 8, 2, 5, 2048, 128, 128, True, [2048, 4, 1000], 0, "none", 300),
    ("decode", torch.float32, 3, 4, 2, 2, 700, 64, 64, True, [700, 1, 300], 0, "none", 128),
    # with a bias (the few-row kernel stages it through LDS)
    ("decode", torch.bfloat16, 3, 8, 2, 2, 3000, 128, 128, True, [3000, 17, 1500], 0, "dense", 512),
    ("decode", torch.bfloat16, 4, 16, 4, 1, 2048, 64, 128, True, [2048, 1, 777, 0], 0, "keys", 256),
    ("fwd", torch.bfloat16, 4, 16, 4, 4, 2000, 128, 128, True, [2000, 3, 1000, 0], 0, "none", None),
    ("fwd", torch.bfloat16, 3, 4, 2, 300, 1000, 128, 128, True, [1000, 300, 100], 0, "none", None),
    ("fwd", torch.bfloat16, 2, 4, 4, 200, 600, 64, 128, True, [600, 250], 0, "dense", None),
    ("fwd", torch.bfloat16, 2, 4, 2, 260, 900, 128, 64, True, [900, 500], 200, "none", None),
    ("fwd", torch.float32, 2, 2, 1, 50, 200, 40, 24, False, [200, 30], 0, "none", None),
]


@pytest.mark.parametrize("case", KV_CASES,
                         ids=lambda c: f"{c[0]}-{str(c[1])[6:]}-B{c[2]}H{c[3]}/{c[4]}-T{c[5]}x{c[6]}-d{c[7]}/{c[8]}-W{c[11]}-{c[12]}")
def test_kvlens_parity(case):
    entry, dt, b, hq, hkv, tq, tk, dh, dv, causal, lens, w, bias, split = case
    print("case:", case, flush=True)
    wl = inputs.make_random(b, hq, hkv, tq, tk, dh, dv, dtype=dt, seed=_seed(case), causal=causal,
                            bias=bias)
    dd = dev()
    lens_t = torch.tensor(lens, dtype=torch.int32, device=dd)
    m = None if wl.bias is None else wl.bias.to(dd)
    if entry == "decode":
        # Workspace pre-filled with NaN bytes: slots of ranges past a batch's
        # length are not written, so the merge must not read them.
        nbytes = attn.attn_decode_workspace_bytes(wl.q, wl.k, wl.v, split_size=split, scale=wl.scale,
                                                  causal=causal, window=w, seqlens_k=lens_t.cpu())
        ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=dd)
        o, lse, _ = attn.attn_decode_splitkv(wl.q.to(dd), wl.k.to(dd), wl.v.to(dd), split_size=split,
                                             scale=wl.scale, causal=causal, window=w, seqlens_k=lens_t,
                                             bias=m, workspace=ws)
        n = None
        o2 = lse2 = None
    else:
        o, lse, n = attn.attn_fwd(wl.q.to(dd), wl.k.to(dd), wl.v.to(dd), scale=wl.scale, causal=causal,
                                  window=w, seqlens_k=lens_t, bias=m, return_n_legal=True)
        # Without counts (the few-row kernel takes few rows per KV head only then).
        o2, lse2 = attn.attn_fwd(wl.q.to(dd), wl.k.to(dd), wl.v.to(dd), scale=wl.scale, causal=causal,
                                 window=w, seqlens_k=lens_t, bias=m)
    torch.cuda.synchronize()
    o_ref, l_ref, n_ref = oracle.attention_kvlens(f64(wl.q), f64(wl.k), f64(wl.v), lens, scale=wl.scale,
                                                  causal=causal, window=w,
                                                  bias=None if wl.bias is None else f64(wl.bias))
    assert_close(o, lse, o_ref, l_ref, dt, what=str(case))
    if n is not None:
        assert np.array_equal(n.cpu().numpy(), n_ref), "n_legal differs"
    if o2 is not None:
        assert_close(o2, lse2, o_ref, l_ref, dt, what=str(case) + " (no counts)")


def test_kvlens_full_lengths_equal_dense_bitwise():
    """Every length = T_k: the same arithmetic as the dense call with
    q_offset = T_k - T_q, for the prefill, few-row and decode kernels."""
    dd = dev()
    for (b, hq, hkv, tq, tk) in ((2, 4, 2, 300, 700), (3, 16, 4, 4, 1500)):
        wl = inputs.make_random(b, hq, hkv, tq, tk, 128, 128, seed=tq)
        q, k, v = wl.q.to(dd), wl.k.to(dd), wl.v.to(dd)
        lens = torch.full((b,), tk, dtype=torch.int32, device=dd)
        o, lse = attn.attn_fwd(q, k, v, scale=wl.scale, causal=True, seqlens_k=lens)
        o2, lse2 = attn.attn_fwd(q, k, v, scale=wl.scale, causal=True, q_offset=tk - tq)
        od, ld, _ = attn.attn_decode_splitkv(q, k, v, split_size=256, scale=wl.scale, seqlens_k=lens)
        od2, ld2, _ = attn.attn_decode_splitkv(q, k, v, split_size=256, scale=wl.scale)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))
        assert torch.equal(od.view(torch.int16), od2.view(torch.int16))
        assert torch.equal(ld.view(torch.int32), ld2.view(torch.int32))


def test_kvlens_decode_full_size_sampled():
    """The cached-decode workload (batch 16, 32 query heads on 8 KV heads,
    T_k = 32768, d = 128, splits of 512) with per-batch lengths uniform in
    [1, 32768]: every batch's rows of four query heads against the oracle
    (each row computed on its own over its batch's keys)."""
    wl = inputs.make_config(3)
    lens = inputs.varlen_lengths(16, 32768, 1003)
    print("lengths:", lens, flush=True)
    dd = dev()
    lens_t = torch.tensor(lens, dtype=torch.int32, device=dd)
    o, lse, _ = attn.attn_decode_splitkv(wl.q.to(dd), wl.k.to(dd), wl.v.to(dd), split_size=512,
                                         scale=wl.scale, seqlens_k=lens_t)
    torch.cuda.synchronize()
    got_o, got_l, ref_o, ref_l = [], [], [], []
    for b, L in enumerate(lens):
        rows = [(0, h, 0) for h in (0, 7, 20, 31)]
        ro, rl, _ = oracle.attention_rows(wl.q[b:b + 1], wl.k[b:b + 1, :, :L], wl.v[b:b + 1, :, :L], rows,
                                          scale=wl.scale, causal=True, q_offset=L - 1)
        ref_o.append(ro); ref_l.append(rl)
        got_o.append(np.stack([f64(o[b, h, 0]) for _, h, _ in rows]))
        got_l.append(np.array([float(lse[b, h, 0]) for _, h, _ in rows]))
    assert_close(np.concatenate(got_o), np.concatenate(got_l), np.concatenate(ref_o), np.concatenate(ref_l),
                 torch.bfloat16, what="decode per-batch lengths")
