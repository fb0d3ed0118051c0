"""Benchmark of the hot path on one MI355X.

One step = one causal bf16 prefill (batch 1, 32 heads, T = 8192, d = 128,
through attn_fwd) plus one split-KV GQA decode (batch 16, 32 query heads on 8
KV heads, T_k = 32768, d = 128, 64 splits of 512 keys, through
attn_decode_splitkv: partial kernel + merge kernel).  Inputs are seeded
synthetic tensors, resident in HBM before timing starts.  Each launch is
bracketed by HIP events on the stream it runs on.

Prints one JSON line.  ``value`` is the prefill's algorithmic TFLOP/s
(2 (d_h + d_v) flops per legal query-key pair); the decode's algorithmic
KV GB/s (Q + K + V + O + LSE bytes once) is reported beside it.  After the
timed steps, the same prefill and decode are timed once more with a sliding
window (``--window``, keys j >= pos - W + 1) and reported under
``sliding_window``, the prefill's backward (``attn_bwd``, upstream
gradient N(0,1)) under ``backward``, unpadded variable-length batches
(packed prefill and its backward against the padded batch, decode over
per-batch KV lengths) under ``varlen``, the single-head fp32 problem, the
multi-query verify and the padded batch with its dense bias under
``workloads``, each with its own algorithmic counts, a library GEMM and a
device copy of the same session under ``achievable``, and the unit rates of
the part (HBM stream, exp, LDS reads, MFMA; libattn_probes.so) under
``ceilings``.  ``roofline.traffic``
and ``roofline.counters`` come from the committed rocprofv3 runs
(profiles/traffic.json) and are null when the kernel's sources changed since.
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill attention TFLOP/s + decode KV GB/s, as % of MI355X peak"
PEAK_BF16_TFLOPS = 2516.6     # dense bf16 MFMA, 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBS = 8000.0
PEAK_FP32_TFLOPS = 157.3      # fp32 vector (256 CU x 2.4 GHz x 256 flop/clk)


def prefill_counts(t: int, heads: int, batch: int, d_h: int, d_v: int):
    pairs = batch * heads * t * (t + 1) // 2          # causal, offset 0
    flops = 2 * (d_h + d_v) * pairs
    bytes_ = batch * heads * t * (d_h + d_h + d_v + d_v) * 2 + batch * heads * t * 4
    return pairs, flops, bytes_


def decode_counts(batch, hq, hkv, t_q, t_k, d_h, d_v):
    kv = batch * hkv * t_k * (d_h + d_v) * 2
    qo = batch * hq * t_q * (d_h + d_v) * 2 + batch * hq * t_q * 4
    pairs = batch * hq * t_q * t_k
    return kv + qo, 2 * (d_h + d_v) * pairs


def window_prefill_counts(t: int, heads: int, d_h: int, d_v: int, w: int):
    """Causal prefill with a sliding window of w keys: row i has min(i + 1, w)
    legal keys; each of Q, K, V, O and LSE is moved once."""
    pairs = heads * sum(min(i + 1, w) for i in range(t))
    return 2 * (d_h + d_v) * pairs, heads * t * (2 * d_h + 2 * d_v) * 2 + heads * t * 4


def window_decode_counts(batch, hq, hkv, t_q, w, d_h, d_v):
    """Decode with a sliding window of w keys: only the K/V rows inside the
    window are read (each KV head once)."""
    kv = batch * hkv * w * (d_h + d_v) * 2
    qo = batch * hq * t_q * (d_h + d_v) * 2 + batch * hq * t_q * 4
    return kv + qo, 2 * (d_h + d_v) * batch * hq * t_q * w


def varlen_counts(lengths, heads: int, d_h: int, d_v: int):
    """Packed causal prefill with every sequence's rows at its own keys
    (L_q = L_k = L): sum L (L + 1) / 2 legal pairs per head; Q, K, V, O and
    LSE of the packed tokens are moved once."""
    pairs = heads * sum(n * (n + 1) // 2 for n in lengths)
    tokens = sum(lengths)
    return 2 * (d_h + d_v) * pairs, heads * tokens * (2 * d_h + 2 * d_v) * 2 + heads * tokens * 4


def kvlens_decode_bytes(lengths, hq, hkv, t_q, d_h, d_v):
    """Decode over per-batch KV lengths: each batch's first L_b K/V rows of
    every KV head read once, plus Q, O and LSE."""
    kv = hkv * sum(lengths) * (d_h + d_v) * 2
    return kv + len(lengths) * hq * t_q * ((d_h + d_v) * 2 + 4)


def varlen_section(torch, attn, inputs, dev, dk, dv_, dq, dec, ws, timed):
    """Unpadded variable-length batches: the padded workload's eight lengths
    (uniform in [1, 4096]) packed, against the same sequences padded to 4096
    with a -inf bias on the padded keys; and the cached decode with per-batch
    KV lengths uniform in [1, 32768]."""
    lengths = inputs.varlen_lengths(8, 4096, 1005)
    hq, d_h, d_v, t = 16, 64, 128, 4096
    q, k, v, _, cu_q, cu_k = inputs.make_packed(lengths, lengths, hq, hq, d_h, d_v, seed=1005)
    q, k, v, cu_q, cu_k = (x.to(dev) for x in (q, k, v, cu_q, cu_k))
    o = torch.empty(1, hq, q.shape[2], d_v, dtype=q.dtype, device=dev)
    lse = torch.empty(1, hq, q.shape[2], device=dev)
    scale = inputs.default_scale(d_h)
    packed_ms = timed(lambda: attn.attn_fwd(q, k, v, scale=scale, causal=True, out=o, lse=lse,
                                            cu_seqlens_q=cu_q, cu_seqlens_k=cu_k,
                                            max_seqlen_q=max(lengths)))
    qp = torch.zeros(8, hq, t, d_h, dtype=q.dtype, device=dev)
    kp = torch.zeros_like(qp)
    vp = torch.zeros(8, hq, t, d_v, dtype=q.dtype, device=dev)
    bias = torch.zeros(8, 1, 1, t, device=dev)
    for b, n in enumerate(lengths):
        s0 = int(cu_q[b])
        qp[b, :, :n], kp[b, :, :n], vp[b, :, :n] = q[0, :, s0:s0 + n], k[0, :, s0:s0 + n], v[0, :, s0:s0 + n]
        bias[b, 0, 0, n:] = float("-inf")
    op = torch.empty(8, hq, t, d_v, dtype=q.dtype, device=dev)
    lp = torch.empty(8, hq, t, device=dev)
    padded_ms = timed(lambda: attn.attn_fwd(qp, kp, vp, scale=scale, causal=True, bias=bias, out=op, lse=lp))
    flops, bytes_ = varlen_counts(lengths, hq, d_h, d_v)
    pt = flops / (packed_ms * 1e-3) / 1e12

    # Backward of the same packed batch, against the padded batch's backward
    # (causal masking alone keeps real rows off padded keys, and a zero
    # upstream gradient on padded rows adds nothing to real keys).
    g = torch.randn(o.shape, generator=torch.Generator().manual_seed(1006)).to(q.dtype).to(dev)
    gq, gk, gv = torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v)
    wsb = torch.empty(hq * q.shape[2] * 4 + 256, dtype=torch.uint8, device=dev)
    pbwd_ms = timed(lambda: attn.attn_bwd(q, k, v, o, lse, g, scale=scale, causal=True, cu_seqlens_q=cu_q,
                                          cu_seqlens_k=cu_k, max_seqlen_q=max(lengths), d_q=gq, d_k=gk, d_v=gv,
                                          workspace=wsb))
    attn.attn_fwd(qp, kp, vp, scale=scale, causal=True, out=op, lse=lp)
    gp = torch.zeros_like(op)
    for b, n in enumerate(lengths):
        s0 = int(cu_q[b])
        gp[b, :, :n] = g[0, :, s0:s0 + n]
    gqp, gkp, gvp = torch.empty_like(qp), torch.empty_like(kp), torch.empty_like(vp)
    wsp = torch.empty(8 * hq * t * 4, dtype=torch.uint8, device=dev)
    padbwd_ms = timed(lambda: attn.attn_bwd(qp, kp, vp, op, lp, gp, scale=scale, causal=True, d_q=gqp, d_k=gkp,
                                            d_v=gvp, workspace=wsp))
    b_flops = flops // (2 * (d_h + d_v)) * 2 * (3 * d_h + 2 * d_v)
    bt = b_flops / (pbwd_ms * 1e-3) / 1e12
    del qp, kp, vp, op, lp, gp, gqp, gkp, gvp

    kv_lens = inputs.varlen_lengths(16, 32768, 1003)
    lens_t = torch.tensor(kv_lens, dtype=torch.int32, device=dev)
    od = torch.empty(dq.shape[:3] + (dv_.shape[3],), dtype=dq.dtype, device=dev)
    ld = torch.empty(dq.shape[:3], device=dev)
    dec_ms = timed(lambda: attn.attn_decode_splitkv(dq, dk, dv_, split_size=dec.split_size, scale=dec.scale,
                                                    causal=True, seqlens_k=lens_t, workspace=ws, out=od,
                                                    lse=ld))
    d_bytes = kvlens_decode_bytes(kv_lens, 32, 8, 1, 128, 128)
    dg = d_bytes / (dec_ms * 1e-3) / 1e9
    return {
        "prefill": {"workload": f"packed causal prefill, 8 sequences of lengths {lengths}, H=16, "
                                "d_h=64, d_v=128 (attn_fwd with cu_seqlens)",
                    "ms": round(packed_ms, 4), "value": round(pt, 2), "unit": "TFLOP/s",
                    "padded_ms": round(padded_ms, 4),
                    "padded": "the same sequences padded to 4096 with a -inf bias on padded keys",
                    "speedup_vs_padded": round(padded_ms / packed_ms, 3),
                    "roofline": {"bound": "mfma", "achieved": round(pt, 2), "peak": PEAK_BF16_TFLOPS,
                                 "unit": "TFLOP/s", "frac": round(pt / PEAK_BF16_TFLOPS, 4),
                                 "traffic": recorded_traffic("packed_prefill"),
                                 "per_launch_flops": flops, "per_launch_bytes": bytes_}},
        "backward": {"workload": f"backward of the packed causal prefill above (attn_bwd with cu_seqlens: "
                                 "D, dQ, dV, dK kernels)",
                     "ms": round(pbwd_ms, 4), "value": round(bt, 2), "unit": "TFLOP/s",
                     "padded_ms": round(padbwd_ms, 4),
                     "padded": "the same sequences padded to 4096 (B=8), dense causal attn_bwd",
                     "speedup_vs_padded": round(padbwd_ms / pbwd_ms, 3),
                     "roofline": {"bound": "mfma", "achieved": round(bt, 2), "peak": PEAK_BF16_TFLOPS,
                                  "unit": "TFLOP/s", "frac": round(bt / PEAK_BF16_TFLOPS, 4),
                                  "traffic": backward_traffic(packed=True),
                                  "per_launch_flops": b_flops,
                                  "flops_per_pair": "2 (3 d_h + 2 d_v): recomputed scores, dP, dV, dQ, dK"}},
        "decode": {"workload": "GQA split-KV decode B=16 Hq=32 Hkv=8 Tk<=32768 d=128 S=512 with per-batch "
                               f"KV lengths uniform in [1, 32768] (sum {sum(kv_lens)}; attn_decode_splitkv "
                               "with seqlens_k)",
                   "ms": round(dec_ms, 4), "value": round(dg, 1), "unit": "GB/s",
                   "roofline": {"bound": "hbm", "achieved": round(dg, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                "frac": round(dg / PEAK_HBM_GBS, 4),
                                "traffic": recorded_traffic("kvlens_decode_partials"),
                                "per_launch_bytes": d_bytes}},
    }


def padded_counts(lengths, masked_rows, heads: int, t: int, d_h: int, d_v: int):
    """Padded causal batch with a dense bias: row i of sequence b has
    min(i + 1, L_b) legal keys (keys past L_b are padding, masked by the bias)
    unless it is one of the two wholly masked rows.  Bytes: Q, K, V, O, LSE
    once, plus the bias entries in the causally visible region once (the bias
    is shared by the heads)."""
    pairs = 0
    for L, rows in zip(lengths, masked_rows):
        per = sum(min(i + 1, L) for i in range(t)) - sum(min(r + 1, L) for r in rows)
        pairs += heads * per
    b = len(lengths)
    bytes_ = b * heads * t * (2 * d_h + 2 * d_v) * 2 + b * heads * t * 4 + b * t * (t + 1) // 2 * 4
    return 2 * (d_h + d_v) * pairs, bytes_


def workloads_section(torch, attn, inputs, dev, timed):
    """The single-head fp32 problem (128 rows, d = 64: latency bound, timed
    beside a one-element fill kernel as the launch floor), the
    multi-query verify (32 x 32 heads, 5 queries at the end of 4096 keys)
    against HBM and the matrix cores, and the padded variable-length batch with
    its dense bias (8 x 16 heads, T = 4096, d_h = 64, d_v = 128) against both
    ceilings."""
    out = {}
    wl = inputs.make_config(1)
    q, k, v = (t.to(dev) for t in (wl.q, wl.k, wl.v))
    o = torch.empty(q.shape[:3] + (v.shape[3],), dtype=q.dtype, device=dev)
    lse = torch.empty(q.shape[:3], device=dev)
    ms = timed(lambda: attn.attn_fwd(q, k, v, scale=wl.scale, causal=True, out=o, lse=lse))
    one = torch.empty(1, device=dev)
    floor_ms = timed(lambda: one.fill_(0.0))
    fl = 2 * (64 + 64) * (128 * 129 // 2)
    tf = fl / (ms * 1e-3) / 1e12
    out["fp32_single_head"] = {"workload": "fp32 causal B=1 H=1 T=128 d=64 (attn_fwd, fp32 MFMA key-split kernel)",
                               "us": round(ms * 1e3, 2), "launch_floor_us": round(floor_ms * 1e3, 2),
                               "value": round(tf, 4), "unit": "TFLOP/s",
                               "roofline": {"bound": "launch", "achieved": round(tf, 4), "peak": PEAK_FP32_TFLOPS,
                                            "unit": "TFLOP/s", "frac": round(tf / PEAK_FP32_TFLOPS, 6),
                                            "traffic": recorded_traffic("fp32_single_head"), "per_launch_flops": fl,
                                            "note": "2.1 MFLOP per call in four workgroups of 32 rows "
                                                    "whose wavefronts take one 32-key tile each: the time "
                                                    "is the launch plus one tile's dependent MFMA chain "
                                                    "and the merge, not arithmetic"}}
    del q, k, v, o, lse, wl
    wl = inputs.make_config(4)
    q, k, v = (t.to(dev) for t in (wl.q, wl.k, wl.v))
    o = torch.empty(q.shape[:3] + (v.shape[3],), dtype=q.dtype, device=dev)
    lse = torch.empty(q.shape[:3], device=dev)
    ms = timed(lambda: attn.attn_fwd(q, k, v, scale=wl.scale, causal=True, q_offset=wl.q_offset, out=o, lse=lse))
    by, fl = decode_counts(32, 32, 32, 5, 4096, 128, 128)
    gbs = by / (ms * 1e-3) / 1e9
    out["verify"] = {"workload": "multi-query verify B=32 H=32 T_q=5 at positions 4091..4095, T_k=4096, d=128 "
                                 "(attn_fwd)", "ms": round(ms, 4), "value": round(gbs, 1), "unit": "GB/s",
                     "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                  "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": recorded_traffic("verify"),
                                  "per_launch_bytes": by, "per_launch_flops": fl,
                                  "mfma_frac": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 5)}}
    del q, k, v, o, lse, wl
    wl = inputs.make_config(5)
    q, k, v, m = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.bias))
    o = torch.empty(q.shape[:3] + (v.shape[3],), dtype=q.dtype, device=dev)
    lse = torch.empty(q.shape[:3], device=dev)
    ms = timed(lambda: attn.attn_fwd(q, k, v, scale=wl.scale, causal=True, bias=m, out=o, lse=lse))
    fl, by = padded_counts(wl.extras["lengths"], wl.extras["masked_rows"], 16, 4096, 64, 128)
    tf = fl / (ms * 1e-3) / 1e12
    gbs = by / (ms * 1e-3) / 1e9
    out["padded_bias"] = {"workload": "padded variable-length batch B=8 H=16 T=4096 d_h=64 d_v=128, dense fp32 bias "
                                      "[8,1,4096,4096] with -inf padding and 2 masked rows per sequence (attn_fwd)",
                          "ms": round(ms, 4), "value": round(tf, 2), "unit": "TFLOP/s",
                          "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                                       "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                                       "traffic": recorded_traffic("padded_bias"), "counters": recorded_mfma("padded_bias"),
                                       "per_launch_flops": fl, "per_launch_bytes": by,
                                       "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}}
    return out


def achievable_section(torch, dev, timed, p_tflops, d_gbs):
    """Ceilings measured in the same session, as context for the fractions of
    the published peaks: a library bf16 GEMM (torch.matmul, hipBLASLt) for the
    matrix cores under a dense MFMA load, and a 1 GiB device-to-device copy
    (reads and writes 1 GiB each) for HBM."""
    n = 8192
    g = torch.Generator(device="cpu").manual_seed(7)
    a = torch.randn(n, n, generator=g).to(torch.bfloat16).to(dev)
    b = torch.randn(n, n, generator=g).to(torch.bfloat16).to(dev)
    c = torch.empty(n, n, dtype=torch.bfloat16, device=dev)
    mm_ms = timed(lambda: torch.matmul(a, b, out=c))
    mm_t = 2 * n ** 3 / (mm_ms * 1e-3) / 1e12
    del a, b, c
    src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    cp_ms = timed(lambda: dst.copy_(src))
    cp_g = 2 * (1 << 30) / (cp_ms * 1e-3) / 1e9
    del src, dst
    return {"gemm_bf16": {"shape": "8192 x 8192 x 8192 (torch.matmul)", "ms": round(mm_ms, 4),
                          "value": round(mm_t, 1), "unit": "TFLOP/s",
                          "prefill_over_gemm": round(p_tflops / mm_t, 4)},
            "copy": {"bytes": 2 * (1 << 30), "ms": round(cp_ms, 4), "value": round(cp_g, 1), "unit": "GB/s",
                     "decode_over_copy": round(d_gbs / cp_g, 4)}}


def ceilings_section(torch, dev, stream):
    """Unit rates measured on the part itself (libattn_probes.so): an HBM
    streaming read of 2 GiB, the v_exp_f32 rate, the LDS read rate with
    16-byte and with transposed 8-byte reads, and the bf16 MFMA rate of
    independent v_mfma_f32_32x32x16_bf16 chains.  The cost model bounds a
    kernel by its work over the rate of the unit doing it, so these are the
    ceilings its fractions are read against (next to the published peaks)."""
    from online_softmax_exact_amd import _probes

    blocks = 2048                                    # 8 workgroups of 4 waves per CU
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)

    def run(fn, n=10):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a_, b_ in evs:
            a_.record(stream)
            fn()
            b_.record(stream)
        torch.cuda.synchronize()
        ts = sorted(a_.elapsed_time(b_) for a_, b_ in evs)
        return ts[len(ts) // 2] * 1e-3               # seconds, median

    # The streaming read on two workgroups per CU, each striding over the
    # whole buffer: the fastest grid in a sweep of 2, 4, 8 and 16 per CU
    # (about 7.0 TB/s against 5.8-6.0 with 8 per CU).
    blocks_rd = 2 * 256
    src = torch.ones(2 << 30, dtype=torch.uint8, device=dev)
    t_rd = run(lambda: _probes.stream_read(src, out, blocks_rd, stream))
    del src
    iters_exp = 2048
    t_exp = run(lambda: _probes.exp_rate(out, blocks, iters_exp, stream))
    iters_lds = 64
    t_lds = run(lambda: _probes.lds_read(out, blocks, iters_lds, False, stream))
    t_tr = run(lambda: _probes.lds_read(out, blocks, iters_lds, True, stream))
    iters_mfma = 256
    t_mf = run(lambda: _probes.mfma_rate(out, blocks, iters_mfma, stream))
    cus, nominal_ghz = 256, 2.4
    rd = (2 << 30) / t_rd / 1e9
    ex = blocks * 256 * 8 * iters_exp / t_exp
    lds = blocks * 4 * 65536 * iters_lds / t_lds
    ldt = blocks * 4 * 32768 * iters_lds / t_tr
    mf = blocks * 4 * 4 * iters_mfma * 32768 / t_mf / 1e12
    return {
        "hbm_stream_read": {"bytes": 2 << 30, "ms": round(t_rd * 1e3, 4), "value": round(rd, 1), "unit": "GB/s",
                            "frac_of_peak": round(rd / PEAK_HBM_GBS, 4), "workgroups": blocks_rd,
                            "note": "non-temporal 16-byte loads, 4 in flight per thread, grid-stride"},
        "exp_f32": {"value": round(ex / 1e9, 1), "unit": "G exp/s (8 independent chains of exp2 and a multiply)",
                    "per_cu_per_nominal_clock": round(ex / cus / (nominal_ghz * 1e9), 2)},
        "lds_read_b128": {"value": round(lds / 1e12, 2), "unit": "TB/s",
                          "bytes_per_cu_per_nominal_clock": round(lds / cus / (nominal_ghz * 1e9), 1)},
        "lds_read_tr_b64": {"value": round(ldt / 1e12, 2), "unit": "TB/s",
                            "bytes_per_cu_per_nominal_clock": round(ldt / cus / (nominal_ghz * 1e9), 1)},
        "mfma_bf16": {"value": round(mf, 1), "unit": "TFLOP/s", "frac_of_peak": round(mf / PEAK_BF16_TFLOPS, 4),
                      "note": "independent 32x32x16 bf16 MFMA chains, no memory traffic"},
    }


def _recorded(key: str):
    """The committed rocprofv3 record of kernel `key` (profiles/traffic.json),
    or None when the kernel's sources have changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))["kernels"][key]
    except (OSError, KeyError, ValueError):
        return None
    h = hashlib.sha256()
    for f in rec["sources"]:
        with open(os.path.join(ROOT, "online_softmax_exact_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return rec if h.hexdigest() == rec["source_sha256"] else None


def recorded_traffic(key: str):
    """HBM bytes per launch of kernel `key` from the committed byte counters,
    or None when stale."""
    rec = _recorded(key)
    return None if rec is None else int(rec["traffic_bytes"])


def recorded_mfma(key: str):
    """MFMA counters of kernel `key` from the committed profile (MfmaUtil in
    percent, executed over algorithmic bf16 MFMA flops, the clock under the
    counters), or None when stale or not recorded."""
    rec = _recorded(key)
    m = None if rec is None else rec.get("mfma")
    if not m:
        return None
    alg = m.get("algorithmic_flops")
    return {"mfma_util_pct": round(m["util_pct"], 1), "clock_ghz": round(m["clock_ghz"], 2),
            "executed_over_algorithmic": round(m["executed_flops"] / alg, 4) if alg else None}


def backward_traffic(packed: bool = False):
    """HBM bytes of one attn_bwd call: its kernels' recorded traffic, or None
    if any is stale: the dQ kernel (which also computes D) and the fused
    dK/dV kernel, for dense batches and packed sequences alike."""
    keys = ("packed_bwd_dq", "packed_bwd_kvf") if packed else ("bwd_dq", "bwd_kvf")
    parts = [recorded_traffic(k) for k in keys]
    return None if None in parts else sum(parts)


def cpu_baseline(wl, heads: int):
    """The fp64 oracle as it stands, on `heads` heads of the prefill workload:
    one oracle call per head on a thread pool of the CPUs this process may
    run on (numpy releases the GIL in its products and ufuncs), BLAS pinned
    to one thread per worker, and no more workers than the host memory holds
    (each materialises three T x T fp64 matrices)."""
    import concurrent.futures as cf

    import oracle
    from threadpoolctl import threadpool_limits

    t = wl.q.shape[2]
    cpus = len(os.sched_getaffinity(0))
    per_worker = 3 * t * t * 8 + 4 * t * wl.q.shape[3] * 8
    try:
        avail = os.sysconf("SC_AVPHYS_PAGES") * os.sysconf("SC_PAGE_SIZE")
    except (ValueError, OSError):  # pragma: no cover
        avail = per_worker * cpus
    workers = max(1, min(cpus, heads, int(0.5 * avail // per_worker)))

    def one(h):
        with threadpool_limits(limits=1):
            oracle.attention(wl.q[:, h:h + 1].double().numpy(), wl.k[:, h:h + 1].double().numpy(),
                             wl.v[:, h:h + 1].double().numpy(), scale=wl.scale, causal=True, q_offset=0)

    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(one, range(heads)))
    dt = time.perf_counter() - t0
    _, flops, _ = prefill_counts(t, heads, 1, wl.q.shape[3], wl.v.shape[3])
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(workers), "kind": "oracle",
            "sample": f"{heads} of 32 heads of the causal prefill (T=8192, d=128), fp64 numpy, one "
                      f"oracle call per head on {workers} threads ({cpus} CPUs available), "
                      f"{dt:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=60,
                    help="untimed steps at least; warm-up goes on until --warmup-s has passed too")
    ap.add_argument("--warmup-s", type=float, default=1.0,
                    help="seconds of untimed steps at least (the clock ramps over the first ~0.5 s "
                         "of load)")
    ap.add_argument("--cpu-heads", type=int, default=32,
                    help="heads of the prefill the CPU oracle baseline times")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward measurement")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the multi-query verify and padded-bias measurements")
    ap.add_argument("--no-achievable", action="store_true",
                    help="skip the same-session ceilings (library bf16 GEMM, device copy)")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the unit microbenchmarks (HBM stream, exp, LDS, MFMA rates)")
    ap.add_argument("--no-varlen", action="store_true",
                    help="skip the variable-length (packed prefill, per-batch KV length decode) measurement")
    ap.add_argument("--window", type=int, default=4096,
                    help="sliding window of the extra windowed prefill/decode measurement (0: skip)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after timing, run two device copies of this many MiB (a kernel of "
                         "known traffic to scale hardware byte counters against)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import online_softmax_exact_amd as attn
    from online_softmax_exact_amd import _lib, inputs

    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    print("bench: generating inputs", file=sys.stderr, flush=True)
    pre = inputs.make_config(2)
    dec = inputs.make_config(3)
    pq, pk, pv = (t.to(dev) for t in (pre.q, pre.k, pre.v))
    dq, dk, dv_ = (t.to(dev) for t in (dec.q, dec.k, dec.v))
    po = torch.empty_like(pq)
    pl = torch.empty(pq.shape[:3], dtype=torch.float32, device=dev)
    do = torch.empty_like(dq)
    dl = torch.empty(dq.shape[:3], dtype=torch.float32, device=dev)
    ws_bytes = attn.attn_decode_workspace_bytes(dq, dk, dv_, split_size=dec.split_size,
                                                scale=dec.scale, q_offset=dec.q_offset)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    def run_prefill():
        attn.attn_fwd(pq, pk, pv, scale=pre.scale, causal=True, q_offset=0, out=po, lse=pl)

    def run_decode():
        attn.attn_decode_splitkv(dq, dk, dv_, split_size=dec.split_size, scale=dec.scale,
                                 causal=True, q_offset=dec.q_offset, workspace=ws, out=do,
                                 lse=dl)

    print("bench: timing", file=sys.stderr, flush=True)
    # Warm-up: at least --warmup steps and at least --warmup-s seconds, so the
    # timed steps see the steady-state clock (it ramps over the first tens of
    # launches after idle; a few steps alone leave the early ones slow).
    warmed, t_w = 0, time.perf_counter()
    while warmed < args.warmup or time.perf_counter() - t_w < args.warmup_s:
        run_prefill()
        run_decode()
        warmed += 1
        if warmed % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    warm_s = time.perf_counter() - t_w
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t_start = time.perf_counter()
    for e in ev:
        e[0].record(stream)
        run_prefill()
        e[1].record(stream)
        run_decode()
        e[2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    pre_ms = [a.elapsed_time(b) for a, b, _ in ev]
    dec_ms = [b.elapsed_time(c) for _, b, c in ev]
    step_ms = [a.elapsed_time(c) for a, _, c in ev]

    _, p_flops, p_bytes = prefill_counts(8192, 32, 1, 128, 128)
    d_bytes, d_flops = decode_counts(16, 32, 8, 1, 32768, 128, 128)
    p_avg = sum(pre_ms) / len(pre_ms)
    d_avg = sum(dec_ms) / len(dec_ms)
    p_tflops = p_flops / (p_avg * 1e-3) / 1e12
    d_gbs = d_bytes / (d_avg * 1e-3) / 1e9

    out = {
        "metric": METRIC,
        "value": round(p_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sum(step_ms) / len(step_ms), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), resident in HBM)",
        "config": {"workload": "causal prefill B=1 H=32 T=8192 d=128 (attn_fwd) + "
                               "GQA split-KV decode B=16 Hq=32 Hkv=8 Tk=32768 d=128 S=512 "
                               "(attn_decode_splitkv)",
                   "prefill_ms": round(p_avg, 4), "prefill_ms_min": round(min(pre_ms), 4),
                   "prefill_ms_median": round(statistics.median(pre_ms), 4),
                   "decode_ms": round(d_avg, 4), "decode_ms_min": round(min(dec_ms), 4),
                   "decode_ms_median": round(statistics.median(dec_ms), 4),
                   "wall_s": round(wall, 3), "warmup_steps_run": warmed,
                   "warmup_s": round(warm_s, 3)},
        "roofline": {"bound": "mfma", "achieved": round(p_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(p_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic("prefill"), "kernel": "attn_fwd prefill",
                     "counters": recorded_mfma("prefill"),
                     "per_launch_flops": p_flops, "per_launch_bytes": p_bytes},
        "decode": {"value": round(d_gbs, 1), "unit": "GB/s", "ms": round(d_avg, 4),
                   "roofline": {"bound": "hbm", "achieved": round(d_gbs, 1), "peak": PEAK_HBM_GBS,
                                "unit": "GB/s", "frac": round(d_gbs / PEAK_HBM_GBS, 4),
                                "traffic": recorded_traffic("decode_partials"),
                                "per_launch_bytes": d_bytes,
                                "per_launch_flops": d_flops}},
        "cpu_baseline": None,
    }

    def timed(fn, n=20):
        """Average of n launches of fn, HIP events on the stream, after at
        least 10 untimed launches and 0.25 s of them: after the host work
        between sections the clock ramps up over the first tens of launches
        (measured on the packed prefill: 0.376 ms for the first launch, 0.29
        from about the 40th on)."""
        t0, k = time.perf_counter(), 0
        while k < 10 or time.perf_counter() - t0 < 0.25:
            fn()
            k += 1
            if k % 10 == 0:
                torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for a_, b_ in evs:
            a_.record(stream)
            fn()
            b_.record(stream)
        torch.cuda.synchronize()
        return sum(a_.elapsed_time(b_) for a_, b_ in evs) / n

    if not args.no_backward:
        gd = torch.randn(pq.shape, generator=torch.Generator().manual_seed(4242)).to(torch.bfloat16).to(dev)
        run_prefill()                      # o and lse of the forward
        gq, gk, gv = torch.empty_like(pq), torch.empty_like(pk), torch.empty_like(pv)
        ws_b = torch.empty(32 * 8192 * 4, dtype=torch.uint8, device=dev)   # fp32 D per query row

        def run_backward():
            attn.attn_bwd(pq, pk, pv, po, pl, gd, scale=pre.scale, causal=True,
                          d_q=gq, d_k=gk, d_v=gv, workspace=ws_b)

        b_ms = timed(run_backward)
        pairs, _, _ = prefill_counts(8192, 32, 1, 128, 128)
        b_flops = 2 * (3 * 128 + 2 * 128) * pairs
        b_t = b_flops / (b_ms * 1e-3) / 1e12
        out["backward"] = {
            "workload": "causal backward B=1 H=32 T=8192 d=128 (attn_bwd: a dQ kernel that also forms D, then one fused dK/dV kernel)",
            "ms": round(b_ms, 4), "value": round(b_t, 2), "unit": "TFLOP/s",
            "roofline": {"bound": "mfma", "achieved": round(b_t, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(b_t / PEAK_BF16_TFLOPS, 4),
                         "traffic": backward_traffic(),
                         "per_launch_flops": b_flops,
                         "flops_per_pair": "2 (3 d_h + 2 d_v): recomputed scores, dP, dV, dQ, dK"}}

    if args.window > 0:
        w = args.window
        ww = torch.empty(attn.attn_decode_workspace_bytes(dq, dk, dv_, split_size=dec.split_size,
                                                          scale=dec.scale, q_offset=dec.q_offset,
                                                          window=w), dtype=torch.uint8, device=dev)

        wp_ms = timed(lambda: attn.attn_fwd(pq, pk, pv, scale=pre.scale, causal=True, window=w,
                                            out=po, lse=pl))
        wd_ms = timed(lambda: attn.attn_decode_splitkv(dq, dk, dv_, split_size=dec.split_size,
                                                       scale=dec.scale, causal=True,
                                                       q_offset=dec.q_offset, window=w,
                                                       workspace=ww, out=do, lse=dl))
        wp_flops, wp_bytes = window_prefill_counts(8192, 32, 128, 128, w)
        wd_bytes, wd_flops = window_decode_counts(16, 32, 8, 1, w, 128, 128)
        wp_t = wp_flops / (wp_ms * 1e-3) / 1e12
        wd_g = wd_bytes / (wd_ms * 1e-3) / 1e9
        out["sliding_window"] = {
            "window": w,
            "prefill": {"workload": f"causal prefill B=1 H=32 T=8192 d=128, window {w} (attn_fwd)",
                        "ms": round(wp_ms, 4), "value": round(wp_t, 2), "unit": "TFLOP/s",
                        "roofline": {"bound": "mfma", "achieved": round(wp_t, 2),
                                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                     "frac": round(wp_t / PEAK_BF16_TFLOPS, 4), "traffic": None,
                                     "per_launch_flops": wp_flops, "per_launch_bytes": wp_bytes}},
            "decode": {"workload": f"GQA split-KV decode B=16 Hq=32 Hkv=8 Tk=32768 d=128 S=512, "
                                   f"window {w} (attn_decode_splitkv)",
                       "ms": round(wd_ms, 4), "value": round(wd_g, 1), "unit": "GB/s",
                       "roofline": {"bound": "hbm", "achieved": round(wd_g, 1), "peak": PEAK_HBM_GBS,
                                    "unit": "GB/s", "frac": round(wd_g / PEAK_HBM_GBS, 4),
                                    "traffic": None, "per_launch_bytes": wd_bytes,
                                    "per_launch_flops": wd_flops}},
        }
    if not args.no_varlen:
        print("bench: variable-length batches", file=sys.stderr, flush=True)
        out["varlen"] = varlen_section(torch, attn, inputs, dev, dk, dv_, dq, dec, ws, timed)
    if not args.no_workloads:
        print("bench: verify and padded-bias workloads", file=sys.stderr, flush=True)
        out["workloads"] = workloads_section(torch, attn, inputs, dev, timed)
    if not args.no_achievable:
        print("bench: achievable ceilings", file=sys.stderr, flush=True)
        out["achievable"] = achievable_section(torch, dev, timed, p_tflops, d_gbs)
    if not args.no_ceilings:
        print("bench: unit microbenchmarks", file=sys.stderr, flush=True)
        out["ceilings"] = ceilings_section(torch, dev, stream)
    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        print("bench: CPU oracle baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(pre, args.cpu_heads)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
