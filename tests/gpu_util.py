"""Helpers for the GPU parity tests: run the HIP path through the C ABI on
seeded inputs and compare with the fp64 oracle element by element."""

import os

import numpy as np
import torch

import oracle
from online_softmax_exact_amd import _lib

# Tolerances on O (absolute) and LSE (absolute, natural log).
TOL = {torch.bfloat16: dict(o_max=1e-2, o_mean=1e-3, lse=1e-3),
       torch.float32: dict(o_max=1e-5, o_mean=1e-6, lse=1e-5)}


def ensure_built():
    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()


def dev():
    return torch.device("cuda:0")


def f64(t):
    return t.detach().cpu().to(torch.float64).numpy()


def oracle_full(wl, key_range=None, window=0):
    return oracle.attention(f64(wl.q), f64(wl.k), f64(wl.v), scale=wl.scale, causal=wl.causal,
                            q_offset=wl.q_offset,
                            bias=None if wl.bias is None else f64(wl.bias),
                            key_range=key_range, window=window)


def to_dev(wl):
    d = dev()
    return (wl.q.to(d), wl.k.to(d), wl.v.to(d), None if wl.bias is None else wl.bias.to(d))


def rounding_floor(o_ref, dtype):
    """|round(o) - o| for the exact result o rounded to the output dtype
    (round to nearest even, through fp32 as a kernel's fp32 result is): the
    error of a perfectly computed output.  bf16 numbers in [4, 8) are 2^-5
    apart, so there it reaches 0.0156."""
    if dtype != torch.bfloat16:
        return np.zeros_like(o_ref)
    return np.abs(torch.from_numpy(o_ref).to(torch.bfloat16).to(torch.float64).numpy() - o_ref)


def o_max_allowed(o_ref, dtype):
    """Per-element bound on |dO|: the tolerance, or, on an element whose exact
    value is itself farther than the tolerance from every number of the
    output dtype, that rounding plus the mean tolerance."""
    tol = TOL[dtype]
    return np.maximum(tol["o_max"], rounding_floor(o_ref, dtype) + tol["o_mean"])


def assert_close(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what=""):
    """Element-wise parity; masked rows (oracle LSE = -inf) must be bit-exact
    (+0.0 output, -inf LSE) and no NaN may appear anywhere.  |dO| is held to
    the tolerance except where the exact value's own rounding to the output
    dtype already exceeds it (``o_max_allowed``)."""
    tol = TOL[dtype]
    og = o_gpu if isinstance(o_gpu, np.ndarray) else f64(o_gpu)
    lg = lse_gpu if isinstance(lse_gpu, np.ndarray) else f64(lse_gpu)
    assert og.shape == o_ref.shape, (og.shape, o_ref.shape)
    assert not np.isnan(og).any() and not np.isnan(lg).any(), f"{what}: NaN in output"
    dead = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lg), dead), f"{what}: masked-row flags differ"
    if dead.any():
        raw = o_gpu if isinstance(o_gpu, np.ndarray) else o_gpu.detach().cpu()
        if isinstance(raw, torch.Tensor):
            bits = raw.view(torch.int16) if raw.dtype == torch.bfloat16 else raw.view(torch.int32)
            assert bool((bits[torch.from_numpy(dead)] == 0).all()), f"{what}: masked row not +0.0"
        else:
            assert np.all(og[dead] == 0) and not np.signbit(og[dead]).any()
    live = ~dead
    if live.any():
        err = np.abs(og[live] - o_ref[live])
        bound = o_max_allowed(o_ref[live], dtype)
        worst = np.argmax(err - bound)
        assert err.flat[worst] <= bound.flat[worst], (
            f"{what}: |dO| {err.flat[worst]:.3e} > {bound.flat[worst]:.3e} allowed "
            f"(max |dO| {err.max():.3e}, tolerance {tol['o_max']})")
        assert err.mean() <= tol["o_mean"], f"{what}: mean |dO| {err.mean():.3e} > {tol['o_mean']}"
        le = np.abs(lg[live] - lse_ref[live])
        assert le.max() <= tol["lse"], f"{what}: max |dLSE| {le.max():.3e} > {tol['lse']}"
    return dict(o_max=float(np.abs(og - o_ref).max()) if og.size else 0.0)


def visible_splits(t_q, t_k, q_offset, split_size, window=0, causal=True):
    """Key ranges [s0, s1) of a split-KV decode that hold a key some row may
    see (below the last causal position + 1, at or past the first window
    start): the ranges whose partials the decode writes and merges."""
    n = max(1, -(-t_k // split_size))
    k_lo, k_hi = 0, t_k
    if causal:
        k_hi = min(k_hi, q_offset + t_q)
    if window > 0:
        k_lo = max(k_lo, q_offset - window + 1)
    if k_hi <= k_lo:
        return 0, 0
    return k_lo // split_size, min(n, (k_hi - 1) // split_size + 1)


def host_workers():
    """Threads for the CPU oracle: the CPUs this process may run on."""
    return max(1, len(os.sched_getaffinity(0)))


def oracle_by_group(wl, fn=None, **kw):
    """Run the oracle over every (batch, KV head) group of a workload in a
    thread pool (numpy releases the GIL in its matrix products and ufuncs; BLAS
    pinned to one thread per worker) and stitch the results back together.

    Each call sees the group's query heads, its one KV head and its bias slice,
    which is exactly what the oracle computes for those heads in one call over
    the whole workload.  ``fn`` is ``oracle.attention`` (returns o, lse,
    n_legal) or ``oracle.split_partials`` (returns the per-split o, lse)."""
    import concurrent.futures as cf
    from threadpoolctl import threadpool_limits

    fn = fn or oracle.attention
    bsz, h_q = wl.q.shape[:2]
    h_kv = wl.k.shape[1]
    g = h_q // h_kv
    bias = wl.bias

    def one(job):
        b, kvh = job
        hs = slice(kvh * g, (kvh + 1) * g)
        bb = None
        if bias is not None:
            bsel = slice(b, b + 1) if bias.shape[0] > 1 else slice(0, 1)
            hsel = hs if bias.shape[1] > 1 else slice(0, 1)
            bb = f64(bias[bsel, hsel])
        with threadpool_limits(limits=1):
            return job, fn(f64(wl.q[b:b + 1, hs]), f64(wl.k[b:b + 1, kvh:kvh + 1]),
                           f64(wl.v[b:b + 1, kvh:kvh + 1]), scale=wl.scale, causal=wl.causal,
                           q_offset=wl.q_offset, bias=bb, **kw)

    jobs = [(b, kvh) for b in range(bsz) for kvh in range(h_kv)]
    out = None
    with cf.ThreadPoolExecutor(max_workers=min(host_workers(), len(jobs), 32)) as ex:
        for (b, kvh), res in ex.map(one, jobs):
            if out is None:
                out = [np.zeros((bsz, h_q) + r.shape[2:], dtype=r.dtype) for r in res]
            for dst, r in zip(out, res):
                dst[b, kvh * g:(kvh + 1) * g] = r[0]
    return tuple(out)


def assert_close_full(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what=""):
    """``assert_close`` over a whole [B, H, T, d] output, one (batch, head)
    at a time so the fp64 copies stay small; the mean error is over every
    live element of the tensor, the maximum over all of them."""
    tol = TOL[dtype]
    bsz, h = o_ref.shape[:2]
    err_sum, err_n, err_max, lse_max, n_floor = 0.0, 0, 0.0, 0.0, 0
    for b in range(bsz):
        for hh in range(h):
            raw = o_gpu[b, hh].detach().cpu()
            og = raw.to(torch.float64).numpy()
            lg = lse_gpu[b, hh].detach().cpu().to(torch.float64).numpy()
            ref, lref = o_ref[b, hh], lse_ref[b, hh]
            where = f"{what} (b={b}, h={hh})"
            assert not np.isnan(og).any() and not np.isnan(lg).any(), f"{where}: NaN in output"
            dead = np.isneginf(lref)
            assert np.array_equal(np.isneginf(lg), dead), f"{where}: masked-row flags differ"
            if dead.any():
                bits = raw.view(torch.int16) if raw.dtype == torch.bfloat16 else raw.view(torch.int32)
                assert bool((bits[torch.from_numpy(dead)] == 0).all()), f"{where}: masked row not +0.0"
            live = ~dead
            if live.any():
                e = np.abs(og[live] - ref[live])
                err_sum += float(e.sum())
                err_n += e.size
                err_max = max(err_max, float(e.max()))
                bound = o_max_allowed(ref[live], dtype)
                n_floor += int((bound > tol["o_max"]).sum())
                worst = int(np.argmax(e - bound))
                assert e.flat[worst] <= bound.flat[worst], (
                    f"{where}: |dO| {e.flat[worst]:.3e} > {bound.flat[worst]:.3e} allowed at row "
                    f"{int(np.argwhere(live)[np.unravel_index(worst, e.shape)[0]][0])}")
                lse_max = max(lse_max, float(np.abs(lg[live] - lref[live]).max()))
                assert lse_max <= tol["lse"], f"{where}: max |dLSE| {lse_max:.3e} > {tol['lse']}"
    mean = err_sum / max(err_n, 1)
    assert mean <= tol["o_mean"], f"{what}: mean |dO| {mean:.3e} > {tol['o_mean']}"
    print(f"{what}: max |dO| {err_max:.3e}, mean |dO| {mean:.3e}, max |dLSE| {lse_max:.3e} "
          f"over {err_n} elements ({n_floor} whose exact value rounds farther than "
          f"{tol['o_max']})", flush=True)
    return dict(o_max=err_max, o_mean=mean, lse_max=lse_max, n_floor=n_floor)
