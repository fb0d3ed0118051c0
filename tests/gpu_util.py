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


def assert_close(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what=""):
    """Element-wise parity; masked rows (oracle LSE = -inf) must be bit-exact
    (+0.0 output, -inf LSE) and no NaN may appear anywhere."""
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
        assert err.max() <= tol["o_max"], f"{what}: max |dO| {err.max():.3e} > {tol['o_max']}"
        assert err.mean() <= tol["o_mean"], f"{what}: mean |dO| {err.mean():.3e} > {tol['o_mean']}"
        le = np.abs(lg[live] - lse_ref[live])
        assert le.max() <= tol["lse"], f"{what}: max |dLSE| {le.max():.3e} > {tol['lse']}"
    return dict(o_max=float(np.abs(og - o_ref).max()) if og.size else 0.0)
