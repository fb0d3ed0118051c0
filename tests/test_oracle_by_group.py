"""The threaded helper that runs the oracle over (batch, KV head) groups for
the full-size parity tests gives exactly what one oracle call over the whole
workload gives (CPU only)."""

import numpy as np

import oracle
from online_softmax_exact_amd import inputs
from gpu_util import f64, oracle_by_group


def test_by_group_equals_whole_call():
    wl = inputs.make_random(3, 8, 2, 37, 50, 64, 32, seed=11, causal=True, q_offset=13,
                            bias="shared", masked_frac=0.1)
    want = oracle.attention(f64(wl.q), f64(wl.k), f64(wl.v), scale=wl.scale, causal=True,
                            q_offset=wl.q_offset, bias=f64(wl.bias))
    got = oracle_by_group(wl)
    for g, w in zip(got, want):
        assert g.shape == w.shape
        assert np.array_equal(g, w)


def test_by_group_split_partials():
    wl = inputs.make_random(2, 4, 4, 3, 70, 64, 64, seed=12, causal=True, q_offset=40)
    want = oracle.split_partials(f64(wl.q), f64(wl.k), f64(wl.v), scale=wl.scale, causal=True,
                                 q_offset=wl.q_offset, split_size=16)
    got = oracle_by_group(wl, fn=oracle.split_partials, split_size=16)
    for g, w in zip(got, want):
        assert g.shape == w.shape
        assert np.array_equal(g, w)
