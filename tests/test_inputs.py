"""The seeded input generators: shapes, dtypes, determinism and the masking
structure of the padded variable-length workload."""

import torch

from online_softmax_exact_amd import inputs


def test_small_configs_shapes_and_determinism():
    for k in (1, 4):
        a = inputs.make_config(k)
        b = inputs.make_config(k)
        spec = inputs.SPECS[k]
        assert a.q.shape == (spec["batch"], spec["heads_q"], spec["t_q"], spec["d_h"])
        assert a.k.shape == (spec["batch"], spec["heads_kv"], spec["t_k"], spec["d_h"])
        assert a.v.shape == (spec["batch"], spec["heads_kv"], spec["t_k"], spec["d_v"])
        assert a.q.dtype == spec["dtype"]
        assert torch.equal(a.q, b.q) and torch.equal(a.k, b.k) and torch.equal(a.v, b.v)
        assert a.scale == float(torch.tensor(spec["d_h"] ** -0.5, dtype=torch.float32))


def test_padded_bias_structure():
    bias, lengths, rows = inputs.padded_bias(4, 64, 64, 123)
    assert bias.shape == (4, 1, 64, 64) and bias.dtype == torch.float32
    for b in range(4):
        L = lengths[b]
        assert 1 <= L <= 64
        assert torch.all(torch.isneginf(bias[b, 0, :, L:]))
        dead = torch.isneginf(bias[b, 0]).all(dim=1)
        assert sorted(torch.nonzero(dead).flatten().tolist()) == sorted(rows[b])
        assert len(set(rows[b])) == 2


def test_random_bias_kinds():
    for kind, shape in (("dense", (2, 4, 3, 5)), ("shared", (2, 1, 3, 5)),
                        ("keys", (2, 1, 1, 5)), ("rows", (2, 1, 3, 1))):
        w = inputs.make_random(2, 4, 2, 3, 5, 8, 8, bias=kind, seed=3)
        assert w.bias.shape == shape


def test_chunked_draw_is_thread_independent(monkeypatch):
    a = inputs._draw((3, 5, 300, 40), 9, 1, torch.bfloat16)
    monkeypatch.setattr(inputs.os, "cpu_count", lambda: 1)
    b = inputs._draw((3, 5, 300, 40), 9, 1, torch.bfloat16)
    assert torch.equal(a, b)
    assert abs(float(a.float().mean())) < 0.01 and abs(float(a.float().std()) - 1) < 0.01


def test_varlen_lengths_are_the_padded_workload_lengths():
    _, lengths, _ = inputs.padded_bias(4, 64, 64, 123)
    assert inputs.varlen_lengths(4, 64, 123) == lengths


def test_make_packed_layout():
    q, k, v, m, cu_q, cu_k = inputs.make_packed([3, 0, 5], [4, 2, 5], 4, 2, 8, 6, seed=1,
                                                bias="keys", masked_frac=0.3)
    assert cu_q.tolist() == [0, 3, 3, 8] and cu_k.tolist() == [0, 4, 6, 11]
    assert q.shape == (1, 4, 8, 8) and k.shape == (1, 2, 11, 8) and v.shape == (1, 2, 11, 6)
    assert m.shape == (1, 1, 1, 11) and m.dtype == torch.float32
    assert cu_q.dtype == torch.int32
