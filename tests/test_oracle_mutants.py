"""Plant a plausible mistake in a copy of the oracle (on the CPU) and check
that the pin suite catches it: the pins are strong enough to notice a dropped
term, a wrong sign or index, or a transposed operand."""

import importlib.util
import os
import sys
import types

import pytest

from pin_checks import ALL_CHECKS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "reference.py")

MUTANTS = {
    "causal_off_by_one": ("legal = j <= (q_offset + i)", "legal = j < (q_offset + i)"),
    "gqa_modulo": ("kvh = hq // group\n            m_rows", "kvh = hq % h_kv\n            m_rows"),
    "scale_dropped": ("s = scale * (q[b, hq] @ k[b, kvh].T)", "s = (q[b, hq] @ k[b, kvh].T)"),
    "bias_scaled": ("s = s + np.where(m_rows == NEG_INF, 0.0, m_rows)",
                    "s = s + scale * np.where(m_rows == NEG_INF, 0.0, m_rows)"),
    "lse_drops_max": ("lse[live] = m + np.log(ell)", "lse[live] = np.log(ell)"),
    "exp_sign": ("w = np.exp(s - m[:, None])", "w = np.exp(s + m[:, None])"),
    "no_normalise": ("o[live] = (w @ values) / ell[:, None]", "o[live] = (w @ values)"),
    "transposed_kv": ("s = scale * (q[b, hq] @ k[b, kvh].T)", "s = scale * (q[b, hq] @ k[b, kvh].T).T[: q.shape[2], : k.shape[2]] if q.shape[2] == k.shape[2] else scale * (q[b, hq] @ k[b, kvh].T)"),
    "merge_wrong_weight": ("cb = arith.exp_diff(m_b, m)", "cb = arith.exp_diff(m_a, m)"),
    "merge_unweighted_u": ("u = [ca * x + cb * y for x, y in zip(u_a, u_b)]",
                           "u = [x + y for x, y in zip(u_a, u_b)]"),
    "merge_keeps_first_max": ("m = m_a if not arith.gt(m_b, m_a) else m_b", "m = m_a"),
    "stats_first_key_max": ("        if arith.gt(z[j], m):\n            m = z[j]", "        pass"),
    "masked_row_nan": ("live = n_legal > 0", "live = n_legal >= 0"),
    "empty_block_not_skipped": ("    if not idx:\n        return None",
                                "    if not idx:\n        return (0.0, 0.0, [0.0] * len(values[0]))"),
    "partitions_no_singleton": ("        yield [[first]] + part\n", "\n"),
    "partitions_first_block_only": ("        for i in range(len(part)):", "        for i in [0] * len(part):"),
    "split_range_inclusive": ("legal = legal & (j >= lo) & (j < hi)", "legal = legal & (j >= lo) & (j <= hi)"),
    "rows_offset_ignored": ("pos = q_offset + i", "pos = i"),
    "window_off_by_one": ("legal = legal & (j >= q_offset + i - window + 1)",
                          "legal = legal & (j > q_offset + i - window + 1)"),
    "window_ignores_offset": ("legal = legal & (j >= q_offset + i - window + 1)",
                              "legal = legal & (j >= i - window + 1)"),
    "window_rows_off_by_one": ("legal = legal & (j >= pos - window + 1)",
                               "legal = legal & (j >= pos - window)"),
    "window_split_dropped": ("                                window=window)",
                             "                                window=0)"),
    "bwd_no_row_mean": ("g_s = p * (g_p - (p * g_p).sum(axis=1, keepdims=True))", "g_s = p * g_p"),
    "bwd_row_mean_unweighted": ("g_s = p * (g_p - (p * g_p).sum(axis=1, keepdims=True))",
                                "g_s = p * (g_p - g_p.mean(axis=1, keepdims=True))"),
    "bwd_dq_scale_dropped": ("dq[b, hq] = scale * (g_s @ k[b, kvh])", "dq[b, hq] = (g_s @ k[b, kvh])"),
    "bwd_dk_from_dq_side": ("dk[b, kvh] += scale * (g_s.T @ q[b, hq])",
                            "dk[b, kvh] += scale * (p.T @ q[b, hq])"),
    "bwd_gqa_overwrites": ("dv[b, kvh] += p.T @ g_o", "dv[b, kvh] = p.T @ g_o"),
    "bwd_dp_uses_k": ("g_p = g_o @ v[b, kvh].T", "g_p = g_o @ v[b, kvh].T[:, ::-1]"),
    "varlen_top_left": ("causal=causal, q_offset=q_offset + (k1 - k0) - (q1 - q0),",
                        "causal=causal, q_offset=q_offset,"),
    "varlen_keys_shifted": ("k[:, :, k0:k1], v[:, :, k0:k1]", "k[:, :, q0:q0 + k1 - k0], v[:, :, k0:k1]"),
    "varlen_bias_rows_unshifted": ("(slice(q0, q1) if bb.shape[2] != 1", "(slice(0, q1 - q0) if bb.shape[2] != 1"),
    "kvlens_top_left": ("q_offset=q_offset + n_k - t_q, bias=b_s", "q_offset=q_offset, bias=b_s"),
    "kvlens_keeps_all_keys": ("k[b:b + 1, :, :n_k], v[b:b + 1, :, :n_k]", "k[b:b + 1], v[b:b + 1]"),
    "varlen_bwd_top_left": ("scale=scale, causal=causal, q_offset=q_offset + (k1 - k0) - (q1 - q0),\n                               bias=b_s",
                            "scale=scale, causal=causal, q_offset=q_offset,\n                               bias=b_s"),
    "varlen_bwd_dk_rows": ("dq[:, :, q0:q1], dk[:, :, k0:k1], dv[:, :, k0:k1] = g",
                           "dq[:, :, q0:q1], dk[:, :, q0:q0 + k1 - k0], dv[:, :, k0:k1] = g"),
    "kvlens_bwd_top_left": ("d_o[b:b + 1],\n                               scale=scale, causal=causal, q_offset=q_offset + n_k - t_q",
                            "d_o[b:b + 1],\n                               scale=scale, causal=causal, q_offset=q_offset"),
    "kvlens_bwd_keys_at_end": ("dq[b:b + 1], dk[b:b + 1, :, :n_k], dv[b:b + 1, :, :n_k] = g",
                               "dq[b:b + 1], dk[b:b + 1, :, k.shape[2] - n_k:], dv[b:b + 1, :, :n_k] = g"),
}


def _load_mutant(name, old, new):
    src = open(SRC, encoding="utf-8").read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    src = src.replace(old, new, 1)
    mod = types.ModuleType(f"oracle_mutant_{name}")
    mod.__file__ = SRC
    sys.modules[mod.__name__] = mod
    exec(compile(src, f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    mod = _load_mutant(name, old, new)
    caught = []
    for check in ALL_CHECKS:
        try:
            check(mod)
        except Exception as e:  # AssertionError, or a crash the mistake causes
            caught.append((check.__name__, type(e).__name__))
    assert caught, f"planted mistake {name!r} passed every pin"
