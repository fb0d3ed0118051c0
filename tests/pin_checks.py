"""Checks that pin the oracle to facts outside itself.

Each ``check_*`` takes the oracle module (``oracle.reference`` or a mutated
copy of it) and raises AssertionError when the oracle disagrees with the
pages' printed values, a closed form, an invariant, a brute force over block
partitions or an independent library softmax.  ``test_oracle_pins.py`` runs
them on the real oracle; ``test_oracle_mutants.py`` runs them on copies with a
planted mistake and expects at least one to fail.
"""

import itertools
import math
from fractions import Fraction

import numpy as np

from conftest import load_golden

LN = math.log


def _row_problem(bias_row, values, d_h=4):
    """q = 0 so every score equals its bias: z_j = M_j (eq 33.2)."""
    t_k = len(bias_row)
    d_v = len(values[0])
    q = np.zeros((1, 1, 1, d_h))
    k = np.random.default_rng(7).standard_normal((1, 1, t_k, d_h))
    v = np.array(values, dtype=np.float64).reshape(1, 1, t_k, d_v)
    bias = np.array(bias_row, dtype=np.float64).reshape(1, 1, 1, t_k)
    return q, k, v, bias


# --- the pages' printed examples ------------------------------------------

def check_example_25_1_exact(R):
    g = load_golden("example_25_1.json")
    z = [R.LogOf(a) for a in g["scores_are_log_of"]]
    vals = [[Fraction(x)] for x in g["values"]]
    legal = [True] * 3
    blk_a, blk_b = g["blocks"]
    st_a = R.block_stats([z[j] for j in blk_a], [vals[j] for j in blk_a],
                         [True] * len(blk_a), R.EXACT)
    st_b = R.block_stats([z[j] for j in blk_b], [vals[j] for j in blk_b],
                         [True] * len(blk_b), R.EXACT)
    for st, ref in ((st_a, g["block_A"]), (st_b, g["block_B"])):
        m, ell, u = st
        assert m == R.LogOf(ref["m_is_log_of"]), (m, ref)
        assert ell == Fraction(ref["ell"]), (ell, ref)
        assert u == [Fraction(ref["u"])], (u, ref)
        o_loc, _ = R.finalize(st, 1, R.EXACT)
        assert o_loc == [Fraction(ref["local_output"])]
    merged = R.merge_stats(st_a, st_b, R.EXACT)
    assert merged[0] == R.LogOf(g["merged"]["m_is_log_of"])
    assert merged[1] == Fraction(g["merged"]["ell"])
    assert merged[2] == [Fraction(g["merged"]["u"])]
    o, lse = R.finalize(merged, 1, R.EXACT)
    assert o == [Fraction(g["output"])]
    # LSE is derived, not printed: ln(2 + 1 + 6) = ln 9.
    assert lse == R.LogOf(9)
    # The full computation the example prints: (2*1 + 1*4 + 6*5)/(2+1+6).
    full = R.blocked_single_query(z, vals, legal, [[0, 1, 2]], R.EXACT)[0]
    num = Fraction(g["full_computation"]["numerator"])
    den = Fraction(g["full_computation"]["denominator"])
    assert full == [num / den] == [Fraction(g["output"])]
    # The wrong answers must not come out.
    for wrong in g["wrong_answers"].values():
        assert o != [Fraction(wrong)]
    # eq 33.3 defines m as the block maximum whatever the key order.
    st_rev = R.block_stats([z[1], z[0]], [vals[1], vals[0]], [True, True], R.EXACT)
    assert st_rev == st_a, st_rev
    # The merge scale of block A and the two global masses.
    assert R.EXACT.exp_diff(st_a[0], merged[0]) == Fraction(g["scale_of_A_in_merge"])
    masses = [R.EXACT.exp_diff(st[0], R.LogOf(1)) * st[1] for st in (st_a, st_b)]
    assert masses == [Fraction(x) for x in g["global_masses"]]


def check_example_25_1_fp64(R):
    g = load_golden("example_25_1.json")
    bias = [LN(a) for a in g["scores_are_log_of"]]
    vals = [[float(x), 0.0] for x in g["values"]]
    q, k, v, m = _row_problem(bias, vals)
    o, lse, n = R.attention(q, k, v, scale=0.125, causal=False, bias=m)
    assert abs(o[0, 0, 0, 0] - 4.0) <= 1e-15 * 4
    assert o[0, 0, 0, 1] == 0.0
    assert abs(lse[0, 0, 0] - LN(9)) <= 1e-15 * 3
    assert n[0, 0, 0] == 3
    # Split into blocks of two keys: partials (2, ln 3) and (5, ln 6).
    op, lp = R.split_partials(q, k, v, scale=0.125, causal=False, q_offset=0,
                              split_size=2, bias=m)
    assert op.shape == (1, 1, 1, 2, 2)
    assert abs(op[0, 0, 0, 0, 0] - 2.0) <= 1e-15 * 2
    assert abs(op[0, 0, 0, 1, 0] - 5.0) <= 1e-15 * 5
    assert abs(lp[0, 0, 0, 0] - LN(3)) <= 1e-15
    assert abs(lp[0, 0, 0, 1] - LN(6)) <= 1e-15 * 2
    om, lm = R.merge_partials(op, lp)
    assert abs(om[0, 0, 0, 0] - 4.0) <= 1e-15 * 4
    assert abs(lm[0, 0, 0] - LN(9)) <= 1e-15 * 3


def check_exercise_33_2(R):
    g = load_golden("exercise_33_2.json")
    masses = [float(Fraction(x)) for x in g["block_masses"]]
    vals = [float(Fraction(x)) for x in g["block_values"]]
    want = float(Fraction(g["output"]))
    o_parts = np.array([[[vals[0]], [vals[1]]]])
    l_parts = np.array([[LN(masses[0]), LN(masses[1])]])
    o, lse = R.merge_partials(o_parts, l_parts)
    assert abs(o[0, 0] - want) <= 1e-15 * want
    assert abs(o[0, 0] - float(Fraction(g["wrong_equal_weight_mean"]))) > 0.5
    assert abs(lse[0] - LN(masses[0] + masses[1])) <= 1e-15
    # The same through the materialised definition (two keys with z = ln mass).
    q, k, v, m = _row_problem([LN(x) for x in masses], [[x] for x in vals])
    o2, l2, _ = R.attention(q, k, v, scale=1.0, causal=False, bias=m)
    assert abs(o2[0, 0, 0, 0] - want) <= 1e-15 * want
    assert abs(l2[0, 0, 0] - LN(4)) <= 1e-15


def check_kv_cache_vectors(R):
    """Incremental (one query at position t over the first t+1 keys) equals
    the full causal computation, with q = k = v = the page's vectors."""
    g = load_golden("kv_cache_vectors.json")
    vecs = np.array(g["vectors"])
    x = vecs.reshape(1, 1, 4, 2)
    scale = 1.0 / math.sqrt(2.0)
    o_full, l_full, _ = R.attention(x, x, x, scale=scale, causal=True)
    for t in range(4):
        o_t, l_t, n_t = R.attention(x[:, :, t:t + 1], x[:, :, :t + 1],
                                    x[:, :, :t + 1], scale=scale, causal=True,
                                    q_offset=t)
        assert n_t[0, 0, 0] == t + 1
        assert np.max(np.abs(o_t[0, 0, 0] - o_full[0, 0, t])) < g["tolerance"]
        # Brute force by hand on the tiny input: weights e^{s_j}/sum e^{s}.
        s = [float(vecs[t] @ vecs[j]) * scale for j in range(t + 1)]
        e = [math.exp(a) for a in s]
        ref = [sum(e[j] * vecs[j][d] for j in range(t + 1)) / sum(e) for d in range(2)]
        assert max(abs(a - b) for a, b in zip(ref, o_full[0, 0, t])) < g["tolerance"]
        assert abs(l_full[0, 0, t] - math.log(sum(e))) < g["tolerance"]


# --- closed forms and special cases ---------------------------------------

def check_equal_scores_mean(R):
    """q = 0, no bias: every legal score is 0, so causal row i averages
    v_0..v_{q_offset+i} and its LSE is ln(q_offset + i + 1)."""
    rng = np.random.default_rng(1)
    t_q, t_k, d = 6, 11, 5
    v = rng.standard_normal((1, 1, t_k, d))
    k = rng.standard_normal((1, 1, t_k, d))
    q = np.zeros((1, 1, t_q, d))
    for off in (0, 3, t_k - t_q):
        o, lse, n = R.attention(q, k, v, scale=0.3, causal=True, q_offset=off)
        for i in range(t_q):
            cnt = min(off + i + 1, t_k)
            assert n[0, 0, i] == cnt
            np.testing.assert_allclose(o[0, 0, i], v[0, 0, :cnt].mean(0), rtol=0, atol=1e-14)
            assert abs(lse[0, 0, i] - math.log(cnt)) <= 1e-14
    # A constant bias c shifts the LSE by c only.
    bias = np.full((1, 1, t_q, t_k), 2.5)
    o, lse, _ = R.attention(q, k, v, scale=0.3, causal=False, bias=bias)
    np.testing.assert_allclose(o[0, 0, 0], v[0, 0].mean(0), rtol=0, atol=1e-14)
    assert abs(lse[0, 0, 0] - (2.5 + math.log(t_k))) <= 1e-14


def check_single_and_two_keys(R):
    rng = np.random.default_rng(2)
    t_k, d = 7, 3
    v = rng.standard_normal((1, 1, t_k, d))
    k = rng.standard_normal((1, 1, t_k, d))
    q = np.zeros((1, 1, 1, d))
    for j in range(t_k):
        bias = np.full((1, 1, 1, t_k), -np.inf)
        bias[..., j] = 1.75
        o, lse, n = R.attention(q, k, v, scale=1.0, causal=False, bias=bias)
        assert n[0, 0, 0] == 1
        assert np.array_equal(o[0, 0, 0], v[0, 0, j])
        assert lse[0, 0, 0] == 1.75
    # Two legal keys whose scores differ by delta: logistic weights.
    for delta in (-3.0, 0.0, 0.7, 5.0):
        bias = np.full((1, 1, 1, t_k), -np.inf)
        bias[..., 1] = 0.0
        bias[..., 4] = delta
        o, lse, _ = R.attention(q, k, v, scale=1.0, causal=False, bias=bias)
        w4 = 1.0 / (1.0 + math.exp(-delta))
        want = (1 - w4) * v[0, 0, 1] + w4 * v[0, 0, 4]
        np.testing.assert_allclose(o[0, 0, 0], want, rtol=0, atol=1e-14)
        assert abs(lse[0, 0, 0] - math.log1p(math.exp(delta))) <= 1e-14


def check_invariants(R):
    rng = np.random.default_rng(3)
    b, hq, hkv, t_q, t_k, d_h, d_v = 1, 2, 1, 5, 9, 4, 3
    q = rng.standard_normal((b, hq, t_q, d_h))
    k = rng.standard_normal((b, hkv, t_k, d_h))
    v = rng.standard_normal((b, hkv, t_k, d_v))
    bias = rng.standard_normal((b, 1, t_q, t_k))
    o, lse, _ = R.attention(q, k, v, scale=0.5, causal=False, bias=bias)
    # Shift: +c on a row's scores leaves o and moves lse by c.
    o2, lse2, _ = R.attention(q, k, v, scale=0.5, causal=False, bias=bias + 3.25)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, lse + 3.25, rtol=0, atol=1e-13)
    # Key permutation (keys, values and bias together) changes nothing.
    perm = rng.permutation(t_k)
    o3, lse3, _ = R.attention(q, k[:, :, perm], v[:, :, perm], scale=0.5,
                              causal=False, bias=bias[..., perm])
    np.testing.assert_allclose(o3, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse3, lse, rtol=0, atol=1e-13)
    # Convex hull: each component lies between the legal values' extremes.
    lo = v.min(axis=2)[:, :, None, :]
    hi = v.max(axis=2)[:, :, None, :]
    assert np.all(o >= lo - 1e-14) and np.all(o <= hi + 1e-14)


def check_partitions_exact(R):
    """Every set partition of 6 keys, blocks taken in every order (first 24
    orders), equals the direct weighted average, exactly (eq 33.3-33.5 with
    e^{z} = a rational mass)."""
    masses = [Fraction(3), Fraction(1, 2), Fraction(7), Fraction(2), Fraction(5, 3), Fraction(1)]
    vals = [[Fraction(2), Fraction(-1)], [Fraction(5)], [Fraction(-3)],
            [Fraction(1, 4)], [Fraction(9)], [Fraction(0)]]
    vals = [[x[0], x[0] * 2 - 1] for x in vals]
    legal = [True, True, False, True, True, True]  # key 2 masked
    z = [R.LogOf(a) for a in masses]
    num = [sum(masses[j] * vals[j][d] for j in range(6) if legal[j]) for d in range(2)]
    den = sum(masses[j] for j in range(6) if legal[j])
    want = [x / den for x in num]
    seen = set()
    for part in R.set_partitions(list(range(6))):
        seen.add(tuple(sorted(tuple(sorted(b)) for b in part)))
        for order in itertools.islice(itertools.permutations(part), 24):
            o, lse = R.blocked_single_query(z, vals, legal, list(order), R.EXACT)
            assert o == want, (order, o, want)
            assert lse == R.LogOf(den)
    assert len(seen) == 203  # Bell(6): every partition of the 6 keys was merged


def check_set_partitions(R):
    """The partition generator behind the brute force yields every set
    partition exactly once: Bell numbers 1, 1, 2, 5, 15, 52, 203, 877 for
    n = 0..7 (OEIS A000110), each yield a true partition (non-empty disjoint
    blocks covering the items), no partition twice."""
    bell = [1, 1, 2, 5, 15, 52, 203, 877]
    for n, want in enumerate(bell):
        items = list(range(n))
        seen = set()
        for part in R.set_partitions(items):
            assert all(len(b) > 0 for b in part), part
            flat = sorted(x for b in part for x in b)
            assert flat == items, part
            canon = tuple(sorted(tuple(sorted(b)) for b in part))
            assert canon not in seen, ("repeated", part)
            seen.add(canon)
        assert len(seen) == want, (n, len(seen), want)


def check_partitions_fp64(R):
    """Every contiguous partition of 10 keys (2^9 of them) through Algorithm
    33.1 equals the materialised definition within 1e-13."""
    rng = np.random.default_rng(4)
    t_k, d = 10, 3
    z = list(rng.standard_normal(t_k) * 3)
    vals = rng.standard_normal((t_k, d))
    legal = [True] * t_k
    legal[6] = False
    o_ref, l_ref, _ = R.softmax_rows(np.array([z]), np.array([legal]), vals)
    for cuts in range(1 << (t_k - 1)):
        blocks, cur = [], [0]
        for j in range(1, t_k):
            if cuts >> (j - 1) & 1:
                blocks.append(cur)
                cur = []
            cur.append(j)
        blocks.append(cur)
        o, lse = R.blocked_single_query(z, vals.tolist(), legal, blocks, R.FP64)
        assert np.max(np.abs(np.array(o) - o_ref[0])) <= 1e-13
        assert abs(lse - l_ref[0]) <= 1e-13


def check_masked_blocks_and_rows(R):
    rng = np.random.default_rng(5)
    t_q, t_k, d = 4, 8, 3
    q = rng.standard_normal((1, 1, t_q, d))
    k = rng.standard_normal((1, 1, t_k, d))
    v = rng.standard_normal((1, 1, t_k, d))
    bias = np.zeros((1, 1, t_q, t_k))
    bias[0, 0, 1, :] = -np.inf          # row 1: no legal key
    bias[0, 0, 2, 2:6] = -np.inf        # row 2: a masked block in the middle
    o, lse, n = R.attention(q, k, v, scale=0.7, causal=False, bias=bias)
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    assert np.all(o[0, 0, 1] == 0.0) and not np.signbit(o[0, 0, 1]).any()
    assert lse[0, 0, 1] == -np.inf and n[0, 0, 1] == 0
    keep = [0, 1, 6, 7]
    o2, lse2, _ = R.attention(q[:, :, 2:3], k[:, :, keep], v[:, :, keep],
                              scale=0.7, causal=False)
    np.testing.assert_allclose(o[0, 0, 2], o2[0, 0, 0], rtol=0, atol=1e-14)
    assert abs(lse[0, 0, 2] - lse2[0, 0, 0]) <= 1e-14
    # Algorithm 33.1 over blocks that are all empty returns the defined row.
    z = [0.0] * 4
    o3, l3 = R.blocked_single_query(z, [[1.0]] * 4, [False] * 4, [[0, 1], [2, 3]])
    assert o3 == [0.0] and l3 == -np.inf
    # Causal rows before position 0 (negative offset) have no legal key.
    o4, l4, n4 = R.attention(q, k, v, scale=0.7, causal=True, q_offset=-2)
    assert np.all(n4[0, 0, :2] == 0) and np.all(l4[0, 0, :2] == -np.inf)
    assert np.all(o4[0, 0, :2] == 0.0)
    assert n4[0, 0, 2] == 1 and np.array_equal(o4[0, 0, 2], v[0, 0, 0])
    # Empty key set: every row is masked.
    o5, l5, n5 = R.attention(q, k[:, :, :0], v[:, :, :0], scale=0.7, causal=True)
    assert np.all(o5 == 0.0) and np.all(l5 == -np.inf) and np.all(n5 == 0)


def check_alignment(R):
    """A cached decode query sits at the newest position: with the right
    offset it equals non-causal attention; aligned at local index 0 it sees
    key 0 only (the §33.3 pitfall) and must come out different."""
    rng = np.random.default_rng(6)
    t_k, d = 9, 4
    q = rng.standard_normal((1, 1, 1, d))
    k = rng.standard_normal((1, 1, t_k, d))
    v = rng.standard_normal((1, 1, t_k, d))
    o_right, l_right, _ = R.attention(q, k, v, scale=0.5, causal=True, q_offset=t_k - 1)
    o_full, l_full, _ = R.attention(q, k, v, scale=0.5, causal=False)
    np.testing.assert_allclose(o_right, o_full, rtol=0, atol=1e-15)
    o_wrong, _, n_wrong = R.attention(q, k, v, scale=0.5, causal=True, q_offset=0)
    assert n_wrong[0, 0, 0] == 1
    assert np.array_equal(o_wrong[0, 0, 0], v[0, 0, 0])
    assert np.max(np.abs(o_wrong - o_right)) > 1e-3
    # Multi-query verify: row r at offset T_k-5+r sees keys 0..T_k-5+r.
    q5 = rng.standard_normal((1, 1, 5, d))
    o5, _, n5 = R.attention(q5, k, v, scale=0.5, causal=True, q_offset=t_k - 5)
    assert list(n5[0, 0]) == [t_k - 4, t_k - 3, t_k - 2, t_k - 1, t_k]
    for r in range(5):
        keep = t_k - 4 + r
        o_r, _, _ = R.attention(q5[:, :, r:r + 1], k[:, :, :keep], v[:, :, :keep],
                                scale=0.5, causal=False)
        np.testing.assert_allclose(o5[0, 0, r], o_r[0, 0, 0], rtol=0, atol=1e-14)
    # An offset past the end makes every key visible.
    o6, _, _ = R.attention(q5, k, v, scale=0.5, causal=True, q_offset=10 * t_k)
    o7, _, _ = R.attention(q5, k, v, scale=0.5, causal=False)
    np.testing.assert_allclose(o6, o7, rtol=0, atol=0)


def check_gqa_mapping(R):
    """Query head hq reads KV head hq // (H_q/H_kv): with q = 0 each output
    is the mean of its KV head's values, which differ per KV head."""
    t_k, d = 5, 2
    hq, hkv = 6, 3
    v = np.zeros((1, hkv, t_k, d))
    for h in range(hkv):
        v[0, h] = 10.0 * h + np.arange(t_k * d).reshape(t_k, d)
    k = np.ones((1, hkv, t_k, d))
    q = np.zeros((1, hq, 1, d))
    o, _, _ = R.attention(q, k, v, scale=1.0, causal=False)
    for h in range(hq):
        np.testing.assert_allclose(o[0, h, 0], v[0, h // 2].mean(0), rtol=0, atol=1e-13)


def check_split_merge(R):
    rng = np.random.default_rng(8)
    b, hq, hkv, t_q, t_k, d_h, d_v = 2, 4, 2, 3, 23, 5, 6
    q = rng.standard_normal((b, hq, t_q, d_h))
    k = rng.standard_normal((b, hkv, t_k, d_h))
    v = rng.standard_normal((b, hkv, t_k, d_v))
    bias = rng.standard_normal((b, 1, t_q, t_k))
    bias[0, 0, 1, :] = -np.inf
    for off, split in ((t_k - t_q, 5), (4, 4), (t_k + 3, 23), (0, 1)):
        o, lse, _ = R.attention(q, k, v, scale=0.4, causal=True, q_offset=off, bias=bias)
        op, lp = R.split_partials(q, k, v, scale=0.4, causal=True, q_offset=off,
                                  split_size=split, bias=bias)
        assert op.shape[3] == -(-t_k // split)
        om, lm = R.merge_partials(op, lp)
        np.testing.assert_allclose(om, o, rtol=0, atol=1e-13)
        assert np.array_equal(np.isneginf(lm), np.isneginf(lse))
        fin = ~np.isneginf(lse)
        np.testing.assert_allclose(lm[fin], lse[fin], rtol=0, atol=1e-13)


def check_rows_match_full(R):
    rng = np.random.default_rng(9)
    b, hq, hkv, t_q, t_k, d_h, d_v = 2, 4, 2, 6, 13, 4, 3
    q = rng.standard_normal((b, hq, t_q, d_h))
    k = rng.standard_normal((b, hkv, t_k, d_h))
    v = rng.standard_normal((b, hkv, t_k, d_v))
    bias = rng.standard_normal((b, 1, t_q, t_k))
    bias[1, 0, 2] = -np.inf
    o, lse, n = R.attention(q, k, v, scale=0.6, causal=True, q_offset=5, bias=bias)
    rows = [(bb, h, i) for bb in range(b) for h in range(hq) for i in range(t_q)]
    o2, l2, n2 = R.attention_rows(q, k, v, rows, scale=0.6, causal=True,
                                  q_offset=5, bias=bias)
    np.testing.assert_allclose(o2, o.reshape(-1, d_v), rtol=0, atol=1e-14)
    assert np.array_equal(n2, n.reshape(-1))
    assert np.array_equal(np.isneginf(l2), np.isneginf(lse.reshape(-1)))


def check_library_softmax(R):
    """Cross-check with torch's own float64 CPU attention and logsumexp, with
    an explicit boolean mask and the KV heads expanded per group."""
    import torch
    rng = np.random.default_rng(10)
    for (b, hq, hkv, t_q, t_k, d_h, d_v, off) in ((2, 6, 3, 7, 19, 8, 5, 9),
                                                  (1, 2, 2, 12, 12, 6, 7, 0)):
        q = rng.standard_normal((b, hq, t_q, d_h))
        k = rng.standard_normal((b, hkv, t_k, d_h))
        v = rng.standard_normal((b, hkv, t_k, d_v))
        bias = rng.standard_normal((b, 1, t_q, t_k))
        bias[rng.random(bias.shape) < 0.2] = -np.inf
        bias[b - 1, 0, 4, :] = -np.inf
        scale = 0.37
        o, lse, n = R.attention(q, k, v, scale=scale, causal=True, q_offset=off, bias=bias)
        tq = torch.from_numpy(q)
        tk = torch.from_numpy(k).repeat_interleave(hq // hkv, dim=1)
        tv = torch.from_numpy(v).repeat_interleave(hq // hkv, dim=1)
        pos = torch.arange(t_q)[:, None] + off
        vis = torch.arange(t_k)[None, :] <= pos
        tb = torch.from_numpy(bias).expand(b, hq, t_q, t_k)
        allowed = vis & torch.isfinite(tb)
        addmask = torch.where(allowed, tb, torch.tensor(float("-inf"), dtype=torch.float64))
        live = allowed.any(-1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, attn_mask=addmask, scale=scale)
        scores = (tq @ tk.transpose(-1, -2).contiguous()) * scale + addmask
        ref_lse = torch.logsumexp(scores, dim=-1)
        o_t = torch.from_numpy(o)
        assert torch.allclose(o_t[live], ref[live], rtol=0, atol=1e-12)
        assert torch.allclose(torch.from_numpy(lse)[live], ref_lse[live], rtol=0, atol=1e-12)
        assert torch.equal(torch.from_numpy(n), allowed.sum(-1))
        assert bool((~live).any())  # the case holds at least one fully masked row
        assert torch.all(o_t[~live] == 0)
        assert torch.all(torch.from_numpy(lse)[~live] == float("-inf"))


def check_bias_broadcast(R):
    rng = np.random.default_rng(11)
    b, hq, t_q, t_k, d = 2, 3, 4, 6, 3
    q = rng.standard_normal((b, hq, t_q, d))
    k = rng.standard_normal((b, hq, t_k, d))
    v = rng.standard_normal((b, hq, t_k, d))
    keyrow = rng.standard_normal((b, 1, 1, t_k))
    keyrow[0, 0, 0, 1] = -np.inf
    dense = np.broadcast_to(keyrow, (b, hq, t_q, t_k)).copy()
    o1, l1, n1 = R.attention(q, k, v, scale=0.5, causal=True, q_offset=1, bias=keyrow)
    o2, l2, n2 = R.attention(q, k, v, scale=0.5, causal=True, q_offset=1, bias=dense)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2) and np.array_equal(n1, n2)


# --- sliding window (§33.7, the sliding-window paragraph and eq 33.16) ------

def _window_count(pos, window, t_k, causal):
    """Integers j in [0, t_k) with pos - window + 1 <= j (<= pos if causal)."""
    lo = max(0, pos - window + 1)
    hi = min(pos, t_k - 1) if causal else t_k - 1
    return max(0, hi - lo + 1)


def check_window_counts(R):
    rng = np.random.default_rng(12)
    t_q, t_k, d = 9, 17, 3
    q = rng.standard_normal((1, 2, t_q, d))
    k = rng.standard_normal((1, 2, t_k, d))
    v = rng.standard_normal((1, 2, t_k, d))
    for causal in (True, False):
        for off in (-4, 0, 5, t_k - t_q, t_k + 2):
            for w in (1, 2, 5, 16, 40):
                _, lse, n = R.attention(q, k, v, scale=0.3, causal=causal, q_offset=off, window=w)
                want = np.array([_window_count(off + i, w, t_k, causal) for i in range(t_q)])
                assert np.array_equal(n[0, 0], want), (causal, off, w)
                assert np.array_equal(np.isneginf(lse[0, 0]), want == 0)
                rows = [(0, 1, i) for i in range(t_q)]
                _, _, n2 = R.attention_rows(q, k, v, rows, scale=0.3, causal=causal, q_offset=off, window=w)
                assert np.array_equal(n2, want), (causal, off, w)


def check_window_single_key(R):
    """W = 1 with causal masking leaves exactly the row's own position."""
    rng = np.random.default_rng(13)
    t_q, t_k, d_h, d_v = 6, 8, 4, 3
    q = rng.standard_normal((1, 1, t_q, d_h))
    k = rng.standard_normal((1, 1, t_k, d_h))
    v = rng.standard_normal((1, 1, t_k, d_v))
    for off in (-2, 0, 3, 5):
        o, lse, n = R.attention(q, k, v, scale=0.7, causal=True, q_offset=off, window=1)
        for i in range(t_q):
            pos = off + i
            if 0 <= pos < t_k:
                np.testing.assert_allclose(o[0, 0, i], v[0, 0, pos], rtol=0, atol=1e-15)
                assert abs(lse[0, 0, i] - 0.7 * float(q[0, 0, i] @ k[0, 0, pos])) < 1e-14
                assert n[0, 0, i] == 1
            else:
                assert n[0, 0, i] == 0 and lse[0, 0, i] == -np.inf and np.all(o[0, 0, i] == 0)


def check_window_as_bias(R):
    """A window is the -inf bias on keys j < q_offset + i - W + 1."""
    rng = np.random.default_rng(14)
    b, hq, hkv, t_q, t_k, d_h, d_v = 2, 4, 2, 7, 21, 5, 4
    q = rng.standard_normal((b, hq, t_q, d_h))
    k = rng.standard_normal((b, hkv, t_k, d_h))
    v = rng.standard_normal((b, hkv, t_k, d_v))
    for causal, off, w in ((True, 14, 6), (True, 3, 2), (False, 10, 9), (True, -3, 4)):
        i = np.arange(t_q)[:, None]
        j = np.arange(t_k)[None, :]
        bias = np.where(j >= off + i - w + 1, 0.0, -np.inf).reshape(1, 1, t_q, t_k)
        o1, l1, n1 = R.attention(q, k, v, scale=0.5, causal=causal, q_offset=off, window=w)
        o2, l2, n2 = R.attention(q, k, v, scale=0.5, causal=causal, q_offset=off, bias=bias)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2) and np.array_equal(n1, n2)


def check_window_truncation_bound(R):
    """eq 33.16 and its proof: with delta the full-attention mass of the keys
    the window drops, o = (1 - delta) o' + delta o_drop, so
    ||o - o'|| <= 2 delta M when every ||v_j|| <= M."""
    rng = np.random.default_rng(15)
    t_k, d_h, d_v = 40, 6, 5
    k = rng.standard_normal((1, 1, t_k, d_h))
    v = rng.standard_normal((1, 1, t_k, d_v))
    big_m = float(np.linalg.norm(v[0, 0], axis=1).max())
    for pos, w, temp in ((39, 10, 1.0), (25, 3, 2.0), (30, 29, 0.3), (12, 1, 1.5)):
        q = temp * rng.standard_normal((1, 1, 1, d_h))
        o, lse, _ = R.attention(q, k, v, scale=1.0, causal=True, q_offset=pos)
        o_w, lse_w, _ = R.attention(q, k, v, scale=1.0, causal=True, q_offset=pos, window=w)
        lo = pos - w + 1
        o_d, lse_d, _ = R.attention(q, k, v, scale=1.0, causal=True, q_offset=pos, key_range=(0, lo))
        delta = math.exp(lse_d[0, 0, 0] - lse[0, 0, 0])
        assert abs(math.exp(lse_w[0, 0, 0] - lse[0, 0, 0]) + delta - 1.0) < 1e-12
        np.testing.assert_allclose(o[0, 0, 0], (1 - delta) * o_w[0, 0, 0] + delta * o_d[0, 0, 0],
                                   rtol=0, atol=1e-12)
        assert 0 < delta < 1
        assert np.linalg.norm(o[0, 0, 0] - o_w[0, 0, 0]) <= 2 * delta * big_m + 1e-12


def check_window_split_merge(R):
    rng = np.random.default_rng(16)
    b, hq, hkv, t_q, t_k, d_h, d_v = 1, 4, 2, 3, 37, 4, 3
    q = rng.standard_normal((b, hq, t_q, d_h))
    k = rng.standard_normal((b, hkv, t_k, d_h))
    v = rng.standard_normal((b, hkv, t_k, d_v))
    for off, w, split in ((34, 9, 4), (34, 30, 7), (20, 2, 5)):
        o, lse, _ = R.attention(q, k, v, scale=0.4, causal=True, q_offset=off, window=w)
        op, lp = R.split_partials(q, k, v, scale=0.4, causal=True, q_offset=off,
                                  split_size=split, window=w)
        om, lm = R.merge_partials(op, lp)
        np.testing.assert_allclose(om, o, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lm, lse, rtol=0, atol=1e-13)
        assert bool(np.isneginf(lp).any())   # splits wholly outside the window are empty


# --- backward (eqs 33.6-33.8, Exercise 33.4) --------------------------------

def _bwd_problem(seed, b=1, hq=2, hkv=1, t_q=4, t_k=6, d_h=3, d_v=2):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((b, hq, t_q, d_h)), rng.standard_normal((b, hkv, t_k, d_h)),
            rng.standard_normal((b, hkv, t_k, d_v)), rng.standard_normal((b, hq, t_q, d_v)))


def check_backward_finite_differences(R):
    """Central differences of L = sum(G_O * O) through the forward oracle."""
    q, k, v, g = _bwd_problem(20)
    bias = np.random.default_rng(21).standard_normal((1, 2, 4, 6))
    bias[0, 0, 1, 2] = -np.inf
    bias[0, 1, 0, :] = -np.inf            # one fully masked row
    for kw in (dict(causal=True, q_offset=2, bias=bias), dict(causal=True, q_offset=3, window=2),
               dict(causal=False, q_offset=0)):
        def loss(q_, k_, v_):
            o, _, _ = R.attention(q_, k_, v_, scale=0.7, **kw)
            return float((g * o).sum())
        dq, dk, dv = R.attention_backward(q, k, v, g, scale=0.7, **kw)
        for x, dx in ((q, dq), (k, dk), (v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                old = x[idx]
                x[idx] = old + 1e-6
                up = loss(q, k, v)
                x[idx] = old - 1e-6
                dn = loss(q, k, v)
                x[idx] = old
                num[idx] = (up - dn) / 2e-6
            np.testing.assert_allclose(dx, num, rtol=0, atol=1e-7)


def check_backward_shift_direction(R):
    """Exercise 33.4: the row-mean term makes the gradient along a common
    shift of a row's scores zero; with every key equal, all scores of a row
    are equal, so G_Q = scale * sum_j (G_S)_ij k = 0."""
    q, k, v, g = _bwd_problem(22, t_q=5, t_k=7)
    k[:] = k[:, :, :1, :]
    dq, dk, _ = R.attention_backward(q, k, v, g, scale=0.9, causal=True, q_offset=2)
    assert np.abs(dq).max() < 1e-14
    assert np.abs(dk).max() > 1e-3          # K itself still gets a gradient


def check_backward_identities(R):
    """sum <G_Q, Q> = sum <G_K, K> (both scale * sum_ij (G_S)_ij <q_i, k_j>),
    and sum_j G_V_j = sum of G_O over rows with a legal key (rows of P sum to 1)."""
    q, k, v, g = _bwd_problem(23, b=2, hq=4, hkv=2, t_q=5, t_k=9, d_h=4, d_v=3)
    for off, w in ((0, 0), (4, 3), (-2, 0)):
        dq, dk, dv = R.attention_backward(q, k, v, g, scale=0.5, causal=True, q_offset=off, window=w)
        _, lse, _ = R.attention(q, k, v, scale=0.5, causal=True, q_offset=off, window=w)
        for bb in range(2):
            for kvh in range(2):
                heads = [2 * kvh, 2 * kvh + 1]
                lhs = sum(float((dq[bb, h] * q[bb, h]).sum()) for h in heads)
                rhs = float((dk[bb, kvh] * k[bb, kvh]).sum())
                assert abs(lhs - rhs) < 1e-12
                live = sum(g[bb, h][~np.isneginf(lse[bb, h])].sum(axis=0) for h in heads)
                np.testing.assert_allclose(dv[bb, kvh].sum(axis=0), live, rtol=0, atol=1e-12)


def check_backward_single_key(R):
    """A window of one key: P is one-hot, so G_S = 0 (G_Q = G_K = 0) and G_V
    of key j is the upstream gradient of the row at position j."""
    q, k, v, g = _bwd_problem(24, t_q=4, t_k=6)
    dq, dk, dv = R.attention_backward(q, k, v, g, scale=1.1, causal=True, q_offset=1, window=1)
    assert np.abs(dq).max() < 1e-15 and np.abs(dk).max() < 1e-15
    want = np.zeros_like(dv)
    for i in range(4):
        want[0, 0, 1 + i] += g[0, 0, i] + g[0, 1, i]
    np.testing.assert_allclose(dv, want, rtol=0, atol=1e-15)


def check_backward_library_autograd(R):
    """torch's float64 autograd through an explicitly masked softmax attention
    (rows with at least one legal key; KV heads expanded per group)."""
    import torch
    q, k, v, g = _bwd_problem(25, b=2, hq=4, hkv=2, t_q=6, t_k=11, d_h=5, d_v=4)
    off, w, scale = 5, 7, 0.45
    dq, dk, dv = R.attention_backward(q, k, v, g, scale=scale, causal=True, q_offset=off, window=w)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    i = torch.arange(6)[:, None] + off
    j = torch.arange(11)[None, :]
    allowed = (j <= i) & (j >= i - w + 1)
    assert bool(allowed.any(-1).all())
    kk = tk.repeat_interleave(2, dim=1)
    vv = tv.repeat_interleave(2, dim=1)
    s = scale * tq @ kk.transpose(-1, -2)
    p = torch.softmax(s.masked_fill(~allowed, float("-inf")), dim=-1)
    (p @ vv * torch.tensor(g)).sum().backward()
    assert np.allclose(tq.grad.numpy(), dq, rtol=0, atol=1e-12)
    assert np.allclose(tk.grad.numpy(), dk, rtol=0, atol=1e-12)
    assert np.allclose(tv.grad.numpy(), dv, rtol=0, atol=1e-12)


def check_backward_sampled_matches_full(R):
    q, k, v, g = _bwd_problem(26, b=2, hq=4, hkv=2, t_q=7, t_k=12, d_h=4, d_v=3)
    for kw in (dict(causal=True, q_offset=5), dict(causal=True, q_offset=6, window=4), dict(causal=False)):
        dq, dk, dv = R.attention_backward(q, k, v, g, scale=0.6, **kw)
        rows = [(1, 3, 6), (0, 0, 0), (0, 2, 3)]
        keys = [(1, 1, 11), (0, 0, 0), (0, 1, 5)]
        sq, sk, sv = R.attention_backward_sampled(q, k, v, g, rows=rows, keys=keys, scale=0.6, **kw)
        np.testing.assert_allclose(sq, np.array([dq[r] for r in rows]), rtol=0, atol=1e-13)
        np.testing.assert_allclose(sk, np.array([dk[x] for x in keys]), rtol=0, atol=1e-13)
        np.testing.assert_allclose(sv, np.array([dv[x] for x in keys]), rtol=0, atol=1e-13)


# --- unpadded variable-length batches (§33.4, shape bucketing) ---------------

def check_varlen_equals_padded(R):
    """Packing the sequences equals the padded batch the pages describe: each
    sequence padded to a bucket, padded keys masked by a -inf bias, the rows of
    the sequence placed at the end of its key positions; the padded rows are
    dropped.  Also the legal-pair saving: sum of n_legal over the padded rows
    minus the unpadded sum is the work the bucket adds."""
    rng = np.random.default_rng(30)
    lq, lk = [3, 0, 7, 1, 5], [6, 4, 7, 9, 5]
    hq, hkv, d_h, d_v, bucket = 4, 2, 5, 3, 10
    cu_q = np.concatenate([[0], np.cumsum(lq)])
    cu_k = np.concatenate([[0], np.cumsum(lk)])
    q = rng.standard_normal((1, hq, cu_q[-1], d_h))
    k = rng.standard_normal((1, hkv, cu_k[-1], d_h))
    v = rng.standard_normal((1, hkv, cu_k[-1], d_v))
    # A bias indexed by packed row and key, with -inf entries (masked pairs
    # and one whole row), read only on each sequence's diagonal block.
    mb = rng.standard_normal((1, hq, cu_q[-1], cu_k[-1]))
    mb[rng.random(mb.shape) < 0.2] = -np.inf
    mb[:, :, 2, :] = -np.inf
    for causal, w, use_bias in ((True, 0, False), (True, 3, False), (False, 0, False),
                                (True, 0, True), (False, 2, True)):
        o, lse, n = R.attention_varlen(q, k, v, cu_q, cu_k, scale=0.6, causal=causal, window=w,
                                       bias=mb if use_bias else None)
        nb = len(lq)
        qp = np.zeros((nb, hq, bucket, d_h)); kp = np.zeros((nb, hkv, bucket, d_h))
        vp = np.zeros((nb, hkv, bucket, d_v)); bias = np.zeros((nb, 1, bucket, bucket))
        for s in range(nb):
            # rows at the end of the bucket, keys at the start: row i sits at
            # position (L_k - L_q) + i when q_offset = bucket - L_q and keys
            # past L_k are masked; here every row is placed at bucket - L_q + i
            # with keys shifted so that position p is key p.
            qp[s, :, bucket - lq[s]:] = q[0, :, cu_q[s]:cu_q[s + 1]]
            kp[s, :, :lk[s]] = k[0, :, cu_k[s]:cu_k[s + 1]]
            vp[s, :, :lk[s]] = v[0, :, cu_k[s]:cu_k[s + 1]]
            bias[s, 0, :, lk[s]:] = -np.inf
        if use_bias:
            bias = np.broadcast_to(bias, (nb, hq, bucket, bucket)).copy()
            for s in range(nb):
                bias[s, :, bucket - lq[s]:, :lk[s]] = mb[0, :, cu_q[s]:cu_q[s + 1], cu_k[s]:cu_k[s + 1]]
        # q_offset per sequence differs (L_k - L_q - (bucket - L_q) = L_k - bucket),
        # so run the padded batch one sequence at a time with that offset.
        for s in range(nb):
            op, lp, npad = R.attention(qp[s:s + 1], kp[s:s + 1], vp[s:s + 1], scale=0.6, causal=causal,
                                       q_offset=lk[s] - bucket, bias=bias[s:s + 1], window=w)
            rows = slice(bucket - lq[s], bucket)
            np.testing.assert_allclose(o[0, :, cu_q[s]:cu_q[s + 1]], op[0, :, rows], rtol=0, atol=1e-14)
            assert np.array_equal(np.isneginf(lse[0, :, cu_q[s]:cu_q[s + 1]]), np.isneginf(lp[0, :, rows]))
            assert np.array_equal(n[0, :, cu_q[s]:cu_q[s + 1]], npad[0, :, rows])
        if use_bias:
            assert np.isneginf(lse[0, :, 2]).all()   # the row the bias masks whole
        if causal and w == 0 and not use_bias:
            # Row i of sequence s sees min(L_k - L_q + i + 1, L_k) keys.
            want = np.concatenate([[min(lk[s] - lq[s] + i + 1, lk[s]) for i in range(lq[s])]
                                   for s in range(nb)]).astype(np.int64)
            assert np.array_equal(n[0, 0], want)


def check_varlen_sequences_independent(R):
    """Changing one sequence's values changes only that sequence's rows."""
    rng = np.random.default_rng(31)
    cu_q, cu_k = [0, 4, 9, 11], [0, 6, 9, 20]
    q = rng.standard_normal((1, 2, 11, 4))
    k = rng.standard_normal((1, 1, 20, 4))
    v = rng.standard_normal((1, 1, 20, 3))
    o1, l1, _ = R.attention_varlen(q, k, v, cu_q, cu_k, scale=0.5, causal=True)
    v2 = v.copy(); v2[0, 0, 6:9] += 1.0
    o2, l2, _ = R.attention_varlen(q, k, v2, cu_q, cu_k, scale=0.5, causal=True)
    assert np.array_equal(l1, l2)
    changed = np.any(o1 != o2, axis=(0, 1, 3))
    # Sequence 1 has 5 rows over 3 keys: its first two rows sit before every
    # key (causal), stay masked and cannot change.
    assert not changed[:6].any() and changed[6:9].all() and not changed[9:].any()
    assert np.isneginf(l1[0, :, 4:6]).all() and np.isfinite(l1[0, :, 6:9]).all()


def check_varlen_key_bias_broadcast(R):
    """A per-key bias [1, 1, 1, sum L_k] (one M_j per packed key) equals the
    same values written out densely for every row."""
    rng = np.random.default_rng(32)
    cu_q, cu_k = [0, 3, 3, 8], [0, 5, 6, 14]
    q = rng.standard_normal((1, 2, 8, 4))
    k = rng.standard_normal((1, 2, 14, 4))
    v = rng.standard_normal((1, 2, 14, 2))
    mj = rng.standard_normal((1, 1, 1, 14))
    mj[0, 0, 0, [1, 9]] = -np.inf
    a = R.attention_varlen(q, k, v, cu_q, cu_k, scale=0.7, causal=True, bias=mj)
    b = R.attention_varlen(q, k, v, cu_q, cu_k, scale=0.7, causal=True,
                           bias=np.broadcast_to(mj, (1, 2, 8, 14)).copy())
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def check_kvlens_equals_padded(R):
    """Per-batch KV lengths equal the padded cache the pages describe: keys
    past L_b masked by a -inf bias, rows at positions L_b - T_q + i."""
    rng = np.random.default_rng(33)
    bsz, hq, hkv, t_q, t_k = 5, 4, 2, 3, 9
    lens = [9, 0, 1, 4, 2]
    q = rng.standard_normal((bsz, hq, t_q, 6))
    k = rng.standard_normal((bsz, hkv, t_k, 6))
    v = rng.standard_normal((bsz, hkv, t_k, 5))
    for causal, w in ((True, 0), (False, 0), (True, 2)):
        o, lse, n = R.attention_kvlens(q, k, v, lens, scale=0.4, causal=causal, window=w)
        for b in range(bsz):
            bias = np.zeros((1, 1, 1, t_k))
            bias[..., lens[b]:] = -np.inf
            op, lp, npad = R.attention(q[b:b + 1], k[b:b + 1], v[b:b + 1], scale=0.4, causal=causal,
                                       q_offset=lens[b] - t_q, bias=bias, window=w)
            np.testing.assert_allclose(o[b], op[0], rtol=0, atol=1e-14)
            assert np.array_equal(np.isneginf(lse[b]), np.isneginf(lp[0]))
            assert np.array_equal(n[b], npad[0])
        assert np.isneginf(lse[1]).all() and (o[1] == 0).all()   # the empty cache
        if causal and w == 0:
            # Row i of batch b sees min(L_b - T_q + i + 1, L_b) keys (>= 0).
            want = np.array([[max(0, min(L - t_q + i + 1, L)) for i in range(t_q)] for L in lens])
            assert np.array_equal(n[:, 0], want)
    # Full lengths: the dense problem with the rows at the end of the keys.
    o, lse, _ = R.attention_kvlens(q, k, v, [t_k] * bsz, scale=0.4, causal=True)
    od, ld, _ = R.attention(q, k, v, scale=0.4, causal=True, q_offset=t_k - t_q)
    assert np.array_equal(o, od) and np.array_equal(lse, ld)


def check_varlen_backward(R):
    """Packed-sequence gradients: (a) central finite differences of
    sum(G_O * O) through the packed forward ``attention_varlen`` (rows at the
    end of their keys, L_q > L_k with masked leading rows, an empty sequence,
    GQA, a packed bias with -inf entries); (b) equal to the padded batch's
    gradients on legal rows and real keys (padded keys masked by a -inf bias,
    padded rows given zero upstream gradient); (c) rows and keys outside every
    sequence get zero."""
    rng = np.random.default_rng(34)
    lq, lk = [3, 5, 0, 2], [4, 3, 2, 6]
    cu_q = np.concatenate([[0], np.cumsum(lq)]).tolist()
    cu_k = np.concatenate([[0], np.cumsum(lk)]).tolist()
    hq, hkv, d_h, d_v = 4, 2, 3, 2
    tq, tk = sum(lq) + 1, sum(lk) + 2          # one row and two keys outside every sequence
    q = rng.standard_normal((1, hq, tq, d_h))
    k = rng.standard_normal((1, hkv, tk, d_h))
    v = rng.standard_normal((1, hkv, tk, d_v))
    g = rng.standard_normal((1, hq, tq, d_v))
    mb = rng.standard_normal((1, hq, tq, tk))
    mb[rng.random(mb.shape) < 0.15] = -np.inf
    for causal, w, bias in ((True, 0, None), (False, 0, mb), (True, 2, mb)):
        kw = dict(scale=0.7, causal=causal, bias=bias, window=w)
        dq, dk, dv = R.attention_varlen_backward(q, k, v, g, cu_q, cu_k, **kw)
        # (c)
        assert not dq[:, :, sum(lq):].any() and not dk[:, :, sum(lk):].any() and not dv[:, :, sum(lk):].any()

        def loss(qq, kk, vv):
            o, _, _ = R.attention_varlen(qq, kk, vv, cu_q, cu_k, **kw)
            return float((o * g).sum())
        eps = 1e-6
        for name, x, grad in (("dq", q, dq), ("dk", k, dk), ("dv", v, dv)):
            for idx in [tuple(rng.integers(0, n) for n in x.shape) for _ in range(12)]:
                xp, xm = x.copy(), x.copy()
                xp[idx] += eps
                xm[idx] -= eps
                args_p = [xp if y is x else y for y in (q, k, v)]
                args_m = [xm if y is x else y for y in (q, k, v)]
                fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
                assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])
        # (b) the padded batch, one sequence at a time
        for s in range(len(lq)):
            q0, q1, k0, k1 = cu_q[s], cu_q[s + 1], cu_k[s], cu_k[s + 1]
            bucket = 7
            qp = np.zeros((1, hq, bucket, d_h)); gp = np.zeros((1, hq, bucket, d_v))
            kp = np.zeros((1, hkv, bucket, d_h)); vp = np.zeros((1, hkv, bucket, d_v))
            bp = np.zeros((1, hq, bucket, bucket))
            qp[:, :, bucket - (q1 - q0):] = q[:, :, q0:q1]
            gp[:, :, bucket - (q1 - q0):] = g[:, :, q0:q1]
            kp[:, :, :k1 - k0] = k[:, :, k0:k1]
            vp[:, :, :k1 - k0] = v[:, :, k0:k1]
            bp[:, :, :, k1 - k0:] = -np.inf
            if bias is not None:
                bp[:, :, bucket - (q1 - q0):, :k1 - k0] = bias[:, :, q0:q1, k0:k1]
            pq, pk, pv = R.attention_backward(qp, kp, vp, gp, scale=0.7, causal=causal,
                                              q_offset=(k1 - k0) - bucket, bias=bp, window=w)
            np.testing.assert_allclose(dq[:, :, q0:q1], pq[:, :, bucket - (q1 - q0):], rtol=0, atol=1e-12)
            np.testing.assert_allclose(dk[:, :, k0:k1], pk[:, :, :k1 - k0], rtol=0, atol=1e-12)
            np.testing.assert_allclose(dv[:, :, k0:k1], pv[:, :, :k1 - k0], rtol=0, atol=1e-12)


def check_kvlens_backward(R):
    """Gradients with per-batch KV lengths: (a) central finite differences of
    sum(G_O * O) through the forward ``attention_kvlens`` (rows at the end of
    each batch's keys, a batch with more rows than keys, an empty key set,
    GQA, a bias with -inf entries, a window); (b) equal to the full-length
    batch's gradients when the keys past kv_lens[b] are masked by a -inf bias
    (the padded form); (c) keys past kv_lens[b] get zero."""
    rng = np.random.default_rng(35)
    b_n, hq, hkv, tq, tk, d_h, d_v = 3, 4, 2, 3, 6, 3, 2
    lens = [6, 2, 0]
    q = rng.standard_normal((b_n, hq, tq, d_h))
    k = rng.standard_normal((b_n, hkv, tk, d_h))
    v = rng.standard_normal((b_n, hkv, tk, d_v))
    g = rng.standard_normal((b_n, hq, tq, d_v))
    mb = rng.standard_normal((b_n, hq, tq, tk))
    mb[rng.random(mb.shape) < 0.15] = -np.inf
    for causal, w, bias in ((True, 0, None), (False, 0, mb), (True, 2, mb)):
        kw = dict(scale=0.7, causal=causal, bias=bias, window=w)
        dq, dk, dv = R.attention_kvlens_backward(q, k, v, g, lens, **kw)
        for b, n in enumerate(lens):   # (c)
            assert not dk[b, :, n:].any() and not dv[b, :, n:].any()

        def loss(qq, kk, vv):
            o, _, _ = R.attention_kvlens(qq, kk, vv, lens, **kw)
            return float((o * g).sum())
        eps = 1e-6
        for name, x, grad in (("dq", q, dq), ("dk", k, dk), ("dv", v, dv)):
            for idx in [tuple(rng.integers(0, n) for n in x.shape) for _ in range(12)]:
                xp, xm = x.copy(), x.copy()
                xp[idx] += eps
                xm[idx] -= eps
                args_p = [xp if y is x else y for y in (q, k, v)]
                args_m = [xm if y is x else y for y in (q, k, v)]
                fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
                assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])
        # (b) batch by batch: all T_k keys, those past the length masked, rows
        # at positions q_offset + L_b - T_q + i
        for b, n in enumerate(lens):
            bp = np.zeros((1, hq, tq, tk)) if bias is None else bias[b:b + 1].copy()
            bp[..., n:] = -np.inf
            pq, pk, pv = R.attention_backward(q[b:b + 1], k[b:b + 1], v[b:b + 1], g[b:b + 1], scale=0.7,
                                              causal=causal, q_offset=n - tq, bias=bp, window=w)
            np.testing.assert_allclose(dq[b:b + 1], pq, rtol=0, atol=1e-12)
            np.testing.assert_allclose(dk[b:b + 1], pk, rtol=0, atol=1e-12)
            np.testing.assert_allclose(dv[b:b + 1], pv, rtol=0, atol=1e-12)


ALL_CHECKS = [
    check_example_25_1_exact, check_example_25_1_fp64, check_exercise_33_2,
    check_kv_cache_vectors, check_equal_scores_mean, check_single_and_two_keys,
    check_invariants, check_set_partitions, check_partitions_exact, check_partitions_fp64,
    check_masked_blocks_and_rows, check_alignment, check_gqa_mapping,
    check_split_merge, check_rows_match_full, check_library_softmax,
    check_bias_broadcast, check_window_counts, check_window_single_key,
    check_window_as_bias, check_window_truncation_bound, check_window_split_merge,
    check_backward_finite_differences, check_backward_shift_direction, check_backward_identities,
    check_backward_single_key, check_backward_library_autograd, check_backward_sampled_matches_full,
    check_varlen_equals_padded, check_varlen_sequences_independent, check_varlen_key_bias_broadcast,
    check_kvlens_equals_padded, check_varlen_backward, check_kvlens_backward,
]
