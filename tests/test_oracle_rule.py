"""Pins of the oracle's verification rule (oracle/verify.py).

Each test fixes part of the rule against something other than the oracle:
hand-worked fixtures, exact enumeration, library routines (numpy's
searchsorted and argmax semantics, scipy's logsumexp/softmax, torch's bf16
decode) and invariants that follow from the rule's definition.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st
from scipy import special

from oracle import philox
from oracle import verify as ov

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rows(fracs):
    return [np.array([float(Fraction(v)) for v in row]) for row in fracs]


def _logits(prob_rows):
    with np.errstate(divide="ignore"):
        return [np.log(r) for r in prob_rows]


# ---------------------------------------------------------------- exactness ---

@pytest.mark.parametrize("case", _load("dyadic_cases.json")["cases"],
                         ids=lambda c: c["name"][:40])
def test_exact_law_by_enumeration(case):
    """Emitted token at each reached position has the target's law, exactly.

    All thresholds are multiples of 1/16, so evaluating the rule at the 16
    midpoints of each uniform and weighting drafted tokens by q is an exact
    integral. The rule runs on softmax rows of log-probabilities.
    """
    p_exp = _rows(case["p"])
    q_exp = _rows(case["q"])
    k, V = len(q_exp), len(p_exp[0])
    p_rows = [ov.softmax_row(z, 1.0)[2] for z in _logits(p_exp)]
    q_rows = [ov.softmax_row(z, 1.0)[2] for z in _logits(q_exp)]
    grid = [(g + 0.5) / 16.0 for g in range(16)]
    cell = 16.0 ** -(k + 1)
    emitted = np.zeros((k + 1, V))
    reached = np.zeros(k + 1)
    for drafted in itertools.product(range(V), repeat=k):
        weight = math.prod(q_exp[i][drafted[i]] for i in range(k))
        if weight == 0.0:
            continue
        for us in itertools.product(grid, repeat=k + 1):
            d = ov.decide_sampled(p_rows, q_rows, list(drafted), us[:k], [us[k]] * (k + 1))
            for i, tok in enumerate(d.tokens):
                emitted[i, tok] += weight * cell
                reached[i] += weight * cell
    survive = [float(Fraction(s)) for s in case["survive"]]
    reach_exp = np.cumprod([1.0] + survive)
    np.testing.assert_allclose(reached, reach_exp, rtol=0, atol=1e-12)
    for i in range(k + 1):
        np.testing.assert_allclose(emitted[i], reached[i] * p_exp[i], rtol=0, atol=1e-12)


# ------------------------------------------------------------------- greedy ---

def test_greedy_golden_cases():
    g = _load("greedy_cases.json")
    target = np.array(g["target"], dtype=np.float64)
    for case in g["cases"]:
        k = case["budget"]
        d = ov.decide_greedy(target[: k + 1], np.array(case["drafted"], dtype=np.int64))
        assert d.n_accepted == case["n_accepted"]
        assert d.tokens == case["emitted"]


def _brute_greedy(rows, drafted):
    best = []
    for row in rows:
        top = None
        for v, val in enumerate(row):          # strict '>' keeps the lowest index
            if top is None or val > row[top]:
                top = v
        best.append(top)
    out = []
    for i, x in enumerate(drafted):
        if x != best[i]:
            return i, out + [best[i]]
        out.append(int(x))
    return len(drafted), out + [best[len(drafted)]]


def test_greedy_matches_brute_force_with_ties():
    rng = np.random.default_rng(5)
    for _ in range(300):
        k = int(rng.integers(0, 6))
        V = int(rng.integers(1, 12))
        rows = rng.integers(-2, 3, size=(k + 1, V)).astype(np.float64)   # many ties
        best = [int(np.argmax(r)) for r in rows]
        drafted = np.array([best[i] if rng.random() < 0.7 else int(rng.integers(0, V))
                            for i in range(k)], dtype=np.int64)
        d = ov.decide_greedy(rows, drafted)
        j, toks = _brute_greedy(rows.tolist(), drafted.tolist())
        assert (d.n_accepted, d.tokens) == (j, toks)


def test_low_temperature_reproduces_greedy():
    """T -> 0+: with well-separated logits the sampled rule becomes greedy."""
    rng = np.random.default_rng(8)
    for b in range(40):
        k, V = 4, 50
        base = rng.permutation(V).astype(np.float64) * 0.1      # gaps of 0.1
        target = np.stack([rng.permutation(base) for _ in range(k + 1)])
        draft = target[:k] + rng.normal(0, 0.2, size=(k, V))
        drafted = np.argmax(draft, axis=1)
        sampled = ov.verify_request(b, target, draft, drafted, 1e-3, 99)
        greedy = ov.decide_greedy(target, drafted)
        assert (sampled.n_accepted, sampled.tokens) == (greedy.n_accepted, greedy.tokens)


# ------------------------------------------------------ sampled special cases ---

def test_q_equal_p_accepts_everything():
    """Identical drafter and target rows: p/q == 1, so every token survives and
    the bonus is the inverse-CDF draw from p_k (numpy searchsorted)."""
    rng = np.random.default_rng(3)
    for b in range(200):
        k, V, T = int(rng.integers(0, 7)), 64, float(rng.uniform(0.3, 2.0))
        target = rng.normal(0, 2, size=(k + 1, V))
        drafted = rng.integers(0, V, size=k)
        d = ov.verify_request(b, target, target[:k].copy(), drafted, T, 1234)
        assert d.n_accepted == k and d.mode == ov.BONUS
        assert d.tokens[:k] == [int(x) for x in drafted]
        p = special.softmax(target[k] / T)
        u = philox.position_uniforms(1234, b, k)[1]
        assert d.tokens[k] == int(np.searchsorted(np.cumsum(p), u * p.sum(), side="right"))


def test_zero_target_mass_is_never_accepted():
    p = [np.array([0.0, 0.5, 0.5]), np.array([0.2, 0.3, 0.5])]
    q = [np.array([0.9, 0.05, 0.05])]
    d = ov.decide_sampled(p, q, [0], [0.0], [0.3, 0.3])      # u = 0 exactly
    assert d.n_accepted == 0 and d.tokens[0] != 0


def test_target_at_least_drafter_is_always_accepted():
    p = [np.array([0.6, 0.2, 0.2]), np.array([0.2, 0.3, 0.5])]
    q = [np.array([0.6, 0.3, 0.1])]
    top_u = 1.0 - 2.0 ** -24
    for x in (0, 2):                                          # p(x) >= q(x)
        d = ov.decide_sampled(p, q, [x], [top_u], [0.5, 0.5])
        assert d.n_accepted == 1


def test_zero_drafter_mass():
    """q(x) == 0: accepted when p(x) > 0, rejected when p(x) == 0."""
    p = [np.array([0.5, 0.5, 0.0]), np.array([1.0, 0.0, 0.0])]
    q = [np.array([0.0, 0.0, 1.0])]
    assert ov.decide_sampled(p, q, [0], [0.999], [0.1, 0.1]).n_accepted == 1
    p2 = [np.array([0.0, 1.0, 0.0]), np.array([1.0, 0.0, 0.0])]
    assert ov.decide_sampled(p2, q, [0], [0.0], [0.1, 0.1]).n_accepted == 0


def test_inverse_cdf_skips_zero_mass_and_is_strict():
    mass = np.array([0.0, 0.0, 0.25, 0.0, 0.75])
    assert ov.inverse_cdf(mass, 0.0)[0] == 2           # u = 0: first positive token
    assert ov.inverse_cdf(mass, 0.25)[0] == 4          # C(2)/R = 0.25 is not > 0.25
    assert ov.inverse_cdf(mass, 0.25 - 2.0 ** -24)[0] == 2
    assert ov.inverse_cdf(mass, 1.0 - 2.0 ** -24)[0] == 4


@settings(max_examples=300, deadline=None)
@given(st.integers(1, 40), st.integers(0, 2**32 - 1), st.floats(0.0, 1.0 - 2.0**-24))
def test_inverse_cdf_matches_searchsorted(V, seed, u):
    rng = np.random.default_rng(seed)
    mass = rng.exponential(size=V) * (rng.random(V) < 0.6)
    if not np.any(mass > 0):
        mass[rng.integers(0, V)] = 1.0
    y, margin, total = ov.inverse_cdf(mass, u)
    ref = int(np.searchsorted(np.cumsum(mass), u * mass.sum(), side="right"))
    if ref == V:                                 # rounding: no crossing at all
        ref = int(np.nonzero(mass > 0)[0][-1])
    assert y == ref
    assert mass[y] > 0 and margin >= 0.0 and total == pytest.approx(mass.sum())


@settings(max_examples=300, deadline=None)
@given(st.integers(1, 6), st.integers(2, 10), st.integers(0, 2**32 - 1))
def test_residual_only_emits_tokens_where_target_exceeds_drafter(k, V, seed):
    rng = np.random.default_rng(seed)
    zt = rng.normal(0, 2, size=(k + 1, V))
    zd = rng.normal(0, 2, size=(k, V))
    drafted = rng.integers(0, V, size=k)
    b = int(rng.integers(0, 1000))
    d = ov.verify_request(b, zt, zd, drafted, 1.0, seed)
    if d.mode == ov.RESIDUAL:
        j, y = d.n_accepted, d.tokens[-1]
        p = special.softmax(zt[j])
        q = special.softmax(zd[j])
        assert p[y] > q[y]
        assert y != drafted[j]                   # rejection implies p(x) < q(x)
    # Acceptance at position i uses word 0 of counter (b, i, 0, 0): every kept
    # position passed u < min(1, p/q) and the first rejected one failed it.
    for i in range(min(d.n_accepted + 1, k)):
        p = special.softmax(zt[i])[drafted[i]]
        q = special.softmax(zd[i])[drafted[i]]
        u = philox.position_uniforms(seed, b, i)[0]
        if i < d.n_accepted:
            assert u < min(1.0, p / q) + 1e-12
        else:
            assert u >= min(1.0, p / q) - 1e-12


def test_bonus_is_drawn_from_row_of_the_budget():
    """A ragged budget k < K draws the bonus from target row k, not row K."""
    rng = np.random.default_rng(4)
    K, V = 5, 32
    target = rng.normal(0, 1, size=(1, K + 1, V))
    tokens = rng.integers(0, V, size=(1, K))
    for k in range(K + 1):
        res = ov.verify_batch(target, target[:, :K].copy(), tokens, np.array([k]), 1.0, 77)
        d = res.decisions[0]
        assert d.n_accepted == k
        p = special.softmax(target[0, k])
        u = philox.position_uniforms(77, 0, k)[1]
        assert d.tokens[-1] == int(np.searchsorted(np.cumsum(p), u * p.sum(), side="right"))
        assert list(res.tokens[0, k + 1:]) == [-1] * (K - k)


# ----------------------------------------------------------------- numerics ---

def test_softmax_normaliser_matches_logsumexp():
    rng = np.random.default_rng(6)
    for T in (0.25, 0.8, 1.0, 3.0):
        z = rng.normal(0, 3, size=151936)
        z[rng.integers(0, z.size, 50)] = -np.inf
        m, s, p = ov.softmax_row(z, T)
        assert m == np.max(z)
        ref = special.logsumexp(z / T)
        assert math.log(s) + m / T == pytest.approx(ref, rel=1e-13, abs=1e-12)
        np.testing.assert_allclose(p, special.softmax(z / T), rtol=1e-12, atol=1e-300)


def test_bf16_decode_matches_torch_for_every_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = ov.decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_preconditions_are_checked():
    t = np.zeros((2, 4, 8))
    d = np.zeros((2, 3, 8))
    x = np.zeros((2, 3), dtype=np.int64)
    with pytest.raises(ValueError):
        ov.verify_batch(t, d, x, np.array([4, 1]), 1.0, 0)        # budget > K
    with pytest.raises(ValueError):
        ov.verify_batch(t, d, x, np.array([-1, 1]), 1.0, 0)
    bad = x.copy()
    bad[1, 0] = 8
    with pytest.raises(ValueError):
        ov.verify_batch(t, d, bad, np.array([1, 1]), 1.0, 0)      # token >= V
    with pytest.raises(ValueError):
        ov.verify_batch(t, d, x, np.array([1, 1]), -1.0, 0)
    with pytest.raises(ValueError):
        ov.verify_batch(t, d, x, np.array([1, 1]), float("nan"), 0)
    # A token beyond the budget is never looked at.
    ok = x.copy()
    ok[1, 2] = 1000
    ov.verify_batch(t, d, ok, np.array([1, 1]), 1.0, 0)
