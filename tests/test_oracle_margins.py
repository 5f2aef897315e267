"""Pins of the oracle's near-tie margins and of the parity checker that uses them.

The sampled parity bar excuses a library/oracle mismatch only where the
oracle's decision lay within 1e-6 of its threshold ("Speculative decoding
becomes standard: DSpark and multi-token drafters", section "Why
draft-and-verify does not change the output", paragraph 2: a drafted token
survives with probability min(1, p/q) and a rejected one is redrawn from the
renormalised residual). So the margins decide which mismatches pass, and are
pinned here to exact values on hand-built dyadic cases, where every quantity
is a short binary fraction and fp64 arithmetic is exact:

* acceptance margin |u - min(1, p/q)|, for u below and above the threshold
  and with the ratio capped at one;
* draw margin: the distance from u to the nearer edge of the drawn token's
  interval [C(y-1)/R, C(y)/R) of the normalised running sum, at both edges,
  across a zero-mass token, and for a residual draw whose R is not 1.

Each pin is then run against planted mistakes in the oracle (a margin that
is always 0, a margin not divided by R, the wrong CDF edge, an uncapped
ratio, a residual normalised by the wrong total): every mutant must fail a
pin. Finally the checker itself (tests/helpers.compare_sampled) is pinned:
a near-tie is excused only at a decision the oracle took within the band,
and a kept token that is not the drafted one, or a drawn token that is not
a neighbour across the near CDF edge, never is.
"""
import math

import numpy as np
import pytest

from oracle import verify as ov
from tests.helpers import compare_sampled


# --------------------------------------------------------------- the pins ---

def pin_acceptance_margin():
    # p/q = (3/8)/(1/2) = 3/4; u = 5/8 lies 1/8 below (kept), u = 7/8 1/8 above.
    assert ov.accept_decision(5 / 8, 3 / 8, 1 / 2) == (True, 1 / 8)
    assert ov.accept_decision(7 / 8, 3 / 8, 1 / 2) == (False, 1 / 8)
    # p/q = 2 is capped at 1: u = 3/4 lies 1/4 below the cap.
    assert ov.accept_decision(3 / 4, 1 / 2, 1 / 4) == (True, 1 / 4)
    # u = 0 against p/q = 1/16 exactly.
    assert ov.accept_decision(0.0, 1 / 32, 1 / 2) == (True, 1 / 16)


def pin_draw_margin():
    # mass [1, 2, 1], R = 4: token 1 owns [1/4, 3/4).
    m = np.array([1.0, 2.0, 1.0])
    assert ov.inverse_cdf(m, 5 / 16) == (1, 1 / 16, 4.0)       # 1/16 above the lower edge
    assert ov.inverse_cdf(m, 11 / 16) == (1, 1 / 16, 4.0)      # 1/16 below the upper edge
    assert ov.inverse_cdf(m, 1 / 8) == (0, 1 / 8, 4.0)         # token 0: [0, 1/4)
    # A zero-mass token between: mass [1, 2, 0, 1]; token 3 owns [3/4, 1).
    m0 = np.array([1.0, 2.0, 0.0, 1.0])
    assert ov.inverse_cdf(m0, 13 / 16) == (3, 1 / 16, 4.0)
    assert ov.cdf_interval(m0, 3) == (3 / 4, 1.0)
    assert ov.cdf_interval(m0, 2) == (3 / 4, 3 / 4)             # no mass, empty interval


def pin_residual_draw_margin():
    # p = [1/2, 1/8, 1/4, 1/8], q = [1/8, 1/2, 1/8, 1/4]; drafted token 1 has
    # p/q = 1/4, so u_acc = 1/2 rejects it with margin 1/4. The residual is
    # [3/8, 0, 1/8, 0] with R = 1/2; token 0 owns [0, 3/4) of it, and
    # u_smp = 5/8 lies 1/8 below that edge.
    p = [np.array([0.5, 0.125, 0.25, 0.125]), np.array([0.25, 0.25, 0.25, 0.25])]
    q = [np.array([0.125, 0.5, 0.125, 0.25])]
    d = ov.decide_sampled(p, q, [1], [0.5], [0.625, 0.0])
    assert d.n_accepted == 0 and d.mode == ov.RESIDUAL
    assert d.tokens == [0]
    assert d.acc_margin == [0.25]
    assert d.mass_total == 0.5
    assert d.cdf_margin == 0.125
    # u_smp = 13/16: threshold 13/32 > 3/8, so token 2 ([3/4, 1)) at 1/16.
    d2 = ov.decide_sampled(p, q, [1], [0.5], [0.8125, 0.0])
    assert d2.tokens == [2] and d2.cdf_margin == 0.0625
    np.testing.assert_array_equal(ov.draw_mass(p, q, 0, 1), [0.375, 0.0, 0.125, 0.0])


PINS = [pin_acceptance_margin, pin_draw_margin, pin_residual_draw_margin]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_margin_pins_hold_on_the_oracle(pin):
    pin()


# ------------------------------------------------------- planted mistakes ---

def _inverse_cdf_with(margin_of):
    def mutant(mass, u):
        total = float(np.sum(mass))
        cdf = np.cumsum(mass)
        hits = np.nonzero(cdf > u * total)[0]
        y = int(hits[0]) if hits.size else int(np.nonzero(mass > 0.0)[0][-1])
        return y, margin_of(cdf, total, y, u), total
    return mutant


def _margin_zero(cdf, total, y, u):
    return 0.0


def _margin_not_normalised(cdf, total, y, u):
    c_prev = float(cdf[y - 1]) if y > 0 else 0.0
    return min(abs(u - c_prev), abs(float(cdf[y]) - u))


def _margin_next_edge(cdf, total, y, u):
    # Upper edge taken one token too far.
    c_prev = float(cdf[y - 1]) if y > 0 else 0.0
    c_hi = float(cdf[min(y + 1, len(cdf) - 1)])
    return min(abs(u - c_prev / total), abs(c_hi / total - u))


def _margin_lower_edge_only(cdf, total, y, u):
    c_prev = float(cdf[y - 1]) if y > 0 else 0.0
    return abs(u - c_prev / total)


_ORIGINAL_ACCEPT = ov.accept_decision


def _accept_margin_zero(u, p_x, q_x):
    ok, _ = _ORIGINAL_ACCEPT(u, p_x, q_x)
    return ok, 0.0


def _accept_uncapped(u, p_x, q_x):
    if q_x > 0.0:
        return u < min(1.0, p_x / q_x), abs(u - p_x / q_x)
    return (p_x > 0.0), math.inf


def _draw_mass_unnormalised_q(p_rows, q_rows, j, k):
    # Residual against a drafter row scaled by 2 (a normaliser taken twice).
    if j < k:
        return np.maximum(0.0, np.asarray(p_rows[j]) - 0.5 * np.asarray(q_rows[j]))
    return np.asarray(p_rows[k], dtype=np.float64)


MUTANTS = {
    "draw margin always 0": ("inverse_cdf", _inverse_cdf_with(_margin_zero)),
    "draw margin not divided by R": ("inverse_cdf", _inverse_cdf_with(_margin_not_normalised)),
    "draw margin at the next token's edge": ("inverse_cdf", _inverse_cdf_with(_margin_next_edge)),
    "draw margin at the lower edge only": ("inverse_cdf",
                                           _inverse_cdf_with(_margin_lower_edge_only)),
    "acceptance margin always 0": ("accept_decision", _accept_margin_zero),
    "acceptance margin against the uncapped ratio": ("accept_decision", _accept_uncapped),
    "residual against a mis-normalised drafter row": ("draw_mass", _draw_mass_unnormalised_q),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_every_planted_mistake_fails_a_pin(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(ov, attr, fn)          # planted in the oracle module
    failed = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {name!r} passed every pin"


# ------------------------------------------------------------- the checker ---

def _decision(p, q, drafted, u_acc, u_smp):
    return ov.decide_sampled(p, q, drafted, u_acc, u_smp)


P = [np.array([0.5, 0.125, 0.25, 0.125]), np.array([0.25, 0.25, 0.25, 0.25])]
Q = [np.array([0.125, 0.5, 0.125, 0.25])]


def _mass_fn(decisions):
    return lambda n: ov.draw_mass(P, Q, decisions[n].n_accepted, 1)


def test_checker_passes_identical_outputs():
    d = _decision(P, Q, [1], [0.5], [0.625, 0.0])
    cmp = compare_sampled([[0, -1]], [0], [d], 1, [[1]], _mass_fn([d]))
    assert cmp.unexcused == [] and cmp.n_excused == 0


def test_checker_excuses_an_acceptance_within_the_band_only():
    # p/q = 1/4: u_acc just below it keeps the token; the library rejecting
    # instead is excused only while the oracle's margin is under 1e-6.
    near = _decision(P, Q, [1], [0.25 - 2.0 ** -24], [0.625, 0.0])
    assert near.n_accepted == 1
    cmp = compare_sampled([[0, -1]], [0], [near], 1, [[1]], _mass_fn([near]))
    assert cmp.unexcused == [] and cmp.excused[0][1] == "accept"
    far = _decision(P, Q, [1], [0.125], [0.625, 0.0])
    cmp = compare_sampled([[0, -1]], [0], [far], 1, [[1]], _mass_fn([far]))
    assert cmp.unexcused and cmp.unexcused[0][1] == "accept"


def test_checker_never_excuses_a_kept_token_that_was_not_drafted():
    near = _decision(P, Q, [1], [0.25 - 2.0 ** -24], [0.625, 0.0])
    # Count 1 (kept) agrees with the oracle, but the kept token is wrong.
    cmp = compare_sampled([[3, 0]], [1], [near], 1, [[1]], _mass_fn([near]))
    assert cmp.unexcused and "drafted" in cmp.unexcused[0][1]
    cmp = compare_sampled([[1, 0]], [1], [near], 1, [[1]], _mass_fn([near]))
    assert cmp.unexcused == []


def test_checker_excuses_only_a_neighbour_across_the_near_edge():
    # Residual [3/8, 0, 1/8, 0] / R: token 0 owns [0, 3/4), token 2 [3/4, 1).
    at_edge = _decision(P, Q, [1], [0.5], [0.75 - 2.0 ** -24, 0.0])
    assert at_edge.tokens == [0]
    ok = compare_sampled([[2, -1]], [0], [at_edge], 1, [[1]], _mass_fn([at_edge]))
    assert ok.unexcused == [] and ok.excused[0][1] == "sample"
    # Token 1 and token 3 have no residual mass: never excused.
    for bad in (1, 3):
        cmp = compare_sampled([[bad, -1]], [0], [at_edge], 1, [[1]], _mass_fn([at_edge]))
        assert cmp.unexcused, bad
    # Far from any edge, the neighbour is not excused either.
    mid = _decision(P, Q, [1], [0.5], [0.375, 0.0])
    cmp = compare_sampled([[2, -1]], [0], [mid], 1, [[1]], _mass_fn([mid]))
    assert cmp.unexcused and cmp.unexcused[0][1] == "sample"


def test_checker_rejects_bad_padding_and_counts():
    d = _decision(P, Q, [1], [0.5], [0.625, 0.0])
    assert compare_sampled([[0, 5]], [0], [d], 1, [[1]], _mass_fn([d])).unexcused
    assert compare_sampled([[0, -1]], [2], [d], 1, [[1]], _mass_fn([d])).unexcused
