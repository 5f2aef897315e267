"""Pins of the scheduler oracle (oracle/schedule.py): hand-worked budgets,
brute-force optimality on tiny batches, the meaning of the objective by
simulation, and invariants."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import schedule as osch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "schedule_cases.json")


def test_golden_budgets():
    cases = json.load(open(GOLDEN))["cases"]
    for case in cases:
        conf = np.asarray(case["conf"], dtype=np.float32)
        for run in case["runs"]:
            got = osch.schedule(conf, run["N"], run["tau"])
            assert got.tolist() == run["budgets"], (case["conf"], run)


def _brute_best(conf, n_total, tau):
    """max over all budget vectors with sum <= N of sum_b E_b(k_b) - tau * sum_b k_b,
    with E_b(k) summed directly from the conditional survival chances."""
    c = np.asarray(conf, dtype=np.float64)
    B, K = c.shape
    best = -1.0
    for ks in itertools.product(range(K + 1), repeat=B):
        if sum(ks) > n_total:
            continue
        val = 0.0
        for b, k in enumerate(ks):
            alive = 1.0
            for n in range(k):
                alive *= c[b, n]
                val += alive - tau
        best = max(best, val)
    return best


@pytest.mark.parametrize("seed", range(12))
def test_allocation_is_optimal_by_brute_force(seed):
    rng = np.random.default_rng(seed)
    B, K = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    conf = rng.uniform(0.05, 1.0, size=(B, K)).astype(np.float32)
    for n_total in range(0, B * K + 2):
        for tau in (0.0, 0.3):
            ks = osch.schedule(conf, n_total, tau)
            val = osch.expected_accepted(conf, ks) - tau * int(ks.sum())
            best = _brute_best(conf, n_total, tau)
            # fp32 gains decide; the objective is fp64: equal up to fp32 rounding
            assert val >= best - 1e-6 * max(1.0, abs(best)), (n_total, tau, ks, val, best)


def test_expected_accepted_matches_simulation():
    """E_b(k) is the mean number of accepted drafts when position l survives
    with chance c[l] given that the earlier ones did."""
    rng = np.random.default_rng(5)
    conf = np.array([[0.9, 0.7, 0.8, 0.6, 0.95]], dtype=np.float32)
    trials = 200_000
    u = rng.random((trials, 5))
    survive = u < conf.astype(np.float64)[0]
    for k in range(6):
        accepted = np.cumprod(survive[:, :k], axis=1).sum(axis=1) if k else np.zeros(trials)
        mean = accepted.mean()
        exact = osch.expected_accepted(conf, [k])
        sd = accepted.std() / np.sqrt(trials)
        assert abs(mean - exact) < 5 * sd + 1e-12, (k, mean, exact)


def test_invariants_random():
    rng = np.random.default_rng(11)
    for _ in range(30):
        B, K = int(rng.integers(1, 40)), int(rng.integers(0, 9))
        conf = rng.uniform(0.0, 1.0, size=(B, K)).astype(np.float32)
        conf[rng.random((B, K)) < 0.1] = 1.0
        tau = float(rng.choice([0.0, 0.1, 0.5]))
        g = osch.gains_fp32(conf)
        above = int((g > np.float32(tau)).sum())
        prev = np.zeros(B, dtype=np.int32)
        for n_total in (0, 1, B, 2 * B, B * K, B * K + 3):
            ks = osch.schedule(conf, n_total, tau)
            assert ks.min() >= 0 and ks.max() <= K
            assert int(ks.sum()) == min(n_total, above)
            assert (ks >= prev).all()                      # monotone in N
            prev = ks
            for b in range(B):                             # taken set is every gain above the cut
                assert (g[b, : ks[b]] > np.float32(tau)).all()


def test_all_ones_fill_level_by_level():
    B, K = 7, 4
    conf = np.ones((B, K), dtype=np.float32)
    for n_total in range(B * K + 1):
        ks = osch.schedule(conf, n_total, 0.0)
        want = np.array([n_total // B + (1 if b < n_total % B else 0) for b in range(B)])
        assert ks.tolist() == want.tolist()


def test_clamping_and_gains():
    conf = np.array([[np.nan, 0.5], [1.5, -0.25], [0.5, 0.5]], dtype=np.float32)
    c = osch.clamp_confidences(conf)
    assert c.tolist() == [[0.0, 0.5], [1.0, 0.0], [0.5, 0.5]]
    g = osch.gains_fp32(conf)
    assert g.tolist() == [[0.0, 0.0], [1.0, 0.0], [0.5, 0.25]]
    assert g.dtype == np.float32
