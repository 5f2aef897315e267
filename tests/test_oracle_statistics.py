"""Statistical pins of the oracle on the tiny workload (B=1, K=4, V=32, T=1).

* Exactness (pages: "Speculative decoding becomes standard", section "Why
  draft-and-verify does not change the output", paragraph 2): over many
  independent trials with drafted tokens drawn from the drafter, the token
  emitted at each position (given the position is reached) follows the
  target's softmax. Checked with scipy's chi-square for a close, an
  adversarial and a very noisy drafter; the expected frequencies come from
  scipy's softmax, not from the oracle.
* Acceptance closed form: under x ~ q the chance that position i survives is
  sum_v min(p_i(v), q_i(v)), so the mean accepted count is
  sum_{n=1..k} prod_{l<n} alpha_l. The Monte-Carlo mean must sit within 4
  standard errors.

Each trial is one request of a batch of 20,000 identical requests; the
request index makes every trial's Philox numbers distinct, and the drafted
tokens come from a separate Gumbel-max draw (torch generator).
"""
import functools

import numpy as np
import pytest
from scipy import special, stats

from oracle import verify as ov
from tests.helpers import to_oracle
from workloads import make_inputs

TRIALS = 20000
SEED = 0x5EED0001


@functools.lru_cache(maxsize=None)
def _run(variant):
    inp = make_inputs("tiny", B=TRIALS, variant=variant)
    t, fmt = to_oracle(inp["target"])
    d, _ = to_oracle(inp["draft"])
    res = ov.verify_batch(t, d, inp["tokens"].numpy(), inp["budgets"].numpy(),
                          inp["temperature"], SEED, logits_format=fmt)
    return inp, t[0], d[0], res


def _chi2_pvalue(observed, expected_p):
    n = observed.sum()
    exp = expected_p * n
    order = np.argsort(exp)
    # Merge the smallest expected bins until each merged bin expects >= 5.
    obs_m, exp_m, acc_o, acc_e = [], [], 0.0, 0.0
    for idx in order:
        acc_o += observed[idx]
        acc_e += exp[idx]
        if acc_e >= 5.0:
            obs_m.append(acc_o)
            exp_m.append(acc_e)
            acc_o = acc_e = 0.0
    if acc_e > 0 and exp_m:
        obs_m[-1] += acc_o
        exp_m[-1] += acc_e
    obs_m, exp_m = np.array(obs_m), np.array(exp_m)
    exp_m *= obs_m.sum() / exp_m.sum()
    return stats.chisquare(obs_m, exp_m).pvalue


@pytest.mark.parametrize("variant", ["sampled", "adversarial", "noisy"])
def test_emitted_tokens_follow_target(variant):
    inp, zt, zd, res = _run(variant)
    K = zd.shape[0]
    T = inp["temperature"]
    for i in range(K + 1):
        reached = res.n_accepted >= i
        emitted = res.tokens[reached, i]
        assert np.all(emitted >= 0)
        if emitted.size < 200:
            continue
        observed = np.bincount(emitted, minlength=zt.shape[1]).astype(float)
        p = special.softmax(zt[i].astype(np.float64) / T)
        assert _chi2_pvalue(observed, p) > 1e-3, (variant, i)


@pytest.mark.parametrize("variant", ["sampled", "adversarial"])
def test_mean_accepted_matches_closed_form(variant):
    inp, zt, zd, res = _run(variant)
    K = zd.shape[0]
    T = inp["temperature"]
    alpha = []
    for i in range(K):
        p = special.softmax(zt[i].astype(np.float64) / T)
        q = special.softmax(zd[i].astype(np.float64) / T)
        alpha.append(np.minimum(p, q).sum())
    expected = sum(np.prod(alpha[:n]) for n in range(1, K + 1))
    got = res.n_accepted.astype(float)
    se = got.std(ddof=1) / np.sqrt(got.size)
    assert abs(got.mean() - expected) < 4 * se + 1e-12, (got.mean(), expected, se)


def test_q_equal_p_variant_accepts_every_token():
    inp = make_inputs("tiny", B=500, variant="q_eq_p")
    t, fmt = to_oracle(inp["target"])
    d, _ = to_oracle(inp["draft"])
    res = ov.verify_batch(t, d, inp["tokens"].numpy(), inp["budgets"].numpy(), 1.0, 3,
                          logits_format=fmt)
    assert np.all(res.n_accepted == 4)
