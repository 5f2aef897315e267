"""Pins of the hidden-state verify oracle (oracle/hidden.py).

* Greedy on a head that is the identity (bf16-exact), so each position's
  logits are its hidden state and the target's token is known by
  construction; expected outputs are written out by hand from the greedy
  rule (pages: "Speculative decoding becomes standard", section "Why
  draft-and-verify does not change the output", paragraph 1).
* q = p: drafter states equal to the target's give identical rows, so every
  drafted token survives (paragraph 2 of the same section: the ratio is 1).
* Exactness: with drafted tokens drawn from the drafter, the emitted token at
  each reached position follows softmax(h_t W^T / T), computed here with
  torch's own bf16 decoding and scipy's softmax; and the mean accepted count
  matches the closed form sum_n prod_{l<n} sum_v min(p_l, q_l). A swap of the
  two models' states or a shifted position fails these.
"""
import functools

import numpy as np
import pytest
import torch
from scipy import special, stats

from oracle import hidden as ohid
from workloads import make_hidden_inputs


def _bits(x: torch.Tensor) -> np.ndarray:
    return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _identity_case(targets, drafted, budgets, H=16):
    """Requests whose target token at position i is targets[b][i] (one-hot
    states, identity head)."""
    B = len(targets)
    K = len(drafted[0])
    th = torch.zeros(B, K + 1, H)
    for b in range(B):
        for i, a in enumerate(targets[b]):
            th[b, i, a] = 1.0
    head = torch.eye(H)
    return (_bits(th.to(torch.bfloat16)), _bits(head.to(torch.bfloat16)),
            np.asarray(drafted, dtype=np.int64), np.asarray(budgets, dtype=np.int64))


def test_greedy_identity_head_by_hand():
    targets = [[3, 1, 4, 1, 5], [2, 7, 1, 8, 2], [0, 0, 0, 0, 0], [6, 6, 6, 6, 6]]
    drafted = [[3, 1, 4, 2], [5, 7, 1, 8], [0, 0, 0, 0], [6, 6, 1, 6]]
    budgets = [4, 4, 2, 4]
    th, head, tok, bud = _identity_case(targets, drafted, budgets)
    res = ohid.verify_from_hidden(th, None, head, tok, bud, 0.0, seed=1)
    # Request 0: 3, 1, 4 agree, 2 != 1 -> keep 3 drafted, emit 1.
    # Request 1: 5 != 2 at once -> emit 2.
    # Request 2: budget 2, both agree -> bonus is the target token at row 2 (0).
    # Request 3: 6, 6 agree, 1 != 6 -> emit 6.
    assert list(res.n_accepted) == [3, 0, 2, 2]
    assert res.tokens[0].tolist() == [3, 1, 4, 1, -1]
    assert res.tokens[1].tolist() == [2, -1, -1, -1, -1]
    assert res.tokens[2].tolist() == [0, 0, 0, -1, -1]
    assert res.tokens[3].tolist() == [6, 6, 6, -1, -1]
    assert np.all(np.isnan(res.p_x)) and np.all(np.isnan(res.q_x))


def test_greedy_tie_takes_the_lowest_index():
    H = 8
    th = torch.zeros(1, 2, H)
    th[0, 0, 5] = th[0, 0, 2] = 1.0          # tie between 2 and 5
    th[0, 1, 7] = 1.0
    res = ohid.verify_from_hidden(_bits(th.to(torch.bfloat16)), None,
                                  _bits(torch.eye(H).to(torch.bfloat16)),
                                  np.array([[5]]), np.array([1]), 0.0, seed=0)
    assert res.n_accepted[0] == 0 and res.tokens[0].tolist() == [2, -1]


def test_q_equal_p_accepts_every_drafted_token():
    inp = make_hidden_inputs(64, 4, 32, 200, 11, device="cpu", variant="q_eq_p")
    res = ohid.verify_from_hidden(_bits(inp["target_hidden"]), _bits(inp["draft_hidden"]),
                                  _bits(inp["head"]), inp["tokens"].numpy(),
                                  inp["budgets"].numpy(), 1.0, seed=5)
    assert np.array_equal(res.n_accepted, inp["budgets"].numpy())
    for n, d in enumerate(res.decisions):
        assert d.mode == "bonus"
        assert np.allclose(d.p_x, d.q_x, rtol=0, atol=0)


TRIALS = 20000
SEED = 0x5EED0002


@functools.lru_cache(maxsize=None)
def _sampled_run(T):
    inp = make_hidden_inputs(TRIALS, 2, 16, 16, 21, device="cpu", variant="sampled",
                             temperature=T)
    res = ohid.verify_from_hidden(_bits(inp["target_hidden"]), _bits(inp["draft_hidden"]),
                                  _bits(inp["head"]), inp["tokens"].numpy(),
                                  inp["budgets"].numpy(), T, SEED)
    # Expected laws from torch's bf16 decoding and scipy, not from the oracle.
    w = inp["head"].float().double().numpy()
    zt = inp["target_hidden"][0].float().double().numpy() @ w.T
    zd = inp["draft_hidden"][0].float().double().numpy() @ w.T
    return res, special.softmax(zt / T, axis=1), special.softmax(zd / T, axis=1)


def _chi2_pvalue(observed, expected_p):
    exp = expected_p * observed.sum()
    order = np.argsort(exp)
    obs_m, exp_m, acc_o, acc_e = [], [], 0.0, 0.0
    for idx in order:                 # merge small bins until each expects >= 5
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


@pytest.mark.parametrize("T", [1.0, 0.6])
def test_emitted_tokens_follow_the_target_softmax(T):
    res, p, _ = _sampled_run(T)
    for i in range(p.shape[0]):
        reached = res.n_accepted >= i
        emitted = res.tokens[reached, i]
        assert np.all(emitted >= 0)
        observed = np.bincount(emitted, minlength=p.shape[1]).astype(float)
        assert _chi2_pvalue(observed, p[i]) > 1e-3, (T, i)


@pytest.mark.parametrize("T", [1.0, 0.6])
def test_mean_accepted_matches_closed_form(T):
    res, p, q = _sampled_run(T)
    K = q.shape[0]
    alpha = [np.minimum(p[i], q[i]).sum() for i in range(K)]
    expected = sum(np.prod(alpha[:n]) for n in range(1, K + 1))
    got = res.n_accepted.astype(float)
    se = got.std(ddof=1) / np.sqrt(got.size)
    assert abs(got.mean() - expected) < 4 * se, (got.mean(), expected, se)
