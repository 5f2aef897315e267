"""GPU parity of verification from hidden states (spec_verify_hidden) against
the fp64 oracle (oracle/hidden.py) on the same bf16 inputs, through the C ABI.

Tolerances follow from the arithmetic. Each logit is an fp32 sum of H exact
bf16 products, within E = 4 sqrt(H) 2^-24 max_v sum_i |h_i w_vi| of the fp64
value (the output head's bound, a factor 4 of margin). A logit error of at
most E moves ln p(x) by at most 2E / T, so:

* p_i(x_i), q_i(x_i): relative error within 1e-5 + 2E / T (E of that row);
* acceptance: the ratio p/q moves by at most (2E_t + 2E_d) / T relative plus
  the fp32 rounding of both, so a first divergence is excused when the
  oracle's |u - min(1, p/q)| is within 1e-6 + min(1, p/q) (2E_t + 2E_d) / T
  + 2e-5 of the threshold;
* the draw: the mass vector moves by at most (eps_p + eps_q) in total
  (eps = 2E / T + 1e-5 relative per row), so each normalised CDF edge moves by
  at most 2 (eps_p + eps_q) / R, and a different token is excused within
  1e-6 plus that of an edge;
* greedy: the target's token must be the oracle's argmax unless the oracle's
  top two logits are within 2E; then it must point at a logit within 2E of
  the maximum (checked at the first diverging position).

Excused cases are counted and printed.
"""
import math
import sys

import numpy as np
import pytest
import torch
from scipy import special, stats

from draft_verify_sampling_spec_amd import HiddenVerify, binding
from oracle import head as oh
from oracle import hidden as ohid
from tests.helpers import NEAR_TIE, PROB_RTOL, assert_sampled, check_probabilities, padded
from oracle import verify as ov
from workloads import make_hidden_inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _gpu(inp, T, seed, hv=None, stream=None):
    B, K1, _ = inp["target_hidden"].shape
    V = inp["head"].shape[0]
    hv = hv or HiddenVerify(DEV, B, K1 - 1, V)
    dh = inp["draft_hidden"] if T > 0 else None
    out = hv.run(inp["target_hidden"], dh, inp["head"], inp["tokens"], inp["budgets"], T, seed,
                 stream=stream)
    torch.cuda.synchronize()
    return tuple(x.cpu().numpy() for x in out)


class Host:
    """Host copies of one input set, with the fp64 head decoded once."""

    def __init__(self, inp):
        self.th = _bits(inp["target_hidden"])
        self.dh = _bits(inp["draft_hidden"])
        self.w64 = oh.bf16_bits_to_f64(_bits(inp["head"]))
        self.aw = np.abs(self.w64)
        self.tokens = inp["tokens"].cpu().numpy()
        self.budgets = inp["budgets"].cpu().numpy()
        self.H = self.th.shape[2]

    def bound(self, rows_bits):
        """E for each row of hidden states (bf16 bits [n, H])."""
        h = np.abs(oh.bf16_bits_to_f64(rows_bits))
        return 4.0 * math.sqrt(self.H) * 2.0 ** -24 * (h @ self.aw.T).max(axis=1)

    def oracle(self, T, seed, requests):
        return ohid.verify_from_hidden(self.th, self.dh if T > 0 else None, None, self.tokens,
                                       self.budgets, T, seed, requests=requests,
                                       head_f64=self.w64)


def _assert_greedy(host, gpu, res, reqs, tag):
    toks, nacc, p, q, status = gpu
    K = host.tokens.shape[1]
    excused = 0
    for n, b in enumerate(reqs):
        d = res.decisions[n]
        g_tok = [int(t) for t in toks[b]]
        if int(nacc[b]) == d.n_accepted and g_tok == padded(d.tokens, K):
            continue
        # First position where the two runs took a different target token.
        i = min(int(nacc[b]), d.n_accepted)
        g_choice = g_tok[i]
        z = oh.logits(oh.bf16_bits_to_f64(host.th[b, i:i + 1]), host.w64)[0]
        e = host.bound(host.th[b, i:i + 1])[0]
        top = np.sort(z)[-2:] if z.size > 1 else np.array([-np.inf, z[0]])
        assert top[1] - top[0] <= 2 * e, (tag, int(b), i, "argmax not a near-tie")
        assert 0 <= g_choice < z.size and z[g_choice] >= top[1] - 2 * e, (tag, int(b), i)
        excused += 1
    assert np.all(np.isnan(p[reqs])) and np.all(np.isnan(q[reqs]))
    _log(f"[{tag}] greedy requests={len(reqs)} excused near-ties={excused}")


def _assert_sampled(host, gpu, res, reqs, T, tag):
    toks, nacc, p, q, status = gpu
    K = host.tokens.shape[1]
    budgets = host.budgets[reqs]
    ora_p = np.full((len(reqs), K), np.nan)
    ora_q = np.full((len(reqs), K), np.nan)
    rt_p = np.full((len(reqs), K), PROB_RTOL)
    rt_q = np.full((len(reqs), K), PROB_RTOL)
    acc_w, cdf_w = [], []
    for n, b in enumerate(reqs):
        d = res.decisions[n]
        k = int(budgets[n])
        et = host.bound(host.th[b, : k + 1])
        ed = host.bound(host.dh[b, :k]) if k else np.zeros(0)
        ora_p[n, :k] = d.p_x
        ora_q[n, :k] = d.q_x
        rt_p[n, :k] += 2 * et[:k] / T
        rt_q[n, :k] += 2 * ed / T
        ratio = np.array([min(1.0, px / qx) if qx > 0 else 1.0 for px, qx in zip(d.p_x, d.q_x)])
        acc_w.append(NEAR_TIE + ratio * (2 * et[:k] + 2 * ed) / T + 2e-5)
        j = d.n_accepted
        eps_p = 2 * et[j] / T + 1e-5
        eps_q = (2 * ed[j] / T + 1e-5) if j < k else 0.0
        cdf_w.append(NEAR_TIE + 2 * (eps_p + eps_q) / max(d.mass_total, 1e-300))
    bad_p = check_probabilities(p[reqs], ora_p, budgets, rtol=rt_p)
    bad_q = check_probabilities(q[reqs], ora_q, budgets, rtol=rt_q)
    assert not bad_p, (tag, "p_x", bad_p[:5])
    assert not bad_q, (tag, "q_x", bad_q[:5])
    for n, kb in enumerate(budgets):
        assert np.all(np.isnan(p[reqs[n], kb:])) and np.all(np.isnan(q[reqs[n], kb:]))
    def mass_fn(n):
        b, k = int(reqs[n]), int(budgets[n])
        zt = oh.logits(ohid.decode_states(host.th[b, : k + 1]), host.w64)
        zd = oh.logits(ohid.decode_states(host.dh[b, :k]), host.w64)
        return ov.request_draw_mass(zt, zd, res.decisions[n].n_accepted, k, T)

    assert_sampled(tag, toks[reqs], nacc[reqs], res.decisions, K, host.tokens[reqs], mass_fn,
                   log=_log, acc_window=acc_w, cdf_window=cdf_w)


def _check(inp, T, seed, tag, reqs=None, gpu=None):
    gpu = gpu or _gpu(inp, T, seed)
    assert int(gpu[4][0]) == 0, f"status flags {int(gpu[4][0]):#x}"
    host = Host(inp)
    B = host.tokens.shape[0]
    reqs = np.arange(B) if reqs is None else np.asarray(reqs)
    res = host.oracle(T, seed, reqs)
    if T == 0:
        _assert_greedy(host, gpu, res, reqs, tag)
    else:
        _assert_sampled(host, gpu, res, reqs, T, tag)
    return gpu


# Shapes spanning several row and vocabulary tiles with ragged tails, an H
# that is not a multiple of the 64-wide k-step, K = 0, and budgets from 0 to K.
SHAPES = [(7, 4, 64, 1000), (16, 3, 72, 517), (5, 0, 64, 300), (33, 6, 136, 4099),
          (40, 8, 256, 2048), (3, 2, 8, 5)]


@pytest.mark.parametrize("B,K,H,V", SHAPES)
@pytest.mark.parametrize("T", [1.0, 0.7, 0.0])
def test_small_shapes_match_oracle(B, K, H, V, T):
    seed = (B << 32) | (K * 131 + V)
    _log(f"[hidden] B={B} K={K} H={H} V={V} T={T}")
    rng = np.random.default_rng(B + V)
    budgets = rng.integers(0, K + 1, size=B) if K else np.zeros(B, dtype=np.int64)
    inp = make_hidden_inputs(B, K, H, V, seed=B * 31 + V, device=DEV, budgets=budgets)
    _check(inp, T, seed, f"B={B} K={K} H={H} V={V} T={T}")


@pytest.mark.parametrize("T", [1.0, 0.0])
def test_many_row_products_every_request(T):
    """A batch large enough for the many-row product in both launches: the
    scored rows' statistics (at least 1,536 rows bound, 40 vocabulary tiles)
    and, sampled, the draw rows' logits (B = 512 gives 1,024 draw rows; at
    least 64 vocabulary tiles), with V not a multiple of 4 (the logits'
    4-wide stores fall back to single ones): every request against the
    oracle."""
    B, K, H, V = 512, 3, 64, 16421
    _log(f"[hidden] many-row products B={B} K={K} H={H} V={V} T={T}")
    rng = np.random.default_rng(77)
    budgets = rng.integers(0, K + 1, size=B)
    inp = make_hidden_inputs(B, K, H, V, seed=77, device=DEV, budgets=budgets)
    _check(inp, T, (77 << 32) | 5, f"many-row B={B} K={K} H={H} V={V} T={T}")


def test_paired_draw_rows_with_a_partial_group_of_eight():
    """The draw masses' paired rows when B is not a multiple of 8 (B = 517:
    requests 512..516 share a group of eight with three padding requests,
    whose rows are rows of zeros), with budgets from 0 to K: every request
    against the oracle."""
    B, K, H, V = 517, 2, 64, 16421
    _log(f"[hidden] paired rows B={B} K={K} H={H} V={V}")
    rng = np.random.default_rng(78)
    budgets = rng.integers(0, K + 1, size=B)
    inp = make_hidden_inputs(B, K, H, V, seed=78, device=DEV, budgets=budgets)
    _check(inp, 1.0, (78 << 32) | 5, f"paired B={B} K={K} H={H} V={V}")


def test_q_equal_p_accepts_everything():
    inp = make_hidden_inputs(64, 5, 128, 3000, seed=3, device=DEV, variant="q_eq_p")
    toks, nacc, p, q, status = _gpu(inp, 1.0, 77)
    assert int(status[0]) == 0
    assert np.array_equal(nacc, inp["budgets"].cpu().numpy())
    assert np.array_equal(p, q, equal_nan=True)


def _chi2_pvalue(observed, expected_p):
    exp = expected_p * observed.sum()
    order = np.argsort(exp)
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


def test_emitted_tokens_follow_the_target_softmax():
    """16,000 independent trials of one position set (drafted tokens drawn
    from q): the emitted token at each reached position follows
    softmax(h_t W^T / T) (scipy on fp64 logits), and the mean accepted count
    matches sum_n prod_{l<n} sum_v min(p_l, q_l)."""
    T, B, K, H, V = 1.0, 16000, 2, 16, 16
    inp = make_hidden_inputs(B, K, H, V, seed=21, device=DEV, variant="sampled", temperature=T)
    toks, nacc, p, q, status = _gpu(inp, T, 0x5EED0003)
    assert int(status[0]) == 0
    w = inp["head"].float().double().cpu().numpy()
    zt = inp["target_hidden"][0].float().double().cpu().numpy() @ w.T
    zd = inp["draft_hidden"][0].float().double().cpu().numpy() @ w.T
    pt, qd = special.softmax(zt / T, axis=1), special.softmax(zd / T, axis=1)
    for i in range(K + 1):
        emitted = toks[nacc >= i, i]
        assert np.all((emitted >= 0) & (emitted < V))
        observed = np.bincount(emitted, minlength=V).astype(float)
        assert _chi2_pvalue(observed, pt[i]) > 1e-3, i
    alpha = [np.minimum(pt[i], qd[i]).sum() for i in range(K)]
    expected = sum(np.prod(alpha[:n]) for n in range(1, K + 1))
    se = nacc.std(ddof=1) / np.sqrt(B)
    assert abs(nacc.mean() - expected) < 4 * se, (nacc.mean(), expected, se)


@pytest.fixture(scope="module")
def heavy():
    """The heavy batch from hidden states: B = 512, K = 8, H = 2,560,
    V = 151,936, budgets 2 + Binomial(6, 1/3)."""
    _log("[hidden] heavy inputs")
    inp = make_hidden_inputs(512, 8, 2560, 151936, seed=5, device=DEV)
    return inp, HiddenVerify(DEV, 512, 8, 151936)


def _invariants(inp, gpu, T):
    toks, nacc, p, q, status = gpu
    budgets = inp["budgets"].cpu().numpy()
    V = inp["head"].shape[0]
    assert int(status[0]) == 0
    assert np.all((nacc >= 0) & (nacc <= budgets))
    for b in range(len(budgets)):
        j = int(nacc[b])
        assert np.all((toks[b, : j + 1] >= 0) & (toks[b, : j + 1] < V))
        assert np.all(toks[b, j + 1:] == -1)
        if T > 0:
            k = int(budgets[b])
            assert np.all((p[b, :k] >= 0) & (p[b, :k] <= 1) & (q[b, :k] >= 0) & (q[b, :k] <= 1))


def test_heavy_sampled_full_launch(heavy):
    inp, hv = heavy
    seed = (5 << 32) | 1
    gpu = _gpu(inp, 1.0, seed, hv=hv)
    _invariants(inp, gpu, 1.0)
    toks, nacc = gpu[0], gpu[1]
    budgets = inp["budgets"].cpu().numpy()
    # The oracle recomputes a few requests: residual draws and bonus draws.
    resid = [b for b in range(512) if nacc[b] < budgets[b]][:4]
    bonus = [b for b in range(512) if nacc[b] == budgets[b]][:2]
    _log(f"[hidden] heavy sampled: oracle on requests {resid + bonus}")
    _check(inp, 1.0, seed, "heavy sampled", reqs=resid + bonus, gpu=gpu)


def test_heavy_greedy(heavy):
    inp, hv = heavy
    gpu = _gpu(inp, 0.0, 0, hv=hv)
    _invariants(inp, gpu, 0.0)
    _log("[hidden] heavy greedy: oracle on 12 requests")
    _check(inp, 0.0, 0, "heavy greedy", reqs=list(range(0, 512, 43)), gpu=gpu)


def test_bad_budget_and_token_set_status_flags():
    B, K, H, V = 6, 3, 64, 700
    budgets = np.array([3, -1, 2, 4, 1, 3])
    inp = make_hidden_inputs(B, K, H, V, seed=9, device=DEV, budgets=budgets)
    inp["tokens"][4, 0] = -5
    inp["tokens"][5, 1] = V
    for T, want in ((1.0, 0x3), (0.0, 0x3)):
        toks, nacc, p, q, status = _gpu(inp, T, 4)
        assert int(status[0]) == want
    # A clean call writes (does not accumulate) the flags.
    good = make_hidden_inputs(B, K, H, V, seed=9, device=DEV)
    assert int(_gpu(good, 1.0, 4)[4][0]) == 0


def test_empty_batch_is_a_no_op():
    out = torch.full((4,), 7, dtype=torch.int32, device=DEV)
    rc = binding.spec_verify_hidden(None, None, None, None, None, 0, 4, 64, 100, 1.0, 0,
                                    out.data_ptr(), out.data_ptr(), None, None, None, None, 0,
                                    None)
    torch.cuda.synchronize()
    assert rc == binding.SV_OK and out.cpu().tolist() == [7, 7, 7, 7]


def test_repeat_calls_are_deterministic_and_stream_ordered():
    inp = make_hidden_inputs(24, 5, 128, 4000, seed=12, device=DEV)
    hv = HiddenVerify(DEV, 24, 5, 4000)
    a = _gpu(inp, 0.8, 99, hv=hv)
    s = torch.cuda.Stream(device=DEV)
    with torch.cuda.stream(s):
        b = _gpu(inp, 0.8, 99, hv=hv, stream=s)
    for x, y in zip(a, b):
        assert np.array_equal(x, y, equal_nan=True)
