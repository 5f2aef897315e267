"""Shared test plumbing: moving tensors into the oracle's numpy layout and
comparing library outputs with the oracle under the parity bar.

The parity bar (for sampled verification the method is randomised, so the
oracle runs the same algorithm with the same Philox numbers):

* greedy (T == 0): accepted counts and emitted tokens bit-exact;
* p_i(x_i) and q_i(x_i): |gpu - oracle| <= 1e-5 * oracle where the oracle's
  value is >= 1e-30; below that the library's value must itself be <= 1e-30;
* sampled decisions identical, except where a decision of the oracle lies
  within 1e-6 of its threshold. What may be excused, and what never is:
  - the library's kept tokens must always be the drafted tokens, its padding
    -1, and its count within the budget;
  - every acceptance the library's count implies (kept before it, rejected at
    it) must equal the oracle's at that position, unless the oracle's margin
    |u_acc - min(1, p/q)| there is below 1e-6;
  - on the same acceptance path, a different drawn token is excused only if
    it has mass in the oracle's draw and u_smp lies within 1e-6 of that
    token's own normalised CDF interval [C(y-1)/R, C(y)/R) (so it is a
    neighbour across the near edge, never an arbitrary token).
  Excused requests are counted per test in NEAR_TIES, with the smallest
  residual mass R seen, and reported at the end of the session.
"""
from __future__ import annotations

import math

import numpy as np
import torch

PROB_RTOL = 1e-5
PROB_FLOOR = 1e-30
NEAR_TIE = 1e-6

# tag -> {"requests", "excused_accept", "excused_sample", "unexcused",
#         "min_residual_R", "excused_R"}: filled by record_near_ties().
NEAR_TIES: dict = {}


def to_oracle(x: torch.Tensor):
    """A logits tensor as the oracle's storage: float array or bf16 bit patterns."""
    x = x.detach().cpu()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view(np.uint16), "bf16"
    return x.numpy(), "f32"


def check_probabilities(gpu_p, ora_p, budgets, rtol=None):
    """p_x / q_x parity on every budgeted position (rtol: an array of
    per-position relative tolerances, default PROB_RTOL everywhere)."""
    gpu_p = np.asarray(gpu_p, dtype=np.float64)
    bad = []
    for n, k in enumerate(budgets):
        for i in range(int(k)):
            o, g = ora_p[n, i], gpu_p[n, i]
            tol = PROB_RTOL if rtol is None else float(rtol[n, i])
            if o >= PROB_FLOOR:
                ok = abs(g - o) <= tol * o
            else:
                ok = 0.0 <= g <= PROB_FLOOR
            if not ok:
                bad.append((n, i, float(g), float(o)))
    return bad


def padded(tokens, K):
    out = [int(t) for t in tokens] + [-1] * (K + 1 - len(tokens))
    return out


class Comparison:
    """Outcome of compare_sampled over a set of requests."""

    def __init__(self):
        self.requests = 0
        self.excused = []        # (request, "accept"|"sample", position, margin, R)
        self.unexcused = []      # (request, reason, details...)
        self.min_residual_R = math.inf

    @property
    def n_excused(self):
        return len(self.excused)


def compare_sampled(gpu_tokens, gpu_n, decisions, K, drafted, mass_fn,
                    acc_window=None, cdf_window=None) -> Comparison:
    """Compare sampled outputs with the oracle's decisions, excusing near-ties.

    drafted[n]: request n's drafted tokens (at least its budget's worth).
    mass_fn(n): the oracle's draw mass vector of request n (called only when
    the drawn tokens differ on the same acceptance path).
    acc_window[n][i] and cdf_window[n] widen the near-tie band of request n's
    acceptance at position i and of its draw (default NEAR_TIE).
    """
    out = Comparison()
    for n, d in enumerate(decisions):
        out.requests += 1
        k = len(d.accepted)
        if d.mode == "residual":
            out.min_residual_R = min(out.min_residual_R, float(d.mass_total))
        g_n = int(gpu_n[n])
        g_tok = [int(t) for t in gpu_tokens[n]]
        if not 0 <= g_n <= k:
            out.unexcused.append((n, "count outside the budget", g_n, k))
            continue
        if g_tok[:g_n] != [int(x) for x in drafted[n][:g_n]]:
            out.unexcused.append((n, "kept tokens are not the drafted ones", g_tok, g_n))
            continue
        if any(t != -1 for t in g_tok[g_n + 1:]):
            out.unexcused.append((n, "padding is not -1", g_tok))
            continue
        # Every acceptance the library's count implies, against the oracle's.
        flipped = []
        for i in range(min(g_n + 1, k)):
            g_acc = i < g_n
            if g_acc != bool(d.accepted[i]):
                flipped.append(i)
        bad_flip = False
        for i in flipped:
            band = NEAR_TIE if acc_window is None else float(acc_window[n][i])
            if d.acc_margin[i] < band:
                out.excused.append((n, "accept", i, float(d.acc_margin[i]), d.mass_total))
            else:
                out.unexcused.append((n, "accept", i, g_n, d.n_accepted, d.acc_margin[i]))
                bad_flip = True
        if bad_flip or g_n != d.n_accepted:
            continue
        # Same acceptance path: only the drawn token can differ.
        y_g, y_o = g_tok[g_n], int(d.tokens[-1])
        if y_g == y_o:
            continue
        band = NEAR_TIE if cdf_window is None else float(cdf_window[n])
        mass = np.asarray(mass_fn(n), dtype=np.float64)
        u = float(d.u_smp[g_n])
        ok = 0 <= y_g < mass.size and mass[y_g] > 0.0
        if ok:
            from oracle import verify as ov
            lo, hi = ov.cdf_interval(mass, y_g)
            ok = lo - band <= u < hi + band
        if ok:
            out.excused.append((n, "sample", g_n, float(d.cdf_margin), d.mass_total))
        else:
            out.unexcused.append((n, "sample", g_n, y_g, y_o, d.cdf_margin, d.mass_total))
    return out


def record_near_ties(tag: str, cmp: Comparison):
    """Add a comparison's counts to the session's near-tie record."""
    rec = NEAR_TIES.setdefault(tag, {"requests": 0, "excused_accept": 0, "excused_sample": 0,
                                     "unexcused": 0, "min_residual_R": math.inf,
                                     "excused_R": []})
    rec["requests"] += cmp.requests
    rec["excused_accept"] += sum(1 for e in cmp.excused if e[1] == "accept")
    rec["excused_sample"] += sum(1 for e in cmp.excused if e[1] == "sample")
    rec["unexcused"] += len(cmp.unexcused)
    rec["min_residual_R"] = min(rec["min_residual_R"], cmp.min_residual_R)
    rec["excused_R"] += [float(e[4]) for e in cmp.excused if e[4] == e[4]]


def near_tie_summary():
    """Totals over the session's record, or None when nothing was compared."""
    if not NEAR_TIES:
        return None
    tot = {"tests": len(NEAR_TIES), "requests": 0, "excused_accept": 0, "excused_sample": 0,
           "unexcused": 0, "min_residual_R": math.inf}
    for rec in NEAR_TIES.values():
        for key in ("requests", "excused_accept", "excused_sample", "unexcused"):
            tot[key] += rec[key]
        tot["min_residual_R"] = min(tot["min_residual_R"], rec["min_residual_R"])
    return tot


def logits_mass_fn(target, draft, budgets, requests, decisions, temperature):
    """mass_fn for compare_sampled on logit inputs: request n of the compared
    set is row requests[n] of target [B, K+1, V] and draft [B, K, V] (torch
    tensors); its draw mass is recomputed by the oracle from those rows."""
    from oracle import verify as ov

    def fn(n):
        b = int(requests[n])
        k = int(budgets[b])
        zt, fmt = to_oracle(target[b, : k + 1])
        zd, _ = to_oracle(draft[b, :k])
        return ov.request_draw_mass(ov.as_f64_rows(zt, fmt), ov.as_f64_rows(zd, fmt),
                                    decisions[n].n_accepted, k, float(temperature))
    return fn


def assert_sampled(tag, gpu_tokens, gpu_n, decisions, K, drafted, mass_fn, log=None,
                   acc_window=None, cdf_window=None) -> Comparison:
    """compare_sampled, recorded under tag; fails on any unexcused request."""
    cmp = compare_sampled(gpu_tokens, gpu_n, decisions, K, drafted, mass_fn,
                          acc_window=acc_window, cdf_window=cdf_window)
    record_near_ties(tag, cmp)
    if log is not None:
        log(f"[{tag}] requests={cmp.requests} excused near-ties={cmp.n_excused} "
            f"unexcused={len(cmp.unexcused)} min residual R={cmp.min_residual_R:.3g}")
    assert not cmp.unexcused, (tag, cmp.unexcused[:5])
    return cmp
