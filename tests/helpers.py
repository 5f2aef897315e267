"""Shared test plumbing: moving tensors into the oracle's numpy layout and
comparing library outputs with the oracle under the parity bar.

The parity bar (for sampled verification the method is randomised, so the
oracle runs the same algorithm with the same Philox numbers):

* greedy (T == 0): accepted counts and emitted tokens bit-exact;
* p_i(x_i) and q_i(x_i): |gpu - oracle| <= 1e-5 * oracle where the oracle's
  value is >= 1e-30; below that the library's value must itself be <= 1e-30;
* sampled decisions identical, except where the oracle's first diverging
  decision lies within 1e-6 of its threshold (|u_acc - min(1, p/q)| < 1e-6,
  or u_smp within 1e-6 of an edge of the chosen token's normalised CDF
  interval); such excused requests are counted and returned.
"""
from __future__ import annotations

import numpy as np
import torch

PROB_RTOL = 1e-5
PROB_FLOOR = 1e-30
NEAR_TIE = 1e-6


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


def compare_sampled(gpu_tokens, gpu_n, decisions, K, acc_window=None, cdf_window=None):
    """Compare sampled outputs with the oracle's decisions, excusing near-ties.

    acc_window[n][i] and cdf_window[n] widen the near-tie band of request n's
    acceptance at position i and of its draw (default NEAR_TIE).
    Returns (n_excused, unexcused) where unexcused lists the requests whose
    first diverging decision was not within the near-tie band.
    """
    excused, unexcused = 0, []
    for n, d in enumerate(decisions):
        g_n = int(gpu_n[n])
        g_tok = [int(t) for t in gpu_tokens[n]]
        o_tok = padded(d.tokens, K)
        if g_n == d.n_accepted and g_tok == o_tok:
            continue
        if g_n != d.n_accepted:
            i = min(g_n, d.n_accepted)        # first position decided differently
            margin = d.acc_margin[i] if i < len(d.acc_margin) else np.inf
            band = NEAR_TIE if acc_window is None else float(acc_window[n][i])
            if margin < band:
                excused += 1
            else:
                unexcused.append((n, "accept", i, g_n, d.n_accepted, margin))
            continue
        # Same acceptance path: only the drawn token can differ.
        band = NEAR_TIE if cdf_window is None else float(cdf_window[n])
        if d.cdf_margin < band:
            excused += 1
        else:
            unexcused.append((n, "sample", d.n_accepted, g_tok, o_tok, d.cdf_margin,
                              d.mass_total))
    return excused, unexcused
