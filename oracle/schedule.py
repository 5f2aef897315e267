"""Plain CPU oracle of the confidence-driven verify-budget scheduler.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. It shares no
code with the HIP library and the library never calls it.

Sources (the pages' own titles and sections):

* "Speculative decoding becomes standard: DSpark and multi-token drafters",
  section "What DSpark adds", paragraph 2: every drafted position carries a
  confidence, read here as the chance it is accepted when all earlier
  positions of its block were; the scheduler sizes each request's verify
  window jointly across the whole batch, to get the most accepted tokens for
  the verification it pays for -- windows of four to six under moderate
  load, shorter ones as the engine fills up.
* "DSpark" (the finds page): the confidence report lets the server spend more
  verification on the requests likely to pay off, scaled to how busy the
  GPUs are.
* The Analytics Vidhya page on DSpark, section "Gotchas and Issues": the
  cutoff is not a static threshold but is recomputed for every batch from
  how busy the system is; only what has positive expected value is verified.

Readings (the pages give no formula; each is stated again in the design
notes of the repository):

* Confidences c[b, i] in [0, 1] are conditional survival probabilities, so
  request b, verified to budget k, accepts on average
  E_b(k) = sum_{n=1..k} prod_{l<n} c[b, l] drafted tokens. Extending its
  budget from k to k + 1 adds the gain g[b, k] = prod_{l<=k} c[b, l].
* The batch's load sets a verify budget of N drafted positions in total; a
  position is worth verifying only if its gain exceeds tau (the cost of a
  verified position in accepted tokens). The scheduler maximises
  sum_b E_b(k_b) subject to sum_b k_b <= N, 0 <= k_b <= K, by taking the N
  largest gains above tau. Gains never increase along a request's block
  (c <= 1), so the taken set is a prefix of every request and k_b is the
  number of positions taken from request b.
* Equal gains are taken in the order (position k ascending, then request b
  ascending), which keeps every request's taken set a prefix.
* The gains decide integers, so they are computed in fp32 (the precision
  the device uses), each as the left-to-right product
  ((c[b,0] * c[b,1]) * c[b,2]) ... rounded after every multiplication.
  Confidences outside [0, 1] are clamped into it; NaN counts as 0.
"""
from __future__ import annotations

import numpy as np


def clamp_confidences(conf) -> np.ndarray:
    """fp32 confidences with NaN -> 0 and values clamped to [0, 1]."""
    c = np.asarray(conf, dtype=np.float32)
    c = np.where(np.isnan(c), np.float32(0.0), c)
    return np.clip(c, np.float32(0.0), np.float32(1.0)).astype(np.float32)


def gains_fp32(conf) -> np.ndarray:
    """g[b, k] = prod_{l<=k} c[b, l], multiplied left to right in fp32
    (one IEEE rounding per product), shape [B, K]."""
    c = clamp_confidences(conf)
    B, K = c.shape
    g = np.zeros((B, K), dtype=np.float32)
    run = np.ones(B, dtype=np.float32)
    for k in range(K):
        run = (run * c[:, k]).astype(np.float32)
        g[:, k] = run
    return g


def expected_accepted(conf, budgets) -> float:
    """sum_b E_b(k_b), E_b(k) = sum_{n=1..k} prod_{l<n} c[b, l], in fp64
    (the objective the scheduler maximises)."""
    c = clamp_confidences(conf).astype(np.float64)
    total = 0.0
    for b, k in enumerate(np.asarray(budgets, dtype=np.int64)):
        run = 1.0
        for n in range(int(k)):
            run *= c[b, n]
            total += run
    return total


def schedule(conf, n_total: int, tau: float) -> np.ndarray:
    """Per-request budgets k_b (int32 [B]): the N largest fp32 gains above
    tau, equal gains in (k, b) order."""
    g = gains_fp32(conf)
    B, K = g.shape
    tau32 = np.float32(tau)
    order = []
    for k in range(K):
        for b in range(B):
            if g[b, k] > tau32:
                order.append((-float(g[b, k]), k, b))
    order.sort()
    take = order[: max(0, int(n_total))]
    budgets = np.zeros(B, dtype=np.int32)
    for _, k, b in take:
        budgets[b] += 1
    return budgets
