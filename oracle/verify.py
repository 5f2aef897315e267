"""Plain fp64 CPU oracle of batched draft verification.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. It shares no
code with the HIP library and the library never calls it.

Sources (the pages' own titles and sections):

* "Speculative decoding becomes standard: DSpark and multi-token drafters",
  section "Why draft-and-verify does not change the output", paragraph 1:
  the target scores the whole drafted block in one pass; drafted tokens are
  kept while the target agrees, the target's own token replaces the first
  disagreeing one, and the rest of the block is thrown away.
* Same section, paragraph 2: the sampled rule of Leviathan, Kalman and
  Matias. A drafted token survives with probability min(1, p/q) (target
  over drafter probability); a rejected one is replaced by a draw from the
  renormalised residual max(0, p - q); the emitted tokens then follow the
  target's distribution however poor the drafter.
* Same page, section "What DSpark adds", paragraph 2: each request carries
  its own verify budget (how many drafted tokens are checked), chosen by a
  scheduler; budgets differ across requests and with load.

Readings where the pages are silent (each is stated again in the design
notes of the repository):

* One temperature T for both models: p = softmax(z_target / T),
  q = softmax(z_draft / T). T == 0 selects greedy verification, where the
  target's token is its argmax (lowest index among equal maxima) and neither
  drafter logits nor random numbers are used.
* Acceptance is the strict test u < min(1, p/q) with u in [0, 1); with
  q(x) == 0 the ratio counts as +inf when p(x) > 0 and the token is rejected
  when p(x) == 0.
* If every drafted token of the budget survives, one more ("bonus") token is
  drawn from the target row right after the budget, row k_b.
* Sampling is the inverse CDF in vocabulary order: the token is the smallest
  v whose inclusive running sum of the (unnormalised) mass exceeds u times
  the total mass. Zero-mass tokens can never be chosen. If the residual has
  no mass at all (possible only through rounding) the target row is used
  instead; if rounding leaves no crossing, the last positive-mass token is
  taken.
* Random numbers come from Philox4x32-10 as laid out in ``oracle.philox``.

Everything below is fp64 on exactly decoded inputs (fp32 and bf16 both embed
exactly in fp64).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from . import philox

GREEDY = "greedy"
RESIDUAL = "residual"
BONUS = "bonus"


def decode_bf16(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) to float64, exactly.

    A bfloat16 value is the upper half of the fp32 value with the same bits,
    so widening the pattern to 32 bits with 16 zero bits below gives the fp32
    number, which fp64 holds exactly.
    """
    bits = np.asarray(bits, dtype=np.uint16)
    wide = bits.astype(np.uint32) << np.uint32(16)
    return wide.view(np.float32).astype(np.float64)


def as_f64_rows(rows, fmt: str) -> np.ndarray:
    """Logit rows in the caller's storage format to float64."""
    if fmt == "bf16":
        return decode_bf16(rows)
    if fmt in ("f32", "f64"):
        return np.asarray(rows, dtype=np.float64)
    raise ValueError(f"unknown logit format {fmt!r}")


def softmax_row(z: np.ndarray, temperature: float):
    """Temperature softmax of one logit row.

    Returns (m, S, p): m = max z, S = sum_v exp((z_v - m) / T) and
    p_v = exp((z_v - m) / T) / S. Subtracting m leaves p unchanged and keeps
    every exponent <= 0.
    """
    m = float(np.max(z))
    w = np.exp((z - m) / temperature)
    s = float(np.sum(w))
    return m, s, w / s


def first_argmax(z: np.ndarray) -> int:
    """Index of the largest logit; the lowest such index when several tie.

    ``np.argmax`` is documented to return the first occurrence of the maximum.
    """
    return int(np.argmax(z))


def accept_decision(u: float, p_x: float, q_x: float):
    """Acceptance of one drafted token: u < min(1, p(x)/q(x)).

    Returns (accepted, margin) where margin = |u - min(1, p/q)| measures how
    close the decision was to flipping (inf when it cannot flip).
    """
    if q_x > 0.0:
        threshold = min(1.0, p_x / q_x)
        return (u < threshold), abs(u - threshold)
    if p_x > 0.0:
        return True, math.inf
    return False, math.inf


def inverse_cdf(mass: np.ndarray, u: float):
    """Inverse-CDF draw over an unnormalised mass vector in vocabulary order.

    y = min{v : sum_{w <= v} mass_w > u * sum_w mass_w}. Returns
    (y, margin, total) where margin is the distance, in normalised units, from
    u to the nearer edge of y's CDF interval [C(y-1)/R, C(y)/R).
    """
    total = float(np.sum(mass))
    cdf = np.cumsum(mass)
    threshold = u * total
    hits = np.nonzero(cdf > threshold)[0]
    if hits.size:
        y = int(hits[0])
    else:                                   # rounding left no crossing
        y = int(np.nonzero(mass > 0.0)[0][-1])
    c_prev = float(cdf[y - 1]) if y > 0 else 0.0
    c_y = float(cdf[y])
    margin = min(abs(u - c_prev / total), abs(c_y / total - u))
    return y, margin, total


def cdf_interval(mass: np.ndarray, y: int):
    """Token y's interval [C(y-1)/R, C(y)/R) of the normalised running sum
    that inverse_cdf draws from (empty when y has no mass)."""
    total = float(np.sum(mass))
    cdf = np.cumsum(mass)
    lo = float(cdf[y - 1]) / total if y > 0 else 0.0
    return lo, float(cdf[y]) / total


def draw_mass(p_rows, q_rows, j: int, k: int) -> np.ndarray:
    """The unnormalised mass of the draw at position j of a request with
    budget k: the residual max(0, p_j - q_j) after a rejection (j < k), p_j
    itself if rounding left that residual without mass, and p_k for the bonus
    token (j == k)."""
    if j < k:
        mass = np.maximum(0.0, np.asarray(p_rows[j]) - np.asarray(q_rows[j]))
        if np.any(mass > 0.0):
            return mass
        return np.asarray(p_rows[j], dtype=np.float64)
    return np.asarray(p_rows[k], dtype=np.float64)


@dataclass
class Decision:
    """Outcome of verifying one request."""
    n_accepted: int                       # j: drafted tokens kept
    tokens: list                          # emitted tokens x_0..x_{j-1}, y
    mode: str                             # greedy / residual / bonus
    p_x: list = field(default_factory=list)         # p_i(x_i), i < k
    q_x: list = field(default_factory=list)         # q_i(x_i), i < k
    acc_margin: list = field(default_factory=list)  # |u_acc - min(1,p/q)|, i < k
    accepted: list = field(default_factory=list)    # acceptance of every i < k
    cdf_margin: float = math.inf
    mass_total: float = math.nan          # R of the sampled row (pair)
    u_acc: list = field(default_factory=list)
    u_smp: list = field(default_factory=list)


def decide_sampled(p_rows, q_rows, drafted, u_acc, u_smp) -> Decision:
    """The sampled rule on probability rows with explicit uniforms.

    p_rows: k+1 target rows, q_rows: k drafter rows, drafted: k tokens,
    u_acc: k uniforms, u_smp: k+1 uniforms (one per position; only the one at
    the sampled position is used).
    """
    k = len(drafted)
    p_x, q_x, margins, accepted = [], [], [], []
    for i in range(k):
        px = float(p_rows[i][drafted[i]])
        qx = float(q_rows[i][drafted[i]])
        ok, margin = accept_decision(float(u_acc[i]), px, qx)
        p_x.append(px)
        q_x.append(qx)
        margins.append(margin)
        accepted.append(bool(ok))
    j = next((i for i in range(k) if not accepted[i]), k)
    mode = RESIDUAL if j < k else BONUS
    mass = draw_mass(p_rows, q_rows, j, k)
    y, cdf_margin, total = inverse_cdf(mass, float(u_smp[j]))
    tokens = [int(t) for t in drafted[:j]] + [y]
    return Decision(n_accepted=j, tokens=tokens, mode=mode, p_x=p_x, q_x=q_x,
                    acc_margin=margins, accepted=accepted, cdf_margin=cdf_margin,
                    mass_total=total, u_acc=list(u_acc), u_smp=list(u_smp))


def decide_greedy(target_rows, drafted) -> Decision:
    """Greedy rule: keep drafted tokens equal to the target's argmax, then the
    target's own token at the first mismatch (or after the whole budget)."""
    k = len(drafted)
    best = [first_argmax(target_rows[i]) for i in range(k + 1)]
    accepted = [int(drafted[i]) == best[i] for i in range(k)]
    j = next((i for i in range(k) if not accepted[i]), k)
    tokens = [int(t) for t in drafted[:j]] + [best[j]]
    return Decision(n_accepted=j, tokens=tokens, mode=GREEDY, accepted=accepted)


def request_draw_mass(target_rows, draft_rows, j: int, k: int, temperature: float):
    """The draw mass of position j of a request from its logits (sampled
    mode): the rows' temperature softmax, then draw_mass."""
    p_rows = [softmax_row(target_rows[i], temperature)[2] for i in range(k + 1)]
    q_rows = [softmax_row(draft_rows[i], temperature)[2] for i in range(k)]
    return draw_mass(p_rows, q_rows, j, k)


def verify_request(b: int, target_rows, draft_rows, drafted, temperature: float,
                   seed: int) -> Decision:
    """Verify request ``b`` (its index fixes its Philox counters).

    target_rows: [k+1, V] float64 logits; draft_rows: [k, V] float64 logits
    (ignored when temperature == 0); drafted: k token ids.
    """
    k = len(drafted)
    if temperature == 0.0:
        return decide_greedy(target_rows, drafted)
    p_rows = [softmax_row(target_rows[i], temperature)[2] for i in range(k + 1)]
    q_rows = [softmax_row(draft_rows[i], temperature)[2] for i in range(k)]
    uniforms = [philox.position_uniforms(seed, b, i) for i in range(k + 1)]
    u_acc = [u[0] for u in uniforms[:k]]
    u_smp = [u[1] for u in uniforms]
    return decide_sampled(p_rows, q_rows, drafted, u_acc, u_smp)


@dataclass
class BatchResult:
    """Oracle outputs over a set of requests, laid out like the library's."""
    requests: np.ndarray          # request indices covered
    tokens: np.ndarray            # [n, K+1] int32, -1 padded
    n_accepted: np.ndarray        # [n] int32
    p_x: np.ndarray               # [n, K] float64, NaN beyond the budget / greedy
    q_x: np.ndarray               # [n, K]
    decisions: list               # one Decision per request


def check_inputs(target_shape, draft_shape, tokens, budgets, temperature):
    """Preconditions of a verify call; raises ValueError on a violation."""
    if len(target_shape) != 3:
        raise ValueError("target logits must be [B, K+1, V]")
    B, K1, V = target_shape
    K = K1 - 1
    if K < 0 or V < 1:
        raise ValueError("need K >= 0 and V >= 1")
    if not (math.isfinite(temperature) and temperature >= 0.0):
        raise ValueError("temperature must be finite and >= 0")
    if temperature > 0.0 and tuple(draft_shape) != (B, K, V):
        raise ValueError("drafter logits must be [B, K, V]")
    tokens = np.asarray(tokens)
    budgets = np.asarray(budgets)
    if tokens.shape != (B, K) or budgets.shape != (B,):
        raise ValueError("drafted tokens must be [B, K] and budgets [B]")
    for b in range(B):
        k = int(budgets[b])
        if not 0 <= k <= K:
            raise ValueError(f"budget of request {b} is {k}, outside [0, {K}]")
        if k and (tokens[b, :k].min() < 0 or tokens[b, :k].max() >= V):
            raise ValueError(f"drafted token of request {b} outside [0, {V})")


def verify_batch(target, draft, tokens, budgets, temperature: float, seed: int,
                 logits_format: str = "f32", requests=None) -> BatchResult:
    """Verify requests of a batch.

    target: [B, K+1, V] logits, draft: [B, K, V] logits (may be None when
    temperature == 0), stored as float arrays or, with
    ``logits_format="bf16"``, as uint16 bfloat16 bit patterns. tokens: [B, K]
    int, budgets: [B] int. ``requests`` selects a subset of request indices
    (default: all); each keeps its own Philox counters.
    """
    target_shape = np.shape(target)
    draft_shape = np.shape(draft) if draft is not None else None
    check_inputs(target_shape, draft_shape, tokens, budgets, float(temperature))
    B, K1, _V = target_shape
    K = K1 - 1
    tokens = np.asarray(tokens, dtype=np.int64)
    budgets = np.asarray(budgets, dtype=np.int64)
    reqs = np.arange(B) if requests is None else np.asarray(requests, dtype=np.int64)
    out_tok = np.full((len(reqs), K + 1), -1, dtype=np.int32)
    out_n = np.zeros(len(reqs), dtype=np.int32)
    out_p = np.full((len(reqs), K), np.nan)
    out_q = np.full((len(reqs), K), np.nan)
    decisions = []
    for n, b in enumerate(reqs):
        k = int(budgets[b])
        zt = as_f64_rows(target[b, : k + 1], logits_format)
        zd = as_f64_rows(draft[b, :k], logits_format) if temperature > 0 else None
        d = verify_request(int(b), zt, zd, tokens[b, :k], float(temperature), seed)
        out_tok[n, : len(d.tokens)] = d.tokens
        out_n[n] = d.n_accepted
        if d.mode != GREEDY:
            out_p[n, :k] = d.p_x
            out_q[n, :k] = d.q_x
        decisions.append(d)
    return BatchResult(requests=reqs, tokens=out_tok, n_accepted=out_n, p_x=out_p,
                       q_x=out_q, decisions=decisions)
