"""Plain CPU oracle of a verify step taken from hidden states through the
shared output head.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. It shares no
code with the HIP library and the library never calls it.

Sources (the pages' own titles and sections):

* "Speculative decoding becomes standard: DSpark and multi-token drafters",
  section "What DSpark adds", paragraph 1: the drafter reuses the target's
  embedding and output projection unchanged, so at a drafted position both
  models' logits are that one projection applied to each model's own hidden
  state.
* Same page, section "Why draft-and-verify does not change the output",
  paragraphs 1 and 2: the greedy and the sampled verification rules, which
  ``oracle.verify`` implements on logits.

Reading: the target's logits for position i of request b are
z_t = h_t[b, i] W^T and the drafter's z_d = h_d[b, i] W^T (``oracle.head``),
in fp64 on the exact bf16 values; the verify step is then ``oracle.verify``'s
on those logit rows, with the same request index (Philox counters), budgets,
drafted tokens, temperature and seed. Only the rows the rule reads are
formed: target rows 0..k_b and, when sampling, drafter rows 0..k_b-1.
"""
from __future__ import annotations

import numpy as np

from . import head as oh
from . import verify as ov


def decode_states(x) -> np.ndarray:
    """bf16 bit patterns (uint16) or float values to float64, exactly."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return oh.bf16_bits_to_f64(x)
    return x.astype(np.float64)


def verify_from_hidden(target_hidden, draft_hidden, head, tokens, budgets,
                       temperature: float, seed: int, requests=None,
                       head_f64=None) -> ov.BatchResult:
    """Verify requests of a batch whose logits come from hidden states.

    target_hidden [B, K+1, H], draft_hidden [B, K, H] (may be None when
    temperature == 0) and head [V, H], as bf16 bit patterns (uint16) or
    floats; tokens [B, K]; budgets [B]. ``requests`` selects request indices
    (default: all). ``head_f64`` may pass the head already decoded to fp64
    (the same values) to save decoding it again.
    """
    th = np.asarray(target_hidden)
    B, K1, H = th.shape
    K = K1 - 1
    W = decode_states(head) if head_f64 is None else head_f64
    V = W.shape[0]
    T = float(temperature)
    tokens = np.asarray(tokens, dtype=np.int64).reshape(B, K)
    budgets = np.asarray(budgets, dtype=np.int64).reshape(B)
    ov.check_inputs((B, K1, V), (B, K, V) if T > 0 else None, tokens, budgets, T)
    reqs = np.arange(B) if requests is None else np.asarray(requests, dtype=np.int64)
    out_tok = np.full((len(reqs), K + 1), -1, dtype=np.int32)
    out_n = np.zeros(len(reqs), dtype=np.int32)
    out_p = np.full((len(reqs), K), np.nan)
    out_q = np.full((len(reqs), K), np.nan)
    decisions = []
    for n, b in enumerate(reqs):
        k = int(budgets[b])
        zt = oh.logits(decode_states(th[b, : k + 1]), W)
        zd = None
        if T > 0:
            zd = oh.logits(decode_states(np.asarray(draft_hidden)[b, :k]), W)
        d = ov.verify_request(int(b), zt, zd, tokens[b, :k], T, seed)
        out_tok[n, : len(d.tokens)] = d.tokens
        out_n[n] = d.n_accepted
        if d.mode != ov.GREEDY:
            out_p[n, :k] = d.p_x
            out_q[n, :k] = d.q_x
        decisions.append(d)
    return ov.BatchResult(requests=reqs, tokens=out_tok, n_accepted=out_n, p_x=out_p,
                          q_x=out_q, decisions=decisions)
