"""Plain CPU oracle of the output head's row statistics.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. It shares no
code with the HIP library and the library never calls it.

Sources (the pages' own titles and sections):

* "Speculative decoding becomes standard: DSpark and multi-token drafters",
  section "What DSpark adds", paragraph 1: the drafter reuses the target's
  embedding and output projection unchanged, so at a given position both
  models' logits are that one projection applied to each model's hidden
  state.
* Same page, section "Why draft-and-verify does not change the output",
  paragraphs 1 and 2: verification needs, per scored position, the target's
  most likely token (greedy) or the probabilities p(x) and q(x) of the drafted
  token under the two softmaxes (sampled).

Reading (the pages give no formula for the head): logits z = h W^T for a
hidden state h (length H) and the head W ([V, H]); the statistics a verify
step needs from a row are its maximum m, the sum S = sum_v 2^((z_v - m) c)
with c = log2(e) / T, the logit of one given token, and the first (lowest
index) argmax; p(x) = 2^((z_x - m) c) / S. Inputs are bf16; everything here
is fp64 on their exact values.
"""
from __future__ import annotations

import numpy as np

LOG2E = 1.4426950408889634


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact values of bf16 bit patterns (uint16) as fp64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def logits(hidden, weight) -> np.ndarray:
    """z[r, v] = sum_i hidden[r, i] * weight[v, i] (fp64 matrix product)."""
    return np.asarray(hidden, dtype=np.float64) @ np.asarray(weight, dtype=np.float64).T


def row_stats(z, tokens, temperature: float):
    """Per row: (max, sum of 2^((z - max) c), z[token] or NaN, first argmax).
    temperature == 0 gives sum = NaN (only the argmax is meaningful)."""
    z = np.asarray(z, dtype=np.float64)
    R, V = z.shape
    m = z.max(axis=1)
    arg = z.argmax(axis=1)                          # numpy returns the first maximum
    if temperature > 0:
        c = LOG2E / temperature
        s = np.exp2((z - m[:, None]) * c).sum(axis=1)
    else:
        s = np.full(R, np.nan)
    tok = np.asarray(tokens, dtype=np.int64)
    zx = np.full(R, np.nan)
    ok = (tok >= 0) & (tok < V)
    zx[ok] = z[np.arange(R)[ok], tok[ok]]
    return m, s, zx, arg.astype(np.int64)


def prob_of(m, s, zx, temperature: float):
    """p(x) = 2^((z_x - m) c) / S from a row's statistics."""
    c = LOG2E / temperature
    return np.exp2((np.asarray(zx) - np.asarray(m)) * c) / np.asarray(s)
