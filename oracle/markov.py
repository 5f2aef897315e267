"""Plain CPU oracle of the drafter's low-rank Markov head.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. It shares no
code with the HIP library and the library never calls it.

Sources (the pages' own titles and sections):

* "Speculative decoding becomes standard: DSpark and multi-token drafters",
  section "What DSpark adds", paragraph 1: a block of tokens comes out of a
  parallel backbone in one pass, and a light sequential correction -- a
  factorised (rank 256) Markov model over consecutive positions -- keeps the
  block's later tokens consistent with its earlier ones.
* "DSpark" (finds page), where it compares two sequential structures: the
  one deployed conditions on nothing but the immediately preceding token,
  through a low-rank matrix.

Reading (the pages give no formula): the Markov head is a first-order
transition term over tokens in factored form. With tables A and Bm, both
[V, r], the logit bias at drafted position i is

    bias_i(v) = sum_j A[x_{i-1}, j] * Bm[v, j],

row x_{i-1} of the rank-r matrix A Bm^T. The drafter's logits at position i
are the parallel backbone's logits plus that bias, z_i = base_i + bias_i,
stored as bf16; the drafted token x_i is the first (lowest index) argmax of
the stored row. x_{-1} is the last token already in the sequence. Positions
run in order, since x_i depends on x_{i-1}. The stored rows are the drafter
logits a verify step then reads.

Precision: the inputs (base logits, A, Bm) are bf16; here the bias and the
sum are fp64 on their exact values, and the sum is rounded once to bf16
(round to nearest, ties to even), which is what the argmax is taken over.
"""
from __future__ import annotations

import numpy as np

BF16_MAX = float.fromhex("0x1.fep127")


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact values of bf16 bit patterns (uint16) as fp64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def round_bf16(x) -> np.ndarray:
    """fp64 values rounded to the nearest bf16 value, ties to even (bf16 has
    8 significant bits, normal exponents down to -126, subnormals to 2^-133);
    magnitudes that round past the largest finite bf16 become infinite."""
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x) & (x != 0.0)
    _, e = np.frexp(x[fin])                    # |x| = m 2^e, 0.5 <= m < 1
    step = np.exp2(np.maximum(e - 8, -133).astype(np.float64))
    r = np.round(x[fin] / step) * step         # numpy rounds halves to even
    r[np.abs(r) > BF16_MAX] = np.copysign(np.inf, r[np.abs(r) > BF16_MAX])
    out[fin] = r
    return out


def markov_bias(A, Bm, prev) -> np.ndarray:
    """bias[b, v] = sum_j A[prev[b], j] Bm[v, j] (fp64); A, Bm [V, r] values."""
    A = np.asarray(A, dtype=np.float64)
    Bm = np.asarray(Bm, dtype=np.float64)
    prev = np.asarray(prev, dtype=np.int64)
    return A[prev] @ Bm.T


def draft_position(base_i, A, Bm, prev):
    """One drafted position for every request: base_i [B, V] values, prev [B]
    the previous tokens. Returns (stored logits [B, V] as bf16 values in fp64,
    drafted tokens [B], the unrounded fp64 sums [B, V])."""
    exact = np.asarray(base_i, dtype=np.float64) + markov_bias(A, Bm, prev)
    z = round_bf16(exact)
    return z, z.argmax(axis=1).astype(np.int64), exact


def draft_block(base, A, Bm, prev):
    """A whole block: base [B, K, V] values, prev [B] the last tokens in the
    sequences. Returns (stored logits [B, K, V], tokens [B, K])."""
    base = np.asarray(base, dtype=np.float64)
    B, K, V = base.shape
    z = np.empty((B, K, V))
    x = np.empty((B, K), dtype=np.int64)
    last = np.asarray(prev, dtype=np.int64)
    for i in range(K):
        z[:, i], x[:, i], _ = draft_position(base[:, i], A, Bm, last)
        last = x[:, i]
    return z, x
