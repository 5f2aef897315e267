"""Pins of the low-rank Markov head oracle (oracle/markov.py).

Pages: "Speculative decoding becomes standard: DSpark and multi-token
drafters", section "What DSpark adds", paragraph 1 (a rank-256 Markov module
over the block's positions); "DSpark" (finds page), the Markov head uses only
the previous token and a low-rank matrix.

* A successor chain built by hand: A = identity, Bm[v] = 4 e_{v-1}, so the
  transition term is 4 exactly when v = x_{i-1} + 1 (mod V); with base logits
  on a coarse grid within (-1, 1), the drafted block from token t is t+1,
  t+2, ... and the stored logits are base + 4 [v = x + 1] exactly.
* No transition term (Bm = 0): every position drafts the first argmax of its
  own base row, whatever the previous token, and stores the base row.
* Low rank: the transition matrix the oracle forms over all previous tokens
  has rank at most r (numpy's SVD rank).
* Rounding to bf16 against torch's float32 -> bfloat16 conversion (ties to
  even) on fp32-exact values, including exact ties and the overflow edge.
* Ties between equal maxima take the lowest index.
A swapped table, a dropped bias or a position that reads its own token
instead of the previous one fails one of these.
"""
import numpy as np
import torch

from oracle import markov as om


def _succ_tables(V):
    A = np.eye(V)
    Bm = np.zeros((V, V))
    for v in range(V):
        Bm[v, (v - 1) % V] = 4.0
    return A, Bm


def test_successor_chain_by_hand():
    V, K = 8, 5
    A, Bm = _succ_tables(V)
    rng = np.random.default_rng(3)
    base = rng.integers(-15, 16, size=(2, K, V)) / 16.0     # bf16-exact, |base| < 1
    z, x = om.draft_block(base, A, Bm, prev=[3, 7])
    assert x.tolist() == [[4, 5, 6, 7, 0], [0, 1, 2, 3, 4]]
    # Stored logits: the base row plus 4 at the drafted token (exact in bf16).
    for b, prev in enumerate([3, 7]):
        last = prev
        for i in range(K):
            want = base[b, i].copy()
            want[(last + 1) % V] += 4.0
            assert np.array_equal(z[b, i], want)
            last = x[b, i]


def test_no_transition_term_drafts_the_base_argmax():
    V, K, r = 50, 4, 6
    rng = np.random.default_rng(5)
    base = om.round_bf16(rng.normal(0, 3, size=(3, K, V)))
    A = om.round_bf16(rng.normal(0, 1, size=(V, r)))
    Bm = np.zeros((V, r))
    z, x = om.draft_block(base, A, Bm, prev=[0, 17, 49])
    assert np.array_equal(z, base)
    assert np.array_equal(x, np.argmax(base, axis=2))


def test_transition_matrix_has_rank_at_most_r():
    V, r = 40, 3
    rng = np.random.default_rng(7)
    A = om.round_bf16(rng.normal(0, 1, size=(V, r)))
    Bm = om.round_bf16(rng.normal(0, 1, size=(V, r)))
    M = om.markov_bias(A, Bm, np.arange(V))                 # row x: bias after token x
    assert M.shape == (V, V)
    assert np.linalg.matrix_rank(M) == r
    # Row x depends on x alone: the same previous token gives the same row.
    assert np.array_equal(om.markov_bias(A, Bm, [5, 5])[0], M[5])


def test_round_bf16_matches_torch_on_fp32_values():
    rng = np.random.default_rng(11)
    f = np.concatenate([
        rng.normal(0, 1, 20000).astype(np.float32),
        rng.normal(0, 1e-38, 2000).astype(np.float32),       # bf16 subnormals
        (rng.normal(0, 1, 2000) * 1e37).astype(np.float32),
        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 3.0e38, -3.0e38,
                  float.fromhex("0x1.fep127"), float.fromhex("0x1.ff8p127")], dtype=np.float32),
    ])
    want = torch.from_numpy(f).to(torch.bfloat16).float().numpy().astype(np.float64)
    got = om.round_bf16(f.astype(np.float64))
    assert np.array_equal(got, want)


def test_ties_take_the_lowest_index():
    V = 6
    base = np.zeros((1, 2, V))
    base[0, 0, [1, 4]] = 2.0
    base[0, 1, [2, 3, 5]] = 1.5
    A = np.zeros((V, 2))
    Bm = np.zeros((V, 2))
    _, x = om.draft_block(base, A, Bm, prev=[0])
    assert x.tolist() == [[1, 2]]


def test_bias_reads_the_previous_token_not_the_current():
    # With the successor chain, a head reading x_i instead of x_{i-1} could
    # not reproduce position 0's draft from the given last token.
    V = 8
    A, Bm = _succ_tables(V)
    base = np.zeros((1, 1, V))
    _, x = om.draft_block(base, A, Bm, prev=[6])
    assert x.tolist() == [[7]]
