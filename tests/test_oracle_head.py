"""Pins of the output-head oracle (oracle/head.py)."""
import numpy as np
import pytest
import torch
from scipy import special

from oracle import head as oh


def test_logits_against_explicit_loops():
    rng = np.random.default_rng(0)
    h = rng.standard_normal((3, 5))
    w = rng.standard_normal((4, 5))
    z = oh.logits(h, w)
    for r in range(3):
        for v in range(4):
            acc = 0.0
            for i in range(5):
                acc += h[r, i] * w[v, i]
            assert abs(z[r, v] - acc) < 1e-12


@pytest.mark.parametrize("T", [0.5, 1.0, 2.0])
def test_stats_against_scipy(T):
    rng = np.random.default_rng(int(T * 10))
    z = rng.standard_normal((6, 50)) * 4
    tok = rng.integers(0, 50, size=6)
    m, s, zx, arg = oh.row_stats(z, tok, T)
    # logsumexp(z / T) = m / T + ln S
    np.testing.assert_allclose(m / T + np.log(s), special.logsumexp(z / T, axis=1), rtol=1e-13)
    # p(x) from the statistics is the softmax at x
    np.testing.assert_allclose(oh.prob_of(m, s, zx, T),
                               special.softmax(z / T, axis=1)[np.arange(6), tok], rtol=1e-12)


def test_first_argmax_and_missing_token():
    z = np.array([[1.0, 3.0, 3.0, 2.0], [5.0, 5.0, 5.0, 5.0], [-1.0, -2.0, -0.5, -0.5]])
    m, s, zx, arg = oh.row_stats(z, [1, -1, 9], 1.0)
    for r in range(3):
        best = 0
        for v in range(4):
            if z[r, v] > z[r, best]:
                best = v
        assert arg[r] == best
    assert zx[0] == 3.0 and np.isnan(zx[1]) and np.isnan(zx[2])
    _, s0, _, _ = oh.row_stats(z, [0, 0, 0], 0.0)
    assert np.isnan(s0).all()


def test_bf16_decoding_matches_torch():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    mine = oh.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    same = (mine == ref) | (np.isnan(mine) & np.isnan(ref))
    assert same.all()
