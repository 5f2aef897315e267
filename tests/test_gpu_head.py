"""GPU parity of the output head's row statistics (spec_head_stats) against
the fp64 oracle on the same bf16 inputs.

Tolerances follow from the arithmetic: each logit is an fp32 sum of H exact
bf16 products, so its error is at most about sqrt(H) * 2^-24 * scale with
scale = sum_i |h_i w_i| (a factor 4 of margin is taken); the row maximum and
the token's logit inherit it; the exp-sum's terms move by at most
2 tol c ln 2 relative, plus fp32 summation; the argmax must be exact unless
the oracle's top two logits are within 2 tol, and is then only required to
point at a logit within 2 tol of the maximum."""
import math
import sys

import numpy as np
import pytest
import torch

from draft_verify_sampling_spec_amd import head_stats
from oracle import head as oh
from workloads import make_head_inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


def _bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _check_rows(z, scale, tokens, T, got, H):
    m_ref, s_ref, z_ref, a_ref = oh.row_stats(z, tokens, T)
    m, s, zx, arg = (x.cpu().numpy() for x in got)
    tol = 4.0 * math.sqrt(H) * 2.0 ** -24 * scale + 1e-30
    assert np.all(np.abs(m - m_ref) <= tol), np.max(np.abs(m - m_ref) / tol)
    ok = ~np.isnan(z_ref)
    assert np.all(np.abs(zx[ok] - z_ref[ok]) <= tol[ok])
    assert np.all(np.isnan(zx[~ok]))
    if T > 0:
        c = oh.LOG2E / T
        rel = 2.0 * tol * c * math.log(2.0) + 1e-5
        assert np.all(np.abs(s / s_ref - 1.0) <= rel), np.max(np.abs(s / s_ref - 1.0) / rel)
        assert np.all(arg == -1)
    else:
        assert np.all(np.isnan(s))
        for r in range(z.shape[0]):
            top = np.sort(z[r])[-2:] if z.shape[1] > 1 else np.array([-np.inf, z[r, 0]])
            if top[1] - top[0] > 2 * tol[r]:
                assert arg[r] == a_ref[r], (r, arg[r], a_ref[r])
            else:
                assert z[r, arg[r]] >= m_ref[r] - 2 * tol[r]


@pytest.mark.parametrize("R,H,V", [(1, 8, 1), (37, 64, 1000), (128, 256, 2048), (200, 96, 3001),
                                   (300, 2560, 5000), (260, 40, 129)])
@pytest.mark.parametrize("T", [0.0, 0.7, 1.0])
def test_small_shapes_match_oracle(R, H, V, T):
    _log(f"[head] R={R} H={H} V={V} T={T}")
    h, w, tok = make_head_inputs(R, H, V, seed=R * 7 + V)
    tok[::5] = -1
    got = head_stats(h, w, tok, T)
    h64, w64 = oh.bf16_bits_to_f64(_bits(h)), oh.bf16_bits_to_f64(_bits(w))
    z = oh.logits(h64, w64)
    scale = (np.abs(h64) @ np.abs(w64).T).max(axis=1)
    _check_rows(z, scale, tok.cpu().numpy(), T, got, H)


@pytest.mark.parametrize("R,H,V", [(1700, 128, 10243), (1541, 192, 10001), (4000, 64, 24576),
                                   (3329, 128, 49153)])
@pytest.mark.parametrize("T", [0.0, 1.0])
def test_many_row_product_every_row(R, H, V, T):
    """Shapes that take the many-row product (at least 1,536 rows, at least
    40 vocabulary tiles of 256, H a multiple of 64) with ragged row and
    vocabulary tails (a partial last row tile and a partial last vocabulary
    tile, a partial last band), and with the side workgroups' columns (1, 0,
    6 and 8 of them, over 1 to 3 bands): every row against the oracle."""
    _log(f"[head] many-row product R={R} H={H} V={V} T={T}")
    h, w, tok = make_head_inputs(R, H, V, seed=R + V)
    tok[::7] = -1
    got = head_stats(h, w, tok, T)
    h64, w64 = oh.bf16_bits_to_f64(_bits(h)), oh.bf16_bits_to_f64(_bits(w))
    z = oh.logits(h64, w64)
    scale = (np.abs(h64) @ np.abs(w64).T).max(axis=1)
    _check_rows(z, scale, tok.cpu().numpy(), T, got, H)


def test_full_size_sampled_rows():
    """The heavy batch's shape: 8,704 rows (4,608 target + 4,096 drafter
    positions), H = 2,560, V = 151,936; the oracle recomputes 6 rows."""
    R, H, V = 8704, 2560, 151936
    _log(f"[head] full size R={R} H={H} V={V}")
    h, w, tok = make_head_inputs(R, H, V, seed=5)
    for T in (1.0, 0.0):
        got = head_stats(h, w, tok, T)
        torch.cuda.synchronize()
        rows = [0, 1, 127, 128, 4607, R - 1]
        h64 = oh.bf16_bits_to_f64(_bits(h[rows]))
        z = np.zeros((len(rows), V))
        scale = np.zeros(len(rows))
        for v0 in range(0, V, 16384):
            w64 = oh.bf16_bits_to_f64(_bits(w[v0:v0 + 16384]))
            z[:, v0:v0 + w64.shape[0]] = oh.logits(h64, w64)
            scale = np.maximum(scale, (np.abs(h64) @ np.abs(w64).T).max(axis=1))
        sub = tuple(x[rows] for x in got)
        _check_rows(z, scale, tok[rows].cpu().numpy(), T, sub, H)
