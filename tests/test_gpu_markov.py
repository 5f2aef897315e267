"""GPU parity of the drafter's low-rank Markov head (spec_markov_draft)
against the fp64 oracle (oracle/markov.py), through the C ABI.

Position i of a request is checked against the oracle given the previous
token the GPU drafted (x_{i-1}; the given last token for i = 0), so every
position is an independent check.

Tolerances follow from the arithmetic. The bias is an fp32 sum of r exact
bf16 products, within E = 4 sqrt(r) 2^-24 sum_j |A[x, j] Bm[v, j]| of its
exact value (a factor 4 of margin); adding the backbone logit in fp32 adds at
most 2^-24 of the sum. With d = E + 2^-23 |z| for the exact sum z, the stored
bf16 value must lie between the bf16 roundings of z - d and z + d (rounding is
monotonic), which is equality with the oracle's rounding except within d of a
rounding boundary. The drafted token must be the first argmax of the GPU's
own stored row (bit-exact, an integer decision on the stored values), and
equal the oracle's first argmax unless another token could be the maximum
under the band (then it must be one of those).
"""
import math
import sys

import numpy as np
import pytest
import torch

from draft_verify_sampling_spec_amd import MarkovDraft, SpecVerify
from oracle import markov as om
from workloads import make_markov_inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _vals(t):
    return om.bf16_bits_to_f64(_bits(t))


def _run(inp, md=None):
    B, K, V = inp["base"].shape
    md = md or MarkovDraft(DEV, B, K, V)
    z, x, st = md.run(inp["base"], inp["markov_a"], inp["markov_b"], inp["prev"])
    torch.cuda.synchronize()
    return z, x.cpu().numpy(), int(st.item())


def _check_positions(inp, z_gpu, x_gpu, requests=None):
    """Every position of the given requests against the oracle (teacher
    forced); returns the number of tokens excused by the band."""
    base = _vals(inp["base"])
    A = _vals(inp["markov_a"])
    Bm = _vals(inp["markov_b"])
    aB = np.abs(Bm)
    prev0 = inp["prev"].cpu().numpy().astype(np.int64)
    zg = _vals(z_gpu)
    B, K, V = base.shape
    r = A.shape[1]
    reqs = range(B) if requests is None else requests
    excused = 0
    for b in reqs:
        last = prev0[b]
        for i in range(K):
            z_ora, x_ora, exact = om.draft_position(base[b, i][None], A, Bm, [last])
            exact = exact[0]
            E = 4.0 * math.sqrt(r) * 2.0 ** -24 * (aB @ np.abs(A[last]))
            d = E + 2.0 ** -23 * np.abs(exact)
            lo, hi = om.round_bf16(exact - d), om.round_bf16(exact + d)
            got = zg[b, i]
            bad = np.nonzero((got < lo) | (got > hi))[0]
            assert bad.size == 0, (b, i, bad[:5], got[bad[:5]], exact[bad[:5]])
            xg = int(x_gpu[b, i])
            # Integer decision on the GPU's own stored values: exact.
            assert xg == int(np.argmax(got)), (b, i)
            if xg != int(x_ora[0]):
                assert hi[xg] >= lo.max(), (b, i, xg, int(x_ora[0]))
                excused += 1
            last = xg
    return excused


SHAPES = [
    (3, 4, 1000, 8),
    (7, 5, 517, 16),          # V not a multiple of 8: element loads
    (16, 8, 4096, 64),
    (5, 3, 40003, 256),
    (2, 2, 5, 8),
    (33, 6, 2048, 256),
    (16, 4, 65536, 128),      # two k-steps, 64 splits (XCD order)
    (9, 3, 30000, 192),       # three k-steps: the last fetch repeats step 2
    (200, 2, 40960, 128),     # two row tiles, 40 splits (XCD order)
    # The streaming product (r a multiple of 16, V of 8): 32-column tiles,
    # stored in pairs; these give an odd tile count (the row's last tile
    # stored alone), a partial last tile alone and as the second of a pair,
    # four groups of 256 requests (the last empty), one request in the
    # second group, a single k-group, and one position.
    (40, 3, 3104, 64),        # 97 tiles: the last one unpaired and full
    (24, 2, 3080, 32),        # 97 tiles: the last one unpaired, 8 columns
    (24, 2, 3048, 48),        # 96 tiles: the last pair's second tile, 8 columns
    (600, 2, 8192, 64),       # four request groups, the fourth empty
    (257, 2, 4096, 16),       # one request in the second group; one k-group
    (64, 1, 16384, 128),      # one position
]


@pytest.mark.parametrize("B,K,V,r", SHAPES)
def test_small_shapes_match_oracle(B, K, V, r):
    _log(f"[markov] B={B} K={K} V={V} r={r}")
    inp = make_markov_inputs(B, K, V, r, seed=B * 1000 + V, device=DEV)
    z, x, st = _run(inp)
    assert st == 0
    n = _check_positions(inp, z, x)
    _log(f"[markov] excused {n} of {B * K} tokens")


def test_no_transition_term_keeps_the_backbone():
    B, K, V, r = 9, 4, 3000, 32
    inp = make_markov_inputs(B, K, V, r, seed=3, device=DEV)
    inp["markov_b"] = torch.zeros_like(inp["markov_b"])
    z, x, st = _run(inp)
    assert st == 0
    assert torch.equal(z.view(torch.int16), inp["base"].view(torch.int16))
    assert np.array_equal(x, torch.argmax(inp["base"].float(), dim=2).cpu().numpy())


def test_successor_chain():
    # A = identity, Bm[v] = 4 e_{v-1}: the transition term is 4 exactly at
    # v = x_{i-1} + 1 (mod V); backbone logits within (-1, 1) on a 1/16 grid.
    V = r = 16
    B, K = 4, 7
    a = torch.eye(V)
    bm = torch.zeros(V, V)
    for v in range(V):
        bm[v, (v - 1) % V] = 4.0
    g = torch.Generator().manual_seed(9)
    base = torch.randint(-15, 16, (B, K, V), generator=g).float() / 16.0
    prev = torch.tensor([0, 5, 15, 9], dtype=torch.int32)
    inp = {"base": base.to(torch.bfloat16).to(DEV), "markov_a": a.to(torch.bfloat16).to(DEV),
           "markov_b": bm.to(torch.bfloat16).to(DEV), "prev": prev.to(DEV)}
    z, x, st = _run(inp)
    assert st == 0
    want = [[(int(p) + 1 + i) % V for i in range(K)] for p in prev]
    assert x.tolist() == want
    zz = z.float().cpu()
    for b in range(B):
        last = int(prev[b])
        for i in range(K):
            row = base[b, i].clone()
            row[(last + 1) % V] += 4.0
            assert torch.equal(zz[b, i], row)
            last = want[b][i]


def test_ties_across_vocabulary_splits():
    # No transition term, so the stored rows are the backbone's; values on a
    # coarse grid tie for the maximum in many vocabulary splits (at
    # V = 40,960: 1,280 tiles of 32 columns over 256 column slots), and the
    # token must be the lowest such column.
    B, K, V, r = 6, 3, 40960, 16
    g = torch.Generator().manual_seed(21)
    base = torch.randint(-2, 3, (B, K, V), generator=g).float()
    base[0, :, :] = 0.0                        # every column ties: token 0
    base[0, 1, :] = -float("inf")              # no value above -inf: token 0
    base[1, :, :] = -1.0
    base[1, :, V - 3] = 2.0                    # the only maximum, in the last split
    base[2, :, :] = 1.0
    base[2, :, 1000] = 1.5
    base[2, :, 30000] = 1.5                    # the first of two maxima in different splits
    inp = make_markov_inputs(B, K, V, r, seed=22, device=DEV)
    inp["base"] = base.to(torch.bfloat16).to(DEV)
    inp["markov_b"] = torch.zeros_like(inp["markov_b"])
    z, x, st = _run(inp)
    assert st == 0
    assert torch.equal(z.view(torch.int16), inp["base"].view(torch.int16))
    want = torch.argmax(base, dim=2).numpy()   # first maximum (-inf rows: 0)
    assert np.array_equal(x, want)
    assert x[0].tolist() == [0, 0, 0] and x[1].tolist() == [V - 3] * K
    assert x[2].tolist() == [1000] * K


def test_heavy_shape_full_launch():
    # The bench's shape: 512 requests, 8 drafted positions, Qwen3-4B's
    # vocabulary, rank 256; the oracle on every 64th request.
    B, K, V, r = 512, 8, 151936, 256
    _log("[markov] heavy shape")
    inp = make_markov_inputs(B, K, V, r, seed=5, device=DEV)
    z, x, st = _run(inp)
    assert st == 0
    assert x.min() >= 0 and x.max() < V
    n = _check_positions(inp, z, x, requests=range(0, B, 64))
    _log(f"[markov] heavy: excused {n} tokens")
    # Every request: the token is the first argmax of its stored row.
    zf = z.float()
    assert torch.equal(torch.argmax(zf, dim=2).to(torch.int32).cpu(), torch.from_numpy(x))


def test_bad_previous_token_sets_the_status_flag():
    B, K, V, r = 6, 3, 1000, 16
    inp = make_markov_inputs(B, K, V, r, seed=11, device=DEV)
    inp["prev"][2] = V
    inp["prev"][4] = -3
    z, x, st = _run(inp)
    assert st == 0x2                                   # SV_FLAG_BAD_TOKEN
    # The other requests are unaffected.
    _check_positions(inp, z, x, requests=[0, 1, 3, 5])


def test_repeat_calls_are_deterministic_and_reuse_the_workspace():
    B, K, V, r = 40, 5, 9000, 64
    inp = make_markov_inputs(B, K, V, r, seed=13, device=DEV)
    md = MarkovDraft(DEV, B, K, V)
    z1, x1, _ = _run(inp, md)
    z1 = z1.clone()
    other = make_markov_inputs(B, K, V, r, seed=14, device=DEV)
    _run(other, md)
    z2, x2, _ = _run(inp, md)
    assert torch.equal(z1.view(torch.int16), z2.view(torch.int16))
    assert np.array_equal(x1, x2)


def test_drafted_block_verifies_against_itself():
    # Draft a block, then verify it with target rows 0..K-1 equal to the
    # drafter's stored rows: p = q at every drafted position, so every drafted
    # token is accepted (sampled mode) and the bonus comes from row K.
    B, K, V, r = 24, 6, 5000, 32
    inp = make_markov_inputs(B, K, V, r, seed=17, device=DEV)
    z, x, st = _run(inp)
    assert st == 0
    g = torch.Generator(device=DEV).manual_seed(18)
    extra = (torch.randn(B, 1, V, generator=g, device=DEV) * 3.0).to(torch.bfloat16)
    target = torch.cat([z, extra], dim=1).contiguous()
    sv = SpecVerify(DEV, max_batch=B, max_k=K, vocab=V, dtype=torch.bfloat16)
    budgets = torch.full((B,), K, dtype=torch.int32, device=DEV)
    xt = torch.from_numpy(x).to(DEV)
    toks, nacc, _, _ = sv.run(target, z, xt, budgets, 1.0, 1234)
    torch.cuda.synchronize()
    assert sv.status() == 0
    assert torch.equal(nacc.cpu(), torch.full((B,), K, dtype=torch.int32))
    assert torch.equal(toks[:, :K].cpu(), xt.cpu())
    sv.close()
