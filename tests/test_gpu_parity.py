"""GPU parity of the HIP library against the fp64 CPU oracle.

Every call goes through the C ABI (ctypes binding). Inputs are the seeded
synthetic workloads; the oracle reads back the exact tensors the library was
given. Bar (see tests/helpers.py): greedy outputs bit-exact; p_i(x_i), q_i(x_i)
within 1e-5 relative; sampled decisions identical except first divergences
inside the 1e-6 near-tie band, which are counted and printed.
"""
import sys

import numpy as np
import pytest
import torch
from scipy import special, stats

from draft_verify_sampling_spec_amd import SpecVerify, binding, philox_words
from oracle import philox
from oracle import verify as ov
from tests.helpers import (assert_sampled, check_probabilities, logits_mass_fn, padded,
                           to_oracle)
from workloads import make_inputs, philox_seed

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


def _run(inp, seed, sv=None, temperature=None):
    T = inp["temperature"] if temperature is None else temperature
    t = inp["target"].to(DEV)
    d = inp["draft"].to(DEV) if T > 0 else None
    x = inp["tokens"].to(DEV)
    k = inp["budgets"].to(DEV)
    B, K1, V = t.shape
    own = sv is None
    if own:
        sv = SpecVerify(DEV, max_batch=max(B, 1), max_k=K1 - 1, vocab=V, dtype=t.dtype)
    toks, nacc, p, q = sv.run(t, d, x, k, T, seed)
    torch.cuda.synchronize()
    flags = sv.status()
    out = (toks.cpu().numpy(), nacc.cpu().numpy(), p.cpu().numpy(), q.cpu().numpy(), flags)
    if own:
        sv.close()
    return out


def _oracle(inp, seed, requests=None, temperature=None, request_base=0):
    """Oracle decisions for the given requests (global indices keep their
    counters; request b's Philox counter is request_base + b)."""
    T = inp["temperature"] if temperature is None else temperature
    budgets = inp["budgets"].cpu().numpy()
    tokens = inp["tokens"].cpu().numpy()
    reqs = range(len(budgets)) if requests is None else requests
    out = []
    for b in reqs:
        k = int(budgets[b])
        zt, fmt = to_oracle(inp["target"][b, : k + 1])
        zt = ov.as_f64_rows(zt, fmt)
        zd = None
        if T > 0:
            zd, _ = to_oracle(inp["draft"][b, :k])
            zd = ov.as_f64_rows(zd, fmt)
        out.append(ov.verify_request(int(request_base) + int(b), zt, zd, tokens[b, :k], float(T),
                                     seed))
    return out


def _assert_parity(inp, seed, gpu, decisions, requests=None, temperature=None, tag=""):
    T = inp["temperature"] if temperature is None else temperature
    toks, nacc, p, q, flags = gpu
    assert flags == 0, f"device status flags {flags:#x}"
    K = inp["tokens"].shape[1]
    reqs = np.arange(len(toks)) if requests is None else np.asarray(requests)
    budgets = inp["budgets"].cpu().numpy()[reqs]
    g_tok, g_n = toks[reqs], nacc[reqs]
    if T == 0:
        for n, d in enumerate(decisions):
            assert int(g_n[n]) == d.n_accepted, (tag, int(reqs[n]))
            assert list(g_tok[n]) == padded(d.tokens, K), (tag, int(reqs[n]))
        assert np.all(np.isnan(p[reqs])) and np.all(np.isnan(q[reqs]))
        return 0
    ora_p = np.full((len(reqs), K), np.nan)
    ora_q = np.full((len(reqs), K), np.nan)
    for n, d in enumerate(decisions):
        ora_p[n, : len(d.p_x)] = d.p_x
        ora_q[n, : len(d.q_x)] = d.q_x
    bad_p = check_probabilities(p[reqs], ora_p, budgets)
    bad_q = check_probabilities(q[reqs], ora_q, budgets)
    assert not bad_p, (tag, "p_x", bad_p[:5])
    assert not bad_q, (tag, "q_x", bad_q[:5])
    for n, kb in enumerate(budgets):                 # padding beyond the budget
        assert np.all(np.isnan(p[reqs[n], kb:])) and np.all(np.isnan(q[reqs[n], kb:]))
    drafted = inp["tokens"].cpu().numpy()[reqs]
    mass_fn = logits_mass_fn(inp["target"], inp["draft"], inp["budgets"].cpu().numpy(), reqs,
                             decisions, T)
    cmp = assert_sampled(tag, g_tok, g_n, decisions, K, drafted, mass_fn, log=_log)
    return cmp.n_excused


# ------------------------------------------------------------------ Philox ---

@pytest.mark.parametrize("seed", [0, 2**64 - 1, (5 << 32) | 17, 0x0123456789ABCDEF])
def test_device_philox_matches_oracle(seed):
    B, P = 1000, 9
    got = philox_words(seed, B, P, DEV).cpu().numpy().astype(np.uint64)
    k0, k1 = philox.seed_key(seed)
    bb, ii = np.meshgrid(np.arange(B, dtype=np.uint64), np.arange(P, dtype=np.uint64),
                         indexing="ij")
    ref = np.stack(philox.philox4x32_np(bb, ii, 0, 0, k0, k1), axis=-1)
    assert np.array_equal(got, ref)


# -------------------------------------------------------------------- tiny ---

def test_tiny_greedy_bit_exact():
    inp = make_inputs("tiny", B=64, variant="greedy", temperature=0.0)
    gpu = _run(inp, 1)
    _assert_parity(inp, 1, gpu, _oracle(inp, 1), tag="tiny-greedy")


def test_tiny_q_equal_p_accepts_all():
    inp = make_inputs("tiny", B=2000, variant="q_eq_p")
    seed = philox_seed(1, 7)
    gpu = _run(inp, seed)
    assert np.all(gpu[1] == 4)
    _assert_parity(inp, seed, gpu, _oracle(inp, seed), tag="tiny-q=p")


@pytest.mark.parametrize("variant", ["sampled", "adversarial"])
def test_tiny_sampled_parity_and_exactness(variant):
    """20,000 trials (one context-free target, drafted tokens drawn from the
    drafter) in two calls of 10,000 with different seeds: oracle parity for
    every trial and a per-position chi-square of the library's emitted tokens
    against the target's softmax."""
    full = make_inputs("tiny", B=20000, variant=variant)
    emitted = [[] for _ in range(5)]
    for call in range(2):
        part = {n: full[n][call * 10000:(call + 1) * 10000]
                for n in ("target", "draft", "tokens", "budgets")}
        part["temperature"] = full["temperature"]
        seed = philox_seed(1, 1000 + call)
        gpu = _run(part, seed)
        _assert_parity(part, seed, gpu, _oracle(part, seed), tag=f"tiny-{variant}-{call}")
        toks, nacc = gpu[0], gpu[1]
        for i in range(5):
            emitted[i].append(toks[nacc >= i, i])
    zt = full["target"][0].double().numpy()
    for i in range(5):
        e = np.concatenate(emitted[i])
        if e.size < 500:
            continue
        obs = np.bincount(e, minlength=32).astype(float)
        exp = special.softmax(zt[i]) * obs.sum()
        keep = exp >= 5
        obs_m = np.append(obs[keep], obs[~keep].sum())
        exp_m = np.append(exp[keep], exp[~keep].sum())
        if exp_m[-1] < 5:
            obs_m[-2] += obs_m[-1]
            exp_m[-2] += exp_m[-1]
            obs_m, exp_m = obs_m[:-1], exp_m[:-1]
        assert stats.chisquare(obs_m, exp_m).pvalue > 1e-3, (variant, i)


# ------------------------------------------------------------ full configs ---

@pytest.mark.parametrize("T", [0.0, 1.0])
def test_qwen3_shaped_fp32(T):
    inp = make_inputs("qwen3", device=DEV)
    seed = philox_seed(2, 3)
    gpu = _run(inp, seed, temperature=T)
    _assert_parity(inp, seed, gpu, _oracle(inp, seed, temperature=T), temperature=T,
                   tag=f"qwen3-T{T}")


def test_ragged_moderate_bf16():
    inp = make_inputs("ragged", device=DEV)
    seed = philox_seed(3, 1)
    gpu = _run(inp, seed)
    _assert_parity(inp, seed, gpu, _oracle(inp, seed), tag="ragged")


def test_gemma_shaped_bf16():
    inp = make_inputs("gemma", device=DEV)
    seed = philox_seed(4, 1)
    gpu = _run(inp, seed)
    reqs = list(range(0, 128, 2))
    _assert_parity(inp, seed, gpu, _oracle(inp, seed, reqs), requests=reqs, tag="gemma")


@pytest.fixture(scope="module")
def heavy():
    return make_inputs("heavy", device=DEV)


def test_heavy_sampled_full_launch(heavy):
    """The benchmark's workload and launch: oracle on a sample of requests,
    structural checks on all of them."""
    seed = philox_seed(5, 0)
    gpu = _run(heavy, seed)
    toks, nacc = gpu[0], gpu[1]
    budgets = heavy["budgets"].cpu().numpy()
    drafted = heavy["tokens"].cpu().numpy()
    V = heavy["target"].shape[2]
    for b in range(len(budgets)):
        j = int(nacc[b])
        assert 0 <= j <= budgets[b]
        assert list(toks[b, :j]) == list(drafted[b, :j])
        assert 0 <= toks[b, j] < V
        assert np.all(toks[b, j + 1:] == -1)
    reqs = list(range(0, 512, 21))
    _assert_parity(heavy, seed, gpu, _oracle(heavy, seed, reqs), requests=reqs, tag="heavy")


def test_heavy_greedy_every_request(heavy):
    seed = philox_seed(5, 1)
    gpu = _run(heavy, seed, temperature=0.0)
    _assert_parity(heavy, seed, gpu, _oracle(heavy, seed, temperature=0.0), temperature=0.0,
                   tag="heavy-greedy")


# -------------------------------------------------------------- edge cases ---

def _edge_inputs(B, K, V, dtype, budgets, seed, masks=False, ties=False):
    g = torch.Generator().manual_seed(seed)
    zt = 2.0 * torch.randn(B, K + 1, V, generator=g)
    zd = zt[:, :K] + 0.7 * torch.randn(B, K, V, generator=g)
    if ties:
        zt = torch.round(zt)
    if masks:
        m = torch.rand(B, K + 1, V, generator=g) < 0.3
        zt[m] = -float("inf")
        zt[..., 0] = 0.0                       # keep every row finite somewhere
        md = torch.rand(B, K, V, generator=g) < 0.3
        zd[md] = -float("inf")
        zd[..., 1 % V] = 0.0
    t = zt.to(dtype)
    d = zd.to(dtype)
    x = torch.argmax(d.float(), dim=-1).to(torch.int32)
    k = torch.tensor(budgets, dtype=torch.int32)
    return {"target": t, "draft": d, "tokens": x, "budgets": k}


EDGE = [
    # B, K, V, dtype, budgets
    (1, 0, 1, torch.float32, [0]),
    (3, 2, 3, torch.bfloat16, [0, 1, 2]),
    (37, 3, 1003, torch.bfloat16, None),          # rows not 16-byte aligned
    (37, 3, 1003, torch.float32, None),
    (9, 8, 16392, torch.bfloat16, None),           # two chunks, ragged tail
    (5, 4, 40003, torch.bfloat16, None),           # several chunks, misaligned rows
    (5, 4, 40003, torch.float32, None),
    (64, 1, 2048, torch.bfloat16, None),           # exactly one sampling tile
]


@pytest.mark.parametrize("B,K,V,dtype,budgets", EDGE)
@pytest.mark.parametrize("T", [0.0, 0.7])
@pytest.mark.parametrize("masks", [False, True])
def test_edge_shapes(B, K, V, dtype, budgets, T, masks):
    if budgets is None:
        budgets = [(b * 7) % (K + 1) for b in range(B)]
    inp = _edge_inputs(B, K, V, dtype, budgets, seed=B * 1000 + V, masks=masks, ties=(T == 0))
    inp["temperature"] = T
    seed = 0xABCDEF00 + B + V
    _log(f"edge B={B} K={K} V={V} {dtype} T={T} masks={masks}")
    gpu = _run(inp, seed, temperature=T)
    _assert_parity(inp, seed, gpu, _oracle(inp, seed, temperature=T), temperature=T,
                   tag=f"edge-{B}-{K}-{V}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_greedy_argmax_ties_signed_zeros_and_masked_rows(dtype):
    """The greedy rule's first argmax where it is easiest to get wrong across
    vocabulary chunks: a -0 and a +0 maximum in different chunks (equal, so
    the lower index), equal positive maxima in different chunks, rows that
    are -inf everywhere (the first index) and a maximum in the last,
    ragged element. Drafted tokens are set to accept or reject on purpose."""
    B, K, V = 6, 3, 40003                      # 2 (bf16) or 3 (fp32) chunks, ragged tail
    g = torch.Generator().manual_seed(4242)
    zt = -1.0 - torch.rand(B, K + 1, V, generator=g)
    x = torch.zeros(B, K, dtype=torch.int32)
    lo, hi = 100, 35000                        # first and last chunk
    zt[0, :, lo] = -0.0
    zt[0, :, hi] = 0.0
    x[0, :] = lo                               # all accepted; bonus = lo
    zt[1, :, lo] = 0.0
    zt[1, :, hi] = -0.0
    x[1, :] = hi                               # rejected at 0; y = lo
    zt[2] = -float("inf")
    x[2, :] = 0                                # -inf rows: argmax 0, all accepted
    zt[3, :, V - 1] = 3.0
    x[3, 0] = V - 1
    x[3, 1] = V - 2                            # rejected at 1; y = V - 1
    zt[4, :, 20] = 5.0
    zt[4, :, 30000] = 5.0
    x[4, :] = 20
    x[4, 2] = 30000                            # rejected at 2; y = 20
    budgets = torch.tensor([3, 3, 3, 2, 3, 0], dtype=torch.int32)
    # The planted values (0, -0, 3, 5, -inf) are exact in bf16 as well.
    inp = {"target": zt.to(dtype), "draft": zt[:, :K].to(dtype).contiguous(), "tokens": x,
           "budgets": budgets, "temperature": 0.0}
    seed = 0x51A0
    gpu = _run(inp, seed, temperature=0.0)
    _assert_parity(inp, seed, gpu, _oracle(inp, seed, temperature=0.0), temperature=0.0,
                   tag=f"greedy-keys-{dtype}")
    n = gpu[1]
    assert list(n) == [3, 0, 3, 1, 2, 0]
    y = [int(gpu[0][b][int(n[b])]) for b in range(B)]
    assert y[:5] == [lo, lo, 0, V - 1, 20]


@pytest.mark.parametrize("V,dtype", [(40003, torch.float32), (151936, torch.bfloat16),
                                     (92161, torch.bfloat16)])
def test_bonus_draws_over_multi_chunk_rows(V, dtype):
    """q = p: every drafted token is accepted, so every request draws its
    bonus token from p_k, whose chunk masses come from the records the
    streaming pass writes for the bonus row (two chunks per unit, the last
    one alone when the chunk count is odd). Rows of 3 (fp32), 5 and 4 (bf16)
    chunks, budgets 0..K."""
    B, K = 48, 3
    budgets = [b % (K + 1) for b in range(B)]
    inp = _edge_inputs(B, K, V, dtype, budgets, seed=V + B)
    inp["draft"] = inp["target"][:, :K].contiguous()
    inp["tokens"] = torch.argmax(inp["draft"].float(), dim=-1).to(torch.int32)
    inp["temperature"] = 1.0
    seed = philox_seed(3, V)
    _log(f"bonus-only B={B} K={K} V={V} {dtype}")
    gpu = _run(inp, seed, temperature=1.0)
    assert list(gpu[1]) == budgets
    _assert_parity(inp, seed, gpu, _oracle(inp, seed, temperature=1.0), temperature=1.0,
                   tag=f"bonus-{V}")


MAXIMA = [
    # B, K, V, dtype, budgets: the header's largest K, vocabulary and batch
    (3, 32, 4099, torch.bfloat16, [32, 17, 0]),
    (2, 2, 1 << 20, torch.bfloat16, [2, 1]),
    (2, 2, 1 << 20, torch.float32, [2, 0]),        # 69 chunks per row: more than one wave's lanes
    (16384, 1, 40, torch.float32, None),           # two launches of 8192 requests
]


@pytest.mark.parametrize("B,K,V,dtype,budgets", MAXIMA)
@pytest.mark.parametrize("T", [0.0, 1.0])
def test_maximum_sizes(B, K, V, dtype, budgets, T):
    if budgets is None:
        budgets = [b % (K + 1) for b in range(B)]
    inp = _edge_inputs(B, K, V, dtype, budgets, seed=B + K + V, ties=(T == 0))
    inp["temperature"] = T
    seed = 0x5EED0000 + B + K
    _log(f"maximum B={B} K={K} V={V} {dtype} T={T}")
    gpu = _run(inp, seed, temperature=T)
    # The oracle on every request of the small batches; on the largest batch,
    # every 41st request and the last ones of both launches.
    reqs = list(range(B)) if B <= 64 else sorted(set(range(0, B, 41)) | set(range(8187, 8197)) |
                                                 set(range(B - 5, B)))
    _assert_parity(inp, seed, gpu, _oracle(inp, seed, requests=reqs, temperature=T),
                   requests=reqs, temperature=T, tag=f"max-{B}-{K}-{V}")


def test_empty_batch_is_a_no_op():
    sv = SpecVerify(DEV, max_batch=4, max_k=2, vocab=64, dtype=torch.float32)
    t = torch.zeros(0, 3, 64, device=DEV)
    d = torch.zeros(0, 2, 64, device=DEV)
    x = torch.zeros(0, 2, dtype=torch.int32, device=DEV)
    k = torch.zeros(0, dtype=torch.int32, device=DEV)
    toks, nacc, p, q = sv.run(t, d, x, k, 1.0, 1)
    torch.cuda.synchronize()
    assert toks.shape == (0, 3) and sv.status() == 0
    sv.close()


def test_bad_budget_and_token_set_status_flags():
    B, K, V = 6, 3, 500
    inp = _edge_inputs(B, K, V, torch.bfloat16, [3, 3, 3, 3, 3, 3], seed=9)
    inp["temperature"] = 1.0
    bad = inp["budgets"].clone()
    bad[1] = 7                                     # > K: clamped to K
    bad[2] = -2                                    # < 0: clamped to 0
    sv = SpecVerify(DEV, max_batch=B, max_k=K, vocab=V, dtype=torch.bfloat16)
    t, d = inp["target"].to(DEV), inp["draft"].to(DEV)
    toks, nacc, _, _ = sv.run(t, d, inp["tokens"].to(DEV), bad.to(DEV), 1.0, 5)
    torch.cuda.synchronize()
    assert sv.status() == binding.SV_FLAG_BAD_BUDGET
    assert sv.status() == 0                        # reading clears it
    clamped = dict(inp)
    clamped["budgets"] = torch.tensor([3, 3, 0, 3, 3, 3], dtype=torch.int32)
    decisions = _oracle(clamped, 5)
    gpu = (toks.cpu().numpy(), nacc.cpu().numpy(), None, None, 0)
    reqs = np.arange(B)
    assert_sampled("bad-budget", gpu[0], gpu[1], decisions, K, inp["tokens"].numpy(),
                   logits_mass_fn(inp["target"], inp["draft"], clamped["budgets"].numpy(), reqs,
                                  decisions, 1.0), log=_log)
    # A drafted token outside [0, V) is rejected and flagged.
    xbad = inp["tokens"].clone()
    xbad[4, 0] = V + 5
    toks, nacc, p, q = sv.run(t, d, xbad.to(DEV), inp["budgets"].to(DEV), 1.0, 5)
    torch.cuda.synchronize()
    assert sv.status() == binding.SV_FLAG_BAD_TOKEN
    assert int(nacc[4]) == 0 and float(p[4, 0]) == 0.0 and float(q[4, 0]) == 0.0
    assert 0 <= int(toks[4, 0]) < V
    sv.close()


def test_repeat_calls_reuse_workspace_and_are_deterministic():
    inp = make_inputs("ragged", device=DEV)
    t, d, x, k = (inp[n].to(DEV) for n in ("target", "draft", "tokens", "budgets"))
    sv = SpecVerify(DEV, max_batch=64, max_k=6, vocab=t.shape[2], dtype=t.dtype)
    outs = []
    for _ in range(3):
        toks, nacc, p, q = sv.run(t, d, x, k, 0.8, 42)
        outs.append((toks.clone(), nacc.clone(), p.clone(), q.clone()))
    # A smaller batch through the same context, then the full one again.
    sub = {n: inp[n][:17] for n in ("target", "draft", "tokens", "budgets")}
    sub["temperature"] = 0.8
    toks_s, nacc_s, _, _ = sv.run(t[:17].contiguous(), d[:17].contiguous(), x[:17].contiguous(),
                                  k[:17].contiguous(), 0.8, 42)
    toks, nacc, p, q = sv.run(t, d, x, k, 0.8, 42)
    outs.append((toks, nacc, p, q))
    torch.cuda.synchronize()
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert torch.equal(a.nan_to_num(-7.0), b.nan_to_num(-7.0))
    assert torch.equal(toks_s, outs[0][0][:17]) and torch.equal(nacc_s, outs[0][1][:17])
    assert sv.status() == 0
    sv.close()


def test_interleaved_modes_and_sizes_on_one_context():
    """Greedy and sampled calls of different batch sizes, with a rejected
    call among them, in turn on one context: every call's outputs equal the
    same call's on a fresh context. The launches alternate between the two
    schedule counters, and the greedy keys and counters must be clear again
    after each call that raised them."""
    inp = make_inputs("ragged", device=DEV)
    t, d, x, k = (inp[n].to(DEV) for n in ("target", "draft", "tokens", "budgets"))
    B, K1, V = t.shape
    sv = SpecVerify(DEV, max_batch=B, max_k=K1 - 1, vocab=V, dtype=t.dtype)

    def call(ctx, n, T, seed):
        dd = d[:n].contiguous() if T > 0 else None
        out = ctx.run(t[:n].contiguous(), dd, x[:n].contiguous(), k[:n].contiguous(), T, seed)
        return tuple(o.clone() for o in out)

    plan = [(B, 0.8, 11), (B, 0.0, 0), (23, 0.0, 0), (B, 0.8, 12), (5, 0.8, 13), None,
            (B, 0.0, 0), (1, 0.8, 14), (B, 0.8, 11)]
    for step in plan:
        if step is None:
            with pytest.raises(ValueError):
                sv.run(t, d, x, k, -1.0, 0)
            continue
        n, T, seed = step
        got = call(sv, n, T, seed)
        fresh = SpecVerify(DEV, max_batch=n, max_k=K1 - 1, vocab=V, dtype=t.dtype)
        want = call(fresh, n, T, seed)
        torch.cuda.synchronize()
        assert fresh.status() == 0
        fresh.close()
        for a, b in zip(got, want):
            assert torch.equal(a.nan_to_num(-7.0), b.nan_to_num(-7.0)), step
    assert sv.status() == 0
    sv.close()


def test_runs_on_a_non_default_stream():
    inp = make_inputs("tiny", B=256, variant="sampled")
    s = torch.cuda.Stream(DEV)
    t, d, x, k = (inp[n].to(DEV) for n in ("target", "draft", "tokens", "budgets"))
    torch.cuda.synchronize()
    sv = SpecVerify(DEV, max_batch=256, max_k=4, vocab=32, dtype=torch.float32)
    with torch.cuda.stream(s):
        toks, nacc, p, q = sv.run(t, d, x, k, 1.0, 11)
    s.synchronize()
    ref = _oracle(inp, 11)
    reqs = np.arange(256)
    assert_sampled("non-default-stream", toks.cpu().numpy(), nacc.cpu().numpy(), ref, 4,
                   inp["tokens"].numpy(),
                   logits_mass_fn(inp["target"], inp["draft"], inp["budgets"].numpy(), reqs, ref,
                                  1.0), log=_log)
    sv.close()


def test_pass_timing_counts_each_pass():
    """Per-pass event timing: sampled runs launch the streaming and the draw
    pass, greedy runs only the streaming pass; batches above the per-launch
    limit of 8192 requests run as several launches of each."""
    inp = make_inputs("tiny", B=8200, variant="sampled")
    t, d, x, k = (inp[n].to(DEV) for n in ("target", "draft", "tokens", "budgets"))
    sv = SpecVerify(DEV, max_batch=8200, max_k=4, vocab=32, dtype=torch.float32)
    sv.run(t, d, x, k, 1.0, 5)                 # not recorded
    sv.timing(True)
    for s in range(3):
        sv.run(t[:100].contiguous(), d[:100].contiguous(), x[:100].contiguous(),
               k[:100].contiguous(), 1.0, s)
    counts, total = sv.pass_times()
    assert counts == [3, 3] and total[0] > 0.0 and total[1] > 0.0
    sv.run(t, None, x, k, 0.0, 0)              # greedy, two launches
    counts, total = sv.pass_times()
    assert counts == [2, 0] and total[0] > 0.0 and total[1] == 0.0
    sv.run(t, d, x, k, 1.0, 9)
    sv.timing(False)                           # discards the record
    sv.timing(True)
    counts, _ = sv.pass_times()
    assert counts == [0, 0]
    sv.timing(False)
    assert sv.status() == 0
    sv.close()


# ---------------------------------------------------- slices of one batch ---

@pytest.mark.parametrize("name,T", [("ragged", 0.8), ("qwen3", 1.0), ("ragged", 0.0)])
def test_request_base_slices_reproduce_the_whole_batch(name, T):
    """Calls over contiguous slices of the batch, each with its global request
    base, give the whole-batch call's outputs bit for bit (how the batch would
    be split across GPUs)."""
    inp = make_inputs(name, device=DEV)
    t, x, k = inp["target"], inp["tokens"], inp["budgets"]
    d = inp["draft"] if T > 0 else None
    B, K1, V = t.shape
    seed = philox_seed(WORKLOAD_SEEDS[name], 77)
    sv = SpecVerify(DEV, max_batch=B, max_k=K1 - 1, vocab=V, dtype=t.dtype)
    whole = [o.clone() for o in sv.run(t, d, x, k, T, seed)]
    cuts = [0, 3, B // 2, B]
    parts = []
    for b0, b1 in zip(cuts[:-1], cuts[1:]):
        out = sv.run(t[b0:b1], None if d is None else d[b0:b1], x[b0:b1], k[b0:b1], T, seed,
                     request_base=b0)
        parts.append([o.clone() for o in out])
    torch.cuda.synchronize()
    assert sv.status() == 0
    for n in range(4):
        joined = torch.cat([p[n] for p in parts])
        assert torch.equal(joined.nan_to_num(-7.0), whole[n].nan_to_num(-7.0)), n
    # The base is the Philox request index: the last slice run without it
    # differs from the whole batch wherever a draw is made.
    if T > 0:
        b0 = B // 2
        moved = sv.run(t[b0:], d[b0:], x[b0:], k[b0:], T, seed, request_base=0)
        torch.cuda.synchronize()
        assert not torch.equal(moved[0], whole[0][b0:])
    sv.close()


WORKLOAD_SEEDS = {"tiny": 1, "qwen3": 2, "ragged": 3, "gemma": 4, "heavy": 5}


@pytest.mark.parametrize("name,T", [("qwen3", 1.0), ("ragged", 0.8)])
def test_request_base_at_the_counter_limit(name, T):
    """The largest request base the ABI accepts, so the device generator runs
    on counter words just below 2^32: every draw and acceptance follows the
    oracle given the same global request indices."""
    inp = make_inputs(name, device=DEV)
    t, d, x, k = inp["target"], inp["draft"], inp["tokens"], inp["budgets"]
    B, K1, V = t.shape
    base = 2 ** 32 - 1 - B
    seed = philox_seed(WORKLOAD_SEEDS[name], 91)
    _log(f"request base {base} {name} T={T}")
    sv = SpecVerify(DEV, max_batch=B, max_k=K1 - 1, vocab=V, dtype=t.dtype)
    toks, nacc, p, q = sv.run(t, d, x, k, T, seed, request_base=base)
    torch.cuda.synchronize()
    gpu = (toks.cpu().numpy(), nacc.cpu().numpy(), p.cpu().numpy(), q.cpu().numpy(), sv.status())
    sv.close()
    decisions = _oracle(inp, seed, temperature=T, request_base=base)
    _assert_parity(inp, seed, gpu, decisions, temperature=T, tag=f"base-{name}")


# ------------------------------------------------------- low temperatures ---

@pytest.mark.parametrize("T", [0.05, 0.3])
@pytest.mark.parametrize("name", ["qwen3", "ragged"])
def test_low_temperature_sampled_parity(name, T):
    """The kernels scale logits by c = log2(e) / T rounded once to fp32, so
    the scaled exponents' error grows as 1/T; the parity bar is unchanged."""
    inp = make_inputs(name, device=DEV)
    seed = philox_seed(WORKLOAD_SEEDS[name], int(T * 1000))
    _log(f"low temperature {name} T={T}")
    gpu = _run(inp, seed, temperature=T)
    _assert_parity(inp, seed, gpu, _oracle(inp, seed, temperature=T), temperature=T,
                   tag=f"{name}-T{T}")


def test_tiny_temperature_reproduces_greedy():
    """T -> 0+: with logits 0.1 apart, sampling at T = 1e-3 keeps and emits
    exactly what greedy verification does (the oracle's own consistency pin,
    here on the library)."""
    B, K, V = 64, 4, 4096
    g = torch.Generator().manual_seed(31)
    base = torch.arange(V, dtype=torch.float32) * 0.1
    zt = torch.stack([base[torch.randperm(V, generator=g)] for _ in range(B * (K + 1))])
    zt = zt.view(B, K + 1, V).contiguous()
    zd = (zt[:, :K] + 0.2 * torch.randn(B, K, V, generator=g)).contiguous()
    x = torch.argmax(zd, dim=-1).to(torch.int32)
    k = torch.full((B,), K, dtype=torch.int32)
    inp = {"target": zt, "draft": zd, "tokens": x, "budgets": k, "temperature": 1e-3}
    seed = 0x7E57
    sampled = _run(inp, seed, temperature=1e-3)
    greedy = _run(inp, seed, temperature=0.0)
    assert np.array_equal(sampled[0], greedy[0]) and np.array_equal(sampled[1], greedy[1])
    _assert_parity(inp, seed, greedy, _oracle(inp, seed, temperature=0.0), temperature=0.0,
                   tag="T0+-greedy")
    assert np.any(greedy[1] < K) and np.any(greedy[1] > 0)


# ------------------------------------------------- partial residency ---

def test_verify_while_another_stream_holds_half_the_cus():
    """A verify call while a bounded kernel on another stream holds half of
    the CUs (each of its workgroups takes a CU's whole LDS): the streaming
    pass's workgroups cannot all be resident at once. No wave of the verify
    kernels waits on another workgroup, so the calls complete, concurrently
    with the other kernel, with the outputs of an unobstructed call and no
    status flag."""
    import ctypes
    from draft_verify_sampling_spec_amd import build
    helper = ctypes.CDLL(build.TEST_LIB_PATH)
    helper.sv_test_occupy.argtypes = [ctypes.c_int, ctypes.c_uint, ctypes.c_void_p,
                                      ctypes.c_void_p]
    helper.sv_test_occupy.restype = ctypes.c_int
    inp = make_inputs("ragged", device=DEV)
    t, d, x, k = inp["target"], inp["draft"], inp["tokens"], inp["budgets"]
    B, K1, V = t.shape
    sv = SpecVerify(DEV, max_batch=B, max_k=K1 - 1, vocab=V, dtype=t.dtype)
    seeds = [philox_seed(3, 900 + i) for i in range(4)]
    modes = [0.8, 0.0, 0.8, 0.0]
    free = []
    for T, seed in zip(modes, seeds):
        free.append([o.clone() for o in sv.run(t, d if T > 0 else None, x, k, T, seed)])
    torch.cuda.synchronize()
    cus = torch.cuda.get_device_properties(DEV).multi_processor_count
    busy_out = torch.zeros(cus // 2, dtype=torch.int32, device=DEV)
    # Streams go to the hardware queues in turn, so of four work streams at
    # least one runs beside the other kernel rather than behind it.
    busy = torch.cuda.Stream(DEV)
    works = [torch.cuda.Stream(DEV) for _ in range(4)]
    b0, b1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
    ends = [torch.cuda.Event(enable_timing=True) for _ in works]
    # Everything that allocates or synchronises (contexts, outputs) comes
    # first; one context per stream, since calls that overlap in time must
    # not share one.
    ctxs = [SpecVerify(DEV, max_batch=B, max_k=K1 - 1, vocab=V, dtype=t.dtype) for _ in works]
    held = [[[torch.empty_like(o) for o in f] for f in free] for _ in works]
    for c, outs in zip(ctxs, held):                 # first calls (launch queries) now
        for (T, seed), o in zip(zip(modes, seeds), outs):
            c.run(t, d if T > 0 else None, x, k, T, seed, out_tokens=o[0], out_num_accepted=o[1],
                  out_p=o[2], out_q=o[3])
    torch.cuda.synchronize()
    for outs in held:
        for o in outs:
            for v in o:
                v.fill_(-5)
    b0.record(busy)
    assert helper.sv_test_occupy(cus // 2, 30000, busy_out.data_ptr(), busy.cuda_stream) == 0
    b1.record(busy)
    for work, end, c, outs in zip(works, ends, ctxs, held):
        for (T, seed), o in zip(zip(modes, seeds), outs):
            c.run(t, d if T > 0 else None, x, k, T, seed, out_tokens=o[0], out_num_accepted=o[1],
                  out_p=o[2], out_q=o[3], stream=work)
        end.record(work)
    torch.cuda.synchronize()
    assert int(busy_out.sum()) == cus // 2
    busy_ms = b0.elapsed_time(b1)
    done_ms = [b0.elapsed_time(e) for e in ends]
    _log(f"occupier: {busy_ms:.2f} ms; verify calls on four streams done after "
         + ", ".join(f"{v:.2f}" for v in done_ms) + " ms")
    assert min(done_ms) < busy_ms, "no call overlapped the other kernel"
    for outs in held:
        for a, b in zip(free, outs):
            for n in range(4):
                assert torch.equal(a[n].nan_to_num(-7.0), b[n].nan_to_num(-7.0)), n
    for c in ctxs + [sv]:
        assert c.status() == 0
        c.close()
