"""GPU parity of the verify-budget scheduler (spec_budget_schedule) against
the oracle: budgets are integers decided by fp32 gains that both sides form
in the same order, so they must agree exactly."""
import json
import os
import sys

import numpy as np
import pytest
import torch

from draft_verify_sampling_spec_amd import SpecVerify, schedule_budgets
from oracle import schedule as osch
from oracle import verify as ov
from tests.helpers import assert_sampled, logits_mass_fn, to_oracle
from workloads import make_confidences, make_inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "schedule_cases.json")


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


def _check(conf_cpu, n_total, tau):
    conf = conf_cpu.to(DEV).contiguous()
    got = schedule_budgets(conf, n_total, tau).cpu().numpy()
    want = osch.schedule(conf_cpu.numpy(), n_total, tau)
    assert got.tolist() == want.tolist(), (conf_cpu.shape, n_total, tau)
    return got


def test_golden_cases():
    for case in json.load(open(GOLDEN))["cases"]:
        conf = torch.tensor(case["conf"], dtype=torch.float32)
        for run in case["runs"]:
            got = schedule_budgets(conf.to(DEV), run["N"], run["tau"]).cpu().tolist()
            assert got == run["budgets"], (case["conf"], run)


@pytest.mark.parametrize("B,K", [(1, 1), (7, 5), (64, 6), (512, 8), (1000, 3), (3000, 32)])
@pytest.mark.parametrize("quantum", [None, 16])
def test_random_confidences_match_oracle(B, K, quantum):
    conf = make_confidences(B, K, seed=B * 100 + K, quantum=quantum)
    _log(f"[schedule] B={B} K={K} quantum={quantum}")
    for n_total in sorted({0, 1, B // 2, B, 4 * B, B * K - 1, B * K, B * K + 5}):
        if n_total < 0:
            continue
        for tau in (0.0, 0.05, 0.3):
            ks = _check(conf, n_total, tau)
            assert ks.sum() <= n_total and ks.max() <= K


def test_full_batch_with_ties():
    conf = make_confidences(16384, 8, seed=7, quantum=8)
    _log("[schedule] B=16384 K=8")
    _check(conf, 4 * 16384, 0.0)
    _check(conf, 16384 * 8, 0.1)


def test_tiny_gains_and_clamping():
    rng = np.random.default_rng(3)
    c = rng.uniform(1e-3, 0.2, size=(40, 32)).astype(np.float32)   # products far below fp32's normal range
    c[0, :] = [np.nan, 2.0, -1.0, -0.0] * 8
    c[1, :] = 1.0
    conf = torch.from_numpy(c)
    for n_total in (0, 10, 100, 40 * 32):
        _check(conf, n_total, 0.0)


def test_zero_positions_and_degenerate_budgets():
    conf = make_confidences(9, 0, seed=1)
    assert schedule_budgets(conf.to(DEV), 10, 0.0).cpu().tolist() == [0] * 9
    conf = make_confidences(9, 4, seed=2)
    assert schedule_budgets(conf.to(DEV), 0, 0.0).cpu().tolist() == [0] * 9
    assert schedule_budgets(conf.to(DEV), 100, 0.999999).cpu().sum().item() == \
        int((osch.gains_fp32(conf.numpy()) > np.float32(0.999999)).sum())


def test_scheduled_budgets_drive_verification_on_one_stream():
    """Scheduler then verifier on one stream: the budgets go straight from
    one call's output to the next call's input, and the verification result
    matches the oracle run with the oracle's budgets."""
    inp = make_inputs("tiny", B=256, variant="sampled")
    B, K1, V = inp["target"].shape
    K = K1 - 1
    conf = make_confidences(B, K, seed=9)
    s = torch.cuda.Stream(DEV)
    t, d, x = (inp[n].to(DEV) for n in ("target", "draft", "tokens"))
    c_dev = conf.to(DEV)
    torch.cuda.synchronize()
    sv = SpecVerify(DEV, max_batch=B, max_k=K, vocab=V, dtype=torch.float32)
    with torch.cuda.stream(s):
        k_dev = schedule_budgets(c_dev, 2 * B, 0.0, stream=s)
        toks, nacc, _, _ = sv.run(t, d, x, k_dev, 1.0, 123, stream=s)
    s.synchronize()
    k_ref = osch.schedule(conf.numpy(), 2 * B, 0.0)
    assert k_dev.cpu().numpy().tolist() == k_ref.tolist()
    ref = []
    for b in range(B):
        zt, fmt = to_oracle(inp["target"][b])
        zd, _ = to_oracle(inp["draft"][b])
        tok = inp["tokens"][b].numpy().copy()
        ref.append(ov.verify_request(b, ov.as_f64_rows(zt, fmt)[: k_ref[b] + 1],
                                     ov.as_f64_rows(zd, fmt)[: k_ref[b]], tok[: k_ref[b]], 1.0, 123))
    assert_sampled("scheduled-budgets", toks.cpu().numpy(), nacc.cpu().numpy(), ref, K,
                   inp["tokens"].numpy(),
                   logits_mass_fn(inp["target"], inp["draft"], k_ref, np.arange(B), ref, 1.0))
    assert sv.status() == 0
    sv.close()
