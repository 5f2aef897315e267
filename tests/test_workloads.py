"""The synthetic workloads: shapes, storage types, budget laws, and the
ragged workload's drafter-noise calibration, re-measured with the oracle."""
import numpy as np
import pytest
import torch

from oracle import verify as ov
from tests.helpers import to_oracle
from workloads import make_inputs, philox_seed
from workloads.configs import CONFIGS
from workloads.gen import SIGMA_CHAT, SIGMA_MATH


@pytest.mark.parametrize("name", ["tiny", "qwen3", "ragged", "gemma", "heavy"])
def test_shapes_and_types(name):
    w = CONFIGS[name]
    B = {"tiny": 16, "qwen3": 2, "ragged": 4, "gemma": 2, "heavy": 4}[name]
    inp = make_inputs(name, B=B)
    t, d, x, k = inp["target"], inp["draft"], inp["tokens"], inp["budgets"]
    assert t.shape == (B, w.K + 1, w.V) and d.shape == (B, w.K, w.V)
    assert x.shape == (B, w.K) and k.shape == (B,)
    assert t.dtype == (torch.bfloat16 if w.fmt == "bf16" else torch.float32)
    assert x.dtype == torch.int32 and k.dtype == torch.int32
    assert bool(((x >= 0) & (x < w.V)).all())
    assert bool(((k >= 0) & (k <= w.K)).all())


def test_heavy_budget_law():
    """Budgets 2 + Binomial(6, 1/3): support 2..8, mean 4, variance 4/3."""
    k = make_inputs("heavy", B=256)["budgets"].numpy()
    assert k.min() >= 2 and k.max() <= 8
    # 256 draws: the sample mean has standard deviation sqrt(4/3 / 256) ~ 0.072.
    assert abs(k.mean() - 4.0) < 0.3
    assert abs(k.var() - 4.0 / 3.0) < 0.5


def test_drafted_tokens_are_drafter_argmax():
    inp = make_inputs("qwen3", B=2)
    assert torch.equal(inp["tokens"], torch.argmax(inp["draft"], dim=-1).to(torch.int32))


def test_ragged_calibration():
    """With the full budget of 6 and T = 0.8, the two halves of the ragged
    workload emit about 3.5 (chat-like) and 5.5 (math/code-like) tokens per
    request on average (accepted + 1); the noise levels SIGMA_CHAT and
    SIGMA_MATH were chosen for that with this oracle."""
    assert SIGMA_CHAT > SIGMA_MATH
    inp = make_inputs("ragged")
    B = inp["target"].shape[0]
    tokens = inp["tokens"].numpy()
    seed = philox_seed(3, 99)
    emitted = []
    for b in range(B):
        zt, fmt = to_oracle(inp["target"][b])
        zd, _ = to_oracle(inp["draft"][b])
        res = ov.verify_request(b, ov.as_f64_rows(zt, fmt), ov.as_f64_rows(zd, fmt), tokens[b], 0.8,
                                seed)
        emitted.append(res.n_accepted + 1)
    emitted = np.asarray(emitted, dtype=float)
    chat, math = emitted[: B // 2].mean(), emitted[B // 2:].mean()
    assert 2.8 < chat < 4.2, chat
    assert 4.8 < math < 6.2, math
