"""Seeded synthetic per-position confidences, standing in for the output of
a confidence head (values in (0, 1), as a logistic function of a learned
score would give).

Request b is chat-like (lower confidence, falling faster along the block) or
math/code-like; c[b, i] = sigmoid(a_b - s_b * i + 0.5 * eps[b, i]) with
a_b ~ U[0.5, 1.5] (chat) or U[2.0, 3.5] (math/code) and s_b ~ U[0.3, 0.6]
(chat) or U[0.1, 0.3] (math/code), eps standard normal. ``quantum`` rounds
the values to multiples of 1/quantum (many exactly equal gains, for tie
tests). No scheduling arithmetic lives here.
"""
from __future__ import annotations

import numpy as np
import torch


def make_confidences(B: int, K: int, seed: int, chat_fraction: float = 0.5,
                     quantum: int | None = None, device=None) -> torch.Tensor:
    rng = np.random.default_rng(seed)
    chat = rng.random(B) < chat_fraction
    a = np.where(chat, rng.uniform(0.5, 1.5, B), rng.uniform(2.0, 3.5, B))
    s = np.where(chat, rng.uniform(0.3, 0.6, B), rng.uniform(0.1, 0.3, B))
    i = np.arange(K)[None, :]
    z = a[:, None] - s[:, None] * i + 0.5 * rng.standard_normal((B, K))
    c = 1.0 / (1.0 + np.exp(-z))
    if quantum:
        c = np.round(c * quantum) / quantum
    t = torch.from_numpy(c.astype(np.float32))
    return t.to(device) if device is not None else t
