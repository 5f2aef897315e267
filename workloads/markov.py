"""Seeded synthetic inputs for the drafter's low-rank Markov head.

Only draws inputs (no part of the head's arithmetic): the backbone's logits
for a drafted block, the two rank-r factors and the last token of each
sequence.
"""
from __future__ import annotations

import torch


def make_markov_inputs(B: int, K: int, V: int, r: int, seed: int, device="cuda",
                       base_sigma: float = 3.0, bias_sigma: float = 1.5):
    """Backbone logits base ~ N(0, base_sigma^2) [B, K, V]; factors A ~ N(0, 1)
    and Bm ~ N(0, bias_sigma^2 / r), both [V, r], so a transition bias
    A[x] Bm^T has standard deviation about bias_sigma; previous tokens uniform
    on [0, V). Everything is drawn in fp32 on `device` and stored as bf16
    (tokens int32). Returns a dict: base, markov_a, markov_b, prev."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    base = (torch.randn(B, K, V, generator=g, device=device) * base_sigma).to(torch.bfloat16)
    a = torch.randn(V, r, generator=g, device=device).to(torch.bfloat16)
    bm = (torch.randn(V, r, generator=g, device=device) * (bias_sigma / r ** 0.5)).to(torch.bfloat16)
    prev = torch.randint(0, V, (B,), generator=g, device=device, dtype=torch.int64).to(torch.int32)
    return {"base": base.contiguous(), "markov_a": a.contiguous(), "markov_b": bm.contiguous(),
            "prev": prev.contiguous()}
