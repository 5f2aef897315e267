"""Seeded synthetic inputs for the output head: hidden states h ~ N(0, 1) and
a head W ~ N(0, 9 / H), both rounded to bf16, so that logits z = h W^T have
standard deviation about 3 (the scale of the verify workloads' logits).
Tokens are uniform over the vocabulary. No head arithmetic lives here."""
from __future__ import annotations

import torch


def make_head_inputs(R: int, H: int, V: int, seed: int, device="cuda"):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    hidden = torch.randn(R, H, generator=g, device=device).to(torch.bfloat16)
    weight = (torch.randn(V, H, generator=g, device=device) * (3.0 / H ** 0.5)).to(torch.bfloat16)
    tokens = torch.randint(0, V, (R,), generator=g, device=device, dtype=torch.int32)
    return hidden, weight, tokens
