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


def make_hidden_inputs(B: int, K: int, H: int, V: int, seed: int, device="cuda",
                       variant: str = "heavy", temperature: float = 1.0, budgets=None):
    """Inputs of a verify step from hidden states through a shared head.

    Head W ~ N(0, 9 / H) [V, H] and target states h_t ~ N(0, 1) [B, K+1, H],
    so the target's logits have standard deviation about 3 (the heavy
    workload's logit law). Drafter states h_d = h_t[:, :K] + (sigma_b / 3)
    eps' with sigma_b ~ U[0.3, 1.5] per request, so the drafter's logits
    differ from the target's by about sigma_b eps' (again the heavy law).
    Everything is drawn in fp32 and stored as bf16.

    variant:
      "heavy"  drafted token = argmax of the drafter's logits (fp32 product of
               the stored bf16 values, first maximum); budgets
               2 + Binomial(6, 1/3), at most K (unless given).
      "sampled" one shared set of rows for every request (a context-free
               target, so the requests are independent trials of one
               position set); drafted tokens drawn from q = softmax(z_d / T)
               by the Gumbel-max trick with this generator (a drafter's own
               draw, independent of the verifier's Philox numbers); budgets K.
      "q_eq_p" h_d = h_t[:, :K] exactly; drafted tokens as "heavy".
    Returns a dict: target_hidden, draft_hidden, head, tokens, budgets (int32).
    """
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    head = (torch.randn(V, H, generator=g, device=device) * (3.0 / H ** 0.5)).to(torch.bfloat16)
    rows = 1 if variant == "sampled" else B
    th = torch.randn(rows, K + 1, H, generator=g, device=device)
    sigma = 0.3 + 1.2 * torch.rand(rows, 1, 1, generator=g, device=device)
    noise = torch.randn(rows, K, H, generator=g, device=device)
    th = th.to(torch.bfloat16)
    if variant == "q_eq_p":
        dh = th[:, :K].clone()
    else:
        dh = (th[:, :K].float() + (sigma / 3.0) * noise).to(torch.bfloat16)
    if variant == "sampled":
        th = th.expand(B, K + 1, H).contiguous()
        dh = dh.expand(B, K, H).contiguous()
    th, dh = th.contiguous(), dh.contiguous()

    wf = head.float()
    tokens = torch.empty(B, K, dtype=torch.int32, device=device)
    step = max(1, (1 << 26) // max(1, K * V))          # requests per chunk of drafter logits
    for b0 in range(0, B, step):
        zd = dh[b0:b0 + step].float() @ wf.T           # [b, K, V]
        if variant == "sampled":
            u = torch.rand(zd.shape, generator=g, device=device).clamp_min(1e-20)
            zd = zd / float(temperature) - torch.log(-torch.log(u))
        tokens[b0:b0 + step] = zd.argmax(dim=-1).to(torch.int32)
    if budgets is None:
        if variant == "heavy":
            draws = torch.rand(B, 6, generator=g, device=device) < (1.0 / 3.0)
            budgets = (2 + draws.sum(dim=1)).clamp_max(K).to(torch.int32)
        else:
            budgets = torch.full((B,), K, dtype=torch.int32, device=device)
    else:
        budgets = torch.as_tensor(budgets, dtype=torch.int32).to(device)
    return {"target_hidden": th, "draft_hidden": dh, "head": head, "tokens": tokens,
            "budgets": budgets.contiguous()}
