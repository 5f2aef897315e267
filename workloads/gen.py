"""Seeded draws of verify inputs with torch generators.

Inputs are drawn once per (workload, seed) on the requested device. The CPU
oracle always reads back the exact tensors the HIP library was given, so the
draws need not agree across devices or torch versions.

Value laws (epsilon terms are independent standard normals):

* tiny:   z_t = 2 eps per position, shared by every trial (a context-free
          target); z_d = z_t + 0.5 eps'. Variants: "sampled" draws each
          trial's drafted tokens from q = softmax(z_d / T) with the Gumbel-max
          trick (argmax of z_d / T plus Gumbel noise, a drafter's own draw that
          is independent of the verifier's Philox stream); "greedy" drafts
          argmax z_d; "q_eq_p" sets z_d = z_t exactly; "adversarial" sets
          z_d = -3 z_t, so the drafter prefers the target's least likely
          tokens; "noisy" uses z_d = z_t + 5 eps'.
* qwen3:  z_t = 3 eps plus 8 on one uniformly chosen token per row;
          z_d = z_t + eps'; drafted token = argmax z_d; budgets = K.
* ragged: z_t = 3 eps; z_d = z_t + sigma_b eps' with sigma_b = SIGMA_CHAT for
          the first half of the requests and SIGMA_MATH for the second;
          budgets uniform on 2..6; drafted token = argmax z_d.
* gemma:  z_t = 2.5 eps - 1.1 ln(rank_v) with rank a random permutation of
          1..V per row (a Zipf(1.1) prior over a random token order);
          z_d = z_t + 0.7 eps'; budgets = K.
* heavy:  z_t = 3 eps; z_d = z_t + sigma_b eps' with sigma_b ~ U[0.3, 1.5] per
          request; budgets 2 + Binomial(6, 1/3) (support 2..8, mean 4).

bf16 workloads draw in fp32 and round to nearest even. The drafted token of
an argmax drafter is taken on the stored (rounded) drafter logits, lowest
index on ties (torch.argmax returns the first maximum).
"""
from __future__ import annotations

import torch

from .configs import get

# Drafter noise of the two halves of the ragged workload. Chosen so that, with
# the full budget of 6 and T = 0.8, the oracle's mean emitted length per
# request (accepted + 1) is close to 3.5 (chat-like) and 5.5 (math/code-like);
# tests/test_workloads.py re-measures this with the oracle.
SIGMA_CHAT = 0.46
SIGMA_MATH = 0.17


def philox_seed(workload_index: int, step: int) -> int:
    """Philox seed of one verify call: workload index in the high word, step low."""
    return ((int(workload_index) & 0xFFFFFFFF) << 32) | (int(step) & 0xFFFFFFFF)


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _store(x: torch.Tensor, fmt: str) -> torch.Tensor:
    if fmt == "bf16":
        return x.to(torch.bfloat16).contiguous()
    if fmt == "f32":
        return x.to(torch.float32).contiguous()
    raise ValueError(fmt)


def _argmax_tokens(draft: torch.Tensor) -> torch.Tensor:
    return torch.argmax(draft.float(), dim=-1).to(torch.int32).contiguous()


def _tiny(w, g, device, B, variant, temperature):
    K, V = w.K, w.V
    zt_rows = 2.0 * torch.randn(K + 1, V, generator=g, device=device)
    noise = torch.randn(K, V, generator=g, device=device)
    if variant == "q_eq_p":
        zd_rows = zt_rows[:K].clone()
    elif variant == "adversarial":
        zd_rows = -3.0 * zt_rows[:K]
    elif variant == "noisy":
        zd_rows = zt_rows[:K] + 5.0 * noise
    else:
        zd_rows = zt_rows[:K] + 0.5 * noise
    target = _store(zt_rows, w.fmt).unsqueeze(0).expand(B, K + 1, V).contiguous()
    draft = _store(zd_rows, w.fmt).unsqueeze(0).expand(B, K, V).contiguous()
    if variant == "greedy" or temperature == 0.0:
        tokens = _argmax_tokens(draft)
    else:
        # Gumbel-max: argmax(z/T + G) with G = -log(-log U) is a draw from softmax(z/T).
        u = torch.rand(B, K, V, generator=g, device=device, dtype=torch.float64)
        u = u.clamp_(min=1e-300)
        gumbel = -torch.log(-torch.log(u))
        tokens = torch.argmax(draft.double() / temperature + gumbel, dim=-1)
        tokens = tokens.to(torch.int32).contiguous()
    budgets = torch.full((B,), K, dtype=torch.int32, device=device)
    return target, draft, tokens, budgets


def _qwen3(w, g, device, B):
    K, V = w.K, w.V
    zt = 3.0 * torch.randn(B, K + 1, V, generator=g, device=device)
    peak = torch.randint(0, V, (B, K + 1), generator=g, device=device)
    zt.scatter_add_(2, peak.unsqueeze(-1), torch.full((B, K + 1, 1), 8.0, device=device))
    zd = zt[:, :K] + torch.randn(B, K, V, generator=g, device=device)
    target, draft = _store(zt, w.fmt), _store(zd, w.fmt)
    budgets = torch.full((B,), K, dtype=torch.int32, device=device)
    return target, draft, _argmax_tokens(draft), budgets


def _ragged(w, g, device, B):
    K, V = w.K, w.V
    zt = 3.0 * torch.randn(B, K + 1, V, generator=g, device=device)
    sigma = torch.where(torch.arange(B, device=device) < B // 2,
                        torch.tensor(SIGMA_CHAT, device=device),
                        torch.tensor(SIGMA_MATH, device=device))
    zd = zt[:, :K] + sigma.view(B, 1, 1) * torch.randn(B, K, V, generator=g, device=device)
    target, draft = _store(zt, w.fmt), _store(zd, w.fmt)
    budgets = torch.randint(2, 7, (B,), generator=g, device=device).to(torch.int32)
    return target, draft, _argmax_tokens(draft), budgets


def _gemma(w, g, device, B):
    K, V = w.K, w.V
    zt = 2.5 * torch.randn(B, K + 1, V, generator=g, device=device)
    # A random ranking per row: argsort of uniform keys is a uniform permutation.
    keys = torch.rand(B * (K + 1), V, generator=g, device=device)
    rank = torch.empty_like(keys)
    order = torch.argsort(keys, dim=1)
    ranks = torch.arange(1, V + 1, device=device, dtype=keys.dtype).expand_as(keys)
    rank.scatter_(1, order, ranks)
    del keys, order
    zt -= 1.1 * torch.log(rank.view(B, K + 1, V))
    del rank
    zd = zt[:, :K] + 0.7 * torch.randn(B, K, V, generator=g, device=device)
    target, draft = _store(zt, w.fmt), _store(zd, w.fmt)
    budgets = torch.full((B,), K, dtype=torch.int32, device=device)
    return target, draft, _argmax_tokens(draft), budgets


def _heavy(w, g, device, B):
    K, V = w.K, w.V
    target = torch.empty(B, K + 1, V, dtype=torch.bfloat16, device=device)
    draft = torch.empty(B, K, V, dtype=torch.bfloat16, device=device)
    sigma = 0.3 + 1.2 * torch.rand(B, generator=g, device=device)
    # Draw request by request blocks to bound the fp32 temporaries.
    step = 64
    for b0 in range(0, B, step):
        b1 = min(B, b0 + step)
        zt = 3.0 * torch.randn(b1 - b0, K + 1, V, generator=g, device=device)
        target[b0:b1] = zt.to(torch.bfloat16)
        zd = zt[:, :K] + sigma[b0:b1].view(-1, 1, 1) * torch.randn(
            b1 - b0, K, V, generator=g, device=device)
        draft[b0:b1] = zd.to(torch.bfloat16)
        del zt, zd
    trials = (torch.rand(B, 6, generator=g, device=device) < (1.0 / 3.0)).sum(dim=1)
    budgets = (2 + trials).to(torch.int32)
    return target, draft, _argmax_tokens(draft), budgets


def make_inputs(name: str, device="cpu", seed=None, B=None, variant="sampled",
                temperature=None):
    """Draw the inputs of workload ``name``.

    Returns a dict with target [B, K+1, V], draft [B, K, V] (torch float32 or
    bfloat16), tokens [B, K] int32, budgets [B] int32, temperature, fmt and
    the Workload record. ``B`` overrides the request count (tiny: trials).
    """
    w = get(name)
    B = w.B if B is None else int(B)
    temperature = w.temperature if temperature is None else float(temperature)
    g = _gen(device, w.data_seed if seed is None else seed)
    if name == "tiny":
        t, d, x, k = _tiny(w, g, device, B, variant, temperature)
    elif name == "qwen3":
        t, d, x, k = _qwen3(w, g, device, B)
    elif name == "ragged":
        t, d, x, k = _ragged(w, g, device, B)
    elif name == "gemma":
        t, d, x, k = _gemma(w, g, device, B)
    elif name == "heavy":
        t, d, x, k = _heavy(w, g, device, B)
    else:
        raise KeyError(name)
    return {"target": t, "draft": d, "tokens": x, "budgets": k,
            "temperature": temperature, "fmt": w.fmt, "workload": w}
