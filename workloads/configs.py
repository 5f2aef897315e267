"""The five synthetic verify workloads (shapes, storage type, temperature).

Shapes follow the pages' models where the pages name them: a Qwen3-4B-shaped
vocabulary of 151,936 tokens and a Gemma-4-shaped one of 262,144; budgets
follow "What DSpark adds" on the first page (per-request verify budgets, four
to six tokens under moderate load against a baseline of two, shorter under
heavy load, with blocks of up to five tokens or eight in the "block8" config
of the third page). Value laws are the synthetic stand-ins described in
``workloads.gen``.
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    B: int             # requests
    K: int             # drafted tokens per request (tensor width)
    V: int             # vocabulary
    fmt: str           # logit storage: "f32" or "bf16"
    temperature: float
    data_seed: int     # seed of the input draws
    summary: str


CONFIGS = {
    "tiny": Workload(
        "tiny", 1, 4, 32, "f32", 1.0, 1,
        "B=1 K=4 V=32 fp32; target N(0,2^2), drafter = target + N(0,0.5^2); "
        "drafted tokens drawn from the drafter; run as many independent trials"),
    "qwen3": Workload(
        "qwen3", 8, 5, 151936, "f32", 1.0, 2,
        "B=8 K=5 V=151936 fp32; target N(0,3^2) plus +8 on one random token per "
        "row; drafter = target + N(0,1); drafted token = drafter argmax; T in {0, 1}"),
    "ragged": Workload(
        "ragged", 64, 6, 151936, "bf16", 0.8, 3,
        "B=64 K=6 V=151936 bf16; budgets uniform on 2..6; target N(0,3^2); "
        "drafter noise per half set for a chat-like and a math/code-like "
        "accepted length; T=0.8"),
    "gemma": Workload(
        "gemma", 128, 5, 262144, "bf16", 1.0, 4,
        "B=128 K=5 V=262144 bf16; target N(0,2.5^2) - 1.1 ln(rank) over a random "
        "per-row ranking (Zipf(1.1) prior); drafter = target + N(0,0.7^2); budget 5"),
    "heavy": Workload(
        "heavy", 512, 8, 151936, "bf16", 1.0, 5,
        "B=512 K=8 V=151936 bf16; budgets 2 + Binomial(6, 1/3) (2..8, mean 4); "
        "target N(0,3^2); drafter noise U[0.3, 1.5] per request; T=1"),
}


def get(name: str) -> Workload:
    try:
        return CONFIGS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; have {sorted(CONFIGS)}") from None
