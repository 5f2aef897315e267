"""Seeded synthetic inputs for batched draft verification.

This package only draws inputs: logits, per-request verify budgets, the
drafted tokens, per-position confidences for the budget scheduler,
hidden states with an output head, and the Markov head's factors. It holds none of the verification rule's arithmetic (no
softmax, no acceptance test, no sampling from p or from the residual), so both
the HIP library's tests and the CPU oracle can take their inputs from it.
"""
from .configs import CONFIGS, Workload, get  # noqa: F401
from .confidence import make_confidences  # noqa: F401
from .head import make_head_inputs, make_hidden_inputs  # noqa: F401
from .gen import make_inputs, philox_seed  # noqa: F401
from .markov import make_markov_inputs  # noqa: F401
