"""CPU oracle of batched draft verification (plain NumPy, fp64).

TEST INFRASTRUCTURE, not product code. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import, call or execute anything in this package. It shares no code with the
HIP library in ``draft_verify_sampling_spec_amd`` and neither imports the
other.

Modules:
  philox  -- Philox4x32-10 from the SC'11 definition, and the stream layout
             (key = seed, counter = (request, position, 0, 0)).
  verify  -- the verification rule itself (greedy and sampled), per request.
  schedule -- the confidence-driven verify-budget scheduler.
  head    -- the shared output head's row statistics.
  hidden  -- a verify step whose logits come from hidden states and the head.
  markov  -- the drafter's low-rank Markov head (previous-token logit bias).

Every function here is pinned by ``tests/test_oracle_*.py`` against facts that
do not come from the oracle itself: library routines (rocRAND's Philox,
scipy's logsumexp and chi-square, numpy's searchsorted), exact enumeration on
dyadic inputs, closed forms and invariants of the rule.
"""
from . import philox, verify  # noqa: F401
