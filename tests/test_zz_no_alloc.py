"""The allocation-free entry point (spec_verify_run_noalloc) against the
context entry point (spec_verify_run_ex) through the C ABI: identical outputs
bit for bit, on two calls in a row (the second smaller), in sampled and
greedy mode; and the size limit of its static scratch."""
import ctypes

import numpy as np
import pytest
import torch

from draft_verify_sampling_spec_amd import SpecVerify, binding, verify_noalloc
from workloads import make_inputs, philox_seed

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _same(a, b):
    return torch.equal(a.nan_to_num(-7.0), b.nan_to_num(-7.0))


@pytest.mark.parametrize("T", [0.8, 0.0])
def test_noalloc_matches_the_context_entry_point(T):
    inp = make_inputs("ragged", device=DEV)
    t, x, k = inp["target"], inp["tokens"], inp["budgets"]
    d = inp["draft"] if T > 0 else None
    B, K1, V = t.shape
    sv = SpecVerify(DEV, max_batch=B, max_k=K1 - 1, vocab=V, dtype=t.dtype)
    calls = [(0, B, 0), (5, 22, 5)]            # (first row, end row, request base)
    for step, (b0, b1, base) in enumerate(calls):
        seed = philox_seed(3, 500 + step)
        args = (t[b0:b1], None if d is None else d[b0:b1], x[b0:b1], k[b0:b1], T, seed)
        want = [o.clone() for o in sv.run(*args, request_base=base)]
        got = verify_noalloc(*args, request_base=base)
        torch.cuda.synchronize()
        for n in range(4):
            assert _same(got[n], want[n]), (step, n)
        assert int(got[4][0]) == 0
    assert sv.status() == 0
    sv.close()


def test_noalloc_flags_a_bad_budget_in_its_status_word():
    inp = make_inputs("ragged", device=DEV)
    t, d, x, k = inp["target"][:4], inp["draft"][:4], inp["tokens"][:4], inp["budgets"][:4]
    bad = k.clone()
    bad[2] = 99
    out = verify_noalloc(t, d, x, bad, 1.0, 3)
    torch.cuda.synchronize()
    assert int(out[4][0]) == binding.SV_FLAG_BAD_BUDGET
    out = verify_noalloc(t, d, x, k, 1.0, 3)            # written, not accumulated
    torch.cuda.synchronize()
    assert int(out[4][0]) == 0


def test_noalloc_rejects_a_call_larger_than_its_scratch():
    A = 0x10000                                        # never dereferenced: refused first
    rc = binding.spec_verify_run_noalloc(151936, binding.SV_DTYPE_BF16, A, A, A, A, 16384, 32,
                                         1.0, 1, 0, A, A, None, None, None, None)
    assert rc == binding.SV_ERR_TOO_BIG
