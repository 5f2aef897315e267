"""The C ABI without a GPU: the library loads, exports every function the
header declares, and its host-side argument checks return the documented
codes. No kernel is launched here."""
import ctypes
import math
import os
import re

import pytest

from draft_verify_sampling_spec_amd import binding as sb
from draft_verify_sampling_spec_amd.build import LIB_PATH

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "spec_verify.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_(?:verify|budget|head|markov)_[a-z_]+)\s*\(", text)))


def _declared_constants():
    text = open(HEADER).read()
    out = dict(re.findall(r"#define\s+(SV_[A-Z_]+)\s+([0-9][0-9a-fA-Fx]*)u?\s", text))
    for name, val in re.findall(r"\b(SV_[A-Z_0-9]+)\s*=\s*(-?\d+)", text):
        out[name] = val
    return out


def test_library_exports_every_declared_function():
    lib = ctypes.CDLL(LIB_PATH)
    declared = _declared_functions()
    assert declared, "no functions parsed from the header"
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(sb.EXPORTED)


def test_binding_constants_match_header():
    consts = _declared_constants()
    for name, val in consts.items():
        if hasattr(sb, name):
            v = int(val, 0) if not val.startswith("(") else None
            assert getattr(sb, name) == v, name
    assert sb.SV_MAX_VOCAB == 1 << 20


def test_strerror_covers_every_code():
    for code in range(0, -9, -1):
        assert sb.spec_verify_strerror(code) != "unknown status code"
    assert sb.spec_verify_strerror(42) == "unknown status code"


def test_chunk_count():
    # A chunk is 960 lanes x 4 sixteen-byte groups: 30720 bf16 or 15360 fp32 values.
    assert sb.spec_verify_chunks(151936, sb.SV_DTYPE_BF16) == 5
    assert sb.spec_verify_chunks(262144, sb.SV_DTYPE_BF16) == 9
    assert sb.spec_verify_chunks(151936, sb.SV_DTYPE_F32) == 10
    assert sb.spec_verify_chunks(30720, sb.SV_DTYPE_BF16) == 1
    assert sb.spec_verify_chunks(30721, sb.SV_DTYPE_BF16) == 2
    assert sb.spec_verify_chunks(32, sb.SV_DTYPE_F32) == 1
    assert sb.spec_verify_chunks(0, sb.SV_DTYPE_F32) == sb.SV_ERR_ARG
    assert sb.spec_verify_chunks(32, 7) == sb.SV_ERR_DTYPE


A = 0x10000  # a 16-byte aligned fake address (never dereferenced)


def _check(**kw):
    args = dict(max_batch=8, max_k=4, vocab=1000, dtype=sb.SV_DTYPE_BF16, target=A,
                draft=A, tokens=A, budgets=A, B=8, K=4, temperature=1.0, out_tokens=A,
                out_num_accepted=A, out_p_draft=None, out_q_draft=None)
    args.update(kw)
    return sb.spec_verify_check_args(**args)


def test_check_args_accepts_valid_calls():
    assert _check() == sb.SV_OK
    assert _check(temperature=0.0, draft=None) == sb.SV_OK          # greedy needs no drafter
    assert _check(B=0, target=None, budgets=None) == sb.SV_OK      # empty batch is a no-op
    assert _check(K=0, draft=None, tokens=None) == sb.SV_OK         # bonus-only requests
    assert _check(out_p_draft=A, out_q_draft=A) == sb.SV_OK
    assert _check(dtype=sb.SV_DTYPE_F32, target=A + 4, draft=A + 8) == sb.SV_OK


@pytest.mark.parametrize("kw, code", [
    (dict(B=9), sb.SV_ERR_ARG),
    (dict(B=-1), sb.SV_ERR_ARG),
    (dict(K=5), sb.SV_ERR_ARG),
    (dict(K=-1), sb.SV_ERR_ARG),
    (dict(temperature=-0.5), sb.SV_ERR_ARG),
    (dict(temperature=math.nan), sb.SV_ERR_ARG),
    (dict(temperature=math.inf), sb.SV_ERR_ARG),
    (dict(dtype=2), sb.SV_ERR_DTYPE),
    (dict(max_batch=0), sb.SV_ERR_ARG),
    (dict(max_batch=sb.SV_MAX_BATCH + 1, B=1), sb.SV_ERR_ARG),
    (dict(max_k=sb.SV_MAX_K + 1), sb.SV_ERR_ARG),
    (dict(vocab=0), sb.SV_ERR_ARG),
    (dict(vocab=sb.SV_MAX_VOCAB + 1), sb.SV_ERR_ARG),
    (dict(target=None), sb.SV_ERR_NULL),
    (dict(draft=None), sb.SV_ERR_NULL),
    (dict(tokens=None), sb.SV_ERR_NULL),
    (dict(budgets=None), sb.SV_ERR_NULL),
    (dict(out_tokens=None), sb.SV_ERR_NULL),
    (dict(out_num_accepted=None), sb.SV_ERR_NULL),
    (dict(target=A + 1), sb.SV_ERR_ALIGN),
    (dict(draft=A + 3), sb.SV_ERR_ALIGN),
    (dict(dtype=sb.SV_DTYPE_F32, target=A + 2), sb.SV_ERR_ALIGN),
    (dict(tokens=A + 2), sb.SV_ERR_ALIGN),
    (dict(budgets=A + 1), sb.SV_ERR_ALIGN),
    (dict(out_tokens=A + 2), sb.SV_ERR_ALIGN),
    (dict(out_p_draft=A + 2), sb.SV_ERR_ALIGN),
])
def test_check_args_rejects(kw, code):
    assert _check(**kw) == code


def test_null_context_paths_do_not_touch_a_device():
    lib = sb.load()
    assert sb.spec_verify_run(None, A, A, A, A, 1, 1, 1.0, 0, A, A, None, None, None) \
        == sb.SV_ERR_STATE
    rc, _ = sb.spec_verify_status(None)
    assert rc == sb.SV_ERR_STATE
    sb.spec_verify_free(None)                         # NULL-safe
    out = ctypes.c_void_p()
    assert lib.spec_verify_init(None, 0, 8, 4, 1000, 1) == sb.SV_ERR_NULL
    assert lib.spec_verify_init(ctypes.byref(out), 0, 8, 4, 1000, 9) == sb.SV_ERR_DTYPE
    assert lib.spec_verify_init(ctypes.byref(out), 0, 0, 4, 1000, 1) == sb.SV_ERR_ARG
    assert lib.spec_verify_init(ctypes.byref(out), -1, 8, 4, 1000, 1) == sb.SV_ERR_ARG
    assert out.value is None
    assert sb.spec_verify_philox_words(0, -1, 1, None, None) == sb.SV_ERR_ARG
    assert sb.spec_verify_philox_words(0, 0, 5, None, None) == sb.SV_OK


def test_init_without_a_device_fails_cleanly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    rc, ctx = sb.spec_verify_init(0, 8, 4, 1000, sb.SV_DTYPE_BF16)
    assert rc == sb.SV_ERR_HIP and ctx is None


_VALID = 1     # marks valid arguments in the table below


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), sb.SV_ERR_ARG),
    (dict(B=sb.SV_MAX_BATCH + 1), sb.SV_ERR_ARG),
    (dict(K=-1), sb.SV_ERR_ARG),
    (dict(K=sb.SV_MAX_K + 1), sb.SV_ERR_ARG),
    (dict(n_total=-1), sb.SV_ERR_ARG),
    (dict(tau=-0.5), sb.SV_ERR_ARG),
    (dict(tau=math.nan), sb.SV_ERR_ARG),
    (dict(tau=math.inf), sb.SV_ERR_ARG),
    (dict(out=None), sb.SV_ERR_NULL),
    (dict(conf=None), sb.SV_ERR_NULL),
    (dict(out=0x1002), sb.SV_ERR_ALIGN),
    (dict(conf=0x2001), sb.SV_ERR_ALIGN),
    (dict(B=0, out=None, conf=None), sb.SV_OK),
])
def test_budget_schedule_argument_checks(kw, code):
    """Host-side checks of spec_budget_schedule: they return before any
    launch, so fake (never dereferenced) pointers are fine."""
    args = dict(conf=0x1000, B=8, K=4, n_total=16, tau=0.0, out=0x2000)
    args.update(kw)
    rc = sb.spec_budget_schedule(args["conf"], args["B"], args["K"], args["n_total"],
                                 args["tau"], args["out"], None)
    assert rc == code


@pytest.mark.parametrize("kw,code", [
    (dict(R=-1), sb.SV_ERR_ARG),
    (dict(H=0), sb.SV_ERR_ARG),
    (dict(H=12), sb.SV_ERR_ARG),
    (dict(V=0), sb.SV_ERR_ARG),
    (dict(V=sb.SV_MAX_VOCAB + 1), sb.SV_ERR_ARG),
    (dict(T=-1.0), sb.SV_ERR_ARG),
    (dict(T=math.nan), sb.SV_ERR_ARG),
    (dict(hid=None), sb.SV_ERR_NULL),
    (dict(ws=None), sb.SV_ERR_NULL),
    (dict(hid=0x1008), sb.SV_ERR_ALIGN),
    (dict(ws_bytes=16), sb.SV_ERR_ARG),
    (dict(R=0, hid=None, w=None, ws=None), sb.SV_OK),
])
def test_head_stats_argument_checks(kw, code):
    """Host-side checks of spec_head_stats (they return before any launch)."""
    args = dict(hid=0x1000, w=0x2000, R=300, H=64, V=1000, tok=None, T=1.0, m=0x3000, s=None,
                z=None, a=None, ws=0x4000, ws_bytes=1 << 30)
    args.update(kw)
    rc = sb.spec_head_stats(args["hid"], args["w"], args["R"], args["H"], args["V"], args["tok"],
                            args["T"], args["m"], args["s"], args["z"], args["a"], args["ws"],
                            args["ws_bytes"], None)
    assert rc == code


def test_head_workspace_size():
    assert sb.spec_head_workspace_bytes(0, 10) == 0
    n = sb.spec_head_workspace_bytes(300, 1000)
    assert n > 0 and n % (300 * 16) == 0


_VALID = 1     # marks valid arguments in the table below


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), sb.SV_ERR_ARG),
    (dict(B=sb.SV_MAX_BATCH + 1), sb.SV_ERR_ARG),
    (dict(K=-1), sb.SV_ERR_ARG),
    (dict(K=sb.SV_MAX_K + 1), sb.SV_ERR_ARG),
    (dict(H=4), sb.SV_ERR_ARG),
    (dict(H=12), sb.SV_ERR_ARG),
    (dict(V=0), sb.SV_ERR_ARG),
    (dict(T=-0.5), sb.SV_ERR_ARG),
    (dict(T=math.inf), sb.SV_ERR_ARG),
    (dict(th=None), sb.SV_ERR_NULL),
    (dict(head=None), sb.SV_ERR_NULL),
    (dict(dh=None), sb.SV_ERR_NULL),
    (dict(dh=None, T=0.0), _VALID),
    (dict(tok=None), sb.SV_ERR_NULL),
    (dict(ws=None), sb.SV_ERR_NULL),
    (dict(th=0x1008), sb.SV_ERR_ALIGN),
    (dict(ws=0x4010), sb.SV_ERR_ALIGN),
    (dict(n=0x3002), sb.SV_ERR_ALIGN),
    (dict(ws_bytes=4096), sb.SV_ERR_ARG),
    (dict(B=0, th=None, dh=None, head=None, tok=None, bud=None, ws=None), sb.SV_OK),
])
def test_verify_hidden_argument_checks(kw, code):
    """Host-side checks of spec_verify_hidden (they return before any launch)."""
    args = dict(th=0x1000, dh=0x2000, head=0x3000, tok=0x5000, bud=0x6000, B=8, K=4, H=64,
                V=1000, T=1.0, out=0x7000, n=0x8000, ws=0x4000, ws_bytes=0)
    args.update(kw)
    if code == _VALID:
        # Valid arguments: only the workspace size check (too small here)
        # stands between them and a launch.
        code = sb.SV_ERR_ARG
    rc = sb.spec_verify_hidden(args["th"], args["dh"], args["head"], args["tok"], args["bud"],
                               args["B"], args["K"], args["H"], args["V"], args["T"], 1,
                               args["out"], args["n"], None, None, None, args["ws"],
                               args["ws_bytes"] if "ws_bytes" in kw else 0, None)
    assert rc == code


def test_verify_hidden_workspace_size():
    assert sb.spec_verify_hidden_workspace_bytes(0, 4, 100) == 0
    assert sb.spec_verify_hidden_workspace_bytes(4, sb.SV_MAX_K + 1, 100) == 0
    n = sb.spec_verify_hidden_workspace_bytes(512, 8, 151936)
    # Dominated by the fp32 logits of two draw rows per request; then the
    # head statistics' 16-byte partials for up to 512 * 17 + 7 packed rows,
    # 40 super-tile slots and up to 594 / 16 + 4 side columns per row.
    partials = (512 * 17 + 7) * (40 + 594 // 16 + 4) * 16
    assert 8 * 512 * 151936 <= n < 8 * 512 * 151936 + partials + (1 << 20)


@pytest.mark.parametrize("kw,code", [
    (dict(), _VALID),
    (dict(B=-1), sb.SV_ERR_ARG),
    (dict(B=sb.SV_MAX_BATCH + 1), sb.SV_ERR_ARG),
    (dict(K=sb.SV_MAX_K + 1), sb.SV_ERR_ARG),
    (dict(r=4), sb.SV_ERR_ARG),
    (dict(r=260), sb.SV_ERR_ARG),
    (dict(V=0), sb.SV_ERR_ARG),
    (dict(V=sb.SV_MAX_VOCAB + 1), sb.SV_ERR_ARG),
    (dict(base=None), sb.SV_ERR_NULL),
    (dict(a=None), sb.SV_ERR_NULL),
    (dict(prev=None), sb.SV_ERR_NULL),
    (dict(ws=None), sb.SV_ERR_NULL),
    (dict(base=0x1008), sb.SV_ERR_ALIGN),
    (dict(out=0x7004), sb.SV_ERR_ALIGN),
    (dict(ws=0x4010), sb.SV_ERR_ALIGN),
    (dict(out=0x1000), sb.SV_ERR_ARG),                 # the output may not be the input
    (dict(ws_bytes=100), sb.SV_ERR_ARG),
    (dict(B=0, base=None, a=None, b=None, prev=None, out=None, tok=None, ws=None), sb.SV_OK),
    (dict(K=0, base=None, a=None, b=None, prev=None, out=None, tok=None, ws=None), sb.SV_OK),
])
def test_markov_draft_argument_checks(kw, code):
    """Host-side checks of spec_markov_draft (they return before any launch)."""
    args = dict(base=0x1000, a=0x2000, b=0x3000, prev=0x5000, B=8, K=4, r=256, V=1000,
                out=0x7000, tok=0x8000, ws=0x4000, ws_bytes=0)
    args.update(kw)
    if code == _VALID:
        # Valid arguments: only the workspace size check (too small here)
        # stands between them and a launch.
        code = sb.SV_ERR_ARG
    rc = sb.spec_markov_draft(args["base"], args["a"], args["b"], args["prev"], args["B"],
                              args["K"], args["r"], args["V"], args["out"], args["tok"], None,
                              args["ws"], args["ws_bytes"] if "ws_bytes" in kw else 0, None)
    assert rc == code


def test_markov_draft_workspace_size():
    assert sb.spec_markov_draft_workspace_bytes(0, 100) == 0
    assert sb.spec_markov_draft_workspace_bytes(4, 0) == 0
    assert sb.spec_markov_draft_workspace_bytes(4, sb.SV_MAX_VOCAB + 1) == 0
    n = sb.spec_markov_draft_workspace_bytes(512, 151936)
    # Two token maps of B entries each, an 8-byte first argmax per request and
    # vocabulary split of the product for other shapes (128 splits), and the
    # streaming path's three arrays of one 8-byte argmax key per request. The
    # bias rows never reach memory.
    want = 2 * 4 * 512 + 128 * 512 * 8 + 3 * 8 * 512
    assert want <= n <= want + 4 * 255


def _noalloc(**kw):
    args = dict(vocab=1000, dtype=sb.SV_DTYPE_BF16, target=A, draft=A, tokens=A, budgets=A, B=8,
                K=4, temperature=1.0, seed=1, request_base=0, out_tokens=A, out_num_accepted=A,
                out_p_draft=None, out_q_draft=None, out_status=None, stream=None)
    args.update(kw)
    return sb.spec_verify_run_noalloc(**args)


@pytest.mark.parametrize("kw, code", [
    (dict(B=-1), sb.SV_ERR_ARG),
    (dict(B=sb.SV_MAX_BATCH + 1), sb.SV_ERR_ARG),
    (dict(K=sb.SV_MAX_K + 1), sb.SV_ERR_ARG),
    (dict(vocab=0), sb.SV_ERR_ARG),
    (dict(dtype=5), sb.SV_ERR_DTYPE),
    (dict(temperature=-1.0), sb.SV_ERR_ARG),
    (dict(target=None), sb.SV_ERR_NULL),
    (dict(draft=None), sb.SV_ERR_NULL),
    (dict(target=A + 1), sb.SV_ERR_ALIGN),
    (dict(out_status=A + 2), sb.SV_ERR_ALIGN),
    (dict(request_base=-1), sb.SV_ERR_ARG),
    (dict(request_base=2**32 - 8), sb.SV_ERR_ARG),   # the last request's counter would wrap
])
def test_noalloc_rejects_bad_arguments_before_any_device_call(kw, code):
    assert _noalloc(**kw) == code


def test_noalloc_empty_batch_is_a_no_op():
    assert _noalloc(B=0, target=None, budgets=None, out_tokens=None,
                    out_num_accepted=None) == sb.SV_OK


def test_run_ex_checks_context_and_request_base():
    assert sb.spec_verify_run_ex(None, A, A, A, A, 8, 4, 1.0, 1, 0, A, A, None, None,
                                 None) == sb.SV_ERR_STATE
