"""Build the HIP library in-tree with hipcc for gfx950.

``python -m draft_verify_sampling_spec_amd.build`` (or ``build_library()``)
compiles ``csrc/spec_verify.hip`` (verification), ``csrc/budget_schedule.hip``
(the verify-budget scheduler), ``csrc/head_stats.hip`` (output-head row
statistics), ``csrc/verify_hidden.hip`` (verification from hidden states) and
``csrc/markov_draft.hip`` (the drafter's low-rank Markov head) into
``libspec_verify.so`` next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
SRC = os.path.join(PKG_DIR, "csrc", "spec_verify.hip")
SOURCES = [SRC, os.path.join(PKG_DIR, "csrc", "budget_schedule.hip"),
           os.path.join(PKG_DIR, "csrc", "head_stats.hip"),
           os.path.join(PKG_DIR, "csrc", "verify_hidden.hip"),
           os.path.join(PKG_DIR, "csrc", "markov_draft.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libspec_verify.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
# A test helper (not part of the library): a bounded kernel that holds CUs.
TEST_SRC = os.path.join(ROOT, "tests", "occupy_kernel.hip")
TEST_LIB_PATH = os.path.join(ROOT, "tests", "libsv_occupy.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def compile_command(out: str = LIB_PATH, sources=None) -> list:
    return [
        hipcc(),
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        # Floating-point expressions are evaluated as written (no FMA
        # contraction), so identical expressions give identical values.
        "-ffp-contract=off",
        # Keep the compiler from emitting packed fp32 VALU instructions.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall",
        "-I", INCLUDE,
        *(SOURCES if sources is None else sources),
        "-o", out,
    ]


def build_library(verbose: bool = True) -> str:
    """Compile the library and the tests' helper (always; outputs are
    replaced atomically)."""
    if os.path.exists(TEST_SRC):
        _compile(compile_command(TEST_LIB_PATH + ".tmp", [TEST_SRC]), TEST_LIB_PATH, verbose)
    return _compile(compile_command(LIB_PATH + ".tmp"), LIB_PATH, verbose)


def _compile(cmd, out, verbose):
    tmp = out + ".tmp"
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    if verbose and res.stderr.strip():
        # Warnings (the host pass does not know the packed-fp32 feature flag).
        lines = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l]
        if any(l.strip() for l in lines):
            sys.stderr.write("\n".join(lines) + "\n")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build_library()
