"""Pins of the oracle's Philox4x32-10 (oracle/philox.py).

The oracle's generator is compared word for word with an independent
implementation of the same function: rocRAND's Philox4x32-10 engine, whose
header is host-compilable. A small host program is compiled here with g++
against ``/opt/rocm/include`` (no GPU involved) and fed counters and keys,
including words at the 2**32 - 1 boundary.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

from oracle import philox

ROCRAND_HEADER = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"

HOST_PROGRAM = r"""
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
#include <cstdint>
#include <vector>
// ten_rounds is protected in the engine; a subclass may call it.
struct Probe : rocrand_device::philox4x32_10_engine {
  uint4 block(uint4 c, uint2 k) { return ten_rounds(c, k); }
};
int main(int argc, char** argv) {
  FILE* in = std::fopen(argv[1], "rb");
  FILE* out = std::fopen(argv[2], "wb");
  if (!in || !out) return 2;
  Probe p;
  uint32_t w[6];
  while (std::fread(w, sizeof(uint32_t), 6, in) == 6) {
    uint4 c = {w[0], w[1], w[2], w[3]};
    uint2 k = {w[4], w[5]};
    uint4 r = p.block(c, k);
    uint32_t o[4] = {r.x, r.y, r.z, r.w};
    std::fwrite(o, sizeof(uint32_t), 4, out);
  }
  std::fclose(in);
  std::fclose(out);
  return 0;
}
"""


@pytest.fixture(scope="module")
def rocrand_block(tmp_path_factory):
    if not os.path.exists(ROCRAND_HEADER) or shutil.which("g++") is None:
        pytest.skip("rocRAND header or g++ not available")
    d = tmp_path_factory.mktemp("rocrand")
    src = d / "probe.cpp"
    exe = d / "probe"
    src.write_text(HOST_PROGRAM)
    subprocess.run(["g++", "-O2", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    str(src), "-o", str(exe)], check=True, capture_output=True)

    def run(words: np.ndarray) -> np.ndarray:
        words = np.ascontiguousarray(words, dtype=np.uint32)
        fin, fout = d / "in.bin", d / "out.bin"
        words.tofile(fin)
        subprocess.run([str(exe), str(fin), str(fout)], check=True)
        return np.fromfile(fout, dtype=np.uint32).reshape(-1, 4)
    return run


def _inputs(n, seed):
    rng = np.random.default_rng(seed)
    words = rng.integers(0, 2 ** 32, size=(n, 6), dtype=np.uint64)
    # Boundary words: all-ones, zeros and counters of the verifier's layout
    # (request, position, 0, 0) near the top of the 32-bit range.
    edge = np.array([
        [0, 0, 0, 0, 0, 0],
        [2**32 - 1] * 6,
        [2**32 - 1, 2**32 - 1, 0, 0, 0x12345678, 0x9ABCDEF0],
        [2**32 - 2, 7, 0, 0, 2**32 - 1, 0],
        [0, 2**32 - 1, 0, 0, 5, 1],
    ], dtype=np.uint64)
    return np.concatenate([edge, words]).astype(np.uint32)


def test_vectorised_matches_rocrand(rocrand_block):
    words = _inputs(1 << 20, 11)
    ref = rocrand_block(words)
    w = words.astype(np.uint64)
    got = philox.philox4x32_np(w[:, 0], w[:, 1], w[:, 2], w[:, 3], w[:, 4], w[:, 5])
    got = np.stack(got, axis=1).astype(np.uint32)
    assert np.array_equal(got, ref)


def test_scalar_matches_rocrand(rocrand_block):
    words = _inputs(2000, 12)
    ref = rocrand_block(words)
    for row, r in zip(words, ref):
        got = philox.philox4x32(row[:4], row[4:])
        assert tuple(int(v) for v in r) == got


def test_uniform_table_matches_scalar_layout():
    seed = (3 << 32) | 17
    u_acc, u_smp = philox.uniforms_table(seed, 40, 9)
    for b in (0, 1, 39):
        for i in (0, 4, 8):
            assert (u_acc[b, i], u_smp[b, i]) == philox.position_uniforms(seed, b, i)


def test_uniform_conversion_edges():
    assert philox.word_to_uniform(0) == 0.0
    top = philox.word_to_uniform(2**32 - 1)
    assert top == 1.0 - 2.0 ** -24 and top < 1.0
    assert philox.word_to_uniform(0x80000000) == 0.5
    # Exactly representable in fp32 (24 significant bits at most).
    vals = np.array([philox.word_to_uniform(w) for w in (1 << 8, 12345678, 2**32 - 257)])
    assert np.array_equal(vals.astype(np.float32).astype(np.float64), vals)


def test_uniforms_are_uniform():
    u_acc, u_smp = philox.uniforms_table(0xDEADBEEF, 4096, 64)
    for u in (u_acc.ravel(), u_smp.ravel()):
        counts, _ = np.histogram(u, bins=256, range=(0.0, 1.0))
        assert stats.chisquare(counts).pvalue > 1e-4
    # The two words drawn per position are not correlated.
    r = np.corrcoef(u_acc.ravel(), u_smp.ravel())[0, 1]
    assert abs(r) < 0.01
