"""Philox4x32-10 counter-based generator, written out from its published definition.

TEST INFRASTRUCTURE. Part of the CPU oracle: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. The product path never does.

Definition followed: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3", SC'11, section on the Philox
family. Philox-4x32 keeps a counter of four 32-bit words and a key of two.
One round multiplies counter words 0 and 2 by two fixed odd multipliers,
giving 64-bit products; the new counter is built from the high halves xored
with the two remaining counter words and the key words, and the low halves,
in the paper's fixed word permutation. Between rounds both key words are
increased by the Weyl constants (golden ratio and sqrt(3) - 1, scaled to 32
bits). Ten rounds make Philox4x32-10.

How the verifier uses it (the pages fix no RNG; this is the library's own
stream layout): the key is the 64-bit call seed split into (low, high) words,
the counter of request ``b`` and position ``i`` is ``(b, i, 0, 0)``; output
word 0 drives the acceptance test of that position and word 1 its sample.
A word ``r`` becomes the uniform ``(r >> 8) * 2**-24``, exact in fp32 and
fp64 and lying in [0, 1).
"""
from __future__ import annotations

import numpy as np

MASK32 = 0xFFFFFFFF
# Round multipliers and key increments of Philox-4x32 (SC'11 paper).
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
PHILOX_ROUNDS = 10


def philox4x32(counter, key, rounds: int = PHILOX_ROUNDS):
    """One Philox-4x32 block with plain Python integers.

    ``counter`` is four 32-bit words, ``key`` two. Returns four 32-bit words.
    """
    c0, c1, c2, c3 = (int(w) & MASK32 for w in counter)
    k0, k1 = (int(w) & MASK32 for w in key)
    for rnd in range(rounds):
        if rnd > 0:
            k0 = (k0 + PHILOX_W0) & MASK32
            k1 = (k1 + PHILOX_W1) & MASK32
        prod0 = PHILOX_M0 * c0          # exact 64-bit product
        prod1 = PHILOX_M1 * c2
        c0, c1, c2, c3 = (
            (prod1 >> 32) ^ c1 ^ k0,
            prod1 & MASK32,
            (prod0 >> 32) ^ c3 ^ k1,
            prod0 & MASK32,
        )
    return c0, c1, c2, c3


def philox4x32_np(c0, c1, c2, c3, k0, k1, rounds: int = PHILOX_ROUNDS):
    """The same block over numpy arrays of counters (broadcasting).

    Every intermediate is held in uint64: a product of two 32-bit words is
    below 2**64, so it is exact; key sums are reduced modulo 2**32.
    """
    m32 = np.uint64(MASK32)
    c0 = np.asarray(c0, dtype=np.uint64) & m32
    c1 = np.asarray(c1, dtype=np.uint64) & m32
    c2 = np.asarray(c2, dtype=np.uint64) & m32
    c3 = np.asarray(c3, dtype=np.uint64) & m32
    k0 = np.asarray(k0, dtype=np.uint64) & m32
    k1 = np.asarray(k1, dtype=np.uint64) & m32
    sh = np.uint64(32)
    for rnd in range(rounds):
        if rnd > 0:
            k0 = (k0 + np.uint64(PHILOX_W0)) & m32
            k1 = (k1 + np.uint64(PHILOX_W1)) & m32
        prod0 = np.uint64(PHILOX_M0) * c0
        prod1 = np.uint64(PHILOX_M1) * c2
        c0, c1, c2, c3 = (
            (prod1 >> sh) ^ c1 ^ k0,
            prod1 & m32,
            (prod0 >> sh) ^ c3 ^ k1,
            prod0 & m32,
        )
    return c0, c1, c2, c3


def seed_key(seed: int):
    """Split a 64-bit seed into the (low, high) key words."""
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return seed & MASK32, seed >> 32


def word_to_uniform(word) -> float:
    """Top 24 bits of a 32-bit word as a dyadic uniform in [0, 1)."""
    return float(int(word) >> 8) * 2.0 ** -24


def position_uniforms(seed: int, b: int, i: int):
    """(u_acc, u_smp) of request ``b``, position ``i`` for call seed ``seed``."""
    r0, r1, _r2, _r3 = philox4x32((b, i, 0, 0), seed_key(seed))
    return word_to_uniform(r0), word_to_uniform(r1)


def uniforms_table(seed: int, B: int, P: int):
    """(u_acc, u_smp) arrays of shape [B, P] for requests 0..B-1, positions 0..P-1."""
    k0, k1 = seed_key(seed)
    bb, ii = np.meshgrid(np.arange(B, dtype=np.uint64), np.arange(P, dtype=np.uint64),
                         indexing="ij")
    r0, r1, _r2, _r3 = philox4x32_np(bb, ii, 0, 0, k0, k1)
    scale = 2.0 ** -24
    u_acc = (r0 >> np.uint64(8)).astype(np.float64) * scale
    u_smp = (r1 >> np.uint64(8)).astype(np.float64) * scale
    return u_acc, u_smp
