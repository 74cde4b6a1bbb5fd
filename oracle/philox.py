"""Philox4x32-10, written from its published definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition (J. Salmon, M. Moraes, R. Dror, D. Shaw, "Parallel random numbers:
as easy as 1, 2, 3", SC'11, section 3.2 "The Philox family"): the state is a
counter of four 32-bit words and a key of two 32-bit words.  One round
multiplies counter words 0 and 2 by the fixed constants 0xD2511F53 and
0xCD9E8D57 into 64-bit products, and outputs

    (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0)).

Between rounds the key is bumped by the Weyl constants 0x9E3779B9 and
0xBB67AE85 (mod 2^32).  Philox4x32-10 applies ten rounds.

The verify method draws its uniforms from this generator by contract: the
source workloads name them "Philox(seed, row, pos)".  The reading taken here:
key = (low 32 bits of seed, high 32 bits of seed); counter = (row, pos, 0, 0);
output word 0 is the acceptance uniform at (row, pos) and word 1 the
resampling uniform.  A word w becomes u = (w >> 8) * 2^-24, a 24-bit grid in
[0, 1 - 2^-24] that float32 and float64 both represent exactly.
"""

import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
_MASK = 0xFFFFFFFF


def philox4x32_10(counter, key):
    """Return the four output words of Philox4x32-10.

    counter: array-like [..., 4] of uint32 words (c0, c1, c2, c3).
    key:     array-like [..., 2] of uint32 words (k0, k1), broadcast against
             the counter's leading shape.
    Returns a uint32 array of shape [..., 4].
    """
    c = np.asarray(counter, dtype=np.uint64) & _MASK
    k = np.asarray(key, dtype=np.uint64) & _MASK
    c0, c1, c2, c3 = (c[..., i].copy() for i in range(4))
    k0 = np.broadcast_to(k[..., 0], c0.shape).copy()
    k1 = np.broadcast_to(k[..., 1], c0.shape).copy()
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + W0) & _MASK
            k1 = (k1 + W1) & _MASK
        p0 = c0 * np.uint64(M0)  # < 2^64: both factors are below 2^32
        p2 = c2 * np.uint64(M1)
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK
        hi2, lo2 = p2 >> np.uint64(32), p2 & _MASK
        c0, c1, c2, c3 = hi2 ^ c1 ^ k0, lo2, hi0 ^ c3 ^ k1, lo0
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def seed_key(seed):
    """Split a 64-bit seed into the two key words (low word first)."""
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return np.array([seed & _MASK, seed >> 32], dtype=np.uint64)


def word_to_uniform(w):
    """Map a 32-bit word to its 24-bit uniform in [0, 1 - 2^-24] (float64)."""
    return (np.asarray(w, dtype=np.uint64) >> np.uint64(8)).astype(np.float64) * 2.0 ** -24


def uniforms(seed, row, pos, stage=0):
    """The (acceptance, resampling) uniforms for counter (row, pos, stage, 0);
    stage 0 is the verify step's own stream."""
    out = philox4x32_10(np.array([row, pos, stage, 0], dtype=np.uint64), seed_key(seed))
    return float(word_to_uniform(out[0])), float(word_to_uniform(out[1]))
