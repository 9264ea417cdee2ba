"""Philox4x32-10 counter-based generator (oracle side).  TEST INFRASTRUCTURE.

The pages draw their uniforms with an unspecified ``uniform_0_1()`` /
``torch.rand`` (pseudo-code 10-1 in "11.1 核心原理"; section 3.3 of the
tutorial) and leave RNG management to the serving system (the remark after
pseudo-code 10-1).  This build fixes it to Philox4x32-10 as published in
Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
(SC'11), written here from that paper's description:

* state: a 128-bit counter (four 32-bit words X0..X3) and a 64-bit key
  (two 32-bit words K0, K1);
* one round: multiply X0 by 0xD2511F53 and X2 by 0xCD9E8D57 as 32x32 -> 64
  bit products (hi, lo); the new counter is
  (hi(X2*M1) ^ X1 ^ K0, lo(X2*M1), hi(X0*M0) ^ X3 ^ K1, lo(X0*M0));
* between rounds the key is bumped by the Weyl constants 0x9E3779B9 and
  0xBB67AE85 (mod 2^32); ten rounds in total.

Keying used by the verify step (one draw per (row, position, purpose, step)):
key = (seed mod 2^32, seed >> 32), counter = (b, i, purpose, step), and the
uniform is word 0 mapped to u = (X0 >> 8) * 2^-24, which is exact in float32
and float64 and lies in [0, 1 - 2^-24].

Parity pin: ``tests/test_philox.py`` compares this implementation with
rocRAND's ``philox4x32_10`` engine (an installed library, run on the host)
over many counters and keys, and checks the uniform mapping's range and
uniformity.
"""

import numpy as np

M0 = np.uint64(0xD2511F53)
M1 = np.uint64(0xCD9E8D57)
W0 = np.uint64(0x9E3779B9)
W1 = np.uint64(0xBB67AE85)
MASK32 = np.uint64(0xFFFFFFFF)
SHIFT32 = np.uint64(32)

PURPOSE_DRAFT = 0      # harness only: drawing d_i from q_i
PURPOSE_ACCEPT = 1     # the accept test at position i
PURPOSE_RESIDUAL = 2   # the correction sample after a rejection at position i
PURPOSE_BONUS = 3      # the bonus sample after all gamma drafts were accepted


def philox4x32_10(counter, key):
    """Return the four 32-bit output words for the given counter(s) and key(s).

    ``counter`` is a sequence of four integer arrays (or scalars), ``key`` a
    sequence of two; they broadcast against each other.  Returns a tuple of
    four ``np.uint64`` arrays holding 32-bit values.
    """
    x0, x1, x2, x3 = (np.asarray(c, dtype=np.uint64) & MASK32 for c in counter)
    k0, k1 = (np.asarray(k, dtype=np.uint64) & MASK32 for k in key)
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + W0) & MASK32
            k1 = (k1 + W1) & MASK32
        prod0 = M0 * x0            # < 2^64, no wrap
        prod1 = M1 * x2
        hi0, lo0 = prod0 >> SHIFT32, prod0 & MASK32
        hi1, lo1 = prod1 >> SHIFT32, prod1 & MASK32
        x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
    return x0, x1, x2, x3


def split_seed(seed):
    """64-bit seed -> (K0, K1)."""
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return seed & 0xFFFFFFFF, seed >> 32


def uniform(seed, b, i, purpose, step=0):
    """u in [0, 1) for draw (row b, position i, purpose, step); float64, exact.

    Arguments may be numpy arrays (broadcast).  The value is a multiple of
    2^-24, so the same number is representable exactly in float32.
    """
    k0, k1 = split_seed(seed)
    x0, _, _, _ = philox4x32_10((b, i, purpose, step), (k0, k1))
    return (x0 >> np.uint64(8)).astype(np.float64) * (2.0 ** -24)
