"""Philox4x32-10 counter-based generator, vectorised in numpy.

Definition: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel
random numbers: as easy as 1, 2, 3", SC'11, section 4 (the Philox family).
A 4x32-bit counter is transformed by 10 rounds under a 2x32-bit key.  Each
round multiplies counter words 0 and 2 by fixed 32-bit multipliers, keeps the
high and low halves of the 64-bit products, and mixes the high halves with the
other two counter words and the round key by XOR.  The key advances by two
Weyl constants (the golden ratio and sqrt(3)-1 scaled to 2^32) between rounds.

The same generator is implemented independently in HIP (workloads/csrc) so
that the GPU can draw multi-gigabyte expert stacks that the CPU re-draws bit
for bit for the few experts it checks.
"""
import numpy as np

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Apply 10 Philox4x32 rounds to counters (arrays or scalars) under key (k0, k1).

    All inputs are unsigned 32-bit values; c0..c3 may be numpy arrays of equal
    shape.  Returns four uint32 arrays.
    """
    c0 = np.asarray(c0, dtype=np.uint64) & _MASK32
    c1 = np.asarray(c1, dtype=np.uint64) & _MASK32
    c2 = np.asarray(c2, dtype=np.uint64) & _MASK32
    c3 = np.asarray(c3, dtype=np.uint64) & _MASK32
    c0, c1, c2, c3 = np.broadcast_arrays(c0, c1, c2, c3)
    c0, c1, c2, c3 = c0.copy(), c1.copy(), c2.copy(), c3.copy()
    key0 = int(k0) & 0xFFFFFFFF
    key1 = int(k1) & 0xFFFFFFFF
    m0 = np.uint64(PHILOX_M0)
    m1 = np.uint64(PHILOX_M1)
    for rnd in range(10):
        if rnd:
            key0 = (key0 + PHILOX_W0) & 0xFFFFFFFF
            key1 = (key1 + PHILOX_W1) & 0xFFFFFFFF
        p0 = m0 * c0          # < 2^64: exact in uint64
        p1 = m1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        n0 = hi1 ^ c1 ^ np.uint64(key0)
        n2 = hi0 ^ c3 ^ np.uint64(key1)
        c0, c1, c2, c3 = n0, lo1, n2, lo0
    return (c0.astype(np.uint32), c1.astype(np.uint32),
            c2.astype(np.uint32), c3.astype(np.uint32))
