"""Philox4x32-10 counter-based generator and SplitMix64, in numpy.

Philox4x32-10 follows its published definition (Salmon, Moraes, Dror and
Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011): a 4x32-bit
counter and a 2x32-bit key; each of the 10 rounds multiplies words 0 and 2
by the constants below, takes high and low halves, and mixes them with words
1 and 3 and the key; the key is bumped by the Weyl constants between rounds.
SplitMix64 is Steele, Lea and Flood's 64-bit mixer ("Fast Splittable
Pseudorandom Number Generators", OOPSLA 2014).

This holds no arithmetic of the attention method; it only draws numbers.
"""
import numpy as np

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x32-10.  Counters may be arrays (broadcast); the key
    is two Python ints.  Returns four uint32 arrays."""
    c0 = np.asarray(c0, dtype=np.uint64) & _MASK32
    c1 = np.asarray(c1, dtype=np.uint64) & _MASK32
    c2 = np.asarray(c2, dtype=np.uint64) & _MASK32
    c3 = np.asarray(c3, dtype=np.uint64) & _MASK32
    c0, c1, c2, c3 = np.broadcast_arrays(c0, c1, c2, c3)
    k0 = int(k0) & 0xFFFFFFFF
    k1 = int(k1) & 0xFFFFFFFF
    m0 = np.uint64(PHILOX_M0)
    m1 = np.uint64(PHILOX_M1)
    s32 = np.uint64(32)
    for r in range(10):
        p0 = c0 * m0
        p1 = c2 * m1
        hi0 = p0 >> s32
        lo0 = p0 & _MASK32
        hi1 = p1 >> s32
        lo1 = p1 & _MASK32
        c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint64(k0), lo1,
                          hi0 ^ c3 ^ np.uint64(k1), lo0)
        if r != 9:
            k0 = (k0 + PHILOX_W0) & 0xFFFFFFFF
            k1 = (k1 + PHILOX_W1) & 0xFFFFFFFF
    return (c0.astype(np.uint32), c1.astype(np.uint32), c2.astype(np.uint32),
            c3.astype(np.uint32))


def splitmix64(x):
    """One SplitMix64 output for state x (Python int)."""
    z = (int(x) + 0x9E3779B97F4A7C15) & 0xFFFFFFFFFFFFFFFF
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & 0xFFFFFFFFFFFFFFFF
    return z ^ (z >> 31)
