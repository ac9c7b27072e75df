"""Known-answer tests of the input generator's random-number primitives.

The seeded inputs of every parity test and of the benchmark come from
Philox4x32-10 and SplitMix64 (synth/philox.py on the host, its device twin
checked bit for bit against it by a GPU test).  These pin the host
definition to published outputs, not to itself:

- Philox4x32-10: the known-answer vectors distributed with the authors'
  Random123 library (Salmon, Moraes, Dror and Shaw, "Parallel Random
  Numbers: As Easy as 1, 2, 3", SC 2011) for the all-zero, all-ones and
  pi-digit counter/key pairs.
- SplitMix64 (Steele, Lea and Flood, OOPSLA 2014): the first output for
  state 0, as the reference implementation prints it.
"""
import numpy as np
import pytest

from synth.philox import philox4x32_10, splitmix64

KAT = [
    # counter (4 words), key (2 words), output (4 words)
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000),
     (0x00000000, 0x00000000),
     (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF),
     (0xFFFFFFFF, 0xFFFFFFFF),
     (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344),
     (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,want", KAT)
def test_philox4x32_10_known_answers(ctr, key, want):
    got = philox4x32_10(*ctr, *key)
    assert tuple(int(x) for x in got) == want


def test_philox_vectorised_equals_scalar():
    """The array form draws each counter independently."""
    ctr = np.array([0, 0xFFFFFFFF, 0x243F6A88], dtype=np.uint64)
    c1 = np.array([0, 0xFFFFFFFF, 0x85A308D3], dtype=np.uint64)
    c2 = np.array([0, 0xFFFFFFFF, 0x13198A2E], dtype=np.uint64)
    c3 = np.array([0, 0xFFFFFFFF, 0x03707344], dtype=np.uint64)
    # one key for the batch: the pi-digit key
    got = philox4x32_10(ctr, c1, c2, c3, 0xA4093822, 0x299F31D0)
    assert int(got[0][2]) == 0xD16CFE09 and int(got[3][2]) == 0x24126EA1
    for i in range(3):
        one = philox4x32_10(int(ctr[i]), int(c1[i]), int(c2[i]), int(c3[i]),
                            0xA4093822, 0x299F31D0)
        assert [int(x) for x in one] == [int(g[i]) for g in got]


def test_splitmix64_first_output():
    assert splitmix64(0) == 0xE220A8397B1DCDAF
