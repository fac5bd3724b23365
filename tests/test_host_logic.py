"""Host-side arithmetic of the library, checked on the CPU.

The scan-direction remap divides a scan step t < 2^31 by W or H with the
multiply-shift constants of Granlund & Montgomery (PLDI 1994): with
s = ceil(log2 d) and m = floor(2^32 (2^s - d) / d) + 1, t // d equals
(umulhi(t, m) + t) >> s.  This restates that formula (as the library computes
it) and checks it against exact integer division, exhaustively for small
divisors and on edge values for large ones.
"""

import random

import pytest


def constants(d):
    s = 0
    while (1 << s) < d:
        s += 1
    m = ((((1 << s) - d) << 32) // d + 1) & 0xFFFFFFFF
    return m, s


def fast_div(t, m, s):
    return (((t * m) >> 32) + t) >> s


def edge_values(d):
    vals = {0, 1, d - 1, d, d + 1, 2 * d - 1, 2 * d, (1 << 31) - 1, (1 << 30), (1 << 30) - 1}
    q = ((1 << 31) - 1) // d
    vals |= {q * d - 1, q * d, q * d + d - 1}
    return [v for v in vals if 0 <= v < (1 << 31)]


@pytest.mark.parametrize("d", list(range(1, 300)) + [1023, 1024, 1025, 4096, 65535, 65536, 1 << 20,
                                                     (1 << 30) - 1, 1 << 30])
def test_fast_division(d):
    m, s = constants(d)
    assert 0 < m < (1 << 32) or d == 1
    rng = random.Random(d)
    for t in edge_values(d) + [rng.randrange(1 << 31) for _ in range(2000)]:
        assert fast_div(t, m, s) == t // d, (t, d)
    if d <= 300:
        for t in range(0, 70 * d):
            assert fast_div(t, m, s) == t // d
