"""The remainder step of the N-gram hash kernel, h mod M for 64-bit h and
1 <= M <= 2^31, checked as integer arithmetic against Python's own %.

The hash maps each N-gram to a table index by a modulus (zhichai.net
TileKernels page, section "5. Engram": engram_hash). The kernel computes it
with a Barrett quotient from R = floor((2^64 - 1) / M) and 32-bit pieces:

    A = h1 R0 + h0 R1 + floor(h0 R0 / 2^32)      (mod 2^64)
    r = h0 + h1 c - floor(A / 2^32) M            (mod 2^32),  c = -(R1 M) mod 2^32
    h mod M = min(r, r - M)                      (unsigned 32-bit)

This file checks that derivation, step for step as written above, on the
values where it could fail: h at the top of the 64-bit range and next to
multiples of M, M = 1, 2, powers of two, 2^31 - 1, 2^31 and random sizes.
The GPU test of the kernel itself steers its hashes to such values.
"""

import random

M32 = (1 << 32) - 1
M64 = (1 << 64) - 1


def folded_remainder(h: int, m: int) -> int:
    R = M64 // m
    h0, h1 = h & M32, h >> 32
    r0, r1 = R & M32, R >> 32
    c = (-(r1 * m)) & M32
    a = (h0 * r1 + h1 * r0 + ((h0 * r0) >> 32)) & M64
    r = (h0 + h1 * c - (a >> 32) * m) & M32
    return min(r, (r - m) & M32)


def edge_hashes(m: int, rng: random.Random) -> list:
    top = M64 // m
    hs = [0, 1, M64, M64 - 1, m - 1, m, m + 1]
    for k in (top, top - 1, 1, 2, rng.randrange(0, top + 1)):
        hs += [k * m - 1, k * m, k * m + m - 1]
    hs += [rng.getrandbits(64) for _ in range(24)]
    return [h for h in hs if 0 <= h <= M64]


def test_folded_barrett_remainder_is_exact():
    rng = random.Random(20261203)
    sizes = [1, 2, 3, 4, 5, 7, 1021, 524287, 524288, (1 << 30) + 1, (1 << 31) - 1, 1 << 31]
    sizes += [1 << e for e in range(1, 31)]
    sizes += [rng.randrange(1, (1 << 31) + 1) for _ in range(1500)]
    checked = 0
    for m in sizes:
        for h in edge_hashes(m, rng):
            assert folded_remainder(h, m) == h % m, (h, m)
            checked += 1
    assert checked > 60000


def test_one_correction_is_needed_and_enough():
    """The quotient can fall one short of floor(h / M), never two: without
    the final correction some remainders come out as r + M, and with it all
    are exact (the cases above)."""
    rng = random.Random(7)
    short = 0
    for _ in range(20000):
        m = rng.randrange(3, (1 << 31) + 1)
        h = rng.getrandbits(64)
        R = M64 // m
        q = (h * R) >> 64
        assert h // m - 1 <= q <= h // m
        short += q != h // m
    assert short > 0
