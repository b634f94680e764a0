"""CPU replay of the table-decode TQ1 tiled kernel's index arithmetic.

The kernel (csrc/tq_tiled.hip, 1.6-bit weight source) copies, for the block b
of a round, the 64 bytes of each weight row that start at floor(256 b / 5)
rounded down to 4, and each lane (g = 0..3) rebuilds the 2-bit fields of
weights 256 b + 64 g .. + 63 from 14 of those bytes: five dword reads, a byte
alignment, a 256-entry table of each byte's five fields, a 160-bit string of
10-bit codes and one funnel shift by twice the trit offset.  This test runs
the same integer steps in Python for every block and lane group at several
K and checks that the four dwords equal the 2-bit packing of the same trits
by the oracle (the project page's "2 bits per weight" layout), and that every
read stays inside the copied window.  No GPU is needed.
"""

import pytest

from oracle import pack_tq1_ref, pack_tq2_ref
from synth import seed_for, ternary_iid

M32 = 0xFFFFFFFF


def table():
    """Byte value -> its five 2-bit fields d' (weight j at bits 2j), by the
    multiply-by-3 decoder: t = 3q, d' = t >> 8, q = t & 255."""
    lut = []
    for v in range(256):
        q, code = v, 0
        for f in range(5):
            t = 3 * q
            code |= (t >> 8) << (2 * f)
            q = t & 255
        lut.append(code)
    return lut


LUT = table()


def alignbyte(hi, lo, s):
    return ((((hi << 32) | lo) >> (8 * (s & 3))) & M32)


def alignbit(hi, lo, s):
    return ((((hi << 32) | lo) >> (s & 31)) & M32)


def lane_dwords(row, b, g, trit_error=0):
    """The four dwords lane group g of a wave gets for block b of one TQ1 row
    (row: its ldq bytes), following the kernel's steps; asserts its bounds.
    trit_error shifts the field string by that many trits less (a planted
    mistake for the mutation check)."""
    ab = ((256 * b) // 5) & ~3  # first byte of the block, rounded down to 4
    window = bytes(row[ab:ab + 64]).ljust(64, b"\0")  # past the row: zeros / next row
    x = 256 * b + 64 * g
    i5 = ((x * 0xCCCCCCCD) >> 32) >> 2  # __umulhi(x, 0xCCCCCCCD) >> 2
    assert i5 == x // 5
    sh = 2 * (x - 5 * i5 - trit_error)
    o = i5 - ab
    assert 0 <= o <= 42
    start = o & ~3
    assert start + 20 <= 64  # five dwords inside the copied 64 bytes
    D = [int.from_bytes(window[start + 4 * u:start + 4 * u + 4], "little") for u in range(5)]
    E = [alignbyte(D[t + 1], D[t], o & 3) for t in range(4)]
    c = [LUT[(E[i >> 2] >> (8 * (i & 3))) & 0xFF] for i in range(14)]
    W = [0] * 5
    W[0] = (c[0] | (c[1] << 10) | (c[2] << 20) | (c[3] << 30)) & M32
    W[1] = ((c[3] >> 2) | (c[4] << 8) | (c[5] << 18) | (c[6] << 28)) & M32
    W[2] = ((c[6] >> 4) | (c[7] << 6) | (c[8] << 16) | (c[9] << 26)) & M32
    W[3] = ((c[9] >> 6) | (c[10] << 4) | (c[11] << 14) | (c[12] << 24)) & M32
    W[4] = ((c[12] >> 8) | (c[13] << 2)) & M32
    # the 14 bytes hold every weight the lane needs
    assert 5 * (i5 + 13) + 4 >= x + 63
    return [alignbit(W[t + 1], W[t], sh) for t in range(4)]


def test_table_matches_the_division_route():
    """The table's fields are the base-3 digits of n = floor(243 v / 256),
    most significant first, each plus one (d' = d + 1 in {0, 1, 2})."""
    for v in range(256):
        n = (v * 243) >> 8
        digits = [(n // p) % 3 for p in (81, 27, 9, 3, 1)]
        assert LUT[v] == sum(d << (2 * j) for j, d in enumerate(digits)), v


@pytest.mark.parametrize("K,ldq", [(256, None), (768, None), (1280, 272), (8192, None),
                                   (28672, 5760)])
def test_every_block_and_lane_group_rebuilds_the_2bit_fields(K, ldq):
    N = 3
    T = ternary_iid(seed_for(31, K), N, K, 0.31)
    q1 = pack_tq1_ref(T, ldq)
    q2 = pack_tq2_ref(T)
    for n in range(N):
        row = q1[n].tobytes()
        for b in range(K // 256):
            for g in range(4):
                want = q2[n, 64 * b + 16 * g:64 * b + 16 * g + 16].tobytes()
                got = b"".join(d.to_bytes(4, "little") for d in lane_dwords(row, b, g))
                assert got == want, (K, n, b, g)


def test_a_wrong_trit_offset_is_caught():
    """Mutation check of the replay: shifting the field string by one trit
    too few breaks every lane whose weights do not start at a byte boundary."""
    K = 1280
    T = ternary_iid(seed_for(32), 1, K, 0.31)
    row = pack_tq1_ref(T)[0].tobytes()
    q2 = pack_tq2_ref(T)
    checked = 0
    for b in range(K // 256):
        for g in range(4):
            if (256 * b + 64 * g) % 5 == 0:
                continue
            checked += 1
            got = b"".join(d.to_bytes(4, "little") for d in lane_dwords(row, b, g, 1))
            assert got != q2[0, 64 * b + 16 * g:64 * b + 16 * g + 16].tobytes(), (b, g)
    assert checked >= 10
