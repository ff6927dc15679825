"""Swizzle model pins: the page's printed CuTe layout, bijection, involution (CPU)."""
import re

import pytest

from oracle import swizzle as Z
from tests.conftest import golden_lines


def _parse_layout():
    ln = golden_lines("tile_layout_128x64.txt")[0]
    B, M, S = (int(x) for x in re.match(r"Sw<(\d+),(\d+),(\d+)>", ln).groups())
    nums = [int(x) for x in re.findall(r"_(\d+)", ln.split(" o ")[-1])]
    # ((r0,r1),(c0,c1)):((sr0,sr1),(sc0,sc1))
    r0, r1, c0, c1, sr0, sr1, sc0, sc1 = nums
    return (B, M, S), (r0, r1, c0, c1), (sr0, sr1, sc0, sc1)


def test_page_layout_is_128B_chunk_xor():
    (B, M, S), (r0, r1, c0, c1), (sr0, sr1, sc0, sc1) = _parse_layout()
    assert (r0 * r1, c0 * c1) == (128, 64)
    sw = Z.cute_swizzle(B, M, S)
    for r in range(128):
        for c in range(64):
            elem = (r % r0) * sr0 + (r // r0) * sr1 + (c % c0) * sc0 + (c // c0) * sc1
            assert sw(2 * elem) == Z.slot_byte_address(r, c, shift=0)
            assert Z.page_tile_byte_address(r, c) == Z.slot_byte_address(r, c, shift=0)


@pytest.mark.parametrize("shift", [0, 1, 2])
def test_chunk_swizzle_bijective_involution(shift):
    seen = set()
    for r in range(128):
        for c in range(8):
            p = Z.chunk_position(r, c, shift)
            assert 0 <= p < 8
            assert Z.chunk_position(r, p, shift) == c  # involution
            seen.add((r, p))
    assert len(seen) == 128 * 8
    addrs = {Z.slot_byte_address(r, c, shift) for r in range(128) for c in range(64)}
    assert addrs == set(range(0, 16384, 2))


def test_bank_model_basics():
    contiguous = [16 * l for l in range(64)]
    assert Z.bank_conflicts(contiguous, 16, nbanks=32) == 0
    assert Z.bank_conflicts(contiguous, 16, nbanks=64) == 0
    column = [128 * l for l in range(64)]  # same chunk of 64 rows, no swizzle
    assert Z.bank_conflicts(column, 16, nbanks=32) > 0
    swz = [Z.slot_byte_address(l, 0, 0) for l in range(64)]
    assert Z.bank_conflicts(swz, 16, nbanks=32) == 0
    broadcast = [64] * 64
    assert Z.bank_conflicts(broadcast, 4, nbanks=32) == 0


@pytest.mark.parametrize("G", [2, 4])
@pytest.mark.parametrize("S,first", [(5, 0), (5, 3), (8, 6), (4, 2)])
def test_grouped_store_reads_are_conflict_free(G, S, first):
    """The grouped copy consumers' wave-wide reads: lane l takes slot
    (first + (l/16) % G) mod S of the ring, row 2*((l/16)/G) + (l/8) % 2 of the
    instruction's 8/G rows, chunk position l % 8. Any 16 consecutive lanes read
    256 contiguous bytes of one slot, so the bank model finds no conflict for
    any instruction, while the plain alternative (8 lanes per tile, the G tiles
    side by side) puts two slots' identical offsets into one 16-lane pass."""
    if G > S:
        pytest.skip("a group must fit the ring")
    rows_per_instr = 8 // G
    for instr in range(16 * G):
        addrs = []
        for lane in range(64):
            g = (lane >> 4) % G
            slot = (first + g) % S
            r = instr * rows_per_instr + 2 * ((lane >> 4) // G) + ((lane >> 3) & 1)
            addrs.append(slot * 16384 + r * 128 + (lane & 7) * 16)
        assert Z.bank_conflicts(addrs, 16, nbanks=64) == 0
        assert Z.bank_conflicts(addrs, 16, nbanks=64, lanes_per_pass=8) == 0
    # the naive lane order: lanes 8g..8g+7 read slot g's row, G slots per 8 rows
    naive = [((first + (l >> 3) % G) % S) * 16384 + ((l >> 3) // G) * 128 + (l & 7) * 16
             for l in range(64)]
    assert Z.bank_conflicts(naive, 16, nbanks=64) > 0


def test_reading_the_slot_unswizzled_gives_wrong_positions():
    """"cute（11）hopper之TMA_copy" section 4: a raw read of the swizzled buffer
    puts elements in the wrong place. Reading chunk c of row r at its logical
    position r*128 + c*16 finds the chunk c ^ (r & 7) instead, which is right
    only on rows r with r & 7 == 0."""
    wrong_rows = set()
    for r in range(128):
        for c in range(8):
            found = Z.chunk_position(r, c, 0)      # the involution: position -> chunk
            if found != c:
                wrong_rows.add(r)
            assert (found == c) == (r % 8 == 0)
    assert len(wrong_rows) == 112


def test_bank_model_matches_the_strided_access_closed_form():
    """The bank model against the textbook count for strided 4-byte accesses:
    n lanes reading words 0, s, 2s, ... (s > 0) over B banks touch
    B / gcd(s, B) distinct banks, each holding ceil(n / (B / gcd(s, B)))
    distinct words, so a pass of n lanes costs that many cycles, i.e. that
    minus one extra. Broadcast (s = 0) costs nothing extra."""
    import math
    for B in (32, 64):
        for n in (16, 32, 64):
            for s in range(0, 70):
                addrs = [4 * s * i for i in range(n)]
                if s == 0:
                    want = 0
                else:
                    distinct_banks = B // math.gcd(s, B)
                    want = -(-n // distinct_banks) - 1
                assert Z.bank_conflicts(addrs, 4, nbanks=B, lanes_per_pass=n) == want, (B, n, s)
    # a wave split into passes: the extras of the passes add up
    addrs = [4 * 64 * i for i in range(64)]          # stride of one full bank row
    assert Z.bank_conflicts(addrs, 4, nbanks=64, lanes_per_pass=16) == 4 * 15
