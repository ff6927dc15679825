"""Swizzle and LDS bank model -- test infrastructure only.

The swizzle never changes a result (a copy through any bijective slot layout
is still the identity), so this module is a model of the layout, not a result
oracle. It restates:
  * "cute（11）hopper之TMA_copy", printed shared-memory layout and section 2.2:
    the 128x64 fp16 tile is stored row-major (row stride 64 elements) under the
    ``Sw<3,4,3>`` swizzle, i.e. a 128-byte XOR pattern on 16-byte units;
  * CuTe's Swizzle<B, M, S> functor (public definition): the B bits starting at
    bit M+S of an offset are XOR-ed into the B bits starting at bit M.

The bank model counts LDS bank collisions of a lane->byte-address pattern for
a parametric bank geometry. It is parity unpinned against gfx950 hardware: the
real geometry is taken from the ``SQ_LDS_BANK_CONFLICT`` counter.
"""
from __future__ import annotations

ROW_BYTES = 128     # one tile row of 64 fp16
CHUNK_BYTES = 16    # one 16-byte unit (one b128 LDS access / one DMA lane)
CHUNKS_PER_ROW = ROW_BYTES // CHUNK_BYTES


def cute_swizzle(B: int, M: int, S: int):
    """CuTe Swizzle<B,M,S> as a function on integer offsets (S > 0)."""
    mask = ((1 << B) - 1) << (M + S)

    def f(x: int) -> int:
        return x ^ ((x & mask) >> S)

    return f


def page_tile_byte_address(r: int, c: int) -> int:
    """Byte address of fp16 element (r, c) of the page's swizzled 128x64 tile.

    Layout printed on the page: ((8,16),(64,1)) : ((64,512),(1,0)) in elements,
    under Sw<3,4,3> applied to the byte address.
    """
    r0, r1 = r % 8, r // 8
    elem = r0 * 64 + r1 * 512 + c * 1
    return cute_swizzle(3, 4, 3)(2 * elem)


def chunk_position(r: int, c: int, shift: int = 0) -> int:
    """Physical 16-byte position of logical chunk c of tile row r.

    XOR of the chunk index with 3 bits of the row index. ``shift`` selects
    which row bits: shift 0 is the page's 128-byte pattern (row & 7).
    """
    return c ^ ((r >> shift) & (CHUNKS_PER_ROW - 1))


def slot_byte_address(r: int, c_elem: int, shift: int = 0) -> int:
    """Byte address inside a slot of fp16 element (r, c_elem) of a 128-byte-row tile."""
    chunk, within = divmod(c_elem * 2, CHUNK_BYTES)
    return r * ROW_BYTES + chunk_position(r, chunk, shift) * CHUNK_BYTES + within


def bank_conflicts(lane_addrs, access_bytes: int, nbanks: int = 64, bank_bytes: int = 4,
                   lanes_per_pass=None) -> int:
    """Extra LDS cycles caused by bank collisions for one wave-wide access.

    Lanes are serviced in groups of ``lanes_per_pass`` consecutive lanes
    (default: as many as fill the bank width once). Within a group, each bank
    serves one distinct 4-byte word per cycle; identical addresses broadcast.
    Returns sum over groups of (max words per bank - 1).
    """
    width = nbanks * bank_bytes
    if lanes_per_pass is None:
        lanes_per_pass = max(1, width // access_bytes)
    extra = 0
    n = len(lane_addrs)
    for g0 in range(0, n, lanes_per_pass):
        per_bank = {}
        for a in lane_addrs[g0:g0 + lanes_per_pass]:
            for w in range(access_bytes // bank_bytes):
                word = a // bank_bytes + w
                per_bank.setdefault(word % nbanks, set()).add(word)
        extra += max(len(v) for v in per_bank.values()) - 1
    return extra
