"""The benchmark's context-only ceiling library (ceilings/, not part of the
tile-stream library): it exports what its header declares and validates its
arguments before any HIP call (no GPU needed)."""
import os
import re

from tests.conftest import ROOT

FAKE = 0x10000  # never dereferenced: every case below fails validation first


def test_ceiling_library_exports_and_validation():
    import ceilings as ceiling
    hdr = open(os.path.join(ROOT, "ceilings", "pipe_ceiling.h")).read()
    hdr = re.sub(r"/\*.*?\*/", "", hdr, flags=re.S)
    declared = sorted(set(re.findall(r"\b(ceil_[a-z_]+)\s*\(", hdr)))
    assert declared == sorted(ceiling.SYMBOLS)
    L = ceiling.lib()
    for name in declared:
        assert hasattr(L, name), name
    # validation runs before any HIP call
    assert L.ceil_copy(None, FAKE, 1024, 8, 4, 1, None) == 1
    assert L.ceil_copy(FAKE, FAKE, 1000, 8, 4, 1, None) == 2
    assert L.ceil_copy(FAKE + 8, FAKE, 1024, 8, 4, 1, None) == 2
    assert L.ceil_copy(FAKE, FAKE, 1024, 0, 4, 1, None) == 3
    assert L.ceil_copy(FAKE, FAKE, 1024, 8, 2, 1, None) == 3
    assert L.ceil_read(FAKE, None, 1024, 8, 1, None) == 1
    assert L.ceil_read(FAKE, FAKE, 1024, 8, 2, None) == 3
    assert L.ceil_memcpy(None, FAKE, 16, None) == 1
    # column strips: rows x width bytes at pitch; grid = strips * split, a multiple of 8
    ok = (1024, 32768, 32768, 128, 1)
    assert L.ceil_strip_copy(None, FAKE, *ok, None) == 1
    assert L.ceil_strip_copy(FAKE + 8, FAKE, *ok, None) == 2
    assert L.ceil_strip_copy(FAKE, FAKE, 1000, 32768, 32768, 128, 1, None) == 2  # partial tile
    assert L.ceil_strip_copy(FAKE, FAKE, 1024, 32768, 32704, 128, 1, None) == 2  # partial strip
    assert L.ceil_strip_copy(FAKE, FAKE, 1024, 16384, 32768, 128, 1, None) == 2  # pitch < width
    assert L.ceil_strip_copy(FAKE, FAKE, 1024, 32768, 32768, 64, 1, None) == 3
    assert L.ceil_strip_copy(FAKE, FAKE, 1024, 32768, 32768, 128, 0, None) == 3
    assert L.ceil_strip_copy(FAKE, FAKE, 1024, 32768, 3 * 512, 512, 1, None) == 3  # grid 3
    assert L.ceil_strip_copy(FAKE, FAKE, 1 << 40, 32768, 32768, 128, 1, None) == 2  # > 2^40 B
    assert L.ceil_strip_read(FAKE, None, *ok, None) == 1
    assert L.ceil_strip_read(FAKE, FAKE + 2, *ok, None) == 2
    assert L.ceil_strip_write(None, *ok, None) == 1
    assert L.ceil_strip_write(FAKE, 1024, 32768, 32768, 1024, 1, None) == 3
    # LDS ceilings: op, src, fold, clocks, grid, iters
    assert L.ceil_lds(0, None, None, FAKE, 8, 10, None) == 1
    assert L.ceil_lds(2, None, FAKE, FAKE, 8, 10, None) == 1  # the DMA op reads src
    assert L.ceil_lds(0, None, FAKE + 2, FAKE, 8, 10, None) == 2
    assert L.ceil_lds(0, None, FAKE, FAKE + 4, 8, 10, None) == 2
    assert L.ceil_lds(0, None, FAKE, FAKE, 0, 10, None) == 3
    assert L.ceil_lds(0, None, FAKE, FAKE, 8, 0, None) == 3
    assert L.ceil_lds(7, None, FAKE, FAKE, 8, 10, None) == 3
    assert L.ceil_lds(4, None, FAKE, FAKE, 8, 10, None) == 1  # DMA half reads src
    assert L.ceil_lds(6, None, FAKE, FAKE, 8, 10, None) == 1
