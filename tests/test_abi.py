"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

import async_stage_tile_amd as pt
from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "pipe_tile.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(pipe_[a-z_]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    L = pt.lib()
    declared = _declared()
    assert len(declared) == 12
    for name in declared:
        assert hasattr(L, name), name
    assert sorted(pt.exported_symbols()) == declared


def test_group_loads_flag_validation():
    GL = pt.PIPE_FLAG_STRIP_GROUPS | pt.PIPE_FLAG_GROUP_LOADS
    q = pt.lib().pipe_query_kernel
    info = pt.pipe_kernel_info_t()

    def status(op, **kw):
        return q(op, ctypes.byref(pt.make_config(op, **kw)), 1024, 1024, 0, ctypes.byref(info))

    assert status(pt.PIPE_OP_COPY, stages=8, flags=GL) == pt.PIPE_OK
    assert info.items == 4 * 4 and info.tiles_per_item == 2 * 4   # 4 strips x 4 segments of 2 tile rows
    assert status(pt.PIPE_OP_COPY, stages=4, producer_waves=2, consumer_waves=8,
                  flags=GL) == pt.PIPE_OK
    assert status(pt.PIPE_OP_COPY, stages=8, flags=pt.PIPE_FLAG_GROUP_LOADS) == \
        pt.PIPE_ERR_CONFIG                                   # needs strip groups
    for S in (2, 3, 5, 6, 7):
        assert status(pt.PIPE_OP_COPY, stages=S, flags=GL) == pt.PIPE_ERR_CONFIG
    assert status(pt.PIPE_OP_COPY, stages=8, producer_waves=1, flags=GL) == pt.PIPE_ERR_CONFIG
    assert status(pt.PIPE_OP_COPY, stages=8, consumer_waves=3, flags=GL) == pt.PIPE_ERR_CONFIG
    assert status(pt.PIPE_OP_COPY, stages=8, flags=GL | pt.PIPE_FLAG_UNIFIED) == \
        pt.PIPE_ERR_CONFIG
    assert status(pt.PIPE_OP_ROWSUM, stages=8, flags=GL) == pt.PIPE_ERR_CONFIG
    assert status(pt.PIPE_OP_GEMM, flags=pt.PIPE_FLAG_GROUP_LOADS) == pt.PIPE_ERR_CONFIG


def test_rowsum_noalloc_validation_needs_no_gpu():
    """The no-allocation row sum checks everything, including that the shape's
    workspace fits the library buffer, before any HIP call."""
    L = pt.lib()
    c = pt.make_config(pt.PIPE_OP_ROWSUM, split=8)
    need = ctypes.c_size_t()
    assert L.pipe_rowsum_workspace_bytes(65536, 4096, ctypes.byref(c), ctypes.byref(need)) == 0
    assert need.value > pt.PIPE_ROWSUM_SCRATCH_BYTES
    assert L.pipe_rowsum_noalloc(FAKE, FAKE, 65536, 4096, 4096, ctypes.byref(c), None) \
        == pt.PIPE_ERR_WORKSPACE
    assert L.pipe_rowsum_noalloc(FAKE, FAKE, 0, 4096, 4096, ctypes.byref(c), None) == pt.PIPE_OK
    assert L.pipe_rowsum_noalloc(FAKE, None, 64, 4096, 4096, ctypes.byref(c), None) \
        == pt.PIPE_ERR_NULL
    assert L.pipe_rowsum_noalloc(FAKE, FAKE, 64, 4090, 4096, ctypes.byref(c), None) \
        == pt.PIPE_ERR_SHAPE
    bad = pt.make_config(pt.PIPE_OP_ROWSUM, stages=9)
    assert L.pipe_rowsum_noalloc(FAKE, FAKE, 64, 4096, 4096, ctypes.byref(bad), None) \
        == pt.PIPE_ERR_STAGES


def test_version_and_status_strings():
    assert pt.abi_version() == 1
    assert pt.status_str(pt.PIPE_OK) == "ok"
    assert "timed out" in pt.status_str(pt.PIPE_ERR_TIMEOUT)
    assert "invariant" in pt.status_str(pt.PIPE_ERR_INVARIANT)
    assert pt.status_str(99) == "unknown status"


def test_status_word_to_error_code():
    """Each status bit maps to its error code; the invariant bit wins over a
    timeout (a broken protocol can also stall a wait)."""
    f = pt.pipe_status_from_word
    assert f(0) == pt.PIPE_OK
    assert f(pt.PIPE_STATUS_TIMEOUT_PRODUCER) == pt.PIPE_ERR_TIMEOUT
    assert f(pt.PIPE_STATUS_TIMEOUT_CONSUMER) == pt.PIPE_ERR_TIMEOUT
    assert f(pt.PIPE_STATUS_TIMEOUT_PRODUCER | pt.PIPE_STATUS_TIMEOUT_CONSUMER) == \
        pt.PIPE_ERR_TIMEOUT
    assert f(pt.PIPE_STATUS_INVARIANT) == pt.PIPE_ERR_INVARIANT
    assert f(pt.PIPE_STATUS_INVARIANT | pt.PIPE_STATUS_TIMEOUT_CONSUMER) == pt.PIPE_ERR_INVARIANT
    assert f(0x80000000) == pt.PIPE_OK      # bits the library never sets


def test_config_defaults():
    c = pt.make_config(pt.PIPE_OP_COPY)
    assert (c.stages, c.tile_m, c.tile_n, c.producer_waves, c.consumer_waves) == (2, 128, 64, 4, 4)
    assert c.flags == (pt.PIPE_FLAG_NONTEMPORAL | pt.PIPE_FLAG_XCD_REMAP |
                       pt.PIPE_FLAG_LAZY_COMMIT)
    r = pt.make_config(pt.PIPE_OP_ROWSUM)
    assert (r.stages, r.producer_waves, r.consumer_waves) == (3, 4, 4)
    assert r.flags == (pt.PIPE_FLAG_NONTEMPORAL | pt.PIPE_FLAG_XCD_REMAP)
    g = pt.make_config(pt.PIPE_OP_GEMM)
    assert (g.stages, g.tile_m, g.tile_n, g.tile_k, g.producer_waves, g.consumer_waves) \
        == (2, 128, 128, 64, 4, 4)
    assert g.flags == pt.PIPE_FLAG_EAGER_NEWEST
    assert pt.lib().pipe_config_default(7, ctypes.byref(c)) == pt.PIPE_ERR_CONFIG
    assert pt.lib().pipe_config_default(0, None) == pt.PIPE_ERR_NULL


def _copy(src, dst, M, N, lds, ldd, cfg=None, chk=None):
    c = cfg if cfg is not None else pt.make_config(pt.PIPE_OP_COPY)
    return pt.lib().pipe_tile_copy(src, dst, M, N, lds, ldd, ctypes.byref(c), chk, None)


FAKE = 0x10000  # never dereferenced: every case below fails validation first


def test_copy_validation():
    assert _copy(None, FAKE, 256, 128, 128, 128) == pt.PIPE_ERR_NULL
    assert _copy(FAKE, FAKE, 200, 100, 128, 128) == pt.PIPE_ERR_SHAPE   # N not a multiple of 8
    assert _copy(FAKE, FAKE, 256, 12, 128, 128) == pt.PIPE_ERR_SHAPE
    assert _copy(FAKE, FAKE, -128, 128, 128, 128) == pt.PIPE_ERR_SHAPE
    assert _copy(FAKE, FAKE, 256, 128, 64, 128) == pt.PIPE_ERR_SHAPE    # ld < N
    assert _copy(FAKE + 8, FAKE, 256, 128, 128, 128) == pt.PIPE_ERR_ALIGN
    assert _copy(FAKE, FAKE, 256, 128, 132, 128) == pt.PIPE_ERR_ALIGN  # pitch not 16 B
    assert _copy(FAKE, FAKE, 256, 128, 128, 128, chk=FAKE + 2) == pt.PIPE_ERR_ALIGN
    for bad in (0, 9):
        assert _copy(FAKE, FAKE, 256, 128, 128, 128, pt.make_config(0, stages=bad)) \
            == pt.PIPE_ERR_STAGES
    for bad in (0, 5, 9):
        assert _copy(FAKE, FAKE, 256, 128, 128, 128, pt.make_config(0, consumer_waves=bad)) \
            == pt.PIPE_ERR_CONFIG
    assert _copy(FAKE, FAKE, 256, 128, 128, 128, pt.make_config(0, tile_n=32)) == pt.PIPE_ERR_CONFIG
    assert _copy(FAKE, FAKE, 256, 128, 128, 128, pt.make_config(0, swizzle_shift=4)) \
        == pt.PIPE_ERR_CONFIG
    assert _copy(FAKE, FAKE, 256, 128, 128, 128, pt.make_config(0, flags=0x80000)) \
        == pt.PIPE_ERR_CONFIG
    assert _copy(FAKE, FAKE, 256, 128, 128, 128, pt.make_config(0, flags=pt.PIPE_FLAG_TRACE)) \
        == pt.PIPE_ERR_NULL
    assert _copy(FAKE, FAKE, 256, 128, 128, 128, pt.make_config(
        0, flags=pt.PIPE_FLAG_LAZY_COMMIT | pt.PIPE_FLAG_EAGER_NEWEST)) == pt.PIPE_ERR_CONFIG
    # empty matrices are a no-op, with or without pointers
    assert _copy(None, None, 0, 128, 128, 128) == pt.PIPE_OK
    assert _copy(None, None, 256, 0, 0, 0) == pt.PIPE_OK


def test_ring_shapes():
    # Deep rings (S > 4) exist for 4 or 8 consumer waves only.
    for kw in (dict(stages=5, consumer_waves=3), dict(stages=8, consumer_waves=2),
               dict(producer_waves=3), dict(producer_waves=0)):
        assert _copy(FAKE, FAKE, 256, 128, 128, 128, pt.make_config(0, **kw)) \
            == pt.PIPE_ERR_CONFIG, kw
    for C in (1, 2, 3):
        q = pt.pipe_query_kernel(pt.PIPE_OP_COPY, 4096, 4096, stages=4, producer_waves=4,
                                 consumer_waves=C)
        assert q["threads"] == 64 * (4 + C)
    for S in range(1, 9):
        for pw in (1, 2, 4):
            q = pt.pipe_query_kernel(pt.PIPE_OP_COPY, 16384, 16384, stages=S, producer_waves=pw,
                                     consumer_waves=8)
            assert q["threads"] == 64 * (pw + 8)
            assert S * 16384 <= q["lds_bytes"] <= 160 * 1024
    q = pt.pipe_query_kernel(pt.PIPE_OP_ROWSUM, 8192, 65536, stages=8, producer_waves=4,
                             consumer_waves=4, flags=pt.PIPE_FLAG_UNIFIED)
    assert q["lds_bytes"] == 8 * 16384 and q["threads"] == 256


def test_unified_variant_constraints():
    U = pt.PIPE_FLAG_UNIFIED
    assert _copy(FAKE, FAKE, 200, 128, 128, 128, pt.make_config(0, flags=U, consumer_waves=4)) \
        == pt.PIPE_ERR_CONFIG                                           # ragged M
    assert _copy(FAKE, FAKE, 256, 128, 128, 128, pt.make_config(0, flags=U, consumer_waves=3)) \
        == pt.PIPE_ERR_CONFIG                                           # 3 waves do not divide 16
    assert _copy(FAKE, FAKE, 256, 128, 128, 128, pt.make_config(0, flags=U, consumer_waves=4),
                 chk=FAKE) == pt.PIPE_ERR_CONFIG                       # no checksums
    q = pt.pipe_query_kernel(pt.PIPE_OP_COPY, 16384, 16384, flags=U, consumer_waves=8, stages=3)
    assert q["threads"] == 512 and q["lds_bytes"] == 3 * 16384


def test_rowsum_and_gemm_validation():
    L = pt.lib()
    c = pt.make_config(pt.PIPE_OP_ROWSUM, split=4)
    need = ctypes.c_size_t()
    assert L.pipe_rowsum_workspace_bytes(1024, 4096, ctypes.byref(c), ctypes.byref(need)) == 0
    assert need.value == 4 * 1024 * 4 + 8 * 4  # partials [4][1024], then 8 strip tickets
    assert L.pipe_rowsum(FAKE, FAKE, 1024, 4096, 4096, ctypes.byref(c), None, 0, None) \
        == pt.PIPE_ERR_WORKSPACE
    assert L.pipe_rowsum(FAKE, FAKE, 1024, 4096, 4096, ctypes.byref(c), FAKE, need.value - 4,
                         None) == pt.PIPE_ERR_WORKSPACE
    assert L.pipe_rowsum(FAKE, FAKE, 1000, 4090, 4096, ctypes.byref(c), FAKE, 1 << 20, None) \
        == pt.PIPE_ERR_SHAPE
    assert L.pipe_rowsum(FAKE, None, 1024, 4096, 4096, ctypes.byref(c), FAKE, 1 << 20, None) \
        == pt.PIPE_ERR_NULL
    assert L.pipe_rowsum(None, None, 0, 4096, 4096, ctypes.byref(c), None, 0, None) == pt.PIPE_OK
    g = pt.make_config(pt.PIPE_OP_GEMM)
    args = lambda M, N, K, **kw: L.pipe_gemm_mainloop(kw.get("A", FAKE), FAKE, FAKE, M, N, K,
                                                       K, N, N, ctypes.byref(kw.get("cfg", g)), None)
    assert args(256, 256, 100) == pt.PIPE_ERR_SHAPE      # K not a multiple of 8
    assert args(256, 196, 128) == pt.PIPE_ERR_SHAPE      # N not a multiple of 8
    # shapes that are not whole tiles are accepted (a masked kernel runs them)
    q = pt.pipe_query_kernel(pt.PIPE_OP_GEMM, 200, 136, 72)
    assert (q["items"], q["tiles_per_item"], q["grid"]) == (2 * 2, 2, 4)
    tr = pt.make_config(2, flags=pt.PIPE_FLAG_TRACE, trace=FAKE, trace_capacity=8)
    assert args(200, 136, 72, cfg=tr) == pt.PIPE_ERR_SHAPE   # the trace takes whole tiles
    assert args(256, 256, 128, A=FAKE + 4) == pt.PIPE_ERR_ALIGN
    assert args(256, 256, 128, cfg=pt.make_config(2, stages=5)) == pt.PIPE_ERR_STAGES
    assert args(256, 256, 128, cfg=pt.make_config(2, consumer_waves=3)) == pt.PIPE_ERR_CONFIG
    # bf16 C: 16-byte aligned base and ldc a multiple of 8
    bf = pt.make_config(2, flags=pt.PIPE_FLAG_GEMM_C_BF16)
    assert L.pipe_gemm_mainloop(FAKE, FAKE, FAKE + 4, 256, 256, 128, 128, 256, 256,
                                ctypes.byref(bf), None) == pt.PIPE_ERR_ALIGN
    assert L.pipe_gemm_mainloop(FAKE, FAKE, FAKE, 256, 256, 128, 128, 256, 260,
                                ctypes.byref(bf), None) == pt.PIPE_ERR_ALIGN
    # the GEMM-only flags are rejected by the stream ops
    for f in (pt.PIPE_FLAG_GEMM_C_BF16, pt.PIPE_FLAG_GEMM_B_LINEAR):
        assert _copy(FAKE, FAKE, 256, 128, 128, 128, pt.make_config(0, flags=f)) \
            == pt.PIPE_ERR_CONFIG
    q = pt.pipe_query_kernel(pt.PIPE_OP_GEMM, 4096, 4096, 4096, flags=pt.PIPE_FLAG_GEMM_C_BF16)
    assert q["threads"] == 64 * (4 + 4) and 2 * q["lds_bytes"] <= 160 * 1024
    q = pt.pipe_query_kernel(pt.PIPE_OP_GEMM, 4096, 4096, 4096,
                             flags=pt.PIPE_FLAG_GEMM_C_BF16 | pt.PIPE_FLAG_GEMM_STORE_WAVE)
    assert q["threads"] == 64 * (4 + 4 + 1) and 2 * q["lds_bytes"] <= 160 * 1024
    sw = pt.make_config(2, flags=pt.PIPE_FLAG_GEMM_STORE_WAVE)   # store wave needs bf16 C
    assert L.pipe_gemm_mainloop(FAKE, FAKE, FAKE, 256, 256, 128, 128, 256, 256,
                                ctypes.byref(sw), None) == pt.PIPE_ERR_CONFIG
    assert args(0, 256, 128) == pt.PIPE_OK


def test_query_geometry():
    q = pt.pipe_query_kernel(pt.PIPE_OP_COPY, 16384, 16384, stages=4)
    assert q["items"] == 256 and q["tiles_per_item"] == 128 and q["grid"] == 256
    assert q["lds_bytes"] >= 4 * 16384 and q["threads"] == 512
    q = pt.pipe_query_kernel(pt.PIPE_OP_COPY, 16384, 16384, split=3, grid=100)
    assert q["split"] == 3 and q["tiles_per_item"] == 43 and q["items"] == 768 and q["grid"] == 100
    q = pt.pipe_query_kernel(pt.PIPE_OP_COPY, 128, 512, grid=1)
    assert (q["items"], q["tiles_per_item"], q["grid"]) == (8, 1, 1)
    q = pt.pipe_query_kernel(pt.PIPE_OP_ROWSUM, 8192, 65536)
    assert q["items"] >= 256 and q["items"] == 64 * q["split"]
    q = pt.pipe_query_kernel(pt.PIPE_OP_GEMM, 4096, 4096, 4096)
    assert (q["items"], q["tiles_per_item"], q["threads"]) == (1024, 64, 512)
    assert q["lds_bytes"] >= 2 * 32768
    q = pt.pipe_query_kernel(pt.PIPE_OP_COPY, 300, 200, split=1)   # ragged: 3 x 4 tiles
    assert (q["items"], q["tiles_per_item"]) == (4, 3)
    q = pt.pipe_query_kernel(pt.PIPE_OP_ROWSUM, 1000, 3000, split=2)
    assert (q["items"], q["tiles_per_item"]) == (8 * 2, 24)
    with pytest.raises(pt.PipeError):
        pt.pipe_query_kernel(pt.PIPE_OP_COPY, 100, 60)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(pt, "_lib", None)
    monkeypatch.setattr(pt, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(pt.PipeBuildError):
        pt.lib()


def test_tile_shapes():
    """16 KiB tiles: the pages' 128 x 64, and the wider 64 x 128 and 32 x 256
    (S 2..4, 2 or 4 producer waves, 4 or 8 consumer waves)."""
    ok = dict(stages=2, producer_waves=4, consumer_waves=4)
    for tm, tn in ((64, 128), (32, 256)):
        q = pt.pipe_query_kernel(pt.PIPE_OP_COPY, 16384, 16384, tile_m=tm, tile_n=tn, **ok)
        assert q["items"] == 16384 // tn and q["tiles_per_item"] == 16384 // tm
        q = pt.pipe_query_kernel(pt.PIPE_OP_ROWSUM, 8192, 65536, tile_m=tm, tile_n=tn,
                                 stages=3, producer_waves=2, consumer_waves=8)
        assert q["items"] == (8192 // tm) * q["split"]
        q = pt.pipe_query_kernel(pt.PIPE_OP_COPY, 4096, 4096, tile_m=tm, tile_n=tn,
                                 flags=pt.PIPE_FLAG_UNIFIED, stages=2, consumer_waves=2)
        assert q["threads"] == 128
    for kw in (dict(tile_m=64, tile_n=64), dict(tile_m=256, tile_n=32),
               dict(tile_m=64, tile_n=128, stages=1), dict(tile_m=64, tile_n=128, stages=6,
                                                           consumer_waves=8),
               dict(tile_m=32, tile_n=256, producer_waves=1),
               dict(tile_m=32, tile_n=256, consumer_waves=2),
               dict(tile_m=32, tile_n=256, flags=pt.PIPE_FLAG_UNIFIED, consumer_waves=8)):
        args = dict(ok)
        args.update(kw)
        assert _copy(FAKE, FAKE, 256, 256, 256, 256, pt.make_config(0, **args)) \
            == pt.PIPE_ERR_CONFIG, kw


def test_barrier_arrival_counts_stay_below_2_31():
    """Barrier words count arrivals in 32 bits: a launch whose workgroup would
    see 2^31 or more arrivals on one barrier is refused before any HIP call."""
    cfg = pt.make_config(0, stages=2, producer_waves=1, consumer_waves=8, grid=1)
    M = 128 << 28                      # 2^28 tiles in one strip, one workgroup
    assert _copy(FAKE, FAKE, M, 64, 64, 64, cfg) == pt.PIPE_ERR_SHAPE


def test_binding_rejects_views_the_kernels_cannot_address():
    """The binding passes (rows, cols, pitch) to the library; a view whose rows
    overlap (a broadcast row, stride 0) or whose columns are not adjacent must
    be refused before anything is launched."""
    g = pt.matrix_geometry
    assert g((4, 8), (8, 1)) == (4, 8, 8)
    assert g((4, 8), (16, 1)) == (4, 8, 16)        # padded rows
    assert g((1, 8), (0, 1)) == (1, 8, 8)          # a single row: its stride is never used
    assert g((4, 1), (1, 1)) == (4, 1, 1)          # one column
    for shape, strides in (((4, 8), (0, 1)),       # broadcast row
                           ((4, 8), (4, 1)),       # overlapping rows
                           ((4, 8), (1, 4)),       # column-major
                           ((4, 8, 2), (16, 2, 1))):
        with pytest.raises(ValueError):
            g(shape, strides)


def test_gemm_b_colmajor_validation():
    """Column-major B takes ldb >= K (not >= N), rejects GEMM_B_LINEAR, and is a
    GEMM-only flag; all checked before any launch."""
    g = pt.make_config(pt.PIPE_OP_GEMM, flags=pt.PIPE_FLAG_GEMM_B_COLMAJOR)
    L = pt.lib()
    # M=256, N=512, K=128: ldb 128 is fine for column-major B, too small for row-major
    assert L.pipe_gemm_mainloop(FAKE, FAKE, FAKE, 256, 512, 128, 128, 100, 512,
                                ctypes.byref(g), None) == pt.PIPE_ERR_SHAPE  # ldb < K
    assert L.pipe_gemm_mainloop(FAKE + 4, FAKE, FAKE, 256, 512, 128, 128, 128, 512,
                                ctypes.byref(g), None) == pt.PIPE_ERR_ALIGN  # checked after shape
    g2 = pt.make_config(pt.PIPE_OP_GEMM)
    assert L.pipe_gemm_mainloop(FAKE + 4, FAKE, FAKE, 256, 512, 128, 128, 128, 512,
                                ctypes.byref(g2), None) == pt.PIPE_ERR_SHAPE  # row-major: ldb < N
    bad = pt.make_config(pt.PIPE_OP_GEMM, flags=pt.PIPE_FLAG_GEMM_B_COLMAJOR |
                         pt.PIPE_FLAG_GEMM_B_LINEAR)
    assert L.pipe_gemm_mainloop(FAKE, FAKE, FAKE, 256, 512, 128, 128, 128, 512,
                                ctypes.byref(bad), None) == pt.PIPE_ERR_CONFIG
    info = pt.pipe_kernel_info_t()
    assert L.pipe_query_kernel(pt.PIPE_OP_GEMM, ctypes.byref(bad), 256, 512, 128,
                               ctypes.byref(info)) == pt.PIPE_ERR_CONFIG
    c = pt.make_config(pt.PIPE_OP_COPY, flags=pt.PIPE_FLAG_GEMM_B_COLMAJOR)
    assert L.pipe_tile_copy(FAKE, FAKE, 256, 128, 128, 128, ctypes.byref(c), None,
                            None) == pt.PIPE_ERR_CONFIG


def test_kernel_resources_validation_runs_before_the_runtime():
    """pipe_kernel_resources checks like the op's entry point, before it asks
    the HIP runtime anything, so these fail the same way without a device."""
    L = pt.lib()
    out = pt.pipe_kernel_resources_t()
    c = pt.make_config(pt.PIPE_OP_COPY)
    assert L.pipe_kernel_resources(pt.PIPE_OP_COPY, ctypes.byref(c), 256, 128, 0, None) == \
        pt.PIPE_ERR_NULL
    assert L.pipe_kernel_resources(7, ctypes.byref(c), 256, 128, 0, ctypes.byref(out)) == \
        pt.PIPE_ERR_CONFIG
    for M, N in ((0, 128), (256, 0), (256, 12), (-1, 128)):
        assert L.pipe_kernel_resources(pt.PIPE_OP_COPY, ctypes.byref(c), M, N, 0,
                                       ctypes.byref(out)) == pt.PIPE_ERR_SHAPE
    bad = pt.make_config(pt.PIPE_OP_COPY, stages=9)
    assert L.pipe_kernel_resources(pt.PIPE_OP_COPY, ctypes.byref(bad), 256, 128, 0,
                                   ctypes.byref(out)) == pt.PIPE_ERR_STAGES
    r = pt.make_config(pt.PIPE_OP_ROWSUM, flags=pt.PIPE_FLAG_ROW_STRIPS)
    assert L.pipe_kernel_resources(pt.PIPE_OP_ROWSUM, ctypes.byref(r), 256, 128, 0,
                                   ctypes.byref(out)) == pt.PIPE_ERR_CONFIG
    g = pt.make_config(pt.PIPE_OP_GEMM)
    for M, N, K in ((256, 256, 0), (256, 100, 128), (0, 256, 128)):
        assert L.pipe_kernel_resources(pt.PIPE_OP_GEMM, ctypes.byref(g), M, N, K,
                                       ctypes.byref(out)) == pt.PIPE_ERR_SHAPE
    gb = pt.make_config(pt.PIPE_OP_GEMM, flags=pt.PIPE_FLAG_GEMM_STORE_WAVE)  # needs bf16 C
    assert L.pipe_kernel_resources(pt.PIPE_OP_GEMM, ctypes.byref(gb), 256, 256, 128,
                                   ctypes.byref(out)) == pt.PIPE_ERR_CONFIG


def test_gemm_query_rejects_what_the_entry_point_rejects():
    """For any configuration, pipe_query_kernel(GEMM) returns the error that
    pipe_gemm_mainloop returns for it (the entry point's configuration checks
    run before any pointer is looked at, so an empty product exposes them)."""
    import random
    rng = random.Random(5)
    L = pt.lib()
    info = pt.pipe_kernel_info_t()
    for _ in range(3000):
        c = pt.make_config(pt.PIPE_OP_GEMM, stages=rng.randrange(0, 7),
                           producer_waves=rng.randrange(0, 6),
                           consumer_waves=rng.choice([0, 1, 2, 3, 4, 5, 8]),
                           split=rng.randrange(0, 3), flags=rng.randrange(0, 0x100000) & ~0x1,
                           tile_m=rng.choice([64, 128, 256]), tile_n=rng.choice([64, 128]))
        entry = L.pipe_gemm_mainloop(None, None, None, 0, 0, 0, 0, 0, 0, ctypes.byref(c), None)
        query = L.pipe_query_kernel(pt.PIPE_OP_GEMM, ctypes.byref(c), 256, 128, 64,
                                    ctypes.byref(info))
        if entry != pt.PIPE_OK:
            assert query == entry, (c.stages, c.producer_waves, c.consumer_waves, c.split,
                                    hex(c.flags), c.tile_m, c.tile_n, entry, query)


def test_stream_query_rejects_what_the_entry_points_reject():
    """pipe_query_kernel applies the copy / row-sum entry points' own
    configuration and shape rules (checked here without any launch)."""
    q = pt.lib().pipe_query_kernel
    info = pt.pipe_kernel_info_t()

    def status(op, M, N, **kw):
        return q(op, ctypes.byref(pt.make_config(op, **kw)), M, N, 0, ctypes.byref(info))

    U = pt.PIPE_FLAG_UNIFIED | pt.PIPE_FLAG_NONTEMPORAL
    assert status(pt.PIPE_OP_ROWSUM, 256, 128, flags=pt.PIPE_FLAG_ROW_STRIPS) == pt.PIPE_ERR_CONFIG
    nbytes = ctypes.c_size_t(0)
    rs = pt.make_config(pt.PIPE_OP_ROWSUM, flags=pt.PIPE_FLAG_ROW_STRIPS)
    assert pt.lib().pipe_rowsum_workspace_bytes(256, 128, ctypes.byref(rs), ctypes.byref(nbytes)) \
        == pt.PIPE_ERR_CONFIG
    assert status(pt.PIPE_OP_COPY, 256, 128, stages=2, consumer_waves=1, flags=U) == \
        pt.PIPE_ERR_CONFIG                                   # unified needs 2, 4 or 8 waves
    assert status(pt.PIPE_OP_COPY, 250, 128, stages=2, consumer_waves=4, flags=U) == \
        pt.PIPE_ERR_CONFIG                                   # unified takes whole tiles only
    assert status(pt.PIPE_OP_COPY, 256, 128, stages=2, consumer_waves=4, flags=U) == pt.PIPE_OK
    assert status(pt.PIPE_OP_COPY, 1 << 60, 1 << 12) == pt.PIPE_ERR_SHAPE  # spans >= 2^62 bytes
    assert status(pt.PIPE_OP_GEMM, 256, 256, flags=pt.PIPE_FLAG_TEST_START_PHASE0) == \
        pt.PIPE_ERR_CONFIG


def test_strip_groups_geometry_and_where_they_apply():
    """PIPE_FLAG_STRIP_GROUPS: strips of 4 (else 2) tile columns where the grouped
    kernels take the launch, the plain geometry elsewhere; never for the GEMM."""
    G = pt.PIPE_FLAG_STRIP_GROUPS
    q = lambda M, N, **kw: pt.pipe_query_kernel(pt.PIPE_OP_COPY, M, N, **kw)

    def group(M, N, **kw):   # with one segment per strip: one item per strip
        return (N // 64) // q(M, N, split=1, **kw)["items"]

    # headline shape: 64 strips of 4 tile columns, default split 4 -> 256 items
    h = q(16384, 16384, stages=5, flags=G)
    assert (h["items"], h["split"], h["tiles_per_item"]) == (256, 4, 128)
    assert group(16384, 16384, stages=5, flags=G) == 4
    assert group(16384, 16384, stages=3, flags=G) == 2          # G <= S
    assert group(16384, 16384, stages=1, flags=G) == 1
    assert group(1024, 384, stages=8, flags=G) == 2             # 6 tile columns
    assert group(1024, 320, stages=8, flags=G) == 1             # 5 tile columns
    assert group(1024, 1024, stages=4, flags=G) == 4
    for kw in (dict(consumer_waves=2), dict(consumer_waves=3), dict(producer_waves=1),
               dict(tile_m=64, tile_n=128)):
        assert q(1024, 1024, stages=4, split=1, flags=G, **kw) == \
            q(1024, 1024, stages=4, split=1, flags=0, **kw), kw
    for flags in (G | pt.PIPE_FLAG_ROW_STRIPS, G | pt.PIPE_FLAG_UNIFIED):
        kw = dict(consumer_waves=4) if flags & pt.PIPE_FLAG_UNIFIED else {}
        plain = q(1024, 1024, stages=4, split=1, flags=flags & ~G, **kw)
        assert q(1024, 1024, stages=4, split=1, flags=flags, **kw) == plain
    # ragged shapes take the plain (masked) path
    assert q(1000, 1024, stages=8, split=1, flags=G) == q(1000, 1024, stages=8, split=1)
    assert q(1024, 1000, stages=8, split=1, flags=G) == q(1024, 1000, stages=8, split=1)
    # the row sum ignores the flag; the GEMM rejects it
    assert pt.pipe_query_kernel(pt.PIPE_OP_ROWSUM, 1024, 4096, flags=G) == \
        pt.pipe_query_kernel(pt.PIPE_OP_ROWSUM, 1024, 4096, flags=0)
    info = pt.pipe_kernel_info_t()
    c = pt.make_config(pt.PIPE_OP_GEMM, flags=G)
    assert pt.lib().pipe_query_kernel(pt.PIPE_OP_GEMM, ctypes.byref(c), 256, 256, 256,
                                      ctypes.byref(info)) == pt.PIPE_ERR_CONFIG


def test_binding_rejects_host_buffers_and_mixed_devices():
    """trace/status must be device tensors, and every tensor of a call must live
    on one device (checked before anything reaches the library)."""
    import torch
    with pytest.raises(ValueError):
        pt.make_config(pt.PIPE_OP_COPY, status=torch.zeros(1, dtype=torch.int32))
    with pytest.raises(ValueError):
        pt.make_config(pt.PIPE_OP_COPY, trace=torch.zeros(64, dtype=torch.int32),
                       trace_capacity=8)
    with pytest.raises(ValueError):
        pt._device(torch.zeros(1), torch.zeros(1, device="meta"))
    assert pt._device(None, torch.zeros(1), None) == torch.device("cpu")
    assert pt._device() is None


def test_register_producer_engine_configs():
    """PIPE_FLAG_PRODUCER_VGPR: 128 x 64 tiles, S 1..4, (C, PW) in {3, 4} x {1, 4};
    not unified, not for the GEMM; grouped strips are then ignored."""
    V = pt.PIPE_FLAG_PRODUCER_VGPR
    info = pt.pipe_kernel_info_t()

    def status(op, **kw):
        c = pt.make_config(op, **kw)
        return pt.lib().pipe_query_kernel(op, ctypes.byref(c), 1024, 1024, 0, ctypes.byref(info))

    for op in (pt.PIPE_OP_COPY, pt.PIPE_OP_ROWSUM):
        for S in (1, 2, 3, 4):
            for C in (3, 4):
                for PW in (1, 4):
                    assert status(op, stages=S, consumer_waves=C, producer_waves=PW,
                                  flags=V) == pt.PIPE_OK, (op, S, C, PW)
        for kw in (dict(stages=5), dict(consumer_waves=8), dict(consumer_waves=2),
                   dict(producer_waves=2), dict(tile_m=32, tile_n=256),
                   dict(flags=V | pt.PIPE_FLAG_UNIFIED, consumer_waves=4)):
            kw.setdefault("flags", V)
            assert status(op, **kw) == pt.PIPE_ERR_CONFIG, (op, kw)
    assert status(pt.PIPE_OP_GEMM, flags=V) == pt.PIPE_ERR_CONFIG
    q = lambda **kw: pt.pipe_query_kernel(pt.PIPE_OP_COPY, 1024, 1024, stages=4, **kw)
    assert q(flags=V | pt.PIPE_FLAG_STRIP_GROUPS) == q(flags=V) == q(flags=0)
    assert q(flags=pt.PIPE_FLAG_STRIP_GROUPS) != q(flags=0)


def test_debug_check_configs():
    """DEBUG_CHECKS: 128 x 64 tiles, S 1..4 with 1 + 3 or 4 + 4 waves; JITTER and
    EARLY_RELEASE only with it; not with UNIFIED or PRODUCER_VGPR; not for the GEMM."""
    Dg, J, E = pt.PIPE_FLAG_DEBUG_CHECKS, pt.PIPE_FLAG_TEST_JITTER, pt.PIPE_FLAG_TEST_EARLY_RELEASE
    info = pt.pipe_kernel_info_t()

    def status(op, **kw):
        c = pt.make_config(op, **kw)
        return pt.lib().pipe_query_kernel(op, ctypes.byref(c), 1024, 1024, 0, ctypes.byref(info))

    for op in (pt.PIPE_OP_COPY, pt.PIPE_OP_ROWSUM):
        for S in (1, 2, 3, 4):
            for C, PW in ((3, 1), (4, 4)):
                for extra in (0, J, E, J | E):
                    assert status(op, stages=S, consumer_waves=C, producer_waves=PW,
                                  flags=Dg | extra) == pt.PIPE_OK
        for kw in (dict(stages=5), dict(consumer_waves=4, producer_waves=1),
                   dict(consumer_waves=8), dict(tile_m=32, tile_n=256),
                   dict(flags=Dg | pt.PIPE_FLAG_UNIFIED),
                   dict(flags=Dg | pt.PIPE_FLAG_PRODUCER_VGPR), dict(flags=J), dict(flags=E)):
            kw.setdefault("flags", Dg)
            assert status(op, **kw) == pt.PIPE_ERR_CONFIG, (op, kw)
    assert status(pt.PIPE_OP_GEMM, flags=Dg) == pt.PIPE_ERR_CONFIG
    q = lambda **kw: pt.pipe_query_kernel(pt.PIPE_OP_COPY, 1024, 1024, stages=4, **kw)
    assert q(flags=Dg | pt.PIPE_FLAG_STRIP_GROUPS) == q(flags=Dg) == q(flags=0)


def test_gemm_trace_needs_fp32_c_and_row_major_b():
    info = pt.pipe_kernel_info_t()
    T = pt.PIPE_FLAG_TRACE
    for flags, want in ((T, pt.PIPE_OK), (T | pt.PIPE_FLAG_GEMM_C_BF16, pt.PIPE_ERR_CONFIG),
                        (T | pt.PIPE_FLAG_GEMM_B_COLMAJOR, pt.PIPE_ERR_CONFIG)):
        c = pt.make_config(pt.PIPE_OP_GEMM, flags=flags | pt.PIPE_FLAG_EAGER_NEWEST)
        c.trace, c.trace_capacity = 64, 8          # any aligned address: nothing is launched
        assert pt.lib().pipe_query_kernel(pt.PIPE_OP_GEMM, ctypes.byref(c), 256, 256, 256,
                                          ctypes.byref(info)) == want, hex(flags)


def test_ring_lds_layout_of_the_three_stage_program():
    """The pages' 3-stage ring (128 x 64 fp16 tiles) on gfx950: 3 slots of 16 KiB,
    then 32-bit full, empty and checksum words per slot and one partial per
    consumer wave and slot (1 producer + 3 consumer waves: 49 224 bytes, against
    the pages' 49 280 with 8-byte mbarriers placed first)."""
    q = pt.pipe_query_kernel(pt.PIPE_OP_COPY, 128, 512, stages=3, producer_waves=1,
                             consumer_waves=3, grid=1)
    assert q["lds_bytes"] == 3 * 16384 + 3 * 4 * (3 + 3) == 49224
    assert q["threads"] == 256 and q["grid"] == 1 and (q["items"], q["tiles_per_item"]) == (8, 1)


def test_gemm_256_row_tiles_geometry_and_rejections():
    """tile_m = 256: 8 MFMA + 4 producer waves, a ring of 256 x 64 A and 64 x 128
    B stages; M must be a multiple of 256; no store wave, no trace, S <= 3
    (S <= 2 with bf16 C, whose staging adds 8 x 16 rows of 144 bytes)."""
    q = lambda M, N, K, **kw: pt.pipe_query_kernel(pt.PIPE_OP_GEMM, M, N, K, **kw)
    T = dict(tile_m=256, consumer_waves=8, producer_waves=4)
    for S in (1, 2, 3):
        g = q(4096, 4096, 4096, stages=S, **T)
        assert (g["items"], g["threads"], g["tiles_per_item"]) == (512, 768, 64)
        assert g["lds_bytes"] == S * (256 * 64 * 2 + 64 * 128 * 2 + 8)
    g = q(4096, 4096, 4096, stages=2, flags=pt.PIPE_FLAG_GEMM_C_BF16, **T)
    assert g["lds_bytes"] == 2 * (48 * 1024 + 8) + 8 * 16 * 144
    assert q(4096, 4096, 4096, **dict(T, tile_m=128, consumer_waves=4))["items"] == 1024
    status = lambda M, **kw: pt.lib().pipe_query_kernel(
        pt.PIPE_OP_GEMM, ctypes.byref(pt.make_config(pt.PIPE_OP_GEMM, **kw)), M, 128, 64,
        ctypes.byref(pt.pipe_kernel_info_t()))
    assert status(256, **T) == pt.PIPE_OK
    assert status(384, **T) == pt.PIPE_OK                 # a ragged tile row (masked kernel)
    assert status(384, **dict(T, flags=pt.PIPE_FLAG_TRACE)) != pt.PIPE_OK
    assert status(256, **dict(T, consumer_waves=4)) == pt.PIPE_ERR_CONFIG
    assert status(256, **dict(T, producer_waves=2)) == pt.PIPE_ERR_CONFIG
    assert status(256, tile_m=128, consumer_waves=8, producer_waves=4) == pt.PIPE_ERR_CONFIG
    assert status(256, stages=4, **T) == pt.PIPE_ERR_STAGES
    assert status(256, stages=3, flags=pt.PIPE_FLAG_GEMM_C_BF16, **T) == pt.PIPE_ERR_STAGES
    assert status(256, flags=pt.PIPE_FLAG_GEMM_C_BF16 | pt.PIPE_FLAG_GEMM_STORE_WAVE, **T) == \
        pt.PIPE_ERR_CONFIG
    assert status(256, flags=pt.PIPE_FLAG_TRACE, **T) != pt.PIPE_OK   # (no trace buffer either)


def test_gemm_unified_validation_and_geometry():
    """The unified GEMM (256 x 256 tiles, 16 waves) is its own configuration:
    its geometry comes back from the host query, and every neighbouring
    setting is rejected before any HIP call."""
    U = dict(tile_m=256, tile_n=256, consumer_waves=16, stages=2, flags=pt.PIPE_FLAG_UNIFIED)
    q = pt.pipe_query_kernel(pt.PIPE_OP_GEMM, 4096, 4096, 4096, **U)
    assert (q["items"], q["grid"], q["threads"], q["lds_bytes"], q["tiles_per_item"]) == \
        (256, 256, 1024, 131072, 64)
    q = pt.pipe_query_kernel(pt.PIPE_OP_GEMM, 1000, 600, 72, **U)
    assert (q["items"], q["tiles_per_item"]) == (4 * 3, 2)
    info = pt.pipe_kernel_info_t()

    def status(**kw):
        c = pt.make_config(pt.PIPE_OP_GEMM, **kw)
        return pt.lib().pipe_query_kernel(pt.PIPE_OP_GEMM, ctypes.byref(c), 512, 512, 512,
                                          ctypes.byref(info))

    assert status(**U) == pt.PIPE_OK
    assert status(**dict(U, stages=3)) == pt.PIPE_ERR_STAGES
    assert status(**dict(U, stages=1)) == pt.PIPE_ERR_STAGES
    assert status(**dict(U, consumer_waves=8)) == pt.PIPE_ERR_CONFIG
    assert status(**dict(U, tile_n=128)) == pt.PIPE_ERR_CONFIG
    assert status(**dict(U, tile_m=128)) == pt.PIPE_ERR_CONFIG
    assert status(**dict(U, flags=pt.PIPE_FLAG_UNIFIED | pt.PIPE_FLAG_GEMM_C_BF16)) == \
        pt.PIPE_ERR_CONFIG
    assert status(**dict(U, flags=pt.PIPE_FLAG_UNIFIED | pt.PIPE_FLAG_GEMM_B_COLMAJOR |
                         pt.PIPE_FLAG_GEMM_B_LINEAR)) == pt.PIPE_ERR_CONFIG
    # The 4-wave kernels: 64-K stages in two slots, or 32-K stages in 3 to 5.
    W = dict(U, consumer_waves=4)
    q = pt.pipe_query_kernel(pt.PIPE_OP_GEMM, 4096, 4096, 4096, **W)
    assert (q["threads"], q["lds_bytes"], q["tiles_per_item"]) == (256, 131072, 64)
    for S in (3, 4, 5):
        q = pt.pipe_query_kernel(pt.PIPE_OP_GEMM, 1000, 600, 72, **dict(W, tile_k=32, stages=S))
        assert (q["items"], q["threads"], q["lds_bytes"], q["tiles_per_item"]) == \
            (12, 256, S * 32768, 3)
        assert status(**dict(W, tile_k=32, stages=S)) == pt.PIPE_OK
    assert status(**W) == pt.PIPE_OK
    assert status(**dict(W, tile_k=32, stages=2)) == pt.PIPE_ERR_STAGES
    assert status(**dict(W, tile_k=32, stages=6)) == pt.PIPE_ERR_STAGES
    assert status(**dict(W, stages=3)) == pt.PIPE_ERR_STAGES
    assert status(**dict(W, tile_k=16, stages=4)) == pt.PIPE_ERR_CONFIG
    assert status(**dict(U, tile_k=32, stages=4)) == pt.PIPE_ERR_CONFIG   # 16 waves: 64-K only
    assert status(**dict(W, consumer_waves=2)) == pt.PIPE_ERR_CONFIG
    # bf16 C: the 32-K kernel only.
    assert status(**dict(W, tile_k=32, stages=4, flags=pt.PIPE_FLAG_UNIFIED |
                         pt.PIPE_FLAG_GEMM_C_BF16)) == pt.PIPE_OK
    assert status(**dict(W, flags=pt.PIPE_FLAG_UNIFIED | pt.PIPE_FLAG_GEMM_C_BF16)) == \
        pt.PIPE_ERR_CONFIG
    # Outside the unified flag, tile_k stays 64 and the ring 1..4 deep.
    assert status(tile_k=32) == pt.PIPE_ERR_CONFIG
    assert status(stages=5) == pt.PIPE_ERR_STAGES
    # 256-column tiles only come with the unified flag, and the flag only with them.
    assert status(tile_m=256, tile_n=256, consumer_waves=16, stages=2) == pt.PIPE_ERR_CONFIG
    assert status(flags=pt.PIPE_FLAG_UNIFIED) == pt.PIPE_ERR_CONFIG
    assert status(tile_m=256, consumer_waves=8, flags=pt.PIPE_FLAG_UNIFIED) == pt.PIPE_ERR_CONFIG


def test_gemm_unified_deep_preset_is_a_valid_config():
    q = pt.pipe_query_kernel(pt.PIPE_OP_GEMM, 4096, 4096, 4096, **pt.GEMM_UNIFIED_DEEP)
    assert (q["items"], q["threads"], q["lds_bytes"], q["tiles_per_item"]) == (256, 256, 131072, 128)
