"""Python binding of libpipetile.so (the pipelined tile stream for MI355X / gfx950).

Argument marshalling only: every step of the path runs in the HIP kernels of
the shared library. PyTorch supplies device memory and the current stream.
The functions carry the C ABI's names (``include/pipe_tile.h``):

    pipe_tile_copy(src, dst=None, checksums=False, **cfg)  -> dst [, checksums]
    pipe_rowsum(A, out=None, workspace=None, **cfg)        -> out
    pipe_rowsum_noalloc(A, out, **cfg)                     -> out
    pipe_gemm_mainloop(A, B, C=None, **cfg)                -> C
    pipe_query_kernel(op, M, N, K=0, **cfg)                -> dict
    pipe_kernel_resources(op, M, N, K=0, **cfg)            -> dict
    pipe_rowsum_workspace_bytes(M, N, **cfg)               -> int
    pipe_device_status(clear=False)                        -> int
    pipe_status_from_word(word)                            -> int (PIPE_OK / _ERR_TIMEOUT / _ERR_INVARIANT)

``cfg`` keywords are the fields of ``pipe_config_t`` (stages, consumer_waves,
grid, split, swizzle_shift, flags, spin_limit, trace, status, ...).

If the shared library has not been built, every call raises ``PipeBuildError``:
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libpipetile.so")

PIPE_OK = 0
PIPE_ERR_NULL = 1
PIPE_ERR_SHAPE = 2
PIPE_ERR_ALIGN = 3
PIPE_ERR_STAGES = 4
PIPE_ERR_CONFIG = 5
PIPE_ERR_WORKSPACE = 6
PIPE_ERR_HIP = 7
PIPE_ERR_TIMEOUT = 8
PIPE_ERR_INVARIANT = 9

PIPE_OP_COPY = 0
PIPE_OP_ROWSUM = 1
PIPE_OP_GEMM = 2

PIPE_FLAG_TRACE = 0x1
PIPE_FLAG_ROW_STRIPS = 0x2
PIPE_FLAG_NONTEMPORAL = 0x4
PIPE_FLAG_GEMM_B_LINEAR = 0x8
PIPE_FLAG_XCD_REMAP = 0x10
PIPE_FLAG_SPLIT_INTERLEAVE = 0x20
PIPE_FLAG_UNIFIED = 0x40
PIPE_FLAG_LAZY_COMMIT = 0x80
PIPE_FLAG_TEST_START_PHASE0 = 0x100
PIPE_FLAG_TEST_NO_RELEASE = 0x200
PIPE_FLAG_EAGER_NEWEST = 0x400
PIPE_FLAG_GEMM_C_BF16 = 0x800
PIPE_FLAG_GEMM_STORE_WAVE = 0x1000
PIPE_FLAG_GEMM_B_COLMAJOR = 0x2000
PIPE_FLAG_STRIP_GROUPS = 0x4000
PIPE_FLAG_PRODUCER_VGPR = 0x8000
PIPE_FLAG_DEBUG_CHECKS = 0x10000
PIPE_FLAG_TEST_JITTER = 0x20000
PIPE_FLAG_TEST_EARLY_RELEASE = 0x40000
PIPE_FLAG_GROUP_LOADS = 0x80000

PIPE_STATUS_TIMEOUT_PRODUCER = 0x1
PIPE_STATUS_TIMEOUT_CONSUMER = 0x2
PIPE_STATUS_INVARIANT = 0x4

PIPE_TRACE_WORDS = 8


class PipeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} (status {status})")


class PipeBuildError(RuntimeError):
    pass


class pipe_config_t(ctypes.Structure):
    _fields_ = [
        ("stages", ctypes.c_int32),
        ("tile_m", ctypes.c_int32),
        ("tile_n", ctypes.c_int32),
        ("tile_k", ctypes.c_int32),
        ("producer_waves", ctypes.c_int32),
        ("consumer_waves", ctypes.c_int32),
        ("grid", ctypes.c_int32),
        ("split", ctypes.c_int32),
        ("swizzle_shift", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("spin_limit", ctypes.c_uint32),
        ("trace_capacity", ctypes.c_int32),
        ("trace", ctypes.c_void_p),
        ("status", ctypes.c_void_p),
    ]


class pipe_kernel_info_t(ctypes.Structure):
    _fields_ = [
        ("lds_bytes", ctypes.c_int32),
        ("threads", ctypes.c_int32),
        ("grid", ctypes.c_int32),
        ("items", ctypes.c_int32),
        ("tiles_per_item", ctypes.c_int32),
        ("split", ctypes.c_int32),
    ]


class pipe_kernel_resources_t(ctypes.Structure):
    _fields_ = [
        ("vgprs", ctypes.c_int32),
        ("lds_bytes", ctypes.c_int32),
        ("scratch_bytes", ctypes.c_int32),
        ("max_threads", ctypes.c_int32),
    ]


_lib = None
_lock = threading.Lock()

_c = ctypes
_SIGS = {
    "pipe_abi_version": (_c.c_int, []),
    "pipe_status_str": (_c.c_char_p, [_c.c_int]),
    "pipe_config_default": (_c.c_int, [_c.c_int, _c.POINTER(pipe_config_t)]),
    "pipe_tile_copy": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_int64, _c.c_int64,
                                  _c.c_int64, _c.POINTER(pipe_config_t), _c.c_void_p,
                                  _c.c_void_p]),
    "pipe_rowsum_workspace_bytes": (_c.c_int, [_c.c_int64, _c.c_int64,
                                               _c.POINTER(pipe_config_t),
                                               _c.POINTER(_c.c_size_t)]),
    "pipe_rowsum": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_int64, _c.c_int64,
                               _c.POINTER(pipe_config_t), _c.c_void_p, _c.c_size_t,
                               _c.c_void_p]),
    "pipe_rowsum_noalloc": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_int64,
                                       _c.c_int64, _c.POINTER(pipe_config_t), _c.c_void_p]),
    "pipe_gemm_mainloop": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int64,
                                      _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int64,
                                      _c.c_int64, _c.POINTER(pipe_config_t), _c.c_void_p]),
    "pipe_query_kernel": (_c.c_int, [_c.c_int, _c.POINTER(pipe_config_t), _c.c_int64,
                                     _c.c_int64, _c.c_int64, _c.POINTER(pipe_kernel_info_t)]),
    "pipe_kernel_resources": (_c.c_int, [_c.c_int, _c.POINTER(pipe_config_t), _c.c_int64,
                                         _c.c_int64, _c.c_int64,
                                         _c.POINTER(pipe_kernel_resources_t)]),
    "pipe_device_status": (_c.c_int, [_c.POINTER(_c.c_uint32), _c.c_int]),
    "pipe_status_from_word": (_c.c_int, [_c.c_uint32]),
}


def lib():
    """The loaded shared library (loaded once; raises PipeBuildError if absent)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise PipeBuildError(
                    f"{LIB_PATH} is missing: build it with `python -m async_stage_tile_amd.build`"
                    " (or __graft_entry__.build())")
            L = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in _SIGS.items():
                fn = getattr(L, name)
                fn.restype = res
                fn.argtypes = args
            _lib = L
    return _lib


def exported_symbols():
    return list(_SIGS)


def abi_version() -> int:
    return int(lib().pipe_abi_version())


def status_str(status: int) -> str:
    return lib().pipe_status_str(int(status)).decode()


def _check(status: int, where: str):
    if status != PIPE_OK:
        raise PipeError(status, where)


def make_config(op: int, **kw) -> pipe_config_t:
    """The op's default config with the given fields replaced. ``trace`` and
    ``status`` may be device tensors (or raw device addresses): a tensor must
    be contiguous and hold ``trace_capacity`` records of PIPE_TRACE_WORDS
    32-bit words, or one 32-bit word for ``status``; the tensors are kept on
    the config (``cfg.buffers``) for the device check of the entry points."""
    cfg = pipe_config_t()
    _check(lib().pipe_config_default(op, ctypes.byref(cfg)), "pipe_config_default")
    buffers = {}
    for k, v in kw.items():
        if not hasattr(cfg, k):
            raise TypeError(f"unknown config field {k!r}")
        if k in ("trace", "status"):
            if v is not None and not isinstance(v, int):
                buffers[k] = v
            v = _ptr(v) if v is not None else None
        setattr(cfg, k, v)
    need = {"trace": 4 * PIPE_TRACE_WORDS * max(0, int(cfg.trace_capacity)), "status": 4}
    for k, t in buffers.items():
        if not (t.is_cuda and t.is_contiguous()):
            raise ValueError(f"{k} must be a contiguous device tensor")
        if t.numel() * t.element_size() < need[k]:
            raise ValueError(f"{k} holds {t.numel() * t.element_size()} bytes, "
                             f"{need[k]} needed")
    cfg.buffers = list(buffers.values())
    return cfg


def _device(*tensors):
    """The one device that all the given tensors (None skipped) live on."""
    dev = None
    for t in tensors:
        if t is None:
            continue
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"tensors on different devices: {dev} and {t.device}")
    return dev


def _ptr(t) -> int:
    if t is None:
        return 0
    if isinstance(t, int):
        return t
    return int(t.data_ptr())


def _stream(stream=None, device=None):
    """The given stream, else the current stream of `device`; it must belong
    to `device`."""
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(device)
    if device is not None and s.device != device:
        raise ValueError(f"stream of {s.device} for tensors on {device}")
    return ctypes.c_void_p(int(s.cuda_stream))


def _hold_for(stream, device, *tensors):
    """Tensors this wrapper allocated, used by work enqueued on `stream`: when
    that is not the device's current stream, tell the caching allocator, so that
    their memory is not handed out again before that stream's work is done."""
    import torch
    if stream is None or stream == torch.cuda.current_stream(device):
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def matrix_geometry(shape, strides, name="matrix"):
    """(rows, cols, row pitch in elements) of a 2-D row-major view, or
    ValueError. Columns must be adjacent (unit stride) and rows must not
    overlap (row stride >= cols): the kernels address row r at r * pitch, so a
    broadcast or overlapping view would make them read or write outside it."""
    if len(shape) != 2:
        raise ValueError(f"{name} must be 2-D")
    rows, cols = int(shape[0]), int(shape[1])
    if cols > 1 and strides[1] != 1:
        raise ValueError(f"{name} must be row-major (unit column stride)")
    if rows > 1 and strides[0] < cols:
        raise ValueError(f"{name} rows overlap (row stride {strides[0]} < {cols} columns)")
    return rows, cols, max(int(strides[0]), cols)


def _check_matrix(t, name, dtypes):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} dtype {t.dtype} not in {dtypes}")
    return matrix_geometry(tuple(t.shape), t.stride() if t.dim() == 2 else (), name)


def _check_vector(t, n, dtype, name):
    if t.dtype != dtype or not t.is_cuda or not t.is_contiguous() or t.numel() < n:
        raise ValueError(f"{name} must be a contiguous {dtype} device tensor of >= {n} elements")


def pipe_tile_copy(src, dst=None, checksums=False, stream=None, **cfg):
    """Copy a 16-bit matrix through the tile ring; optionally per-tile code sums."""
    import torch
    M, N, ld_src = _check_matrix(src, "src", (torch.float16, torch.bfloat16, torch.int16))
    made = []
    if dst is None:
        dst = torch.empty_like(src, memory_format=torch.contiguous_format)
        made.append(dst)
    Md, Nd, ld_dst = _check_matrix(dst, "dst", (src.dtype,))
    if (Md, Nd) != (M, N):
        raise ValueError("dst shape differs from src")
    c = make_config(PIPE_OP_COPY, **cfg)
    dev = _device(src, dst, *c.buffers)
    chk = None
    if checksums:   # one word per tile of the configured shape
        tm, tn = max(1, c.tile_m), max(1, c.tile_n)
        chk = torch.empty(((M + tm - 1) // tm) * ((N + tn - 1) // tn), dtype=torch.int32,
                          device=dev)
        made.append(chk)
    with torch.cuda.device(dev):
        st = lib().pipe_tile_copy(_ptr(src), _ptr(dst), M, N, ld_src, ld_dst, ctypes.byref(c),
                                  _ptr(chk), _stream(stream, dev))
    _check(st, "pipe_tile_copy")
    _hold_for(stream, dev, *made)
    return (dst, chk) if checksums else dst


def pipe_rowsum_workspace_bytes(M, N, **cfg) -> int:
    c = make_config(PIPE_OP_ROWSUM, **cfg)
    out = ctypes.c_size_t(0)
    _check(lib().pipe_rowsum_workspace_bytes(M, N, ctypes.byref(c), ctypes.byref(out)),
           "pipe_rowsum_workspace_bytes")
    return int(out.value)


def pipe_rowsum(A, out=None, workspace=None, stream=None, **cfg):
    """fp32 row sums of an fp16 matrix streamed through the tile ring."""
    import torch
    M, N, lda = _check_matrix(A, "A", (torch.float16,))
    made = []
    if out is None:
        out = torch.empty(M, dtype=torch.float32, device=A.device)
        made.append(out)
    need = pipe_rowsum_workspace_bytes(M, N, **cfg)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=A.device)
        made.append(workspace)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    c = make_config(PIPE_OP_ROWSUM, **cfg)
    dev = _device(A, out, workspace, *c.buffers)
    _check_vector(out, M, torch.float32, "out")
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    with torch.cuda.device(dev):
        st = lib().pipe_rowsum(_ptr(A), _ptr(out), M, N, lda, ctypes.byref(c), _ptr(workspace),
                               wbytes, _stream(stream, dev))
    _check(st, "pipe_rowsum")
    _hold_for(stream, dev, *made)
    return out


PIPE_ROWSUM_SCRATCH_BYTES = 1 << 20


def pipe_rowsum_noalloc(A, out, stream=None, **cfg):
    """pipe_rowsum with the workspace in the library's own per-device buffer
    (for callers that cannot allocate). ``out`` (float32[M] on A's device) is
    required: neither this wrapper nor the entry point allocates."""
    import torch
    M, N, lda = _check_matrix(A, "A", (torch.float16,))
    c = make_config(PIPE_OP_ROWSUM, **cfg)
    dev = _device(A, out, *c.buffers)
    _check_vector(out, M, torch.float32, "out")
    with torch.cuda.device(dev):
        st = lib().pipe_rowsum_noalloc(_ptr(A), _ptr(out), M, N, lda, ctypes.byref(c),
                                       _stream(stream, dev))
    _check(st, "pipe_rowsum_noalloc")
    return out


def _gemm_config(C, cfg, b_colmajor=False):
    """The GEMM config, with PIPE_FLAG_GEMM_C_BF16 set from C's dtype and
    PIPE_FLAG_GEMM_B_COLMAJOR from B's layout."""
    import torch
    c = make_config(PIPE_OP_GEMM, **cfg)
    if C.dtype == torch.bfloat16:
        c.flags |= PIPE_FLAG_GEMM_C_BF16
    else:
        c.flags &= ~PIPE_FLAG_GEMM_C_BF16
    if b_colmajor:
        c.flags |= PIPE_FLAG_GEMM_B_COLMAJOR
    else:
        c.flags &= ~PIPE_FLAG_GEMM_B_COLMAJOR
    return c


def _gemm_b(B):
    """(K, N, ldb, column-major) of the B operand. A row-major B (unit column
    stride) is passed as is; a column-major one (unit row stride, e.g. the
    transpose of a row-major N x K tensor) goes with PIPE_FLAG_GEMM_B_COLMAJOR
    and ldb = its column stride."""
    import torch
    if B.dim() == 2 and B.shape[1] > 1 and B.stride(1) != 1 and B.stride(0) == 1:
        N, K, ldb = _check_matrix(B.t(), "B (column-major)", (torch.bfloat16,))
        return K, N, ldb, True
    K, N, ldb = _check_matrix(B, "B", (torch.bfloat16,))
    return K, N, ldb, False


# The fastest GEMM configuration on MI355X for products with at least 256
# output tiles of 256 x 256 (one per CU; e.g. 4096 x 4096 and up): 4 waves (one
# per SIMD) each own a 128 x 128 block, fed by a four-slot ring of 32-K stages
# (PIPE_FLAG_UNIFIED). Pass it as keyword arguments:
# pipe_gemm_mainloop(A, B, **GEMM_UNIFIED_DEEP). bf16 C is supported. Smaller
# products keep more CUs busy with the default 128 x 128 tiles.
GEMM_UNIFIED_DEEP = dict(tile_m=256, tile_n=256, tile_k=32, consumer_waves=4, stages=4,
                         flags=PIPE_FLAG_UNIFIED)


def pipe_gemm_mainloop(A, B, C=None, stream=None, out_dtype=None, **cfg):
    """C = A @ B (bf16 in, fp32 accumulate) with A/B tiles fed through the ring.

    B may be row-major (K x N) or column-major (a K x N view with unit row
    stride, such as Bt.t() of a row-major N x K Bt). C is fp32 (default) or
    bf16 (out_dtype=torch.bfloat16, or a bf16 C): a bf16 C is rounded to
    nearest even from the fp32 sums and written through the staged
    epilogue."""
    import torch
    M, K, lda = _check_matrix(A, "A", (torch.bfloat16,))
    K2, N, ldb, b_col = _gemm_b(B)
    if K2 != K:
        raise ValueError("inner dimensions differ")
    made = None
    if C is None:
        C = made = torch.empty((M, N), dtype=out_dtype or torch.float32, device=A.device)
    Mc, Nc, ldc = _check_matrix(C, "C", (torch.float32, torch.bfloat16))
    if (Mc, Nc) != (M, N):
        raise ValueError("C shape mismatch")
    c = _gemm_config(C, cfg, b_col)
    dev = _device(A, B, C, *c.buffers)
    with torch.cuda.device(dev):
        st = lib().pipe_gemm_mainloop(_ptr(A), _ptr(B), _ptr(C), M, N, K, lda, ldb, ldc,
                                      ctypes.byref(c), _stream(stream, dev))
    _check(st, "pipe_gemm_mainloop")
    _hold_for(stream, dev, made)
    return C


def pipe_query_kernel(op: int, M: int, N: int, K: int = 0, **cfg) -> dict:
    c = make_config(op, **cfg)
    info = pipe_kernel_info_t()
    _check(lib().pipe_query_kernel(op, ctypes.byref(c), M, N, K, ctypes.byref(info)),
           "pipe_query_kernel")
    return {f: getattr(info, f) for f, _ in pipe_kernel_info_t._fields_}


def pipe_kernel_resources(op: int, M: int, N: int, K: int = 0, **cfg) -> dict:
    """Registers, static LDS, spill bytes and maximum workgroup size of the
    kernel the op would launch for this shape (needs a device)."""
    c = make_config(op, **cfg)
    out = pipe_kernel_resources_t()
    _check(lib().pipe_kernel_resources(op, ctypes.byref(c), M, N, K, ctypes.byref(out)),
           "pipe_kernel_resources")
    return {f: getattr(out, f) for f, _ in pipe_kernel_resources_t._fields_}


def pipe_device_status(clear: bool = False) -> int:
    out = ctypes.c_uint32(0)
    _check(lib().pipe_device_status(ctypes.byref(out), 1 if clear else 0), "pipe_device_status")
    return int(out.value)


def pipe_status_from_word(word: int) -> int:
    """The error code a status word stands for (PIPE_OK, PIPE_ERR_TIMEOUT or
    PIPE_ERR_INVARIANT); host arithmetic in the library, no device access."""
    return int(lib().pipe_status_from_word(int(word) & 0xFFFFFFFF))


# ---------------------------------------------------------------------------
# Pre-marshalled launchers: validate and marshal once, then each call is a
# single C-ABI call (with the tensors' device current) on the stream given, or
# else the device's current stream at creation (for repeated launches on the
# same buffers, e.g. timing loops).
# ---------------------------------------------------------------------------
def copy_launcher(src, dst, checksums=None, stream=None, **cfg):
    import torch
    M, N, ld_src = _check_matrix(src, "src", (torch.float16, torch.bfloat16, torch.int16))
    Md, Nd, ld_dst = _check_matrix(dst, "dst", (src.dtype,))
    if (Md, Nd) != (M, N):
        raise ValueError("dst shape differs from src")
    c = make_config(PIPE_OP_COPY, **cfg)
    dev = _device(src, dst, checksums, *c.buffers)
    if checksums is not None:
        tm, tn = max(1, c.tile_m), max(1, c.tile_n)
        tiles = ((M + tm - 1) // tm) * ((N + tn - 1) // tn)
        if checksums.element_size() != 4:
            raise ValueError("checksums must hold 32-bit words")
        _check_vector(checksums, tiles, checksums.dtype, "checksums")
    fn, args = lib().pipe_tile_copy, (_ptr(src), _ptr(dst), M, N, ld_src, ld_dst,
                                       ctypes.byref(c), _ptr(checksums), _stream(stream, dev))

    def launch():
        with torch.cuda.device(dev):
            _check(fn(*args), "pipe_tile_copy")
    launch.keep = (c, src, dst, checksums)
    return launch


def rowsum_launcher(A, out, workspace=None, stream=None, **cfg):
    import torch
    M, N, lda = _check_matrix(A, "A", (torch.float16,))
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    c = make_config(PIPE_OP_ROWSUM, **cfg)
    dev = _device(A, out, workspace, *c.buffers)
    _check_vector(out, M, torch.float32, "out")
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    fn, args = lib().pipe_rowsum, (_ptr(A), _ptr(out), M, N, lda, ctypes.byref(c),
                                    _ptr(workspace), wbytes, _stream(stream, dev))

    def launch():
        with torch.cuda.device(dev):
            _check(fn(*args), "pipe_rowsum")
    launch.keep = (c, A, out, workspace)
    return launch


def gemm_launcher(A, B, C, stream=None, **cfg):
    import torch
    M, K, lda = _check_matrix(A, "A", (torch.bfloat16,))
    K2, N, ldb, b_col = _gemm_b(B)
    Mc, Nc, ldc = _check_matrix(C, "C", (torch.float32, torch.bfloat16))
    if K2 != K or (Mc, Nc) != (M, N):
        raise ValueError("shape mismatch")
    c = _gemm_config(C, cfg, b_col)
    dev = _device(A, B, C, *c.buffers)
    fn, args = lib().pipe_gemm_mainloop, (_ptr(A), _ptr(B), _ptr(C), M, N, K, lda, ldb, ldc,
                                           ctypes.byref(c), _stream(stream, dev))

    def launch():
        with torch.cuda.device(dev):
            _check(fn(*args), "pipe_gemm_mainloop")
    launch.keep = (c, A, B, C)
    return launch


# short aliases
tile_copy = pipe_tile_copy
rowsum = pipe_rowsum
gemm_mainloop = pipe_gemm_mainloop
query_kernel = pipe_query_kernel
kernel_resources = pipe_kernel_resources
device_status = pipe_device_status
