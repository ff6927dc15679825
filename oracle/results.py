"""Result oracle: the plain definitions of what the pipelined tile stream computes.

Test infrastructure only (see the package docstring). The pipeline changes how
fast a result is produced, never which result: the tile copy is the identity,
the row reduction is the exact row sum, the GEMM mainloop is the matrix
product. Each function is that definition written out.

Sources (pages, by title and section):
  * "cute（11）hopper之TMA_copy", code listing and section 4 (verification):
    each 128x64 tile travels global -> swizzled shared memory -> global and the
    host checks the round trip bit for bit.
  * "cute（12）async_pipeline", code listing (consumer loop): consumers use the
    data of each stage; here the uses are copy-out, per-tile checksum, row sum
    and a matrix-multiply mainloop.
  * "cute（12）async_pipeline", section 8 "实验设计": tile 128x64, 3 stages,
    8 tiles along K.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

TILE_M = 128
TILE_N = 64


def _bits16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    assert a.dtype.itemsize == 2, "16-bit payload expected"
    return a.view(np.uint16)


def tile_grid(M: int, N: int, tile_m: int = TILE_M, tile_n: int = TILE_N):
    """Tiles (i, j) covering an MxN matrix: rows [i*tm, ...), cols [j*tn, ...).

    Ragged edges give partial tiles. Returned in row-major tile order.
    """
    tiles = []
    for i in range(0, (M + tile_m - 1) // tile_m):
        for j in range(0, (N + tile_n - 1) // tile_n):
            r0, c0 = i * tile_m, j * tile_n
            tiles.append((i, j, r0, min(M, r0 + tile_m), c0, min(N, c0 + tile_n)))
    return tiles


def tile_copy(src: np.ndarray, tile_m: int = TILE_M, tile_n: int = TILE_N) -> np.ndarray:
    """Copy every tile back to the same (row, col) of the output, bit for bit."""
    s = _bits16(src)
    M, N = s.shape
    dst = np.zeros_like(s)
    for (_, _, r0, r1, c0, c1) in tile_grid(M, N, tile_m, tile_n):
        dst[r0:r1, c0:c1] = s[r0:r1, c0:c1]
    return dst.view(src.dtype)


def tile_checksums(src: np.ndarray, tile_m: int = TILE_M, tile_n: int = TILE_N) -> np.ndarray:
    """Per-tile sum of the raw 16-bit codes, as uint32, in row-major tile order.

    A 128x64 tile sums at most 8192 * 65535 < 2**30, so uint32 never wraps and
    the value does not depend on summation order.
    """
    s = _bits16(src)
    M, N = s.shape
    out = []
    for (_, _, r0, r1, c0, c1) in tile_grid(M, N, tile_m, tile_n):
        out.append(int(s[r0:r1, c0:c1].astype(np.uint64).sum()))
    return np.array(out, dtype=np.uint64).astype(np.uint32)


def int_to_f32_rne(v: int) -> np.float32:
    """Round an exact integer to the nearest fp32 (ties to even)."""
    if v == 0:
        return np.float32(0.0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    L = a.bit_length()
    if L <= 24:
        return np.float32(sign * a)
    sh = L - 24
    q, rem = divmod(a, 1 << sh)
    half = 1 << (sh - 1)
    if rem > half or (rem == half and (q & 1)):
        q += 1
    return np.float32(sign * float(q) * float(1 << sh))


def fp16_to_scaled_int(a: np.ndarray) -> np.ndarray:
    """Every finite fp16 is k * 2**-24 with |k| < 2**40; return k as int64."""
    k = a.astype(np.float64) * float(1 << 24)
    return k.astype(np.int64)


def rowsum_exact(A: np.ndarray, row_block: int = 256) -> np.ndarray:
    """Row sums of an fp16 matrix: the exact sum, rounded once to fp32.

    Exact because each row's scaled integers sum below 2**56 for N <= 65536.
    """
    assert A.dtype == np.float16
    M, N = A.shape
    assert N <= (1 << 16), "int64 exactness bound"
    out = np.empty(M, dtype=np.float32)
    scale = np.float32(2.0 ** -24)
    for r0 in range(0, M, row_block):
        blk = fp16_to_scaled_int(A[r0:r0 + row_block]).sum(axis=1)
        for i, v in enumerate(blk.tolist()):
            out[r0 + i] = int_to_f32_rne(int(v)) * scale
    return out


def rowsum_fraction(A: np.ndarray) -> list:
    """Brute-force exact row sums as Fractions (tiny inputs only)."""
    return [sum((Fraction(float(x)) for x in row), Fraction(0)) for row in A]


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen raw bf16 codes (uint16) to float32 values (exact)."""
    b = np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def gemm_f64(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """R = A @ B in fp64 from exactly-representable inputs (A MxK, B KxN).

    A bf16*bf16 product is exact in fp64; the fp64 sum error over K terms is
    far below any fp32-accumulate tolerance.
    """
    return A.astype(np.float64) @ B.astype(np.float64)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round real values (given as float64) to the nearest bf16, ties to even.

    bf16 keeps 8 significant bits and fp32's exponent range: a normal value
    m * 2**e (0.5 <= |m| < 1) becomes rint(m * 2**8) * 2**(e - 8); below the
    smallest normal 2**-126 the quantum is fixed at 2**-133 (subnormals);
    beyond the largest finite bf16 the result is +-inf. NaN stays NaN.
    Returns the bf16 values as float32 (every bf16 is exactly an fp32).
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    nan = np.isnan(x)
    m, e = np.frexp(np.where(nan, 0.0, x))
    normal = np.abs(x) >= 2.0 ** -126
    q = np.where(normal, np.rint(m * 256.0) * np.ldexp(1.0, e - 8),
                 np.rint(np.where(nan, 0.0, x) * 2.0 ** 133) * 2.0 ** -133)
    max_bf16 = (2.0 - 2.0 ** -7) * 2.0 ** 127
    q = np.where(np.abs(q) > max_bf16, np.copysign(np.inf, q), q)
    out[...] = np.where(nan, np.nan, q)
    return out.astype(np.float32)


def bf16_bits(values_f32: np.ndarray) -> np.ndarray:
    """Raw 16-bit codes of bf16 values held exactly in float32."""
    v = np.ascontiguousarray(values_f32, dtype=np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def gemm_bf16(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """R = round_to_bf16(A @ B): the product rounded once to bf16 (as float32)."""
    return round_to_bf16(gemm_f64(A, B))


def gemm_fraction(A: np.ndarray, B: np.ndarray) -> list:
    """Brute-force exact product as Fractions (tiny shapes only)."""
    M, K = A.shape
    K2, N = B.shape
    assert K == K2
    return [[sum((Fraction(float(A[i, k])) * Fraction(float(B[k, j])) for k in range(K)),
                 Fraction(0)) for j in range(N)] for i in range(M)]


def within_tol(got: np.ndarray, ref: np.ndarray, rel: float) -> dict:
    """Element-wise check |got - ref| <= rel * max(|ref|, rms(ref)).

    A plain relative bound is ill-posed for entries near zero (a row sum of
    normal data can land arbitrarily close to 0); measuring the error against
    the larger of |ref| and the rms of the whole result keeps the bound
    meaningful there and equals the plain relative bound elsewhere.
    """
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    scale = np.maximum(np.abs(r), rms)
    err = np.abs(g - r)
    bad = err > rel * scale
    return {
        "ok": bool(not bad.any()) and bool(np.isfinite(g).all()),
        "n_bad": int(bad.sum()),
        "max_abs_err": float(err.max()) if err.size else 0.0,
        "max_err_over_rms": float(err.max() / rms) if err.size and rms > 0 else 0.0,
        "n_over_plain_rel": int((err > rel * np.abs(r)).sum()),
        "rms_ref": rms,
    }
