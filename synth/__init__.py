"""Seeded synthetic inputs shared by the CPU oracle and the HIP path.

This module holds none of the pipeline's arithmetic: it only manufactures
input bits. Every generator is counter-based so that any element can be
recomputed on its own, on any device, from (seed, stream, index).

Generator: splitmix64 (Vigna's public-domain generator). Element ``i`` of
stream ``s`` under ``seed`` is ``mix(key_s + (i + 1) * GOLDEN)`` where
``key_s = mix(seed + (s + 1) * GOLDEN)`` and ``mix`` is the splitmix64
output finaliser. The arithmetic is done on int64 tensors with wrapping
multiplication and masked (logical) right shifts, so the same code runs on
the CPU and on a ROCm device and gives identical bits (the CPU tests check
it against a uint64 numpy version and the published test vector).

Distributions (all built from one 64-bit draw per element unless noted):
  * uniform[-1, 1): ``u = (z >> 40) * 2**-24``, ``v = 2u - 1`` (exact in
    fp32), then round-to-nearest-even to fp16 / bf16;
  * normal(0, 1): Box-Muller in fp64 from two draws per element (streams
    ``2s`` and ``2s+1``), ``u1 in (0, 1]``, ``u2 in [0, 1)``, then RNE to
    fp16. Transcendentals may differ in the last fp64 ulp between devices,
    so callers generate once and hand the same bits to both sides;
  * small integers in [lo, hi]: ``lo + (z >> 32) % (hi - lo + 1)``;
  * index codes: ``(r * N + c) mod period`` as exact fp16 integers, and the
    raw 16-bit code ``(r * N + c) mod 65536`` reinterpreted as fp16 bits
    (includes inf / NaN patterns, which a bit copy must move untouched).
"""
from __future__ import annotations

import torch

GOLDEN = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
DEFAULT_SEED = 42


def _s64(x: int) -> int:
    """Two's-complement int64 view of an unsigned 64-bit constant."""
    x &= (1 << 64) - 1
    return x - (1 << 64) if x >= (1 << 63) else x


_G = _s64(GOLDEN)
_C1 = _s64(_M1)
_C2 = _s64(_M2)


def _lsr(z: torch.Tensor, k: int) -> torch.Tensor:
    return (z >> k) & ((1 << (64 - k)) - 1)


def _mix(z: torch.Tensor) -> torch.Tensor:
    z = (z ^ _lsr(z, 30)) * _C1
    z = (z ^ _lsr(z, 27)) * _C2
    return z ^ _lsr(z, 31)


def _mix_int(z: int) -> int:
    m = (1 << 64) - 1
    z &= m
    z = ((z ^ (z >> 30)) * _M1) & m
    z = ((z ^ (z >> 27)) * _M2) & m
    return z ^ (z >> 31)


def stream_key(seed: int, stream: int) -> int:
    """Per-stream key, itself one splitmix64 output of ``seed``."""
    return _s64(_mix_int(seed + (stream + 1) * GOLDEN))


def raw64(n: int, seed: int = DEFAULT_SEED, stream: int = 0, start: int = 0,
          device="cpu") -> torch.Tensor:
    """int64 tensor holding the 64-bit draws ``start .. start+n-1``."""
    key = stream_key(seed, stream)
    idx = torch.arange(start + 1, start + n + 1, dtype=torch.int64, device=device)
    return _mix(idx * _G + key)


def splitmix64_sequence(state: int, n: int) -> list[int]:
    """Plain sequential splitmix64 from ``state`` (for the published test vector)."""
    out = []
    m = (1 << 64) - 1
    for _ in range(n):
        state = (state + GOLDEN) & m
        out.append(_mix_int(state))
    return out


def _chunked(numel: int, fn, out: torch.Tensor, chunk: int = 1 << 24):
    flat = out.view(-1)
    for s in range(0, numel, chunk):
        e = min(numel, s + chunk)
        flat[s:e] = fn(s, e - s)
    return out


def uniform(shape, dtype=torch.float16, seed: int = DEFAULT_SEED, stream: int = 0,
            device="cpu") -> torch.Tensor:
    """Uniform [-1, 1) draws rounded (RNE) to ``dtype``."""
    out = torch.empty(shape, dtype=dtype, device=device)
    numel = out.numel()

    def gen(s, n):
        z = raw64(n, seed, stream, s, device)
        u = _lsr(z, 40).to(torch.float32) * (2.0 ** -24)
        return (2.0 * u - 1.0).to(dtype)

    return _chunked(numel, gen, out)


def normal(shape, dtype=torch.float16, seed: int = DEFAULT_SEED, stream: int = 0,
           device="cpu") -> torch.Tensor:
    """Standard normal draws (Box-Muller in fp64) rounded (RNE) to ``dtype``."""
    out = torch.empty(shape, dtype=dtype, device=device)
    numel = out.numel()

    def gen(s, n):
        z1 = raw64(n, seed, 2 * stream, s, device)
        z2 = raw64(n, seed, 2 * stream + 1, s, device)
        u1 = (_lsr(z1, 11) + 1).to(torch.float64) * (2.0 ** -53)
        u2 = _lsr(z2, 11).to(torch.float64) * (2.0 ** -53)
        r = torch.sqrt(-2.0 * torch.log(u1))
        return (r * torch.cos((2.0 * torch.pi) * u2)).to(dtype)

    return _chunked(numel, gen, out)


def small_int(shape, lo: int, hi: int, dtype=torch.float16, seed: int = DEFAULT_SEED,
              stream: int = 0, device="cpu") -> torch.Tensor:
    """Integers uniform in [lo, hi], exactly representable in ``dtype``."""
    out = torch.empty(shape, dtype=dtype, device=device)
    numel = out.numel()
    span = hi - lo + 1

    def gen(s, n):
        z = raw64(n, seed, stream, s, device)
        return (lo + torch.remainder(_lsr(z, 32), span)).to(dtype)

    return _chunked(numel, gen, out)


def index_coded(M: int, N: int, period: int = 2048, device="cpu") -> torch.Tensor:
    """fp16 matrix with value ``(r*N + c) mod period`` (exact integers)."""
    r = torch.arange(M, dtype=torch.int64, device=device).view(M, 1)
    c = torch.arange(N, dtype=torch.int64, device=device).view(1, N)
    return torch.remainder(r * N + c, period).to(torch.float16)


def unique_codes(M: int, N: int, device="cpu") -> torch.Tensor:
    """fp16-typed matrix whose raw bits are ``(r*N + c) mod 65536``."""
    r = torch.arange(M, dtype=torch.int64, device=device).view(M, 1)
    c = torch.arange(N, dtype=torch.int64, device=device).view(1, N)
    codes = torch.remainder(r * N + c, 65536).to(torch.int32)
    codes = torch.where(codes >= 32768, codes - 65536, codes).to(torch.int16)
    return codes.view(torch.float16)
