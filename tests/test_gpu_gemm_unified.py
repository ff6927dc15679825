"""GPU parity of the unified GEMMs (PIPE_FLAG_UNIFIED: 256 x 256 output tiles
whose waves all load a share of each stage and all compute) against the fp64
CPU oracle: small-integer operands bit for bit (|C| <= 4 K < 2**24 is exact in
fp32 in any order), uniform[-1, 1) operands within the GEMM tolerance. Three
kernels: 16 waves of 64 x 64 output blocks on 64-K stages; 4 waves of
128 x 128 blocks on 64-K stages; the same 4 waves on 32-K stages in rings of
3 to 5 slots, which also write bf16 C."""
import numpy as np
import pytest
import torch

import async_stage_tile_amd as pt
import synth
from oracle import results as R

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
_U = pt.PIPE_FLAG_UNIFIED
KERNELS = {
    "w16": dict(tile_m=256, tile_n=256, consumer_waves=16, stages=2, flags=_U),
    "w4": dict(tile_m=256, tile_n=256, consumer_waves=4, stages=2, flags=_U),
    "w4k32s3": dict(tile_m=256, tile_n=256, tile_k=32, consumer_waves=4, stages=3, flags=_U),
    "w4k32s4": dict(tile_m=256, tile_n=256, tile_k=32, consumer_waves=4, stages=4, flags=_U),
    "w4k32s5": dict(tile_m=256, tile_n=256, tile_k=32, consumer_waves=4, stages=5, flags=_U),
}
U = KERNELS["w16"]


def _f32(t):
    return t.float().cpu().numpy()


def _operands(M, N, K, seed, bcol, kind="int"):
    if kind == "int":
        A = synth.small_int((M, K), -2, 2, torch.bfloat16, seed=seed, stream=0, device=DEV)
        Bt = synth.small_int((N, K), -2, 2, torch.bfloat16, seed=seed, stream=1, device=DEV)
    else:
        A = synth.uniform((M, K), torch.bfloat16, seed=seed, stream=0, device=DEV)
        Bt = synth.uniform((N, K), torch.bfloat16, seed=seed, stream=1, device=DEV)
    B = Bt.t() if bcol else Bt.t().contiguous()   # a K x N view: column-major or row-major
    return A, B, R.gemm_f64(_f32(A), _f32(Bt).T.copy())


def _run(A, B, **cfg):
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    C = pt.pipe_gemm_mainloop(A, B, status=st, **cfg)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    return C


def _assert_exact(C, ref):
    bad = np.argwhere(C.cpu().numpy() != ref)
    assert bad.size == 0, f"{bad.shape[0]} mismatches, first {bad[:4].tolist()}"


@pytest.mark.parametrize("kernel", list(KERNELS))
@pytest.mark.parametrize("shape", [(256, 256, 64), (512, 768, 320), (1000, 1000, 1000),
                                   (300, 264, 72), (1, 8, 8), (257, 520, 136)])
@pytest.mark.parametrize("bcol", [False, True])
def test_unified_gemm_small_integers_bit_exact(kernel, shape, bcol):
    M, N, K = shape
    print(f"[unified] {kernel} {shape} bcol={bcol}", flush=True)
    A, B, ref = _operands(M, N, K, seed=M + N + K, bcol=bcol)
    _assert_exact(_run(A, B, **KERNELS[kernel]), ref)


@pytest.mark.parametrize("kernel", list(KERNELS))
@pytest.mark.parametrize("grid", [1, 3, 5])
def test_unified_gemm_persistent_grid(kernel, grid):
    """Twelve tiles on fewer workgroups: each workgroup's ring runs on from
    one tile into the next."""
    A, B, ref = _operands(1024, 768, 384, seed=grid, bcol=False)
    q = pt.pipe_query_kernel(pt.PIPE_OP_GEMM, 1024, 768, 384, **KERNELS[kernel])
    assert q["items"] == 12
    _assert_exact(_run(A, B, grid=grid, **KERNELS[kernel]), ref)


@pytest.mark.parametrize("kernel", ["w4k32s3", "w4k32s4", "w4k32s5"])
@pytest.mark.parametrize("K", [8, 32, 40, 64, 96, 128, 160])
@pytest.mark.parametrize("bcol", [False, True])
def test_deep_unified_gemm_short_k(kernel, K, bcol):
    """K of 1 to 5 stages of 32: fewer steps than the ring is deep, the
    steady-state loop skipped or run once, ragged last stages; six tiles on
    five workgroups."""
    A, B, ref = _operands(768, 512, K, seed=K, bcol=bcol)
    _assert_exact(_run(A, B, grid=5, **KERNELS[kernel]), ref)


@pytest.mark.parametrize("kernel", list(KERNELS))
@pytest.mark.parametrize("b_linear", [False, True])
def test_unified_gemm_uniform_within_tolerance(kernel, b_linear):
    cfg = dict(KERNELS[kernel])
    cfg["flags"] = cfg["flags"] | (pt.PIPE_FLAG_GEMM_B_LINEAR if b_linear else 0)
    A, B, ref = _operands(1024, 768, 512, seed=7, bcol=False, kind="uniform")
    res = R.within_tol(_run(A, B, **cfg).cpu().numpy(), ref, 1e-2)
    assert res["ok"], res


@pytest.mark.parametrize("kernel", list(KERNELS))
def test_unified_gemm_matches_the_specialised_ring_bitwise(kernel):
    """Each output element is one wave's MFMA chain over K in the same order as
    in the 256 x 128 specialised ring: the kernels give the same bits."""
    A, B, _ = _operands(1000, 1000, 1000, seed=11, bcol=False, kind="uniform")
    T = dict(tile_m=256, consumer_waves=8, producer_waves=4, stages=3,
             flags=pt.PIPE_FLAG_EAGER_NEWEST)
    assert torch.equal(_run(A, B, **KERNELS[kernel]), _run(A, B, **T))


@pytest.mark.parametrize("kernel", ["w16", "w4", "w4k32s4"])
def test_unified_gemm_4096_small_integers_bit_exact(kernel):
    print(f"[unified] {kernel} 4096^3 small integers", flush=True)
    A, B, ref = _operands(4096, 4096, 4096, seed=5, bcol=False)
    _assert_exact(_run(A, B, **KERNELS[kernel]), ref)


def test_deep_unified_gemm_4096_column_major_bit_exact():
    A, B, ref = _operands(4096, 4096, 4096, seed=6, bcol=True)
    _assert_exact(_run(A, B, **KERNELS["w4k32s4"]), ref)


@pytest.mark.parametrize("kernel", ["w4k32s3", "w4k32s4", "w4k32s5"])
@pytest.mark.parametrize("shape", [(256, 256, 64), (1000, 1000, 1000), (300, 264, 72), (1, 8, 8)])
@pytest.mark.parametrize("bcol", [False, True])
def test_deep_unified_gemm_bf16_c_bit_exact(kernel, shape, bcol):
    """bf16 C: each exact fp32 sum of small integers rounded once to bf16, as
    the oracle's gemm_bf16 rounds the fp64 product."""
    M, N, K = shape
    A, B, _ = _operands(M, N, K, seed=M + K, bcol=bcol)
    cfg = dict(KERNELS[kernel], flags=_U | pt.PIPE_FLAG_GEMM_C_BF16)
    C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    _run(A, B, C=C, **cfg)
    ref = R.gemm_bf16(_f32(A), _f32(B.contiguous()))
    got = C.float().cpu().numpy()
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{bad.shape[0]} mismatches, first {bad[:4].tolist()}"


def test_deep_unified_gemm_bf16_c_is_the_fp32_result_rounded():
    """On uniform operands the bf16 C of the deep kernel is its fp32 C rounded
    to nearest even, and its 4096^3 product stays within the GEMM tolerance."""
    A, B, ref = _operands(4096, 4096, 4096, seed=9, bcol=False, kind="uniform")
    cfg = KERNELS["w4k32s4"]
    C32 = _run(A, B, **cfg)
    Cb = torch.empty(4096, 4096, dtype=torch.bfloat16, device=DEV)
    _run(A, B, C=Cb, **dict(cfg, flags=_U | pt.PIPE_FLAG_GEMM_C_BF16))
    assert torch.equal(Cb, C32.to(torch.bfloat16))
    res = R.within_tol(Cb.float().cpu().numpy(), ref, 1e-2)
    assert res["ok"], res


@pytest.mark.parametrize("kernel,c_bf16", [(k, False) for k in KERNELS] +
                         [(k, True) for k in KERNELS if k.startswith("w4k32")])
@pytest.mark.parametrize("bcol", [False, True])
def test_unified_gemm_strided_operands(kernel, c_bf16, bcol):
    """A, B and C as views into wider buffers (lda = K + 64, ldb = N + 128 or
    K + 64 for column-major B, ldc = N + 64); the pitch padding of C stays
    untouched. bf16 C with the 32-K kernels, which alone write it."""
    M, N, K = 520, 384, 328
    Abig = synth.small_int((M, K + 64), -2, 2, torch.bfloat16, seed=71, stream=0, device=DEV)
    A = Abig[:, 32:32 + K]
    if bcol:
        Btbig = synth.small_int((N, K + 64), -2, 2, torch.bfloat16, seed=71, stream=1, device=DEV)
        B = Btbig[:, 16:16 + K].t()                  # K x N, unit row stride, ldb = K + 64
    else:
        Bbig = synth.small_int((K, N + 128), -2, 2, torch.bfloat16, seed=71, stream=1, device=DEV)
        B = Bbig[:, 64:64 + N]
    dt = torch.bfloat16 if c_bf16 else torch.float32
    Cbig = torch.full((M, N + 64), 7.0, dtype=dt, device=DEV)
    C = Cbig[:, 8:8 + N]
    cfg = dict(KERNELS[kernel])
    if c_bf16:
        cfg["flags"] = cfg["flags"] | pt.PIPE_FLAG_GEMM_C_BF16
    _run(A, B, C=C, **cfg)
    a, b = _f32(A.contiguous()), _f32(B.contiguous())
    ref = R.gemm_bf16(a, b) if c_bf16 else R.gemm_f64(a, b)
    assert np.array_equal(C.float().cpu().numpy(), ref)
    pad = Cbig.float().cpu().numpy()
    assert (pad[:, :8] == 7.0).all() and (pad[:, 8 + N:] == 7.0).all()
