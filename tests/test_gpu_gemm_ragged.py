"""GPU parity of the GEMM mainloop on shapes that are not whole tiles (M any,
N and K multiples of 8): chunks outside A and B enter the ring as zeros and
only C's M x N elements are written. Small-integer operands make every fp32
sum exact, so C must equal the oracle's product bit for bit; a guard region
around C must stay untouched."""
import numpy as np
import pytest
import torch

import async_stage_tile_amd as pt
import synth
from oracle import results as R

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
EN = pt.PIPE_FLAG_EAGER_NEWEST


def _f32(t):
    return t.float().cpu().numpy()


def _case(M, N, K, seed):
    A = synth.small_int((M, K), -2, 2, torch.bfloat16, seed=seed, stream=0).to(DEV)
    B = synth.small_int((K, N), -2, 2, torch.bfloat16, seed=seed, stream=1).to(DEV)
    return A, B, R.gemm_f64(_f32(A), _f32(B))


def _guarded_c(M, N, dtype, pad=24):
    """C as an M x N view with `pad` guard columns on the right and a guard row
    below, all holding 7."""
    big = torch.full((M + 1, N + pad), 7.0, dtype=dtype, device=DEV)
    return big, big[:M, :N]


@pytest.mark.parametrize("shape", [(200, 136, 72), (1000, 1000, 1000), (1, 8, 8), (129, 264, 520),
                                   (257, 128, 64), (128, 120, 64), (384, 256, 200)])
@pytest.mark.parametrize("cfg", [dict(), dict(stages=3), dict(stages=1, producer_waves=2),
                                 dict(stages=4, producer_waves=2, flags=pt.PIPE_FLAG_LAZY_COMMIT)],
                         ids=["default", "S3", "S1PW2", "S4PW2lazy"])
def test_ragged_gemm_small_integers_bit_exact(shape, cfg):
    M, N, K = shape
    print(f"[ragged] {shape} {cfg}", flush=True)
    A, B, ref = _case(M, N, K, seed=M + N + K)
    big, C = _guarded_c(M, N, torch.float32)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    pt.pipe_gemm_mainloop(A, B, C, status=st, **cfg)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    got = C.cpu().numpy()
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{bad.shape[0]} mismatches, first {bad[:4].tolist()}"
    assert bool((big[:, N:] == 7.0).all()) and bool((big[M:, :] == 7.0).all())


@pytest.mark.parametrize("shape", [(200, 136, 72), (1000, 1000, 1000), (300, 264, 136)])
@pytest.mark.parametrize("variant", ["tile256", "bf16C", "bf16C_store_wave", "bcol", "bcol_bf16C"])
def test_ragged_gemm_variants_bit_exact(shape, variant):
    M, N, K = shape
    print(f"[ragged] {shape} {variant}", flush=True)
    A, B, ref = _case(M, N, K, seed=3 * M + N)
    cfg, dtype = {}, torch.float32
    if variant == "tile256":
        cfg = dict(tile_m=256, consumer_waves=8, producer_waves=4, stages=3, flags=EN)
    if "bf16C" in variant:
        dtype = torch.bfloat16
    if variant == "bf16C_store_wave":
        cfg = dict(flags=EN | pt.PIPE_FLAG_GEMM_STORE_WAVE)
    if variant.startswith("bcol"):
        B = B.t().contiguous().t()       # the same values, stored column-major
    big, C = _guarded_c(M, N, dtype)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    pt.pipe_gemm_mainloop(A, B, C, status=st, **cfg)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    got = C.float().cpu().numpy()
    want = R.round_to_bf16(ref) if dtype == torch.bfloat16 else ref
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{bad.shape[0]} mismatches, first {bad[:4].tolist()}"
    assert bool((big[:, N:] == 7.0).all()) and bool((big[M:, :] == 7.0).all())


def test_ragged_gemm_uniform_within_tolerance():
    """1000 x 1000 x 1000 bf16 uniform[-1,1): every element within 1e-2 of the
    fp64 product, and edge chunks holding NaN outside the operands' M x K and
    K x N windows do not reach C (they are never loaded)."""
    M = N = K = 1000
    Abig = torch.full((M, K + 24), float("nan"), dtype=torch.bfloat16, device=DEV)
    Bbig = torch.full((K + 8, N + 24), float("nan"), dtype=torch.bfloat16, device=DEV)
    A, B = Abig[:, :K], Bbig[:K, :N]
    A.copy_(synth.uniform((M, K), torch.bfloat16, seed=42, stream=0).to(DEV))
    B.copy_(synth.uniform((K, N), torch.bfloat16, seed=42, stream=1).to(DEV))
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    C = pt.pipe_gemm_mainloop(A, B, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    ref = R.gemm_f64(_f32(A.contiguous()), _f32(B.contiguous()))
    res = R.within_tol(C.cpu().numpy(), ref, 1e-2)
    assert res["ok"], res


def test_ragged_gemm_geometry():
    q = pt.pipe_query_kernel(pt.PIPE_OP_GEMM, 1000, 1000, 1000)
    assert (q["items"], q["tiles_per_item"]) == (8 * 8, 16)
    q = pt.pipe_query_kernel(pt.PIPE_OP_GEMM, 200, 136, 72, tile_m=256, consumer_waves=8,
                             producer_waves=4, stages=3)
    assert (q["items"], q["tiles_per_item"]) == (1 * 2, 2)
