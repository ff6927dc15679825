"""GPU parity of the unified GEMM (PIPE_FLAG_UNIFIED: 256 x 256 output tiles,
16 waves that all load a share of each stage and all compute) against the fp64
CPU oracle: small-integer operands bit for bit (|C| <= 4 K < 2**24 is exact in
fp32 in any order), uniform[-1, 1) operands within the GEMM tolerance."""
import numpy as np
import pytest
import torch

import async_stage_tile_amd as pt
import synth
from oracle import results as R

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
U = dict(tile_m=256, tile_n=256, consumer_waves=16, stages=2, flags=pt.PIPE_FLAG_UNIFIED)


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


@pytest.mark.parametrize("shape", [(256, 256, 64), (512, 768, 320), (1000, 1000, 1000),
                                   (300, 264, 72), (1, 8, 8), (257, 520, 136)])
@pytest.mark.parametrize("bcol", [False, True])
def test_unified_gemm_small_integers_bit_exact(shape, bcol):
    M, N, K = shape
    print(f"[unified] {shape} bcol={bcol}", flush=True)
    A, B, ref = _operands(M, N, K, seed=M + N + K, bcol=bcol)
    bad = np.argwhere(_run(A, B, **U).cpu().numpy() != ref)
    assert bad.size == 0, f"{bad.shape[0]} mismatches, first {bad[:4].tolist()}"


@pytest.mark.parametrize("grid", [1, 3, 5])
def test_unified_gemm_persistent_grid(grid):
    """Twelve tiles on fewer workgroups: each workgroup fetches its next tile's
    first stage during the last K step of the current one."""
    A, B, ref = _operands(1024, 768, 384, seed=grid, bcol=False)
    assert pt.pipe_query_kernel(pt.PIPE_OP_GEMM, 1024, 768, 384, **U)["items"] == 12
    C = _run(A, B, grid=grid, **U)
    assert np.array_equal(C.cpu().numpy(), ref)


@pytest.mark.parametrize("b_linear", [False, True])
def test_unified_gemm_uniform_within_tolerance(b_linear):
    flags = pt.PIPE_FLAG_UNIFIED | (pt.PIPE_FLAG_GEMM_B_LINEAR if b_linear else 0)
    A, B, ref = _operands(1024, 768, 512, seed=7, bcol=False, kind="uniform")
    res = R.within_tol(_run(A, B, **dict(U, flags=flags)).cpu().numpy(), ref, 1e-2)
    assert res["ok"], res


def test_unified_gemm_matches_the_specialised_ring_bitwise():
    """Each output element is one wave's MFMA chain over K in the same order as
    in the 256 x 128 specialised ring: the two give the same bits."""
    A, B, _ = _operands(1000, 1000, 1000, seed=11, bcol=False, kind="uniform")
    T = dict(tile_m=256, consumer_waves=8, producer_waves=4, stages=3,
             flags=pt.PIPE_FLAG_EAGER_NEWEST)
    assert torch.equal(_run(A, B, **U), _run(A, B, **T))


def test_unified_gemm_4096_small_integers_bit_exact():
    print("[unified] 4096^3 small integers", flush=True)
    A, B, ref = _operands(4096, 4096, 4096, seed=5, bcol=False)
    bad = np.argwhere(_run(A, B, **U).cpu().numpy() != ref)
    assert bad.size == 0, f"{bad.shape[0]} mismatches, first {bad[:4].tolist()}"
