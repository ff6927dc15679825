"""GPU parity of the GEMM mainloop with 256 x 128 output tiles (tile_m = 256,
8 MFMA waves, 4 producer waves) against the fp64 CPU oracle.

Each ring stage then holds a 256 x 64 A tile and the 64 x 128 B tile of one
K step; every MFMA wave still owns a 64 x 64 output block and accumulates it
in the same order as with 128-row tiles, so the two tile heights give the same
bits.
"""
import numpy as np
import pytest
import torch

import async_stage_tile_amd as pt
import synth
from oracle import results as R

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TALL = dict(tile_m=256, consumer_waves=8, producer_waves=4)


def _f32(t):
    return t.float().cpu().numpy()


def _colmajor(Bt):
    B = Bt.t()
    assert B.stride(0) == 1
    return B


@pytest.mark.parametrize("S", [1, 2, 3])
@pytest.mark.parametrize("policy", ["eager", "lazy", "newest"])
@pytest.mark.parametrize("b_col", [False, True], ids=["brow", "bcol"])
def test_tall_small_integers_bit_exact(S, policy, b_col):
    """512 x 384 x 512: 6 tiles on 5 persistent workgroups, 8 K steps."""
    M, N, K = 512, 384, 512
    A = synth.small_int((M, K), -2, 2, torch.bfloat16, seed=61, stream=0).to(DEV)
    Bt = synth.small_int((N, K), -2, 2, torch.bfloat16, seed=61, stream=1).to(DEV)
    B = _colmajor(Bt) if b_col else Bt.t().contiguous()
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    flags = {"eager": 0, "lazy": pt.PIPE_FLAG_LAZY_COMMIT,
             "newest": pt.PIPE_FLAG_EAGER_NEWEST}[policy]
    C = pt.pipe_gemm_mainloop(A, B, stages=S, grid=5, status=st, flags=flags, **TALL)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    got = C.cpu().numpy()
    bad = np.argwhere(got != R.gemm_f64(_f32(A), _f32(Bt).T.copy()))
    assert bad.size == 0, f"{bad.shape[0]} mismatches, first {bad[:4].tolist()}"


@pytest.mark.parametrize("S", [1, 2])
@pytest.mark.parametrize("b_col", [False, True], ids=["brow", "bcol"])
def test_tall_bf16_out_small_integers_bit_exact(S, b_col):
    M, N, K = 768, 256, 384
    A = synth.small_int((M, K), -2, 2, torch.bfloat16, seed=62, stream=0).to(DEV)
    Bt = synth.small_int((N, K), -2, 2, torch.bfloat16, seed=62, stream=1).to(DEV)
    B = _colmajor(Bt) if b_col else Bt.t().contiguous()
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    C = pt.pipe_gemm_mainloop(A, B, stages=S, grid=2, status=st, out_dtype=torch.bfloat16,
                              **TALL)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(C.float().cpu().numpy(), R.gemm_bf16(_f32(A), _f32(Bt).T.copy()))


@pytest.mark.parametrize("M,N,K,grid", [
    (256, 128, 64, 0),       # one tile, one K step
    (256, 128, 64, 1),
    (2048, 128, 256, 3),     # tall: 8 tiles on 3 persistent workgroups
    (256, 2048, 256, 0),     # wide
    (768, 640, 192, 1),      # 15 tiles on one workgroup, 3 K steps
    (256, 256, 16384, 0),    # long K: 256 stages through the ring
])
@pytest.mark.parametrize("c_dtype", [torch.float32, torch.bfloat16])
def test_tall_shapes_and_grids_bit_exact(M, N, K, grid, c_dtype):
    """Small-integer data: every partial sum is an integer below 2**24, so C is
    exact in any order and equals the oracle bit for bit."""
    A = synth.small_int((M, K), -2, 2, torch.bfloat16, seed=63, stream=0).to(DEV)
    B = synth.small_int((K, N), -2, 2, torch.bfloat16, seed=63, stream=1).to(DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    C = pt.pipe_gemm_mainloop(A, B, grid=grid, status=st, out_dtype=c_dtype, **TALL)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    if c_dtype == torch.bfloat16:
        assert np.array_equal(C.float().cpu().numpy(), R.gemm_bf16(_f32(A), _f32(B)))
    else:
        assert np.array_equal(C.cpu().numpy(), R.gemm_f64(_f32(A), _f32(B)))


def test_tall_matches_128_row_tiles_bitwise_and_oracle():
    """Uniform data: the same bits as 128-row tiles, and within 1e-2 of fp64."""
    M, N, K = 512, 256, 1024
    A = synth.uniform((M, K), torch.bfloat16, seed=64, stream=0).to(DEV)
    B = synth.uniform((K, N), torch.bfloat16, seed=64, stream=1).to(DEV)
    C128 = pt.pipe_gemm_mainloop(A, B)
    C256 = pt.pipe_gemm_mainloop(A, B, **TALL)
    torch.cuda.synchronize()
    assert torch.equal(C128, C256)
    res = R.within_tol(C256.cpu().numpy(), R.gemm_f64(_f32(A), _f32(B)), 1e-2)
    assert res["ok"], res


def test_tall_strided_operands_and_c():
    """A, B and C as views into wider buffers (lda = K + 64, ldb = N + 128, ldc = N + 32)."""
    M, N, K = 512, 384, 320
    Abig = synth.small_int((M, K + 64), -2, 2, torch.bfloat16, seed=65, stream=0).to(DEV)
    Bbig = synth.small_int((K, N + 128), -2, 2, torch.bfloat16, seed=65, stream=1).to(DEV)
    A, B = Abig[:, 32:32 + K], Bbig[:, 64:64 + N]
    Cbig = torch.full((M, N + 32), 7.0, device=DEV)
    C = Cbig[:, :N]
    pt.pipe_gemm_mainloop(A, B, C, **TALL)
    torch.cuda.synchronize()
    assert np.array_equal(C.cpu().numpy(), R.gemm_f64(_f32(A.contiguous()), _f32(B.contiguous())))
    assert bool((Cbig[:, N:] == 7.0).all())


def test_tall_rejections():
    # (M not a multiple of 256 runs the masked kernel: tests/test_gpu_gemm_ragged.py)
    B = torch.zeros((128, 128), dtype=torch.bfloat16, device=DEV)
    A = torch.zeros((256, 128), dtype=torch.bfloat16, device=DEV)
    for kw in (dict(TALL, consumer_waves=4), dict(TALL, producer_waves=2),
               dict(TALL, stages=4), dict(TALL, stages=3, out_dtype=torch.bfloat16),
               dict(TALL, out_dtype=torch.bfloat16, flags=pt.PIPE_FLAG_GEMM_STORE_WAVE)):
        with pytest.raises(pt.PipeError):
            pt.pipe_gemm_mainloop(A, B, **kw)


@pytest.mark.parametrize("S,c_bf16,b_col", [(1, False, False), (2, False, False),
                                            (3, False, False), (3, False, True),
                                            (2, True, False), (2, True, True)])
def test_tall_kernels_fit_without_spills(S, c_bf16, b_col):
    """The 256-row kernels run 12 waves per workgroup (3 per SIMD), so each
    wave may use up to 168 VGPRs; they must not spill, and their static LDS is
    what pipe_query_kernel reports."""
    flags = (pt.PIPE_FLAG_GEMM_C_BF16 if c_bf16 else 0) | \
            (pt.PIPE_FLAG_GEMM_B_COLMAJOR if b_col else 0)
    cfg = dict(TALL, stages=S, flags=flags | pt.PIPE_FLAG_EAGER_NEWEST)
    r = pt.pipe_kernel_resources(pt.PIPE_OP_GEMM, 512, 256, 256, **cfg)
    q = pt.pipe_query_kernel(pt.PIPE_OP_GEMM, 512, 256, 256, **cfg)
    assert r["scratch_bytes"] == 0, r
    assert r["vgprs"] <= 168, r
    assert r["lds_bytes"] == q["lds_bytes"], (r, q)
    assert r["max_threads"] >= q["threads"] == 768, (r, q)
