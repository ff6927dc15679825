"""GPU parity of the ring-fed GEMM mainloop against the fp64 CPU oracle."""
import numpy as np
import pytest
import torch

import async_stage_tile_amd as pt
import synth
from oracle import protocol as P
from oracle import results as R

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _f32(t):
    return t.float().cpu().numpy()


@pytest.mark.parametrize("S", [1, 2, 3, 4])
@pytest.mark.parametrize("PW", [2, 4])
@pytest.mark.parametrize("policy", ["eager", "lazy", "newest"])
def test_gemm_small_integers_bit_exact(S, PW, policy):
    M, N, K = 256, 384, 512
    A = synth.small_int((M, K), -2, 2, torch.bfloat16, seed=3, stream=0).to(DEV)
    B = synth.small_int((K, N), -2, 2, torch.bfloat16, seed=3, stream=1).to(DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    flags = {"eager": 0, "lazy": pt.PIPE_FLAG_LAZY_COMMIT,
             "newest": pt.PIPE_FLAG_EAGER_NEWEST}[policy]
    C = pt.pipe_gemm_mainloop(A, B, stages=S, producer_waves=PW, grid=5, status=st,
                              flags=flags)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    ref = R.gemm_f64(_f32(A), _f32(B))
    got = C.cpu().numpy()
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{bad.shape[0]} mismatches, first {bad[:4].tolist()}"



@pytest.mark.parametrize("S", [3, 4])
@pytest.mark.parametrize("K", [64, 128, 192])
@pytest.mark.parametrize("PW", [2, 4])
@pytest.mark.parametrize("bcol", [False, True])
def test_gemm_deep_rings_short_k_bit_exact(S, K, PW, bcol):
    """Rings of three or more stages on whole tiles with one, two or three K
    steps (the deep consumer's tail alone, then with one and two loop passes).
    Six output tiles on five workgroups, so one workgroup carries the ring's
    cursor from one tile into the next."""
    M, N = 256, 384
    A = synth.small_int((M, K), -2, 2, torch.bfloat16, seed=K + S, stream=0).to(DEV)
    Bt = synth.small_int((N, K), -2, 2, torch.bfloat16, seed=K + S, stream=1).to(DEV)
    B = _colmajor(Bt) if bcol else Bt.t().contiguous()
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    C = pt.pipe_gemm_mainloop(A, B, stages=S, producer_waves=PW, grid=5, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    ref = R.gemm_f64(_f32(A), _f32(Bt).T.copy())
    bad = np.argwhere(C.cpu().numpy() != ref)
    assert bad.size == 0, f"{bad.shape[0]} mismatches, first {bad[:4].tolist()}"

@pytest.mark.parametrize("shift", [0, 1])
@pytest.mark.parametrize("b_linear", [False, True])
def test_gemm_swizzle_variants_bit_exact(shift, b_linear):
    M, N, K = 256, 256, 256
    A = synth.small_int((M, K), -2, 2, torch.bfloat16, seed=4, stream=0).to(DEV)
    B = synth.small_int((K, N), -2, 2, torch.bfloat16, seed=4, stream=1).to(DEV)
    C = pt.pipe_gemm_mainloop(A, B, swizzle_shift=shift,
                              flags=pt.PIPE_FLAG_GEMM_B_LINEAR if b_linear else 0)
    torch.cuda.synchronize()
    assert np.array_equal(C.cpu().numpy(), R.gemm_f64(_f32(A), _f32(B)))


def test_gemm_identity_operands():
    K = 256
    A = torch.eye(K, dtype=torch.bfloat16, device=DEV)
    B = synth.uniform((K, 128), torch.bfloat16, seed=8).to(DEV)
    C = pt.pipe_gemm_mainloop(A, B)
    torch.cuda.synchronize()
    assert torch.equal(C, B.float())
    A2 = synth.uniform((128, K), torch.bfloat16, seed=9).to(DEV)
    C2 = pt.pipe_gemm_mainloop(A2, torch.eye(K, dtype=torch.bfloat16, device=DEV)[:, :128]
                               .contiguous())
    torch.cuda.synchronize()
    assert torch.equal(C2, A2[:, :128].float())


def test_gemm_uniform_within_tolerance():
    M, N, K = 512, 256, 1024
    A = synth.uniform((M, K), torch.bfloat16, seed=42, stream=0).to(DEV)
    B = synth.uniform((K, N), torch.bfloat16, seed=42, stream=1).to(DEV)
    C = pt.pipe_gemm_mainloop(A, B)
    torch.cuda.synchronize()
    res = R.within_tol(C.cpu().numpy(), R.gemm_f64(_f32(A), _f32(B)), 1e-2)
    assert res["ok"], res


def test_gemm_k_zero_gives_zero():
    A = torch.empty((128, 0), dtype=torch.bfloat16, device=DEV)
    B = torch.empty((0, 128), dtype=torch.bfloat16, device=DEV)
    C = torch.full((128, 128), 3.0, device=DEV)
    pt.pipe_gemm_mainloop(A, B, C)
    torch.cuda.synchronize()
    assert int((C != 0).sum()) == 0


# ---------------------------------------------------------------- bf16 C (staged epilogue)
@pytest.mark.parametrize("S", [1, 2, 3, 4])
@pytest.mark.parametrize("PW", [2, 4])
@pytest.mark.parametrize("store_wave", [False, True])
def test_gemm_bf16_out_small_integers_bit_exact(S, PW, store_wave):
    """Integer sums are exact in fp32, so rounding them once to bf16 must give
    exactly the oracle's rounding of the exact product. Entries 0..3 make the
    sums about 500-2000 (at most 4608), well past bf16's 256 exact integers."""
    M, N, K = 256, 384, 512
    A = synth.small_int((M, K), 0, 3, torch.bfloat16, seed=31, stream=0).to(DEV)
    B = synth.small_int((K, N), 0, 3, torch.bfloat16, seed=31, stream=1).to(DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    flags = pt.PIPE_FLAG_EAGER_NEWEST | (pt.PIPE_FLAG_GEMM_STORE_WAVE if store_wave else 0)
    C = pt.pipe_gemm_mainloop(A, B, out_dtype=torch.bfloat16, stages=S, producer_waves=PW, grid=5,
                              flags=flags, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0 and C.dtype == torch.bfloat16
    ref = R.gemm_bf16(_f32(A), _f32(B))
    got = C.float().cpu().numpy()
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{bad.shape[0]} mismatches, first {bad[:4].tolist()}"
    assert np.abs(ref).max() > 256  # rounding was exercised


@pytest.mark.parametrize("store_wave", [False, True])
def test_gemm_bf16_out_uniform_within_tolerance(store_wave):
    M, N, K = 512, 256, 1024
    A = synth.uniform((M, K), torch.bfloat16, seed=42, stream=0).to(DEV)
    B = synth.uniform((K, N), torch.bfloat16, seed=42, stream=1).to(DEV)
    flags = pt.PIPE_FLAG_EAGER_NEWEST | (pt.PIPE_FLAG_GEMM_STORE_WAVE if store_wave else 0)
    C16 = pt.pipe_gemm_mainloop(A, B, out_dtype=torch.bfloat16, flags=flags)
    C32 = pt.pipe_gemm_mainloop(A, B)
    torch.cuda.synchronize()
    res = R.within_tol(C16.float().cpu().numpy(), R.gemm_f64(_f32(A), _f32(B)), 1e-2)
    assert res["ok"], res
    # the two outputs share the accumulation order: bf16 C is the fp32 C rounded once
    assert np.array_equal(C16.float().cpu().numpy(), R.round_to_bf16(C32.cpu().numpy()))


@pytest.mark.parametrize("store_wave", [False, True])
def test_gemm_bf16_out_strided_c_persistent_grid(store_wave):
    M, N, K = 384, 256, 256
    A = synth.small_int((M, K), 0, 3, torch.bfloat16, seed=33, stream=0).to(DEV)
    B = synth.small_int((K, N), 0, 3, torch.bfloat16, seed=33, stream=1).to(DEV)
    base = torch.full((M, N + 64), 7.0, dtype=torch.bfloat16, device=DEV)
    C = base[:, :N]
    flags = pt.PIPE_FLAG_EAGER_NEWEST | (pt.PIPE_FLAG_GEMM_STORE_WAVE if store_wave else 0)
    pt.pipe_gemm_mainloop(A, B, C, grid=2, flags=flags)   # 6 output tiles on 2 workgroups
    torch.cuda.synchronize()
    assert np.array_equal(C.float().cpu().numpy(), R.gemm_bf16(_f32(A), _f32(B)))
    assert bool((base[:, N:] == 7.0).all())


@pytest.mark.parametrize("store_wave", [False, True])
def test_gemm_bf16_out_full_size_sampled_rows(store_wave):
    n = 4096
    A = synth.uniform((n, n), torch.bfloat16, seed=42, stream=0, device=DEV)
    B = synth.uniform((n, n), torch.bfloat16, seed=42, stream=1, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    flags = pt.PIPE_FLAG_EAGER_NEWEST | (pt.PIPE_FLAG_GEMM_STORE_WAVE if store_wave else 0)
    C = pt.pipe_gemm_mainloop(A, B, out_dtype=torch.bfloat16, flags=flags, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    rows = np.random.default_rng(11).choice(n, 48, replace=False)
    rows.sort()
    ref = R.gemm_f64(_f32(A[rows]), _f32(B))
    res = R.within_tol(C[rows].float().cpu().numpy(), ref, 1e-2)
    assert res["ok"], res


def test_gemm_bf16_out_k_zero_gives_zero():
    A = torch.empty((128, 0), dtype=torch.bfloat16, device=DEV)
    B = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    C = torch.full((128, 256), 3.0, dtype=torch.bfloat16, device=DEV)
    pt.pipe_gemm_mainloop(A, B, C)
    torch.cuda.synchronize()
    assert int((C != 0).sum()) == 0


# ---------------------------------------------------------------------------
# Column-major B (PIPE_FLAG_GEMM_B_COLMAJOR, chosen by the binding for a K x N
# view with unit row stride): the same product, B tiles loaded like A's.
# ---------------------------------------------------------------------------
def _colmajor(Bt, pad=0):
    """K x N column-major view of the row-major N x K matrix Bt, optionally with
    `pad` unused elements after each of its rows (ldb = K + pad)."""
    N, K = Bt.shape
    if pad:
        full = torch.zeros((N, K + pad), dtype=Bt.dtype, device=Bt.device)
        full[:, :K] = Bt
        Bt = full[:, :K]
    B = Bt.t()
    assert B.stride(0) == 1 and B.shape == (K, N)
    return B


@pytest.mark.parametrize("S", [1, 2, 3, 4])
@pytest.mark.parametrize("PW", [2, 4])
@pytest.mark.parametrize("policy", ["eager", "newest"])
def test_gemm_b_colmajor_small_integers_bit_exact(S, PW, policy):
    M, N, K = 256, 384, 512
    A = synth.small_int((M, K), -2, 2, torch.bfloat16, seed=13, stream=0).to(DEV)
    Bt = synth.small_int((N, K), -2, 2, torch.bfloat16, seed=13, stream=1).to(DEV)
    B = _colmajor(Bt)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    C = pt.pipe_gemm_mainloop(A, B, stages=S, producer_waves=PW, grid=5, status=st,
                              flags=pt.PIPE_FLAG_EAGER_NEWEST if policy == "newest" else 0)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    ref = R.gemm_f64(_f32(A), _f32(Bt).T.copy())
    got = C.cpu().numpy()
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{bad.shape[0]} mismatches, first {bad[:4].tolist()}"


@pytest.mark.parametrize("shift", [0, 1, 2])
@pytest.mark.parametrize("pad", [0, 64])
@pytest.mark.parametrize("c_dtype", [torch.float32, torch.bfloat16])
def test_gemm_b_colmajor_pitch_swizzle_and_output(shift, pad, c_dtype):
    """Padded B rows (ldb > K), every swizzle shift, fp32 and bf16 C."""
    M, N, K = 256, 256, 384
    A = synth.small_int((M, K), 0, 3, torch.bfloat16, seed=14, stream=0).to(DEV)
    Bt = synth.small_int((N, K), 0, 3, torch.bfloat16, seed=14, stream=1).to(DEV)
    C = pt.pipe_gemm_mainloop(A, _colmajor(Bt, pad), swizzle_shift=shift, out_dtype=c_dtype)
    torch.cuda.synchronize()
    B_np = _f32(Bt).T.copy()
    if c_dtype == torch.bfloat16:
        assert np.array_equal(C.float().cpu().numpy(), R.gemm_bf16(_f32(A), B_np))
    else:
        assert np.array_equal(C.cpu().numpy(), R.gemm_f64(_f32(A), B_np))


def test_gemm_b_colmajor_matches_row_major_bitwise():
    """The two layouts of one B give the same bits (same accumulation order)."""
    M, N, K = 512, 256, 1024
    A = synth.uniform((M, K), torch.bfloat16, seed=15, stream=0).to(DEV)
    B = synth.uniform((K, N), torch.bfloat16, seed=15, stream=1).to(DEV)
    C_row = pt.pipe_gemm_mainloop(A, B)
    C_col = pt.pipe_gemm_mainloop(A, _colmajor(B.t().contiguous()))
    torch.cuda.synchronize()
    assert torch.equal(C_row, C_col)
    res = R.within_tol(C_col.cpu().numpy(), R.gemm_f64(_f32(A), _f32(B)), 1e-2)
    assert res["ok"], res


def test_gemm_b_colmajor_full_size_sampled_rows():
    """bf16 4096^3 uniform[-1,1), B column-major: 64 sampled rows against fp64."""
    n = 4096
    A = synth.uniform((n, n), torch.bfloat16, seed=42, stream=0, device=DEV)
    Bt = synth.uniform((n, n), torch.bfloat16, seed=42, stream=1, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    C = pt.pipe_gemm_mainloop(A, Bt.t(), status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    rows = np.random.default_rng(7).choice(n, 64, replace=False)
    Bt_np = _f32(Bt)
    ref = R.gemm_f64(_f32(A[torch.as_tensor(rows, device=DEV)]), Bt_np.T.copy())
    res = R.within_tol(C[torch.as_tensor(rows, device=DEV)].cpu().numpy(), ref, 1e-2)
    assert res["ok"], res


def test_gemm_b_colmajor_rejections():
    A = torch.zeros((128, 128), dtype=torch.bfloat16, device=DEV)
    Bt = torch.zeros((128, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(pt.PipeError):  # exclusive with the row-major B swizzle switch
        pt.pipe_gemm_mainloop(A, Bt.t(), flags=pt.PIPE_FLAG_GEMM_B_LINEAR)
    over = torch.zeros(128 * 64 + 64, dtype=torch.bfloat16, device=DEV)
    B_overlap = over.as_strided((128, 128), (1, 64))  # columns 64 apart: rows of B^T overlap
    with pytest.raises(ValueError):
        pt.pipe_gemm_mainloop(A, B_overlap)


@pytest.mark.parametrize("M,N,K,grid", [
    (128, 128, 64, 0),       # one tile, one K step
    (128, 128, 64, 1),
    (2048, 128, 256, 3),     # tall: 16 tiles on 3 persistent workgroups
    (128, 2048, 256, 0),     # wide
    (384, 640, 192, 1),      # 15 tiles on one workgroup, 3 K steps
    (256, 256, 16384, 0),    # long K: 256 stages through the ring
])
@pytest.mark.parametrize("c_dtype", [torch.float32, torch.bfloat16])
def test_gemm_shapes_and_grids_bit_exact(M, N, K, grid, c_dtype):
    """Small-integer data: every fp32 partial sum is an integer below 2**24
    (|C| <= 4 K <= 65536), so C is exact in any order and must equal the oracle
    bit for bit (its bf16 rounding too)."""
    A = synth.small_int((M, K), -2, 2, torch.bfloat16, seed=51, stream=0).to(DEV)
    B = synth.small_int((K, N), -2, 2, torch.bfloat16, seed=51, stream=1).to(DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    C = pt.pipe_gemm_mainloop(A, B, grid=grid, status=st, out_dtype=c_dtype)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    ref = R.gemm_f64(_f32(A), _f32(B))
    if c_dtype == torch.bfloat16:
        assert np.array_equal(C.float().cpu().numpy(), R.gemm_bf16(_f32(A), _f32(B)))
    else:
        assert np.array_equal(C.cpu().numpy(), ref)


def test_gemm_long_k_uniform_within_tolerance():
    """256 x 256 x 16384 uniform[-1, 1): fp32 accumulation over 16384 products
    stays within 1e-2 of the fp64 product (relative to max(|ref|, rms(ref)))."""
    A = synth.uniform((256, 16384), torch.bfloat16, seed=52, stream=0).to(DEV)
    B = synth.uniform((16384, 256), torch.bfloat16, seed=52, stream=1).to(DEV)
    C = pt.pipe_gemm_mainloop(A, B)
    torch.cuda.synchronize()
    res = R.within_tol(C.cpu().numpy(), R.gemm_f64(_f32(A), _f32(B)), 1e-2)
    assert res["ok"], res


def test_gemm_strided_row_major_operands():
    """A and B as views into wider buffers (lda = K + 64, ldb = N + 128)."""
    M, N, K = 256, 384, 320
    Abig = synth.small_int((M, K + 64), -2, 2, torch.bfloat16, seed=53, stream=0).to(DEV)
    Bbig = synth.small_int((K, N + 128), -2, 2, torch.bfloat16, seed=53, stream=1).to(DEV)
    A, B = Abig[:, 32:32 + K], Bbig[:, 64:64 + N]
    C = pt.pipe_gemm_mainloop(A, B)
    torch.cuda.synchronize()
    assert np.array_equal(C.cpu().numpy(), R.gemm_f64(_f32(A.contiguous()), _f32(B.contiguous())))


def test_gemm_trace_cursors():
    """Workgroup 0's trace: the producer acquires stage t and MFMA wave 0 passes
    its wait on stage t at the cursor values of the closed form, the wait after
    the acquire, and slot reuse (stage t + S) only after stage t was waited on."""
    S = 3
    A = synth.small_int((256, 512), -2, 2, torch.bfloat16, seed=61, stream=0).to(DEV)
    B = synth.small_int((512, 128), -2, 2, torch.bfloat16, seed=61, stream=1).to(DEV)
    trace = torch.zeros(32 * pt.PIPE_TRACE_WORDS, dtype=torch.int32, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    C = pt.pipe_gemm_mainloop(A, B, stages=S, grid=1, flags=pt.PIPE_FLAG_TRACE |
                              pt.PIPE_FLAG_EAGER_NEWEST, trace=trace, trace_capacity=32,
                              status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(C.cpu().numpy(), R.gemm_f64(_f32(A), _f32(B)))
    tr = trace.cpu().numpy().view(np.uint32).reshape(32, pt.PIPE_TRACE_WORDS)
    prod, cons = tr[0::2], tr[1::2]      # 2 tiles x 8 K steps = 16 stages
    clock = lambda rec: (int(rec[7]) << 32) | int(rec[6])
    for t in range(16):
        assert tuple(prod[t][:2]) == (0, t) and tuple(cons[t][:2]) == (1, t), t
        assert tuple(prod[t][2:5]) == P.cursor_after(S, t, 1) + (t,)
        assert tuple(cons[t][2:5]) == P.cursor_after(S, t, 0) + (t,)
        assert clock(cons[t]) >= clock(prod[t])
        if t + S < 16:
            assert clock(prod[t + S]) >= clock(cons[t])
