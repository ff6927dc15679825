"""Operands larger than 4 GiB: every byte offset in the kernels is 64-bit.

A 32-bit offset anywhere in address arithmetic would wrap at 4 GiB and move,
sum or multiply the wrong elements past that point. Each case puts a whole
region of its operand beyond the 4 GiB mark, ends in a ragged tile where the
shape allows, and checks rows on both sides of the mark against the oracle:
- copy, fp16 36 901 x 65 536 (4.84 GB each way, the library's default ring):
  the whole output against its input on the device (the oracle's tile copy is
  the identity), and 48 sampled rows against ``tile_copy`` on the host;
- row sum, fp16 32 845 x 65 536 (4.30 GB) of integers in [-8, 8]: 48 sampled
  rows bit for bit against ``rowsum_exact`` (integer partial sums below 2**24
  are exact in any order);
- GEMM, bf16 A of 65 664 x 32 768 (4.30 GB) times 32 768 x 256 (whole tiles)
  and of 65 601 x 32 776 times 32 776 x 200 (the masked kernel), integers in
  [-2, 2]: 48 sampled rows of C bit for bit against ``gemm_f64``
  (|C| <= 4 K < 2**24); the same A through the 4-wave unified GEMM on 32-K
  stages;
- that unified GEMM with a row-major B of 32 768 x 65 664 (4.30 GB), where
  each K step's offset into B grows past 4 GiB: 48 sampled columns of C.
"""
import numpy as np
import pytest
import torch

import async_stage_tile_amd as pt
import synth
from oracle import results as R

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
FOUR_GIB = 1 << 32


def _rows_across(M, row_bytes, seed, n=48):
    """Sample rows: the first and last, the rows around the 4 GiB offset, and random ones."""
    edge = FOUR_GIB // row_bytes
    fixed = {0, 1, edge - 1, edge, edge + 1, M - 2, M - 1}
    rng = np.random.default_rng(seed)
    rest = rng.choice(M, n - len(fixed), replace=False)
    rows = np.array(sorted(fixed | set(int(r) for r in rest)))
    assert rows.max() < M and (rows.max() + 1) * row_bytes > FOUR_GIB
    return rows


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_copy_beyond_4gib_bit_exact():
    M, N = 36901, 65536
    assert M * N * 2 > FOUR_GIB and M % 128
    print(f"[large] copy {M}x{N}", flush=True)
    src = synth.uniform((M, N), torch.float16, seed=91, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    dst = pt.pipe_tile_copy(src, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert torch.equal(dst.view(torch.int16), src.view(torch.int16))
    rows = torch.as_tensor(_rows_across(M, N * 2, seed=1), device=DEV)
    got = dst.index_select(0, rows).cpu().numpy()
    want = R.tile_copy(src.index_select(0, rows).cpu().numpy())
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))
    del src, dst
    _free()


def test_rowsum_beyond_4gib_sampled_rows_bit_exact():
    M, N = 32845, 65536
    assert M * N * 2 > FOUR_GIB and M % 128
    print(f"[large] rowsum {M}x{N}", flush=True)
    A = synth.small_int((M, N), -8, 8, torch.float16, seed=92, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = pt.pipe_rowsum(A, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    rows = _rows_across(M, N * 2, seed=2)
    got = out.cpu().numpy()[rows]
    want = R.rowsum_exact(A.index_select(0, torch.as_tensor(rows, device=DEV)).cpu().numpy())
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    del A, out
    _free()


DEEP = dict(tile_m=256, tile_n=256, tile_k=32, consumer_waves=4, stages=4,
            flags=pt.PIPE_FLAG_UNIFIED)


@pytest.mark.parametrize("M,N,K,cfg", [(65664, 256, 32768, {}), (65601, 200, 32776, {}),
                                       (65664, 256, 32768, DEEP)],
                         ids=["whole_tiles", "masked", "unified_deep"])
def test_gemm_a_beyond_4gib_sampled_rows_bit_exact(M, N, K, cfg):
    assert M * K * 2 > FOUR_GIB
    print(f"[large] gemm {M}x{N}x{K} {cfg}", flush=True)
    A = synth.small_int((M, K), -2, 2, torch.bfloat16, seed=93, stream=0, device=DEV)
    B = synth.small_int((K, N), -2, 2, torch.bfloat16, seed=93, stream=1, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    C = pt.pipe_gemm_mainloop(A, B, status=st, **cfg)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    rows = _rows_across(M, K * 2, seed=3)
    a = A.index_select(0, torch.as_tensor(rows, device=DEV)).float().cpu().numpy()
    want = R.gemm_f64(a, B.float().cpu().numpy())
    got = C.cpu().numpy()[rows]
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{bad.shape[0]} mismatches, first {bad[:4].tolist()}"
    del A, B, C
    _free()


def test_unified_gemm_b_beyond_4gib_sampled_columns_bit_exact():
    M, N, K = 256, 65664, 32768
    assert K * N * 2 > FOUR_GIB
    print(f"[large] unified gemm, B {K}x{N}", flush=True)
    A = synth.small_int((M, K), -2, 2, torch.bfloat16, seed=94, stream=0, device=DEV)
    B = synth.small_int((K, N), -2, 2, torch.bfloat16, seed=94, stream=1, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    C = pt.pipe_gemm_mainloop(A, B, status=st, **DEEP)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    rng = np.random.default_rng(4)
    cols = np.array(sorted({0, 1, N - 2, N - 1} | set(int(c) for c in rng.choice(N, 44, replace=False))))
    idx = torch.as_tensor(cols, device=DEV)
    want = R.gemm_f64(A.float().cpu().numpy(), B.index_select(1, idx).float().cpu().numpy())
    got = C.index_select(1, idx).cpu().numpy()
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{bad.shape[0]} mismatches, first {bad[:4].tolist()}"
    del A, B, C
    _free()
