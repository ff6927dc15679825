"""Pins of the result oracle against closed forms and brute force (CPU)."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth
from oracle import results as R


def test_copy_index_coded_closed_form():
    M, N = 256, 128
    src = synth.unique_codes(M, N).numpy()
    dst = R.tile_copy(src).view(np.uint16)
    r = np.arange(M)[:, None]
    c = np.arange(N)[None, :]
    assert np.array_equal(dst, ((r * N + c) % 65536).astype(np.uint16))


def test_copy_ragged_edges():
    M, N = 200, 72
    src = synth.unique_codes(M, N).numpy()
    assert np.array_equal(R.tile_copy(src).view(np.uint16), src.view(np.uint16))


def test_tile_grid_covers_once():
    M, N = 300, 136
    cover = np.zeros((M, N), dtype=np.int32)
    for (_, _, r0, r1, c0, c1) in R.tile_grid(M, N):
        cover[r0:r1, c0:c1] += 1
    assert (cover == 1).all()
    assert len(R.tile_grid(M, N)) == 3 * 3


def test_checksum_closed_forms():
    one = np.full((128, 64), 1.0, dtype=np.float16)  # fp16 1.0 = 0x3C00
    assert int(R.tile_checksums(one)[0]) == 8192 * 0x3C00
    # index codes: tile j of a 128x512 matrix, brute force with Python ints
    M, N = 128, 512
    src = synth.unique_codes(M, N).numpy()
    chk = R.tile_checksums(src)
    assert len(chk) == 8
    for j in (0, 5, 7):
        tot = 0
        for r in range(128):
            for c in range(64 * j, 64 * j + 64):
                tot += (r * N + c) % 65536
        assert int(chk[j]) == tot
    # maximum code everywhere: 8192 * 65535 still fits uint32
    big = np.full((128, 64), 0xFFFF, dtype=np.uint16).view(np.float16)
    assert int(R.tile_checksums(big)[0]) == 8192 * 65535


def _f32_round_fraction(q: Fraction) -> np.float32:
    """Reference RNE rounding of an exact rational to fp32 (by bracketing)."""
    if q == 0:
        return np.float32(0)
    a = np.float32(float(q))  # within one ulp; fix up by exact comparisons
    cands = [np.nextafter(a, np.float32(-np.inf)), a, np.nextafter(a, np.float32(np.inf))]
    best = min(cands, key=lambda x: (abs(Fraction(float(x)) - q),
                                     int(np.array(x).view(np.uint32)) & 1))
    return np.float32(best)


def test_int_to_f32_rne_ties_and_edges():
    for v in [0, 1, -1, (1 << 24), (1 << 24) + 1, (1 << 24) + 3, -(1 << 24) - 1,
              (1 << 25) + 2, (1 << 25) + 6, (1 << 55) + (1 << 31), 123456789123]:
        assert R.int_to_f32_rne(v) == _f32_round_fraction(Fraction(v)), v
    # 2**24+1 is a tie between 2**24 and 2**24+2: ties to even -> 2**24
    assert R.int_to_f32_rne((1 << 24) + 1) == np.float32(1 << 24)
    assert R.int_to_f32_rne((1 << 24) + 3) == np.float32((1 << 24) + 4)


def test_rowsum_special_cases():
    ones = np.ones((4, 65536), dtype=np.float16)
    assert np.array_equal(R.rowsum_exact(ones), np.full(4, 65536.0, np.float32))
    alt = np.tile(np.array([0.3, -0.3], dtype=np.float16), (3, 512))
    assert np.array_equal(R.rowsum_exact(alt), np.zeros(3, np.float32))
    # smallest subnormal, many times: exact
    tiny = np.full((1, 1000), np.float16(2.0 ** -24))
    assert R.rowsum_exact(tiny)[0] == np.float32(1000 * 2.0 ** -24)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_rowsum_brute_force(seed):
    A = synth.normal((6, 257), torch.float16, seed=seed).numpy()
    A[0, :] *= np.float16(1000)  # wide dynamic range
    got = R.rowsum_exact(A)
    ref = R.rowsum_fraction(A)
    for i in range(A.shape[0]):
        assert got[i] == _f32_round_fraction(ref[i])


def test_rowsum_small_int_any_order_exact():
    A = synth.small_int((8, 4096), -8, 8, torch.float16, seed=9).numpy()
    got = R.rowsum_exact(A)
    np.testing.assert_array_equal(got, A.astype(np.int64).sum(axis=1).astype(np.float32))


def test_gemm_identity_and_brute_force():
    rng = np.random.default_rng(0)
    M, K, N = 5, 7, 3
    A = R.bf16_bits_to_f32(synth.uniform((M, K), torch.bfloat16, seed=4).view(torch.int16).numpy())
    B = R.bf16_bits_to_f32(synth.uniform((K, N), torch.bfloat16, seed=4, stream=1)
                           .view(torch.int16).numpy())
    got = R.gemm_f64(A, B)
    ref = R.gemm_fraction(A, B)
    for i in range(M):
        for j in range(N):
            assert abs(Fraction(got[i, j]) - ref[i][j]) <= Fraction(1, 1 << 45)
    eye = np.eye(K, dtype=np.float32)
    np.testing.assert_array_equal(R.gemm_f64(eye, B), B.astype(np.float64))
    eye_m = np.eye(M, dtype=np.float32)
    np.testing.assert_array_equal(R.gemm_f64(eye_m, A), A.astype(np.float64))
    assert got.shape == (M, N)
    del rng


def test_bf16_widening():
    x = torch.tensor([1.0, -2.5, 3.140625, 0.0], dtype=torch.bfloat16)
    np.testing.assert_array_equal(R.bf16_bits_to_f32(x.view(torch.int16).numpy()),
                                  x.float().numpy())


def test_within_tol():
    ref = np.array([100.0, -50.0, 0.001, 0.0])
    ok = R.within_tol(ref + np.array([0.05, -0.02, 0.03, 0.03]), ref, 1e-3)
    assert ok["ok"]  # rms ~ 55.9 => 0.0559 allowed near zero
    bad = R.within_tol(ref + np.array([0.2, 0.0, 0.0, 0.0]), ref, 1e-3)
    assert not bad["ok"] and bad["n_bad"] == 1
    nan = R.within_tol(np.array([np.nan, 0, 0, 0]), ref, 1e-3)
    assert not nan["ok"]
