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


def test_round_to_bf16_hand_cases():
    """bf16 has 8 significant bits: in [1, 2) the step is 2**-7."""
    s = 2.0 ** -7
    cases = [
        (1.0, 1.0), (-2.5, -2.5), (0.0, 0.0),
        (1.0 + s / 2, 1.0),                 # tie -> even (1.0)
        (1.0 + 3 * s / 2, 1.0 + 2 * s),     # tie -> even (mantissa 2)
        (1.0 + s / 2 + 2.0 ** -30, 1.0 + s),  # just above the tie rounds up
        (1.0 + s / 2 - 2.0 ** -30, 1.0),    # just below rounds down
        (2.0 - 2.0 ** -9, 2.0),             # carry into the exponent
        (-(1.0 + 3 * s / 2), -(1.0 + 2 * s)),
        (255.0, 255.0), (257.0, 256.0), (259.0, 260.0),  # integers above 2**8: step 2
        (16384.0 + 31.0, 16384.0 + 0.0),    # step 128 at 2**14: 16415 -> 16384
        (16384.0 + 64.0, 16384.0),          # tie -> even
        (16384.0 + 192.0, 16384.0 + 256.0),  # tie -> even
        (3 * 2.0 ** -133, 3 * 2.0 ** -133),  # subnormal, exact
        (2.5 * 2.0 ** -133, 2.0 * 2.0 ** -133),  # subnormal tie -> even
        (3.5 * 2.0 ** -133, 4.0 * 2.0 ** -133),
        (2.0 ** -126, 2.0 ** -126),
        (3.5e38, np.inf), (-3.5e38, -np.inf),
    ]
    x = np.array([c[0] for c in cases])
    want = np.array([c[1] for c in cases], dtype=np.float32)
    got = R.round_to_bf16(x)
    assert np.array_equal(got, want), list(zip(x, got, want))
    assert np.isnan(R.round_to_bf16(np.array([np.nan]))[0])
    # the result is always representable: its low 16 fp32 bits are zero
    assert np.all(got.view(np.uint32)[np.isfinite(got)] & 0xFFFF == 0)
    assert R.bf16_bits(np.array([1.0, -2.0], dtype=np.float32)).tolist() == [0x3F80, 0xC000]


def test_round_to_bf16_matches_torch_conversion_of_fp32():
    """For fp32 inputs there is no double rounding: the oracle's rounding of the
    exact value must equal torch's (independent) fp32 -> bf16 conversion."""
    g = torch.Generator().manual_seed(0)
    v = torch.randn(200000, generator=g, dtype=torch.float32) * torch.exp2(
        torch.randint(-40, 40, (200000,), generator=g).float())
    ties = (torch.arange(4096, dtype=torch.int32) << 16) | 0x8000  # exact halfway codes
    v = torch.cat([v, ties.view(torch.float32)[torch.isfinite(ties.view(torch.float32))]])
    ref = v.to(torch.bfloat16).float().numpy()
    got = R.round_to_bf16(v.double().numpy())
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_gemm_bf16_is_rounded_exact_product():
    A = synth.small_int((64, 96), -2, 2, torch.bfloat16, seed=21).float().numpy()
    B = synth.small_int((96, 32), -2, 2, torch.bfloat16, seed=22).float().numpy()
    exact = R.gemm_fraction(A, B)
    got = R.gemm_bf16(A, B)
    for i in range(0, 64, 7):
        for j in range(0, 32, 5):
            e = exact[i][j]
            assert e.denominator == 1
            # integers: exact below 2**8, else the nearest multiple of the step
            v = int(e)
            step = 1 if abs(v) < 256 else 2 ** (abs(v).bit_length() - 8)
            q, r = divmod(abs(v), step)
            if 2 * r > step or (2 * r == step and q % 2 == 1):
                q += 1
            assert got[i, j] == np.float32((1 if v >= 0 else -1) * q * step)
