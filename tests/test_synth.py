"""Input generator checks (CPU): published test vector, cross-implementation
bit equality, value ranges and exactness of the generated codes."""
import numpy as np
import torch

import synth
from tests.conftest import golden_lines


def _np_mix(z):
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        return z ^ (z >> np.uint64(31))


def test_splitmix64_published_vector():
    vals = [int(x) for x in golden_lines("splitmix64_vector.txt")]
    assert synth.splitmix64_sequence(vals[0], 5) == vals[1:]


def test_torch_int64_matches_uint64_numpy():
    key = synth.stream_key(42, 3) & ((1 << 64) - 1)
    n = 200_000
    t = synth.raw64(n, 42, 3).numpy().view(np.uint64)
    with np.errstate(over="ignore"):
        idx = np.arange(1, n + 1, dtype=np.uint64)
        ref = _np_mix(idx * np.uint64(synth.GOLDEN) + np.uint64(key))
    assert np.array_equal(t, ref)
    # counter-based: any window equals the matching slice of the full stream
    w = synth.raw64(1000, 42, 3, start=5000).numpy().view(np.uint64)
    assert np.array_equal(w, ref[5000:6000])


def test_uniform_range_and_exactness():
    u32 = synth.uniform((4096,), torch.float32, seed=7)
    assert float(u32.min()) >= -1.0 and float(u32.max()) < 1.0
    # 2u-1 with u on a 2**-24 grid: v * 2**23 is an integer
    v = u32.double() * 2.0 ** 23
    assert torch.equal(v, torch.round(v))
    h = synth.uniform((4096,), torch.float16, seed=7)
    assert torch.equal(h, u32.half())  # RNE of the same fp32 value
    b = synth.uniform((4096,), torch.bfloat16, seed=7)
    assert torch.equal(b, u32.bfloat16())
    assert abs(float(u32.mean())) < 0.05


def test_normal_moments():
    x = synth.normal((1 << 16,), torch.float16, seed=42).float()
    assert abs(float(x.mean())) < 0.02
    assert abs(float(x.var()) - 1.0) < 0.03
    assert torch.isfinite(x).all()


def test_streams_differ_and_seed_reproducible():
    a = synth.uniform((1024,), torch.float32, seed=42, stream=0)
    b = synth.uniform((1024,), torch.float32, seed=42, stream=1)
    c = synth.uniform((1024,), torch.float32, seed=42, stream=0)
    assert not torch.equal(a, b)
    assert torch.equal(a, c)


def test_index_and_unique_codes():
    x = synth.index_coded(256, 128)
    r, c = 37, 101
    assert float(x[r, c]) == (r * 128 + c) % 2048
    u = synth.unique_codes(256, 128).view(torch.int16).numpy().view(np.uint16)
    assert len(np.unique(u)) == 256 * 128
    assert int(u[200, 3]) == (200 * 128 + 3) % 65536


def test_small_int_range():
    x = synth.small_int((10000,), -8, 8, torch.float16, seed=1)
    assert float(x.min()) == -8 and float(x.max()) == 8
    assert torch.equal(x, torch.round(x))
