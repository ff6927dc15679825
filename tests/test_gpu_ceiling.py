"""The context-only ceiling kernels (include/pipe_ceiling.h) move the bytes
they claim to move: they are timed beside the tile stream, so a kernel that
skipped work would inflate the ceiling."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ceiling():
    from async_stage_tile_amd import ceiling as c
    c.lib()
    return c


def _region(rows=1024, cols=4096, pad=64, seed=3):
    g = torch.Generator(device="cpu").manual_seed(seed)
    full = torch.randint(-32768, 32767, (rows, cols + pad), dtype=torch.int16, generator=g)
    return full.to("cuda")[:, :cols]


@pytest.mark.parametrize("strip_bytes,split", [(128, 1), (128, 2), (256, 2), (512, 4), (512, 1)])
def test_strip_copy_is_exact_and_stays_in_region(ceiling, strip_bytes, split):
    src = _region()
    dst_full = torch.full((src.shape[0], src.stride(0)), 7, dtype=torch.int16, device="cuda")
    dst = dst_full[:, :src.shape[1]]
    ceiling.strip_copy(src, dst, strip_bytes, split)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    assert bool((dst_full[:, src.shape[1]:] == 7).all())  # the pitch padding is untouched


@pytest.mark.parametrize("strip_bytes,split", [(128, 1), (512, 8)])
def test_strip_write_pattern(ceiling, strip_bytes, split):
    rows, cols = 512, 2048  # int32 columns: 8 KiB per row
    full = torch.zeros((rows, cols + 16), dtype=torch.int32, device="cuda")
    dst = full[:, :cols]
    ceiling.strip_write(dst, strip_bytes, split)
    torch.cuda.synchronize()
    r = torch.arange(rows, dtype=torch.int64, device="cuda")[:, None].expand(rows, cols // 4)
    c = (torch.arange(cols // 4, dtype=torch.int64, device="cuda") * 16)[None, :].expand(rows, -1)
    want = torch.stack([r, c, r ^ 0xFFFFFFFF, c ^ 0xFFFFFFFF], dim=-1).reshape(rows, cols)
    want = torch.where(want >= 2**31, want - 2**32, want).to(torch.int32)
    assert torch.equal(dst, want)
    assert bool((full[:, cols:] == 0).all())


def test_strip_read_leaves_sink_alone_on_random_data(ceiling):
    src = _region()
    sink = torch.full((1,), 11, dtype=torch.int32, device="cuda")
    ceiling.strip_read(src, sink, 128, 1)
    torch.cuda.synchronize()
    # The sink is written only when a thread's fold hits one fixed word; on
    # this seeded input no thread's does.
    assert int(sink.item()) == 11
