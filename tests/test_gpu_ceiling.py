"""The context-only ceiling kernels (ceilings/pipe_ceiling.h) move the bytes
they claim to move: they are timed beside the tile stream, so a kernel that
skipped work would inflate the ceiling."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ceiling():
    import ceilings as c
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


def test_lds_read_b128_folds_the_chunks_it_claims_to_read(ceiling):
    """Chunk i of the LDS array holds (i, 1, 2, 3), so a thread's fold is the
    XOR of the chunk indices it read: computed here from the documented
    address pattern (wave w, lane l, iteration t, instruction j:
    ((8w + j) * 1024 + 16 l + 64 t) mod 65536, 16-byte aligned)."""
    grid, iters = 4, 3
    fold = torch.zeros(grid * 512, dtype=torch.int32, device="cuda")
    clocks = torch.zeros(4 * grid, dtype=torch.int64, device="cuda")
    ceiling.lds(0, None, fold, clocks, grid, iters)
    torch.cuda.synchronize()
    want = []
    for t in range(512):
        w, lane = t // 64, t % 64
        acc = 0
        for it in range(iters):
            for j in range(8):
                acc ^= (((8 * w + j) * 1024 + 16 * lane + 64 * it) & 0xFFF0) // 16
        want.append(acc)
    got = fold.view(grid, 512).cpu()
    assert all(got[g].tolist() == want for g in range(grid))
    c = clocks.view(grid, 4).cpu()
    assert bool((c[:, 0] > 0).all()) and bool((c[:, 2] > 0).all())  # waves 0 and 4 timed their loops


@pytest.mark.parametrize("op", [1, 2, 3, 4, 5, 6])
def test_lds_ceiling_ops_run(ceiling, op):
    grid, iters = 8, 4
    src = torch.zeros(65536 + 1024, dtype=torch.uint8, device="cuda")
    fold = torch.full((grid * 512,), 7, dtype=torch.int32, device="cuda")
    clocks = torch.zeros(4 * grid, dtype=torch.int64, device="cuda")
    ceiling.lds(op, src, fold, clocks, grid, iters)
    torch.cuda.synchronize()
    c = clocks.view(grid, 4).cpu()
    assert bool((c[:, 0] > 0).all()) and bool((c[:, 2] > 0).all())
    if op in (2, 3, 6):
        assert bool((fold == 0).all())  # nothing is read into registers
