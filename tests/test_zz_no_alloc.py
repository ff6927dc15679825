"""pipe_rowsum_noalloc (the row sum with the library's own workspace buffer)
against pipe_rowsum on the same inputs: the same kernels, so bit-identical
outputs; on small-integer data both equal the exact row sums of the oracle.
Two calls in a row, the second on a smaller matrix, so the second finds the
first's contents in the shared buffer."""
import numpy as np
import pytest
import torch

import async_stage_tile_amd as pt
import synth
from oracle import results as R

DEV = "cuda:0"


def _both(A, **cfg):
    M = A.shape[0]
    ref = torch.full((M,), float("nan"), device=DEV)
    got = torch.full((M,), float("nan"), device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    pt.pipe_rowsum(A, out=ref, status=st, **cfg)
    pt.pipe_rowsum_noalloc(A, got, status=st, **cfg)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    return ref.cpu().numpy(), got.cpu().numpy()


@pytest.mark.gpu
@pytest.mark.parametrize("cfg", [{}, {"split": 8}, {"stages": 4, "split": 2},
                                 {"flags": pt.PIPE_FLAG_UNIFIED | pt.PIPE_FLAG_NONTEMPORAL,
                                  "stages": 2, "consumer_waves": 2}])
def test_noalloc_rowsum_equals_rowsum_two_calls(cfg):
    print(f"[no_alloc] cfg={cfg}", flush=True)
    # first call: 8192 x 16384 normal data (workspace of split x 8192 partials)
    A1 = synth.normal((8192, 16384), torch.float16, seed=11).to(DEV)
    ref1, got1 = _both(A1, **cfg)
    assert np.array_equal(ref1.view(np.uint32), got1.view(np.uint32))
    # second call, smaller: small integers, so both must equal the exact sums
    M2, N2 = (1024, 4096) if cfg.get("flags", 0) & pt.PIPE_FLAG_UNIFIED else (1000, 3000)
    A2 = synth.small_int((M2, N2), -8, 8, torch.float16, seed=12).to(DEV)
    ref2, got2 = _both(A2, **cfg)
    assert np.array_equal(ref2.view(np.uint32), got2.view(np.uint32))
    assert np.array_equal(got2, R.rowsum_exact(A2.cpu().numpy()))


@pytest.mark.gpu
def test_noalloc_rowsum_full_size_and_rejects_oversized():
    print("[no_alloc] 8192 x 65536 default config", flush=True)
    A = synth.small_int((8192, 65536), -8, 8, torch.float16, seed=13).to(DEV)
    ref, got = _both(A)
    assert np.array_equal(ref.view(np.uint32), got.view(np.uint32))
    assert np.array_equal(got, R.rowsum_exact(A.cpu().numpy()))
    # split 8 over 65536 rows needs 2 MiB of partials: more than the buffer
    big = torch.empty((65536, 4096), dtype=torch.float16, device=DEV)
    out = torch.empty(65536, device=DEV)
    with pytest.raises(pt.PipeError) as e:
        pt.pipe_rowsum_noalloc(big, out, split=8)
    assert e.value.status == pt.PIPE_ERR_WORKSPACE
