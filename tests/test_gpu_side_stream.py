"""Calls on a caller-given side stream, with the outputs and the row sum's
workspace allocated by the Python wrapper: the wrapper marks those tensors as
used by the side stream, so the caching allocator does not hand their memory
to work on the current stream while the kernels still run. Each result is
checked against the oracle after the current stream has reused freed memory."""
import numpy as np
import pytest
import torch

import async_stage_tile_amd as pt
import synth
from oracle import results as R

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _churn():
    # allocate and overwrite memory on the current stream while the side stream runs
    for _ in range(8):
        torch.full((1 << 20,), 7.0, device=DEV).add_(1.0)


def test_rowsum_copy_gemm_on_a_side_stream():
    A = synth.small_int((1024, 8192), -8, 8, torch.float16, seed=21).to(DEV)
    src = synth.unique_codes(512, 768).to(DEV)
    Ga = synth.small_int((256, 512), -2, 2, torch.bfloat16, seed=22, stream=0).to(DEV)
    Gb = synth.small_int((512, 384), -2, 2, torch.bfloat16, seed=22, stream=1).to(DEV)
    side = torch.cuda.Stream(device=DEV)        # default priority
    side.wait_stream(torch.cuda.current_stream())
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    with torch.cuda.stream(torch.cuda.current_stream()):
        rs = pt.pipe_rowsum(A, stream=side, split=4, status=st)
        dst = pt.pipe_tile_copy(src, stream=side, status=st)
        C = pt.pipe_gemm_mainloop(Ga, Gb, stream=side, status=st)
    _churn()
    side.synchronize()
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(rs.cpu().numpy(), R.rowsum_exact(A.cpu().numpy()))
    assert np.array_equal(dst.cpu().numpy().view(np.uint16), src.cpu().numpy().view(np.uint16))
    assert np.array_equal(C.cpu().numpy(), R.gemm_f64(Ga.float().cpu().numpy(),
                                                        Gb.float().cpu().numpy()))
