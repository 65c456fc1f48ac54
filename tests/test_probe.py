"""The matrix-core-only ceiling kernel used by the bench (not part of the
attention path): argument checks on the CPU, one small run on the GPU."""
import ctypes

import pytest


@pytest.fixture(scope="module")
def fa():
    import aware_softmax_amd

    return aware_softmax_amd


def test_mfma_ceiling_validation(fa):
    lib = fa.library()
    p = ctypes.c_void_p(0x7F0000000000)
    assert lib.fa_mfma_ceiling(None, 1, 1, 0, None) == 1              # FA_ERR_NULL
    assert lib.fa_mfma_ceiling(p, 0, 1, 0, None) == 2                 # FA_ERR_SHAPE: iters
    assert lib.fa_mfma_ceiling(p, 1, 0, 0, None) == 2                 # FA_ERR_SHAPE: blocks
    assert lib.fa_mfma_ceiling(p, 1, 1 << 24, 0, None) == 2           # blocks * 256 beyond 2^32 - 1
    assert lib.fa_mfma_ceiling(ctypes.c_void_p(0x7F0000000002), 1, 1, 0, None) == 5  # FA_ERR_ALIGN


@pytest.mark.gpu
def test_mfma_ceiling_runs_and_stores_only_when_asked(fa):
    import torch

    blocks = 8
    sink = torch.full((blocks * 256,), 7.0, dtype=torch.float32, device="cuda:0")
    fa.mfma_ceiling(sink, 4, blocks, store=False)
    torch.cuda.synchronize()
    assert bool((sink == 7.0).all())
    fa.mfma_ceiling(sink, 4, blocks, store=True)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(sink).all())
    assert not bool((sink == 7.0).all())
