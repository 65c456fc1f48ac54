"""Race detection by repetition: every kernel family, on grids large enough
to put several workgroups (and both waves of a SIMD) to work at once, gives
bitwise identical outputs over repeated calls.  No kernel uses atomics, so
any difference is a race (an LDS buffer overwritten while still read, a
register reused while a load is in flight).  Inputs are seeded and
synthetic (synthetic.py); the values themselves are checked by the parity
tests."""
import numpy as np
import pytest

import synthetic

pytestmark = pytest.mark.gpu

REPS = 3


@pytest.fixture(scope="module")
def fa():
    import aware_softmax_amd

    return aware_softmax_amd


def dev16(storage):
    import torch

    return torch.from_numpy(np.ascontiguousarray(storage).view(np.int16)).view(torch.bfloat16).cuda()


def same_every_time(call):
    import torch

    ref = [t.clone() for t in call()]
    for _ in range(REPS):
        out = call()
        torch.cuda.synchronize()
        for a, b in zip(out, ref):
            assert torch.equal(a, b)


@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_and_backward_repeat(fa, d, causal):
    """B2 H16 N2048 (B2 H8 at d = 256): forward and backward, bf16."""
    B, H, N = (2, 8, 2048) if d == 256 else (2, 16, 2048)
    cid = 8800 + d + causal
    q, k, v, do = (dev16(synthetic.full_storage(cid, t, B, H, N, d, "bf16")) for t in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal=causal)
    same_every_time(lambda: fa.fwd(q, k, v, causal=causal))
    same_every_time(lambda: fa.bwd(q, k, v, o, lse, do, causal=causal))


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_forward_repeat(fa, d):
    """B4 H16 N4096 e4m3 causal (the persistent two-waves-per-SIMD kernel
    with V widened in LDS)."""
    import torch

    cid = 8900 + d
    q, k, v = (torch.from_numpy(synthetic.full_storage(cid, t, 4, 16, 4096, d, "e4m3")).cuda()
               for t in ("q", "k", "v"))
    ds = synthetic.E4M3_DESCALE
    same_every_time(lambda: fa.fwd_fp8(q, k, v, ds, ds, ds, causal=True))


def test_decode_repeat(fa):
    """Split-K decode B8 H32 N8192 d128 and its combine."""
    import torch

    g = torch.Generator(device="cuda").manual_seed(8950)
    q = torch.randn(8, 32, 128, device="cuda", generator=g).to(torch.bfloat16)
    k = torch.randn(8, 32, 8192, 128, device="cuda", generator=g).to(torch.bfloat16)
    v = torch.randn(8, 32, 8192, 128, device="cuda", generator=g).to(torch.bfloat16)
    same_every_time(lambda: fa.decode(q, k, v))
