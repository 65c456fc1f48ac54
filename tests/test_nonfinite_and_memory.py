"""GPU checks of what the forward does with non-finite inputs, and that the
library allocates no device memory.

Non-finite inputs.  The 16-bit forward kernels are built without NaN
semantics: the row max (v_max_f32) drops a NaN operand, and the d = 128
kernel's steady-tile overflow test "partial row sum > 2^16" is false for
NaN.  A NaN score is therefore neither caught nor hidden: 2^NaN = NaN
enters P, the row sum and the P.V product.  Hidden scores (behind the
causal mask or past the end) are replaced by -inf with a select before any
arithmetic, and 2^(-inf * c) = 0 for the kernels' c > 0, so a NaN score
never reaches a row that does not see its key.  A NaN value row is
different: P.V multiplies every key of a tile, and 0 * NaN = NaN, so it
reaches every row whose wave multiplies the tile holding it, including
rows that do not see it.  Checked below on the bf16 forward for the d = 128
kernel and the generic d = 64 kernel (two wave groups on this grid):
  * NaN anywhere in query row i: O_i and L_i are NaN, every other row is
    bitwise what it is without the NaN;
  * NaN in key row j: every row that sees key j (causal: i >= j; otherwise
    all) has O and L NaN, the other rows are bitwise unchanged;
  * NaN in value row j: O of every row that sees key j is NaN; L of every
    row is bitwise unchanged, and so is O of every row before the 64-key
    tile holding row j (causal; such rows never multiply that tile).
Other heads are never affected.

Memory.  "PidokuInfra 10 -- FlashAttention", section 10 (hands-on
exercise): the fused method needs memory linear in N (the caller's
tensors), never the N x N matrix.  The library takes every buffer from the
caller: free device memory is the same before and after a series of
forward, backward and decode calls through the C entry points.
"""
import math

import numpy as np
import pytest

import synthetic

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import aware_softmax_amd

    return aware_softmax_amd


def to_device(storage):
    import torch

    return torch.from_numpy(np.ascontiguousarray(storage).view(np.int16)).view(torch.bfloat16).cuda()


def run(fa, st, causal):
    import torch

    q, k, v = (to_device(st[t]) for t in ("q", "k", "v"))
    o, lse = fa.fwd(q, k, v, causal=causal)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def same_bits(a, b):
    return np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("d", [32, 64, 96, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("where", ["q", "k", "v"])
def test_nan_reaches_exactly_the_rows_that_see_it(fa, d, causal, where):
    # d = 96 on a grid above the two-group limit (2048 blocks of 128 rows),
    # so that its two-waves-per-SIMD kernel (LDS rows padded to 128) runs;
    # the others on a small grid (two wave groups for d = 32 and 64)
    B, H, N = (8, 32, 1000) if d == 96 else (1, 2, 1000)
    row = 300  # inside the second 256-row block, not on a tile edge
    st = {t: synthetic.full_storage(7700 + d + causal, t, B, H, N, d, "bf16") for t in ("q", "k", "v")}
    o0, l0 = run(fa, st, causal)
    assert np.isfinite(o0).all() and np.isfinite(l0).all()
    bad = {t: st[t].copy() for t in st}
    bad[where][0, 0, row, :] = 0x7FC0  # bf16 quiet NaN
    o1, l1 = run(fa, bad, causal)

    rows = np.arange(N)
    if where == "q":
        hit = rows == row
    else:
        hit = rows >= row if causal else np.ones(N, dtype=bool)
    # head 1 untouched
    assert same_bits(o1[0, 1], o0[0, 1]) and same_bits(l1[0, 1], l0[0, 1])
    # rows that see the NaN
    assert np.isnan(o1[0, 0][hit]).all()
    if where == "v":
        assert same_bits(l1[0, 0], l0[0, 0])
        # O rows that never multiply the value tile holding the NaN row
        clean = rows < (row // 64) * 64 if causal else np.zeros(N, dtype=bool)
        assert same_bits(o1[0, 0][clean], o0[0, 0][clean])
    else:
        assert np.isnan(l1[0, 0][hit]).all()
        assert same_bits(l1[0, 0][~hit], l0[0, 0][~hit])
        assert same_bits(o1[0, 0][~hit], o0[0, 0][~hit])


def test_free_device_memory_unchanged_by_calls(fa):
    """Forward, backward and decode through the raw C entry points, with
    every buffer allocated beforehand: the device's free memory does not
    move (the library allocates nothing)."""
    import torch

    B, H, N, d = 2, 4, 1024, 128
    st = {t: synthetic.full_storage(7800, t, B, H, N, d, "bf16") for t in ("q", "k", "v", "do")}
    q, k, v, do = (to_device(st[t]) for t in ("q", "k", "v", "do"))
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(fa.bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    qd = q[:, :, 0].contiguous()
    od = torch.empty_like(qd)
    ld = torch.empty((B, H), dtype=torch.float32, device="cuda")
    wsd = torch.empty(max(1, fa.decode_plan(B, H, H, N, d)[2]), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    scale = 1.0 / math.sqrt(d)

    def calls():
        assert fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d, True,
                         scale, fa.DTYPE_BF16, stream) == 0
        assert fa.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                         dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), ws.numel(), B, H, N, d, True,
                         scale, fa.DTYPE_BF16, stream) == 0
        assert fa.fa_decode(qd.data_ptr(), k.data_ptr(), v.data_ptr(), None, od.data_ptr(), ld.data_ptr(),
                            wsd.data_ptr(), wsd.numel(), B, H, H, N, d, scale, 0, fa.DTYPE_BF16, stream) == 0

    calls()  # first launches load the code object
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(5):
        calls()
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0, f"free device memory moved by {free0 - free1} bytes"
    assert torch.isfinite(o.float()).all() and torch.isfinite(dq.float()).all() and torch.isfinite(od.float()).all()
