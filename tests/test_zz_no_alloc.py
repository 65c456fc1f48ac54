"""fa_decode_static, the decode entry point that allocates nothing (its
split partials live in a static device array of the library), against
fa_decode with a caller workspace: bitwise equal outputs, on two calls in a
row with the second smaller than the first (the static array keeps the
first call's partials, which the second must not read), with and without
per-sequence cache lengths, bf16 and fp16; plus the oracle at the decode
tolerances for the first call."""
import math

import numpy as np
import pytest

import oracle
import synthetic

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import aware_softmax_amd

    return aware_softmax_amd


def to_device(storage):
    import torch

    storage = np.ascontiguousarray(storage)
    if storage.dtype == np.float16:
        return torch.from_numpy(storage).cuda()
    return torch.from_numpy(storage.view(np.int16)).view(torch.bfloat16).cuda()


def vals(storage):
    return storage.astype(np.float64) if storage.dtype == np.float16 else synthetic.bf16_bits_to_f32(storage)


def run_pair(fa, cid, B, H, Hkv, N, d, dtype, num_splits=0, seqlens=None):
    """(static o, static lse, workspace o, workspace lse, storage) of one
    problem, both through the raw C entry points."""
    import torch

    st = synthetic.decode_storage(cid, B, H, Hkv, N, d, dtype=dtype)
    q, k, v = (to_device(st[t]) for t in ("q", "k", "v"))
    scale = 1.0 / math.sqrt(d)
    code = fa.DTYPE_BF16 if dtype == "bf16" else fa.DTYPE_F16
    stream = torch.cuda.current_stream().cuda_stream
    sl = None if seqlens is None else torch.tensor(seqlens, dtype=torch.int32, device="cuda")
    sl_ptr = None if sl is None else sl.data_ptr()
    o_s = torch.full_like(q, float("nan"))
    l_s = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
    status = fa.fa_decode_static(q.data_ptr(), k.data_ptr(), v.data_ptr(), sl_ptr, o_s.data_ptr(), l_s.data_ptr(),
                                 B, H, Hkv, N, d, scale, num_splits, code, stream)
    assert status == 0, fa.status_string(status)
    o_w = torch.full_like(q, float("nan"))
    l_w = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, fa.decode_workspace_bytes(B, H, Hkv, N, d, num_splits)), dtype=torch.uint8,
                     device="cuda")
    status = fa.fa_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), sl_ptr, o_w.data_ptr(), l_w.data_ptr(),
                          ws.data_ptr(), ws.numel(), B, H, Hkv, N, d, scale, num_splits, code, stream)
    assert status == 0, fa.status_string(status)
    torch.cuda.synchronize()
    return o_s, l_s, o_w, l_w, st


def assert_same(o_s, l_s, o_w, l_w):
    import torch

    assert torch.equal(o_s.view(torch.int16), o_w.view(torch.int16))
    assert torch.equal(l_s.view(torch.int32), l_w.view(torch.int32))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_static_scratch_matches_workspace_two_calls(fa, dtype):
    # first call: many heads and splits (fills much of the scratch)
    B, H, Hkv, N, d = 4, 16, 4, 5000, 128
    o_s, l_s, o_w, l_w, st = run_pair(fa, 7600, B, H, Hkv, N, d, dtype)
    assert_same(o_s, l_s, o_w, l_w)
    scale = 1.0 / math.sqrt(d)
    tol_o, tol_l = (2e-2, 1e-2) if dtype == "bf16" else (5e-3, 2e-3)
    for b in range(B):
        for h in range(H):
            hk = h // (H // Hkv)
            ref_o, ref_l = oracle.naive_attention(vals(st["q"][b, h][None]), vals(st["k"][b, hk]),
                                                  vals(st["v"][b, hk]), False, scale)
            assert np.max(np.abs(o_s[b, h].float().cpu().numpy() - ref_o[0])) <= tol_o
            assert abs(float(l_s[b, h]) - ref_l[0]) <= tol_l
    # second call, smaller: fewer heads, keys and splits, other head dim
    o_s, l_s, o_w, l_w, _ = run_pair(fa, 7601, 2, 4, 4, 777, 64, dtype)
    assert_same(o_s, l_s, o_w, l_w)


def test_static_scratch_forced_splits_and_cache_lengths(fa):
    # forced split count, then a smaller call with per-sequence cache lengths
    o_s, l_s, o_w, l_w, _ = run_pair(fa, 7602, 3, 32, 8, 4096, 128, "bf16", num_splits=7)
    assert_same(o_s, l_s, o_w, l_w)
    o_s, l_s, o_w, l_w, _ = run_pair(fa, 7603, 3, 8, 8, 1000, 128, "bf16", seqlens=[1000, 0, 321])
    assert_same(o_s, l_s, o_w, l_w)
    assert float(l_s[1, 0]) == -math.inf


def test_static_scratch_rejects_too_large(fa):
    """Too large for the static array: FA_ERR_SCRATCH, nothing launched."""
    import torch

    B, H, N, d = 64, 64, 32768, 256
    assert fa.decode_workspace_bytes(B, H, H, N, d, 8) > fa.DECODE_STATIC_SCRATCH_BYTES
    q = torch.zeros(B, H, d, dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, 3.0)
    lse = torch.full((B, H), 3.0, dtype=torch.float32, device="cuda")
    # k, v: a small real buffer standing in for the cache, never read (the
    # size check rejects the call on the host, before any launch)
    k = torch.zeros(1024, dtype=torch.bfloat16, device="cuda")
    status = fa.fa_decode_static(q.data_ptr(), k.data_ptr(), k.data_ptr(), None, o.data_ptr(), lse.data_ptr(), B, H,
                                 H, N, d, 0.1, 8, fa.DTYPE_BF16, torch.cuda.current_stream().cuda_stream)
    assert status == 10
    torch.cuda.synchronize()
    assert torch.all(o == 3.0) and torch.all(lse == 3.0)
