"""GPU parity of fa_decode (split-K decode) against the fp64 oracle.

Every case draws seeded q [B][H][d] and k, v [B][Hkv][N][d] from
synthetic.py, runs aware_softmax_amd.decode (-> fa_decode through the C
ABI) and compares o and lse of each checked (b, h) with
oracle.naive_attention of that head's single query row against the keys
and values of its key/value head h // (H / Hkv), non-causal (the decoded
token sees the whole cache), on the same bf16 values upcast to fp64.

Tolerance: the bf16 bar of the forward (max |o - ref| <= 2e-2,
max |lse - ref| <= 1e-2) and, because decode keeps P in fp32 and rounds only
o to the output type (relative 2^-9 for bf16, 2^-11 for fp16), a
per-element bound with a 2x margin over that rounding,
|o - ref| <= 2 u |ref| + 1e-4, and |lse - ref| <= 2e-4 max(1, |ref|) (fp32
dot products of length d and fp32 accumulation over N keys).
"""
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


ROUND = {"bf16": 2.0 ** -9, "f16": 2.0 ** -11}


def to_device(x):
    import torch

    x = np.ascontiguousarray(x)
    if x.dtype == np.float16:
        return torch.from_numpy(x).cuda()
    return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()


def vals(x):
    return x.astype(np.float32) if x.dtype == np.float16 else synthetic.bf16_bits_to_f32(x)


def mfma_decode(d, group):
    """Whether fa_decode runs these sizes on its MFMA kernel (P rounded to
    the element type) rather than the VALU kernel (P in fp32)."""
    return d in (64, 128) and group >= 5


def check_heads(st, o, lse, heads, H, Hkv, scale):
    group = H // Hkv
    d = st["q"].shape[-1]
    u = ROUND["f16" if st["q"].dtype == np.float16 else "bf16"]
    # d = 64 or 128 with 5 or more heads per key/value head runs on MFMA and rounds
    # P to the element type (relative error <= u per probability, the row
    # sum taken over the rounded values): o moves by at most
    # u / (1 - u) * max_j |v_j - o| <= 2u max_j |v_j - o| on top of the
    # output rounding.  The VALU kernel keeps P in fp32.
    p_rounded = mfma_decode(d, group)
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    for b, h in heads:
        q = vals(st["q"][b, h])[None, :]
        k = vals(st["k"][b, h // group])
        v = vals(st["v"][b, h // group])
        ref_o, ref_l = oracle.naive_attention(q, k, v, False, scale)
        err_o = np.abs(o[b, h].astype(np.float64) - ref_o[0])
        err_l = abs(float(lse[b, h]) - float(ref_l[0]))
        assert err_o.max() <= 2e-2, f"o[{b},{h}] max err {err_o.max():.3e}"
        assert err_l <= 1e-2, f"lse[{b},{h}] err {err_l:.3e}"
        bound = 2 * u * np.abs(ref_o[0]) + 1e-4
        if p_rounded:
            bound = bound + 2 * u * np.max(np.abs(v.astype(np.float64) - ref_o[0][None, :]), axis=0)
        assert np.all(err_o <= bound), f"o[{b},{h}] exceeds the rounding bound: {np.max(err_o - bound):.3e}"
        l_bound = 2e-4 * max(1.0, abs(float(ref_l[0])))
        if p_rounded:
            l_bound += 2 * u  # the row sum of rounded probabilities: relative error <= u
        assert err_l <= l_bound, f"lse[{b},{h}] err {err_l:.3e}"


def run(fa, cid, B, H, Hkv, N, d, scale=None, num_splits=0, heads=None, st=None, dtype="bf16"):
    import torch

    scale = 1.0 / math.sqrt(d) if scale is None else scale
    st = synthetic.decode_storage(cid, B, H, Hkv, N, d, dtype=dtype) if st is None else st
    q, k, v = (to_device(st[t]) for t in ("q", "k", "v"))
    o, lse = fa.decode(q, k, v, scale=scale, num_splits=num_splits)
    torch.cuda.synchronize()
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    check_heads(st, o, lse, heads, H, Hkv, scale)
    return o, lse


# ------------------------------------------------------------ the workloads


@pytest.mark.parametrize("cid", [6, 7, 8])
@pytest.mark.parametrize("num_splits", [0, 1])
def test_decode_workloads(fa, cid, num_splits):
    """The decode problems at full size, split automatically and unsplit;
    32 seeded heads (all heads for B = 1)."""
    w = synthetic.DECODE_WORKLOADS[cid]
    heads = synthetic.sample_heads(cid, w.B, w.H, 32)
    run(fa, cid, w.B, w.H, w.Hkv, w.N, w.d, num_splits=num_splits, heads=heads)


# ------------------------------------------------------------ shapes and edges


@pytest.mark.parametrize("n", [1, 2, 7, 63, 64, 65, 127, 128, 129, 255, 256, 257, 1000, 4097])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("heads", [(4, 4), (8, 2), (12, 1)])
def test_ragged_decode(fa, n, d, heads):
    H, Hkv = heads
    run(fa, 7000 + n * 8 + (d == 128) * 4 + Hkv, 2, H, Hkv, n, d)


@pytest.mark.parametrize("n", [1, 65, 1000, 4097])
@pytest.mark.parametrize("d", [32, 96, 256])
@pytest.mark.parametrize("heads", [(4, 4), (8, 2), (12, 1)])
def test_head_dims_decode(fa, n, d, heads):
    """The other head dims (lanes per key row 4 or 16, up to 3 chunks per lane)."""
    H, Hkv = heads
    run(fa, 7700 + n * 8 + Hkv + d, 2, H, Hkv, n, d)


@pytest.mark.parametrize("d", [32, 96, 256])
def test_head_dims_decode_long(fa, d):
    run(fa, 7800 + d, 2, 16, 4, 20000, d, heads=synthetic.sample_heads(7800 + d, 2, 16, 8))


@pytest.mark.parametrize("num_splits", [1, 2, 3, 5, 64, 10000])
def test_forced_splits(fa, num_splits):
    run(fa, 7100, 1, 8, 2, 5000, 128, num_splits=num_splits)


@pytest.mark.parametrize("group", [2, 3, 4, 5, 6, 7, 8, 9, 11, 12, 16, 24, 32, 40])
def test_group_sizes(fa, group):
    """Query-head groups of sizes 1..4 (the VALU kernel), 5..40 (the MFMA
    kernel, which serves up to 32 heads of a group per workgroup: 40 runs
    as two workgroups of 20), and 11 (prime)."""
    run(fa, 7200 + group, 2, 2 * group, 2, 777, 128)


@pytest.mark.parametrize("scale", [-0.3, 0.5, 2.0])
def test_other_scales(fa, scale):
    run(fa, 7300 + int(scale * 10), 2, 4, 4, 3000, 128, scale=scale)


def test_scale_zero_is_mean_of_values(fa):
    """No oracle: with scale 0 every weight is 1/N, so o is the mean of the
    value rows and lse = ln N."""
    import torch

    B, H, Hkv, N, d = 1, 4, 2, 2500, 64
    st = synthetic.decode_storage(7400, B, H, Hkv, N, d)
    q, k, v = (to_device(st[t]) for t in ("q", "k", "v"))
    o, lse = fa.decode(q, k, v, scale=0.0)
    torch.cuda.synchronize()
    mean_v = vals(st["v"]).astype(np.float64).mean(axis=2)  # [B][Hkv][d]
    got = o.float().cpu().numpy()
    for h in range(H):
        assert np.all(np.abs(got[0, h] - mean_v[0, h // 2]) <= 2.0 ** -8 * np.abs(mean_v[0, h // 2]) + 1e-4)
    assert np.allclose(lse.cpu().numpy(), math.log(N), atol=1e-5, rtol=0)


def test_deterministic_and_dirty_workspace(fa):
    """No atomics: two calls with the same split agree bitwise, also when
    the workspace starts out full of NaNs."""
    import torch

    B, H, Hkv, N, d = 2, 8, 4, 3333, 128
    st = synthetic.decode_storage(7500, B, H, Hkv, N, d)
    q, k, v = (to_device(st[t]) for t in ("q", "k", "v"))
    need = fa.decode_plan(B, H, Hkv, N, d)[2]
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda")
    o1, l1 = fa.decode(q, k, v, workspace=ws.view(torch.uint8))
    o2, l2 = fa.decode(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
    assert torch.isfinite(o1.float()).all()


def test_outputs_untouched_outside_bounds(fa):
    import torch

    B, H, Hkv, N, d = 1, 4, 4, 300, 64
    st = synthetic.decode_storage(7600, B, H, Hkv, N, d)
    q, k, v = (to_device(st[t]) for t in ("q", "k", "v"))
    size = B * H * d
    ob = torch.full((size + 64,), 7.0, dtype=torch.bfloat16, device="cuda")
    lb = torch.full((B * H + 64,), 7.0, dtype=torch.float32, device="cuda")
    fa.decode(q, k, v, out=ob[:size].view(B, H, d), lse=lb[:B * H].view(B, H))
    torch.cuda.synchronize()
    assert torch.all(ob[size:] == 7.0) and torch.all(lb[B * H:] == 7.0)
    check_heads(st, ob[:size].view(B, H, d), lb[:B * H].view(B, H), [(0, h) for h in range(H)], H, Hkv,
                1.0 / math.sqrt(d))


# ------------------------------------------------------------ float16


@pytest.mark.parametrize("n", [1, 65, 1000, 4097])
@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
@pytest.mark.parametrize("heads", [(4, 4), (8, 2)])
def test_f16_decode(fa, n, d, heads):
    H, Hkv = heads
    run(fa, 7900 + n * 8 + Hkv + d, 2, H, Hkv, n, d, dtype="f16")


def test_f16_decode_long(fa):
    run(fa, 7990, 2, 32, 8, 32768, 128, dtype="f16", heads=synthetic.sample_heads(7990, 2, 32, 8))


@pytest.mark.parametrize("n", [1, 200, 4097])
@pytest.mark.parametrize("num_splits", [0, 1])
@pytest.mark.parametrize("d", [64, 128])
def test_f16_decode_mfma_groups(fa, n, num_splits, d):
    """fp16 through the MFMA decode (8 heads per key/value head)."""
    run(fa, 7995 + n + d, 2, 16, 2, n, d, dtype="f16", num_splits=num_splits)


@pytest.mark.parametrize("group", [5, 8, 16, 32])
@pytest.mark.parametrize("n", [1, 130, 5000])
def test_mfma_decode_d64(fa, group, n):
    """d = 64 through the MFMA decode: groups of 5 to 32 heads, ragged key
    counts (a partial 32-key tile, a partial 128-key stage)."""
    run(fa, 8400 + group * 8 + n % 7, 2, 2 * group, 2, n, 64)


# ------------------------------------------------------------ per-sequence cache lengths


@pytest.mark.parametrize("num_splits", [0, 1, 7])
@pytest.mark.parametrize("d", [64, 128])
def test_cache_seqlens(fa, num_splits, d):
    """Sequence b attends to the first cache_seqlens[b] rows of its cache;
    lengths 0 (o = 0, lse = -inf, the oracle's empty-row reading), 1, the
    full capacity and values in between; splits past a sequence's end."""
    import torch

    B, H, Hkv, N = 6, 8, 2, 3000
    lens = np.array([0, 1, N, 1234, 63, 2049], dtype=np.int32)
    st = synthetic.decode_storage(7998 + d, B, H, Hkv, N, d)
    q, k, v = (to_device(st[t]) for t in ("q", "k", "v"))
    sl = torch.from_numpy(lens).cuda()
    o, lse = fa.decode(q, k, v, num_splits=num_splits, cache_seqlens=sl)
    torch.cuda.synchronize()
    got_o, got_l = o.float().cpu().numpy(), lse.cpu().numpy()
    scale = 1.0 / math.sqrt(d)
    for b in range(B):
        n_b = int(lens[b])
        for h in range(H):
            if n_b == 0:
                assert np.all(got_o[b, h] == 0) and got_l[b, h] == -np.inf
                continue
            ref_o, ref_l = oracle.naive_attention(vals(st["q"][b, h])[None, :], vals(st["k"][b, h // 4][:n_b]),
                                                  vals(st["v"][b, h // 4][:n_b]), False, scale)
            bound = 2.0 ** -8 * np.abs(ref_o[0]) + 1e-4
            l_bound = 2e-4 * max(1.0, abs(ref_l[0]))
            if mfma_decode(d, H // Hkv):  # P rounded (see check_heads)
                vv = vals(st["v"][b, h // 4][:n_b]).astype(np.float64)
                bound = bound + 2.0 ** -8 * np.max(np.abs(vv - ref_o[0][None, :]), axis=0)
                l_bound += 2.0 ** -8
            assert np.all(np.abs(got_o[b, h] - ref_o[0]) <= bound), (b, h)
            assert abs(got_l[b, h] - ref_l[0]) <= l_bound, (b, h)


def test_decode_million_key_cache(fa):
    """A 2^20-row cache (B1 H2 Hkv1 d128, 512 MiB of K and V): many keys per
    split at the automatic plan, the sums and maxima over a long range."""
    run(fa, 7100, 1, 2, 1, 1 << 20, 128)
