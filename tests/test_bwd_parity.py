"""GPU parity of fa_bwd against the fp64 analytic backward of the oracle.

Every case draws seeded Q, K, V, dO from synthetic.py, runs the HIP forward
and backward through the C ABI (aware_softmax_amd.fwd / .bwd -> fa_fwd /
fa_bwd) and compares dQ, dK and dV element by element with
oracle.attention_bwd on the same bf16 values upcast to fp64.

Tolerance (per gradient tensor, over every checked element):
  dQ, dK:  max |got - ref| <= 2e-2 * max(1, max |ref|)
  dV:      max |got - ref| <= 2e-2 * g   (absolute; g = query heads per
           key/value head, 1 without grouping)
  all:     rms(got - ref)  <= 1e-2 * rms(ref) + 1e-4
(the absolute floor covers gradients that are exactly 0, e.g. dQ of a
causal row that sees a single key).  dV = P^T dO involves neither the
scale nor a difference of large terms, so its error does not grow with
the magnitude of the scores; dQ and dK carry the scale and the
cancellation in dP - D, hence the relative form.  With grouped heads dV of
a key/value head is the sum of g per-head gradients, each carrying its own
error, before one final rounding.
Derivation: the kernels round P and dS to bf16 for the MFMAs (relative
2^-9 each), take D_i = dO_i . O_i from the bf16 output O, accumulate in
fp32 and round each gradient to bf16 once (half an ulp: 2^-9 relative).
Replaying exactly those roundings in fp64 NumPy on the B2 H16 N4096 d128
workload gives max-abs errors of 0.007-0.011 against max |ref| of 2-5 and
a relative rms error of 2.4e-3; the bounds leave a 2-4x margin over that
model while a wrong term (a dropped D, a missing scale, a transposed
operand) moves the gradients by O(max |ref|).
float16 rounds P, dS, O and the gradients 4x finer (2^-11 relative), and
its bounds scale down accordingly: max <= 5e-3 * max(1, max |ref|),
rms <= 2.5e-3 * rms(ref) + 1e-4 (dV: 5e-3 * g absolute).
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


TOL = {"bf16": (2e-2, 1e-2), "f16": (5e-3, 2.5e-3)}


def to_device(storage):
    import torch

    storage = np.ascontiguousarray(storage)
    if storage.dtype == np.float16:
        return torch.from_numpy(storage).cuda()
    return torch.from_numpy(storage.view(np.int16)).view(torch.bfloat16).cuda()


def vals(storage):
    return storage.astype(np.float32) if storage.dtype == np.float16 else synthetic.bf16_bits_to_f32(storage)


def assert_grad_close(name, got, ref, dtype="bf16", group=1):
    t_max, t_rms = TOL[dtype]
    max_abs = float(np.abs(got - ref).max())
    if name.startswith("dv"):
        bound = t_max * group
    else:
        bound = t_max * max(1.0, float(np.abs(ref).max()))
    assert max_abs <= bound, f"{name}: max |got - ref| = {max_abs:.3e} > {bound:.3e}"
    rms_err = float(np.sqrt(np.mean((got - ref) ** 2)))
    rms_bound = t_rms * float(np.sqrt(np.mean(ref ** 2))) + 1e-4
    assert rms_err <= rms_bound, f"{name}: rms error {rms_err:.3e} > {rms_bound:.3e}"


def run_bwd(fa, config_id, B, H, N, d, causal, scale=None, heads=None, tensors=None, dtype="bf16"):
    """Runs fwd + bwd on the GPU and checks dQ, dK, dV of the given heads."""
    import torch

    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if tensors is None:
        tensors = {t: synthetic.full_storage(config_id, t, B, H, N, d, dtype) for t in ("q", "k", "v", "do")}
    q, k, v, do = (to_device(tensors[t]) for t in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for b, h in heads:
        v64 = [vals(tensors[t][b, h]) for t in ("q", "k", "v", "do")]
        ref = oracle.attention_bwd(*v64, causal, scale)
        for name, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
            assert_grad_close(f"{name}[{b},{h}]", got[b, h].float().cpu().numpy().astype(np.float64), r, dtype)
    return dq, dk, dv


# ------------------------------------------------------------ the workload


def test_workload5_backward_sampled_heads(fa):
    """B=2, H=16, N=4096, d=128 causal: 4 seeded heads, every row of dQ,
    dK, dV, in the launch configuration the bench times."""
    w = synthetic.WORKLOADS[5]
    heads = synthetic.sample_heads(5, w.B, w.H, 4)
    run_bwd(fa, 5, w.B, w.H, w.N, w.d, w.causal, heads=heads)


def test_raw_fa_bwd_symbol(fa):
    """The C entry points fa_fwd and fa_bwd themselves (not the grouped-head
    entries the Python wrappers use), with device addresses and a
    caller-owned workspace of fa_bwd_workspace_bytes, on a small causal
    problem with a ragged tail; dQ, dK, dV of every head against the
    oracle."""
    import torch

    B, H, N, d = 1, 3, 333, 128
    scale = 1.0 / math.sqrt(d)
    st = {t: synthetic.full_storage(6450, t, B, H, N, d, "bf16") for t in ("q", "k", "v", "do")}
    q, k, v, do = (to_device(st[t]) for t in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(fa.bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    assert fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d, True, scale,
                     fa.DTYPE_BF16, stream) == 0
    status = fa.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                       dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), ws.numel(), B, H, N, d, True, scale,
                       fa.DTYPE_BF16, stream)
    assert status == 0, fa.status_string(status)
    torch.cuda.synchronize()
    for h in range(H):
        ref = oracle.attention_bwd(*(vals(st[t][0, h]) for t in ("q", "k", "v", "do")), True, scale)
        for name, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
            assert_grad_close(f"{name}[{h}]", got[0, h].float().cpu().numpy().astype(np.float64), r)


# ------------------------------------------------------------ shapes and edges


@pytest.mark.parametrize("n", [1, 2, 7, 63, 64, 65, 127, 128, 129, 200, 333, 513])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_bwd(fa, n, d, causal):
    cid = 6000 + n * 4 + (d == 128) * 2 + causal
    run_bwd(fa, cid, 1, 2, n, d, causal)


@pytest.mark.parametrize("n", [1, 7, 63, 65, 129, 333, 513])
@pytest.mark.parametrize("d", [32, 96, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_bwd_head_dims(fa, n, d, causal):
    """d = 32 and 96: LDS rows padded to 64 / 128 elements, the MFMA loops
    over d only.  d = 256: two dK/dV workgroups per key block (one per half
    of the columns) and double-buffered LDS."""
    cid = (20000 if d == 256 else 9000) + n * 4 + (d == 96) * 2 + causal
    run_bwd(fa, cid, 1, 2, n, d, causal)


@pytest.mark.parametrize("d", [32, 96, 256])
def test_bwd_head_dims_long(fa, d):
    """B2 H4 N2048 causal: many query and key tiles per workgroup; 3 seeded
    heads."""
    run_bwd(fa, 9100 + d, 2, 4, 2048, d, True, heads=synthetic.sample_heads(9100 + d, 2, 4, 3))


def test_bwd_d32_large_grid_repeatable(fa):
    """B2 H16 N4096 d32 causal (1024 dQ workgroups, three per CU): 2 seeded
    heads against the oracle, and three runs bitwise equal.  The dQ kernel
    once issued more transposing LDS reads than its d = 32 loop consumed;
    their unused destination registers, still being written by the reads
    in flight, could be handed to live values, which corrupted dQ from run
    to run on this grid only."""
    import torch

    dq, dk, dv = run_bwd(fa, 9150, 2, 16, 4096, 32, True, heads=synthetic.sample_heads(9150, 2, 16, 2))
    st = {t: synthetic.full_storage(9150, t, 2, 16, 4096, 32, "bf16") for t in ("q", "k", "v", "do")}
    q, k, v, do = (to_device(st[t]) for t in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal=True)
    for _ in range(3):
        dq2, dk2, dv2 = fa.bwd(q, k, v, o, lse, do, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(dq2, dq) and torch.equal(dk2, dk) and torch.equal(dv2, dv)


def test_bwd_d256_sampled_heads(fa):
    """B2 H8 N4096 d256 causal: 2 seeded heads, every row of dQ, dK, dV."""
    run_bwd(fa, 9400, 2, 8, 4096, 256, True, heads=synthetic.sample_heads(9400, 2, 8, 2))


@pytest.mark.parametrize("d", [32, 96, 256])
def test_f16_bwd_head_dims(fa, d):
    run_bwd(fa, 9200 + d, 1, 2, 333, d, True, dtype="f16")


@pytest.mark.parametrize("scale", [-0.3, 0.0, 0.35])
def test_other_scales_bwd(fa, scale):
    run_bwd(fa, 6500 + int(scale * 100), 1, 2, 300, 64, True, scale=scale)


def test_noncausal_multi_block(fa):
    run_bwd(fa, 6600, 2, 2, 1000, 128, False)


def test_closed_form_sums(fa):
    """No oracle: every row of P sums to 1, so the dV rows sum to the dO
    rows' sum; the rows of dS sum to 0, so the dK rows sum to 0."""
    import torch

    B, H, N, d = 1, 3, 2048, 128
    st = {t: synthetic.full_storage(6700, t, B, H, N, d, "bf16") for t in ("q", "k", "v", "do")}
    q, k, v, do = (to_device(st[t]) for t in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal=True)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    dov = synthetic.bf16_bits_to_f32(st["do"]).astype(np.float64)
    sum_dv = dv.double().sum(dim=2).cpu().numpy()
    sum_do = dov.sum(axis=2)
    # each of the N bf16 entries carries <= 2^-9 relative rounding
    bound = 2.0 ** -8 * dv.double().abs().sum(dim=2).cpu().numpy() + 1e-3
    assert np.all(np.abs(sum_dv - sum_do) <= bound)
    sum_dk = dk.double().sum(dim=2).cpu().numpy()
    assert np.all(np.abs(sum_dk) <= 2.0 ** -7 * dk.double().abs().sum(dim=2).cpu().numpy() + 1e-3)


def test_deterministic_and_dirty_workspace(fa):
    """No atomics: dQ, dK and dV are bitwise identical across runs, also
    when the workspace starts out full of NaNs (the call overwrites it)."""
    import torch

    B, H, N, d = 2, 2, 777, 128
    st = {t: synthetic.full_storage(6800, t, B, H, N, d, "bf16") for t in ("q", "k", "v", "do")}
    q, k, v, do = (to_device(st[t]) for t in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal=True)
    ws = torch.full((fa.bwd_workspace_bytes(B, H, N, d) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    dq1, dk1, dv1 = fa.bwd(q, k, v, o, lse, do, causal=True, workspace=ws.view(torch.uint8))
    dq2, dk2, dv2 = fa.bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(dk1.view(torch.int16), dk2.view(torch.int16))
    assert torch.equal(dv1.view(torch.int16), dv2.view(torch.int16))
    assert torch.equal(dq1.view(torch.int16), dq2.view(torch.int16))
    assert torch.isfinite(dq1.float()).all()


def test_outputs_untouched_outside_bounds(fa):
    """fa_bwd writes exactly B*H*N rows of dQ, dK and dV."""
    import torch

    B, H, n, d = 1, 2, 129, 64
    st = {t: synthetic.full_storage(6900, t, B, H, n, d, "bf16") for t in ("q", "k", "v", "do")}
    q, k, v, do = (to_device(st[t]) for t in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal=True)
    size = B * H * n * d
    bufs = [torch.full((size + 64,), 7.0, dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    outs = [b[:size].view(B, H, n, d) for b in bufs]
    fa.bwd(q, k, v, o, lse, do, causal=True, dq=outs[0], dk=outs[1], dv=outs[2])
    torch.cuda.synchronize()
    for b in bufs:
        assert torch.all(b[size:] == 7.0)
        assert torch.isfinite(b[:size].float()).all()


# ------------------------------------------------------------ grouped key/value heads


@pytest.mark.parametrize("shape", [(2, 8, 2, 333, 128), (1, 12, 4, 1000, 64), (1, 6, 1, 257, 128),
                                   (1, 8, 2, 2048, 128), (1, 6, 2, 300, 96), (1, 4, 1, 200, 32),
                                   (1, 4, 2, 300, 256)])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_backward(fa, shape, causal):
    """fa_bwd_gqa: dK, dV of a key/value head sum over the query heads of
    its group (oracle.attention_bwd_gqa), dQ per query head."""
    import torch

    B, H, Hkv, N, d = shape
    cid = 6950 + H * 8 + Hkv + (d == 128) + 3 * (d in (32, 96)) + 5 * (d == 256)
    st = {"q": synthetic.full_storage(cid, "q", B, H, N, d, "bf16"),
          "do": synthetic.full_storage(cid, "do", B, H, N, d, "bf16"),
          "k": synthetic.full_storage(cid, "k", B, Hkv, N, d, "bf16"),
          "v": synthetic.full_storage(cid, "v", B, Hkv, N, d, "bf16")}
    q, k, v, do = (to_device(st[t]) for t in ("q", "k", "v", "do"))
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert dk.shape == k.shape and dv.shape == v.shape
    for b in range(B):
        vals = [synthetic.bf16_bits_to_f32(st[t][b]) for t in ("q", "k", "v", "do")]
        ref = oracle.attention_bwd_gqa(*vals, causal, scale)
        for name, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
            for h in range(r.shape[0]):
                assert_grad_close(f"{name}[{b},{h}]", got[b, h].float().cpu().numpy().astype(np.float64), r[h],
                                  group=H // Hkv)


def test_gqa_backward_deterministic(fa):
    import torch

    B, H, Hkv, N, d = 1, 8, 2, 700, 128
    st = {"q": synthetic.full_storage(6990, "q", B, H, N, d, "bf16"),
          "do": synthetic.full_storage(6990, "do", B, H, N, d, "bf16"),
          "k": synthetic.full_storage(6990, "k", B, Hkv, N, d, "bf16"),
          "v": synthetic.full_storage(6990, "v", B, Hkv, N, d, "bf16")}
    q, k, v, do = (to_device(st[t]) for t in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal=True)
    a = fa.bwd(q, k, v, o, lse, do, causal=True)
    b = fa.bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


# ------------------------------------------------------------ float16


@pytest.mark.parametrize("n", [1, 65, 200, 513])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_f16_backward(fa, n, d, causal):
    run_bwd(fa, 8000 + n * 4 + (d == 128) * 2 + causal, 1, 2, n, d, causal, dtype="f16")


def test_f16_backward_workload5_sampled_heads(fa):
    w = synthetic.WORKLOADS[5]
    run_bwd(fa, 8100, w.B, w.H, w.N, w.d, True, heads=synthetic.sample_heads(8100, w.B, w.H, 2), dtype="f16")


# ------------------------------------------------------------ variable length


def varlen_bwd_case(fa, cid, lengths, H, Hkv, d, causal, dtype="bf16"):
    import torch

    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    total = int(cu[-1])
    st = {"q": synthetic.full_storage(cid, "q", 1, H, total, d, dtype)[0],
          "do": synthetic.full_storage(cid, "do", 1, H, total, d, dtype)[0],
          "k": synthetic.full_storage(cid, "k", 1, Hkv, total, d, dtype)[0],
          "v": synthetic.full_storage(cid, "v", 1, Hkv, total, d, dtype)[0]}
    q, k, v, do = (to_device(st[t]) for t in ("q", "k", "v", "do"))
    cu_d = torch.from_numpy(cu).cuda()
    scale = 1.0 / math.sqrt(d)
    mx = int(max(lengths))
    o, lse = fa.fwd_varlen(q, k, v, cu_d, mx, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd_varlen(q, k, v, o, lse, do, cu_d, mx, causal=causal, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.attention_bwd_varlen(*(vals(st[t]) for t in ("q", "k", "v", "do")), cu, causal, scale)
    for b in range(len(lengths)):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        if r1 == r0:
            continue
        for name, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
            for h in range(r.shape[0]):
                assert_grad_close(f"{name}[seq {b}, head {h}]", got[h, r0:r1].float().cpu().numpy().astype(np.float64),
                                  r[h, r0:r1], dtype, group=H // Hkv)


@pytest.mark.parametrize("lengths", [[1], [300], [5, 0, 130, 64, 1, 257], [1000, 17, 513], [64] * 5])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_backward(fa, lengths, d, causal):
    varlen_bwd_case(fa, 8200 + len(lengths) * 8 + (d == 128) * 2 + causal, lengths, 4, 2, d, causal)


@pytest.mark.parametrize("d", [32, 96, 256])
def test_varlen_backward_head_dims(fa, d):
    varlen_bwd_case(fa, 8250 + d, [5, 0, 130, 64, 1, 257], 4, 2, d, True)


def test_varlen_backward_f16(fa):
    varlen_bwd_case(fa, 8300, [700, 3, 1200], 4, 1, 128, True, dtype="f16")


def test_varlen_backward_matches_fixed_length(fa):
    """Equal lengths: packed and batched backward give the same bits."""
    import torch

    B, H, N, d = 2, 4, 384, 128
    st = {t: synthetic.full_storage(8310, t, B, H, N, d, "bf16") for t in ("q", "k", "v", "do")}
    q, k, v, do = (to_device(st[t]) for t in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal=True)
    g = fa.bwd(q, k, v, o, lse, do, causal=True)
    pack = lambda x: x.permute(1, 0, 2, 3).reshape(H, B * N, d).contiguous()
    cu = torch.arange(0, (B + 1) * N, N, dtype=torch.int32, device="cuda")
    lse_p = lse.permute(1, 0, 2).reshape(H, B * N).contiguous()
    g2 = fa.bwd_varlen(pack(q), pack(k), pack(v), pack(o), lse_p, pack(do), cu, N, causal=True)
    torch.cuda.synchronize()
    for a, b in zip(g, g2):
        assert torch.equal(pack(a).view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("shape,causal,dtype", [((1, 8, 2, 700, 128), True, "bf16"),
                                                ((1, 6, 1, 300, 64), True, "bf16"),
                                                ((1, 8, 2, 700, 128), False, "bf16"),
                                                ((1, 8, 2, 513, 128), True, "f16"),
                                                ((1, 6, 1, 300, 64), False, "f16")])
def test_gqa_backward_head_split_matches_unsplit(fa, shape, causal, dtype):
    """The head-split dK/dV pass (workspace of fa_bwd_gqa_workspace_bytes)
    and the one-workgroup-per-key-block pass (fa_bwd_workspace_bytes)
    agree with the oracle and, up to fp32 summation order, with each other;
    each is deterministic.  Causal and not, bf16 and fp16 (the fp16
    instantiation of the partial-sum reduction)."""
    import torch

    B, H, Hkv, N, d = shape
    assert fa.bwd_gqa_workspace_bytes(B, H, Hkv, N, d) > fa.bwd_workspace_bytes(B, H, N, d)
    cid = 6995 + 2 * (not causal) + (dtype == "f16")
    st = {"q": synthetic.full_storage(cid, "q", B, H, N, d, dtype),
          "do": synthetic.full_storage(cid, "do", B, H, N, d, dtype),
          "k": synthetic.full_storage(cid, "k", B, Hkv, N, d, dtype),
          "v": synthetic.full_storage(cid, "v", B, Hkv, N, d, dtype)}
    q, k, v, do = (to_device(st[t]) for t in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal=causal)
    small = torch.empty(fa.bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    big = torch.empty(fa.bwd_gqa_workspace_bytes(B, H, Hkv, N, d), dtype=torch.uint8, device="cuda")
    g_small = fa.bwd(q, k, v, o, lse, do, causal=causal, workspace=small)
    g_big = fa.bwd(q, k, v, o, lse, do, causal=causal, workspace=big)
    g_big2 = fa.bwd(q, k, v, o, lse, do, causal=causal, workspace=big)
    torch.cuda.synchronize()
    vals64 = [vals(st[t][0]) for t in ("q", "k", "v", "do")]
    ref = oracle.attention_bwd_gqa(*vals64, causal, 1.0 / math.sqrt(d))
    for grads in (g_small, g_big):
        for name, got, r in zip(("dq", "dk", "dv"), grads, ref):
            for h in range(r.shape[0]):
                assert_grad_close(f"{name}[{h}]", got[0, h].float().cpu().numpy().astype(np.float64), r[h], dtype,
                                  group=H // Hkv)
    for x, y in zip(g_big, g_big2):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
