"""GPU parity of fa_fwd against the fp64 oracle (element by element).

Every case draws seeded inputs from synthetic.py, runs the HIP path through
the C ABI (aware_softmax_amd.fwd -> fa_fwd) and compares O and L with
oracle.naive_attention on the same bf16/fp32 values upcast to fp64.
Tolerances (max-abs over every checked element): fp32 1e-5 on O and L;
bf16 2e-2 on O and 1e-2 on L (fp32 accumulation); fp16 5e-3 on O and
2e-3 on L: P and O are each rounded once to fp16 (relative 2^-11), so O
moves by at most 2^-11 max|v - O| + half an fp16 ulp of |O| < 4
(together < 3e-3) and L by the relative error of the row sum, < 1e-3.
"""
import math

import numpy as np
import pytest

import oracle
import synthetic

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-5), "bf16": (2e-2, 1e-2), "f16": (5e-3, 2e-3)}


@pytest.fixture(scope="module")
def fa():
    import aware_softmax_amd

    return aware_softmax_amd


def to_device(storage, dtype):
    import torch

    if dtype == "bf16":
        return torch.from_numpy(storage.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(storage)).cuda()


def values(storage, dtype):
    if dtype == "bf16":
        return synthetic.bf16_bits_to_f32(storage)
    return storage.astype(np.float32)


def run_case(fa, config_id, B, H, N, d, dtype, causal, scale=None, heads=None, rows=None,
             tensors=None, stats=False):
    """Runs fa.fwd and returns (max |dO|, max |dL|) against the oracle; with
    stats, also max |O_ref| and max |v| over the checked heads."""
    import torch

    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if tensors is None:
        tensors = {t: synthetic.full_storage(config_id, t, B, H, N, d, dtype) for t in ("q", "k", "v")}
    q, k, v = (to_device(tensors[t], dtype) for t in ("q", "k", "v"))
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    err_o = err_l = 0.0
    o_max = v_max = 0.0
    for b, h in heads:
        ob = o[b, h].float().cpu().numpy().astype(np.float64)
        lb = lse[b, h].cpu().numpy().astype(np.float64)
        ref_o, ref_l = oracle.naive_attention(values(tensors["q"][b, h], dtype), values(tensors["k"][b, h], dtype),
                                              values(tensors["v"][b, h], dtype), causal, scale, rows=rows)
        sel = slice(None) if rows is None else rows
        err_o = max(err_o, float(np.max(np.abs(ob[sel] - ref_o))))
        err_l = max(err_l, float(np.max(np.abs(lb[sel] - ref_l))))
        o_max = max(o_max, float(np.max(np.abs(ref_o))))
        v_max = max(v_max, float(np.max(np.abs(values(tensors["v"][b, h], dtype)))))
    return (err_o, err_l, o_max, v_max) if stats else (err_o, err_l)


def assert_close(errs, dtype, scale_factor=1.0):
    """scale_factor widens the fp32 bound for scores larger than the
    workloads' scale = 1/sqrt(d) gives: an fp32 score carries an absolute
    rounding error proportional to |scale| * |q| * |k| ~ |scale| * sqrt(d)
    (times d unit roundoffs), and O moves by at most that error times
    max|v - O|.  At scale = 1/sqrt(d) the factor is 1."""
    to, tl = TOL[dtype]
    if dtype == "f32":
        to, tl = to * scale_factor, tl * scale_factor
    assert errs[0] <= to, f"max |O - oracle| = {errs[0]:.3e} > {to}"
    assert errs[1] <= tl, f"max |L - oracle| = {errs[1]:.3e} > {tl}"


UNIT_ROUNDOFF = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}


def assert_close_sharp(res, dtype):
    """For adversarial score distributions (a few keys carry almost all of
    a row's weight, so |O| approaches max |v|): the kernels round P to the
    element type for the P.V product while l sums the unrounded fp32 P, so
    O carries a relative perturbation of at most u (unit roundoff) of the
    weights, |dO| <= u max|v|, plus the rounding of O itself, u |O|.  The
    bound is max(tolerance, u (max|v| + max|O_ref|) + 1e-3); on the
    workloads' random scores the fixed tolerance is the binding one."""
    err_o, err_l, o_max, v_max = res
    to, tl = TOL[dtype]
    bound_o = max(to, UNIT_ROUNDOFF[dtype] * (v_max + o_max) + 1e-3)
    assert err_o <= bound_o, f"max |O - oracle| = {err_o:.3e} > {bound_o:.3e}"
    assert err_l <= tl, f"max |L - oracle| = {err_l:.3e} > {tl}"


# ------------------------------------------------------------ the five workloads


def test_workload1_fp32_noncausal(fa):
    w = synthetic.WORKLOADS[1]
    assert_close(run_case(fa, 1, w.B, w.H, w.N, w.d, w.dtype, w.causal), w.dtype)


def test_workload2_bf16_causal_d64(fa):
    w = synthetic.WORKLOADS[2]
    assert_close(run_case(fa, 2, w.B, w.H, w.N, w.d, w.dtype, w.causal), w.dtype)


def test_raw_fa_fwd_symbol_workload2(fa):
    """The C entry point fa_fwd itself (not the grouped-head entry the
    Python wrapper uses), called with device addresses on B=1, H=16,
    N=2048, d=64 causal bf16; every row against the oracle."""
    import torch

    w = synthetic.WORKLOADS[2]
    tensors = synthetic.workload_storage(w)
    q, k, v = (to_device(tensors[t], w.dtype) for t in ("q", "k", "v"))
    o = torch.full_like(q, float("nan"))
    lse = torch.full((w.B, w.H, w.N), float("nan"), dtype=torch.float32, device="cuda")
    status = fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), w.B, w.H, w.N, w.d,
                       w.causal, w.scale, fa.DTYPE_BF16, torch.cuda.current_stream().cuda_stream)
    assert status == 0, fa.status_string(status)
    torch.cuda.synchronize()
    err_o = err_l = 0.0
    for h in range(w.H):
        ref_o, ref_l = oracle.naive_attention(*(values(tensors[t][0, h], w.dtype) for t in ("q", "k", "v")),
                                              w.causal, w.scale)
        err_o = max(err_o, float(np.max(np.abs(o[0, h].float().cpu().numpy() - ref_o))))
        err_l = max(err_l, float(np.max(np.abs(lse[0, h].cpu().numpy() - ref_l))))
    assert_close((err_o, err_l), w.dtype)


@pytest.fixture(scope="module")
def workload3_tensors():
    return synthetic.workload_storage(synthetic.WORKLOADS[3])


def test_workload3_sampled(fa, workload3_tensors):
    """B=8, H=32, N=8192, d=128 causal: 4 seeded heads x 512 seeded rows
    (plus edge rows), in the launch configuration the bench times."""
    w = synthetic.WORKLOADS[3]
    heads = synthetic.sample_heads(3, w.B, w.H, 4)
    rows = synthetic.sample_rows(3, w.N, 512)
    assert_close(run_case(fa, 3, w.B, w.H, w.N, w.d, w.dtype, w.causal, heads=heads, rows=rows,
                          tensors=workload3_tensors), w.dtype)


def test_workload3_every_head(fa, workload3_tensors):
    """B=8, H=32, N=8192, d=128 causal: every one of the 256 heads of the
    full launch (the bench's grid and schedule) at 8 seeded rows per head,
    plus rows in the first and the last query block of every head."""
    import torch

    w = synthetic.WORKLOADS[3]
    tensors = workload3_tensors
    q, k, v = (to_device(tensors[t], w.dtype) for t in ("q", "k", "v"))
    o, lse = fa.fwd(q, k, v, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    err_o = err_l = 0.0
    for b in range(w.B):
        for h in range(w.H):
            rng = np.random.Generator(np.random.PCG64([0xFA, 3, 97, b, h]))
            rows = np.unique(np.concatenate([rng.choice(w.N, 8, replace=False),
                                             [0, 255, 256, w.N - 256, w.N - 1]]))
            ref_o, ref_l = oracle.naive_attention(values(tensors["q"][b, h], w.dtype),
                                                  values(tensors["k"][b, h], w.dtype),
                                                  values(tensors["v"][b, h], w.dtype), w.causal, w.scale, rows=rows)
            err_o = max(err_o, float(np.max(np.abs(o[b, h][rows] - ref_o))))
            err_l = max(err_l, float(np.max(np.abs(lse[b, h][rows] - ref_l))))
    assert_close((err_o, err_l), w.dtype)


def test_workload4_long_context_sampled(fa):
    """B=1, H=16, N=32768, d=128 causal: 256 seeded rows of every head."""
    w = synthetic.WORKLOADS[4]
    rows = synthetic.sample_rows(4, w.N, 256)
    assert_close(run_case(fa, 4, w.B, w.H, w.N, w.d, w.dtype, w.causal, rows=rows), w.dtype)


def test_workload5_forward_all_rows(fa):
    w = synthetic.WORKLOADS[5]
    assert_close(run_case(fa, 5, w.B, w.H, w.N, w.d, w.dtype, w.causal), w.dtype)


# ------------------------------------------------------------ shapes and edges


@pytest.mark.parametrize("n", [1, 2, 7, 63, 64, 65, 127, 128, 129, 200, 333, 1000])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_bf16(fa, n, d, causal):
    cid = 1000 + n * 4 + (d == 128) * 2 + causal
    assert_close(run_case(fa, cid, 2, 3, n, d, "bf16", causal), "bf16")


@pytest.mark.parametrize("n", [1, 7, 63, 65, 129, 333, 1000])
@pytest.mark.parametrize("d", [32, 96, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_head_dims_bf16(fa, n, d, causal):
    """The other head dims the pages list as common (96, 256) and d = 32."""
    cid = 1500 + n * 8 + (d // 32) * 2 + causal
    assert_close(run_case(fa, cid, 2, 3, n, d, "bf16", causal), "bf16")


@pytest.mark.parametrize("d", [32, 96, 256])
def test_head_dims_bf16_long(fa, d):
    """B2 H8 N4096 causal: many key tiles per workgroup, sampled rows."""
    rows = synthetic.sample_rows(1600 + d, 4096, 256)
    assert_close(run_case(fa, 1600 + d, 2, 8, 4096, d, "bf16", True, rows=rows,
                          heads=synthetic.sample_heads(1600 + d, 2, 8, 4)), "bf16")


@pytest.mark.parametrize("d", [32, 64, 96])
@pytest.mark.parametrize("causal", [False, True])
def test_large_grid_single_group(fa, d, causal):
    """B8 H32 N1000: 2048 workgroups, more than the grid size up to which
    the d <= 96 kernel splits the key tiles over two wave groups, so the
    one-group variant runs (the smaller cases above take the two-group
    one); 6 seeded heads, ragged last tile."""
    cid = 1700 + d + causal
    heads = synthetic.sample_heads(cid, 8, 32, 6)
    assert_close(run_case(fa, cid, 8, 32, 1000, d, "bf16", causal, heads=heads), "bf16")


@pytest.mark.parametrize("d", [32, 96])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_padded_lds_rows_large_grid_persistent(fa, d, dtype, causal):
    """B4 H16 N4096 at d = 32 and 96: 2048 blocks of 128 rows, above the
    two-group limit, so the two-waves-per-SIMD kernel runs persistent (N a
    multiple of its 256-row block) with LDS rows of 64 and 128 elements
    (rows of 32 and 96 in HBM); 4 seeded heads, sampled rows plus every
    block edge."""
    cid = 1760 + (dtype == "f16") * 2 + causal + (d == 32) * 4
    rows = synthetic.sample_rows(cid, 4096, 384)
    heads = synthetic.sample_heads(cid, 4, 16, 4)
    assert_close(run_case(fa, cid, 4, 16, 4096, d, dtype, causal, heads=heads, rows=rows), dtype)


@pytest.mark.parametrize("n", [1, 5, 64, 100, 257])
@pytest.mark.parametrize("d", [32, 64, 96, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_fp32(fa, n, d, causal):
    cid = 3000 + n * 16 + (d // 32) * 2 + causal
    assert_close(run_case(fa, cid, 1, 2, n, d, "f32", causal), "f32")


@pytest.mark.parametrize("d", [32, 64, 96, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp32_large_grid(fa, d, causal):
    """B2 H16 N1000 fp32 (512 blocks of 64 rows, above the small-grid limit
    of the fp32 kernel, so four lanes per row; the ragged cases above run
    its small-grid form with 8 or 16 lanes per row); 3 seeded heads."""
    cid = 3500 + d + causal
    assert_close(run_case(fa, cid, 2, 16, 1000, d, "f32", causal, heads=synthetic.sample_heads(cid, 2, 16, 3)),
                 "f32")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("scale", [-0.2, 0.9, 3.0])
def test_other_scales(fa, dtype, scale):
    d = 64
    assert_close(run_case(fa, 4000 + int(scale * 10), 1, 2, 300, d, dtype, True, scale=scale), dtype,
                 scale_factor=max(1.0, abs(scale) * math.sqrt(d)))


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 128), ("bf16", 64), ("bf16", 256), ("f16", 64),
                                     ("f16", 128), ("f32", 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_scale_zero_gives_prefix_means(fa, dtype, d, causal):
    """Closed form, no oracle: scale 0 makes O the mean of the visible V
    rows and L = log(#visible)."""
    import torch

    n = 257
    st = {t: synthetic.full_storage(5000, t, 1, 2, n, d, dtype) for t in ("q", "k", "v")}
    q, k, v = (to_device(st[t], dtype) for t in ("q", "k", "v"))
    o, lse = fa.fwd(q, k, v, causal=causal, scale=0.0)
    torch.cuda.synchronize()
    vv = values(st["v"], dtype).astype(np.float64)
    cnt = np.arange(1, n + 1) if causal else np.full(n, n)
    ref = np.cumsum(vv, axis=2) / cnt[None, None, :, None] if causal else np.repeat(
        vv.mean(axis=2, keepdims=True), n, axis=2)
    tol_o = TOL[dtype][0]
    assert np.max(np.abs(o.float().cpu().numpy() - ref)) <= tol_o
    assert np.max(np.abs(lse.cpu().numpy() - np.log(cnt)[None, None, :])) <= 1e-5


def test_v_all_ones(fa):
    """V = 1 gives O = 1 exactly up to the bf16 rounding of P (2^-8)."""
    import torch

    n, d = 1000, 128
    st = {t: synthetic.full_storage(5100, t, 1, 4, n, d, "bf16") for t in ("q", "k")}
    q, k = (to_device(st[t], "bf16") for t in ("q", "k"))
    v = torch.ones_like(q)
    o, _ = fa.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert float((o.float() - 1.0).abs().max()) <= 2.0 ** -8


def test_deterministic_and_stream(fa):
    """No atomics in the forward: two runs are bitwise identical, also on a
    side stream with caller-provided output buffers."""
    import torch

    st = {t: synthetic.full_storage(5200, t, 2, 4, 777, 128, "bf16") for t in ("q", "k", "v")}
    q, k, v = (to_device(st[t], "bf16") for t in ("q", "k", "v"))
    o1, l1 = fa.fwd(q, k, v, causal=True)
    s = torch.cuda.Stream()
    o2 = torch.full_like(o1, float("nan"))
    l2 = torch.full_like(l1, float("nan"))
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fa.fwd(q, k, v, causal=True, out=o2, lse=l2, stream=s)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_outputs_untouched_outside_bounds(fa):
    """The kernel writes exactly B*H*N rows: a sentinel past the end of the
    output buffers survives."""
    import torch

    B, H, n, d = 1, 3, 129, 64
    st = {t: synthetic.full_storage(5300, t, B, H, n, d, "bf16") for t in ("q", "k", "v")}
    q, k, v = (to_device(st[t], "bf16") for t in ("q", "k", "v"))
    obuf = torch.full((B * H * n * d + 64,), 7.0, dtype=torch.bfloat16, device="cuda")
    lbuf = torch.full((B * H * n + 16,), 7.0, dtype=torch.float32, device="cuda")
    o = obuf[: B * H * n * d].view(B, H, n, d)
    lse = lbuf[: B * H * n].view(B, H, n)
    fa.fwd(q, k, v, causal=False, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(obuf[B * H * n * d:] == 7.0) and torch.all(lbuf[B * H * n:] == 7.0)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scale", [2.0, -1.5])
def test_large_scores_d128(fa, causal, scale):
    """Scores that grow far beyond the row max of a row's first key tile
    (scale * sqrt(d) ~ 23: later tiles exceed it by dozens of log2 units),
    so the d = 128 kernel must raise its reference max mid-row many times."""
    d = 128
    assert_close_sharp(run_case(fa, 4100 + int(scale * 10) + causal, 1, 2, 1000, d, "bf16", causal, scale=scale,
                                stats=True), "bf16")


@pytest.mark.parametrize("causal", [False, True])
def test_key_magnitude_ramp_d128(fa, causal):
    """Key j scaled by 1 + j/16: every new key tile has a larger score range
    than all earlier ones (the worst case for a reference max fixed from
    early tiles)."""
    n, d = 1500, 128
    st = {t: synthetic.full_storage(4200 + causal, t, 1, 2, n, d, "bf16") for t in ("q", "k", "v")}
    kv = synthetic.bf16_bits_to_f32(st["k"]) * (1.0 + np.arange(n, dtype=np.float32) / 16.0)[None, None, :, None]
    st["k"] = synthetic.bf16_round_bits(kv)
    assert_close_sharp(run_case(fa, 0, 1, 2, n, d, "bf16", causal, tensors=st, stats=True), "bf16")


# d = 32, 64 and 96 on grids above the two-group split limit (1024
# workgroups of 128 rows) run the two-waves-per-SIMD kernel's one-group
# form with its reference-max steady loop; these cases force it with 144
# heads.


@pytest.mark.parametrize("d", [32, 64, 96])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scale", [2.0, -1.5])
def test_large_scores_large_grid(fa, d, causal, scale):
    """B2 H72 N1024 (1152 workgroups): scores far beyond the first tile's
    row max, so the reference max is raised mid-row; 3 seeded heads."""
    cid = 4300 + int(scale * 10) + causal + (d != 64) * 3 * d
    heads = synthetic.sample_heads(cid, 2, 72, 3)
    assert_close_sharp(run_case(fa, cid, 2, 72, 1024, d, "bf16", causal, scale=scale, heads=heads, stats=True),
                       "bf16")


@pytest.mark.parametrize("d", [32, 64, 96])
@pytest.mark.parametrize("causal", [False, True])
def test_key_magnitude_ramp_large_grid(fa, d, causal):
    """B2 H72 N1024 with key j scaled by 1 + j/16 (every tile exceeds all
    earlier ones); 3 seeded heads."""
    B, H, n = 2, 72, 1024
    cid = 4400 + causal + (d != 64) * 3 * d
    st = {t: synthetic.full_storage(cid, t, B, H, n, d, "bf16") for t in ("q", "k", "v")}
    kv = synthetic.bf16_bits_to_f32(st["k"]) * (1.0 + np.arange(n, dtype=np.float32) / 16.0)[None, None, :, None]
    st["k"] = synthetic.bf16_round_bits(kv)
    heads = synthetic.sample_heads(4400 + causal, B, H, 3)
    assert_close_sharp(run_case(fa, 0, B, H, n, d, "bf16", causal, tensors=st, heads=heads, stats=True), "bf16")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_d64_throughput_shape_sampled(fa, dtype):
    """B8 H32 N8192 d64 causal (the d = 64 throughput shape): 4 seeded
    heads x 256 rows, including the edges of the 256-row query blocks."""
    cid = 4500 + (dtype == "f16")
    rows = synthetic.sample_rows(cid, 8192, 256)
    assert_close(run_case(fa, cid, 8, 32, 8192, 64, dtype, True, rows=rows,
                          heads=synthetic.sample_heads(cid, 8, 32, 4)), dtype)


# Persistent launches: fixed length, N a multiple of 256 and every XCD
# holding whole heads (B * H * N / 256 a multiple of 8 with the per-XCD
# share a multiple of N / 256) run one workgroup per CU over a snake-ordered
# item list, each item's first K/V tiles copied during the previous one.


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scale", [-0.3, 0.2])
def test_persistent_scales_d128(fa, causal, scale):
    """B2 H8 N1024 d128 (64 items, 8 per XCD): negated Q on every item of a
    workgroup (the negation applies to the Q block loaded by the previous
    item); 4 seeded heads."""
    cid = 4600 + int(scale * 10) + causal
    heads = synthetic.sample_heads(cid, 2, 8, 4)
    assert_close(run_case(fa, cid, 2, 8, 1024, 128, "bf16", causal, scale=scale, heads=heads), "bf16")


@pytest.mark.parametrize("causal", [False, True])
def test_persistent_d64(fa, causal):
    """B4 H72 N512 d64 (576 items of 256 rows; above the two-group limit, so
    the persistent one-group launch); 4 seeded heads, every row."""
    cid = 4700 + causal
    heads = synthetic.sample_heads(cid, 4, 72, 4)
    assert_close(run_case(fa, cid, 4, 72, 512, 64, "bf16", causal, heads=heads), "bf16")


# ------------------------------------------------------------ grouped key/value heads


@pytest.mark.parametrize("shape", [(2, 8, 2, 333, 128), (1, 12, 4, 1000, 64), (2, 6, 1, 129, 96),
                                   (2, 4, 2, 65, 256), (1, 16, 2, 4096, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_forward_bf16(fa, shape, causal):
    """fa_fwd_gqa: query head h reads key/value head h // (H // Hkv);
    compared with oracle.attention_gqa on every head (sampled rows at
    N = 4096)."""
    import torch

    B, H, Hkv, N, d = shape
    cid = 1700 + H * 16 + Hkv + d
    st = {"q": synthetic.full_storage(cid, "q", B, H, N, d, "bf16"),
          "k": synthetic.full_storage(cid, "k", B, Hkv, N, d, "bf16"),
          "v": synthetic.full_storage(cid, "v", B, Hkv, N, d, "bf16")}
    q, k, v = (to_device(st[t], "bf16") for t in ("q", "k", "v"))
    o, lse = fa.fwd(q, k, v, causal=causal)
    torch.cuda.synchronize()
    rows = synthetic.sample_rows(cid, N, 256) if N > 2000 else slice(None)
    for b in range(B):
        vals = [values(st[t][b], "bf16") for t in ("q", "k", "v")]
        if N > 2000:
            g = H // Hkv
            ref = [oracle.naive_attention(vals[0][h], vals[1][h // g], vals[2][h // g], causal, 1 / math.sqrt(d),
                                          rows=rows) for h in range(H)]
            ref_o = np.stack([r[0] for r in ref])
            ref_l = np.stack([r[1] for r in ref])
        else:
            ref_o, ref_l = oracle.attention_gqa(*vals, causal, 1 / math.sqrt(d))
        got_o = o[b].float().cpu().numpy()[:, rows]
        got_l = lse[b].cpu().numpy()[:, rows]
        assert_close((float(np.max(np.abs(got_o - ref_o))), float(np.max(np.abs(got_l - ref_l)))), "bf16")


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_forward_fp32(fa, causal):
    import torch

    B, H, Hkv, N, d = 1, 6, 3, 200, 64
    st = {"q": synthetic.full_storage(1750, "q", B, H, N, d, "f32"),
          "k": synthetic.full_storage(1750, "k", B, Hkv, N, d, "f32"),
          "v": synthetic.full_storage(1750, "v", B, Hkv, N, d, "f32")}
    q, k, v = (to_device(st[t], "f32") for t in ("q", "k", "v"))
    o, lse = fa.fwd(q, k, v, causal=causal)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attention_gqa(st["q"][0], st["k"][0], st["v"][0], causal, 1 / math.sqrt(d))
    assert_close((float(np.max(np.abs(o[0].cpu().numpy() - ref_o))),
                  float(np.max(np.abs(lse[0].cpu().numpy() - ref_l)))), "f32")


# ------------------------------------------------------------ float16


@pytest.mark.parametrize("n", [1, 7, 64, 65, 129, 333, 1000])
@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_f16_forward(fa, n, d, causal):
    """The fp16 instantiation of both MFMA kernels (v_mfma_f32_32x32x16_f16)."""
    cid = 1800 + n * 8 + (d // 32) * 2 + causal
    assert_close(run_case(fa, cid, 2, 3, n, d, "f16", causal), "f16")


def test_f16_forward_throughput_shape_sampled(fa):
    """B2 H16 N4096 d128 causal fp16 (the steady max-free loop over many tiles)."""
    rows = synthetic.sample_rows(1900, 4096, 256)
    assert_close(run_case(fa, 1900, 2, 16, 4096, 128, "f16", True, rows=rows,
                          heads=synthetic.sample_heads(1900, 2, 16, 4)), "f16")


@pytest.mark.parametrize("scale", [2.0, -1.5])
def test_f16_large_scores(fa, scale):
    """Scores of |scale| * q.k up to ~30: probabilities above the fp16 range
    must send the tile through the exact update (the overflow check)."""
    assert_close_sharp(run_case(fa, 1910 + int(scale * 10), 1, 2, 1000, 128, "f16", True, scale=scale, stats=True),
                       "f16")


# ------------------------------------------------------------ variable length


def varlen_case(fa, cid, lengths, H, Hkv, d, dtype, causal, scale=None, check_rows=None):
    """Packs seeded sequences of the given lengths ([H][total][d]), runs
    fa_fwd_varlen and compares with oracle.attention_varlen."""
    import torch

    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    total = int(cu[-1])
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    st = {"q": synthetic.full_storage(cid, "q", 1, H, total, d, dtype)[0],
          "k": synthetic.full_storage(cid, "k", 1, Hkv, total, d, dtype)[0],
          "v": synthetic.full_storage(cid, "v", 1, Hkv, total, d, dtype)[0]}
    q, k, v = (to_device(np.ascontiguousarray(st[t]), dtype) for t in ("q", "k", "v"))
    cu_d = torch.from_numpy(cu).cuda()
    o, lse = fa.fwd_varlen(q, k, v, cu_d, int(max(lengths)), causal=causal, scale=scale)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attention_varlen(*(values(st[t], dtype) for t in ("q", "k", "v")), cu, causal, scale)
    got_o, got_l = o.float().cpu().numpy(), lse.cpu().numpy()
    return float(np.max(np.abs(got_o - ref_o))), float(np.max(np.abs(got_l - ref_l)))


@pytest.mark.parametrize("lengths", [[1], [300], [5, 0, 130, 64, 1, 257], [1000, 17, 513], [64] * 7,
                                     [2048, 1, 700]])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_bf16(fa, lengths, d, causal):
    cid = 1950 + len(lengths) * 8 + (d == 128) * 2 + causal
    assert_close(varlen_case(fa, cid, lengths, 4, 2, d, "bf16", causal), "bf16")


@pytest.mark.parametrize("d", [32, 96, 256])
def test_varlen_head_dims(fa, d):
    assert_close(varlen_case(fa, 1980 + d, [77, 300, 0, 129], 2, 2, d, "bf16", True), "bf16")


@pytest.mark.parametrize("d", [32, 96])
def test_varlen_padded_lds_rows_large_grid(fa, d):
    """Packed lengths 2048, 1000, 17, 513 at H24 Hkv8 causal, d = 32 and
    96: 1536 blocks of 128 rows, above the two-group limit, so the
    two-waves-per-SIMD kernel runs one group over packed rows (grouped
    heads too)."""
    assert_close(varlen_case(fa, 1985 + d, [2048, 1000, 17, 513], 24, 8, d, "bf16", True), "bf16")


def test_varlen_f16(fa):
    assert_close(varlen_case(fa, 1990, [400, 33, 1100], 4, 1, 128, "f16", True), "f16")


def test_varlen_matches_fixed_length(fa):
    """Equal lengths: the packed call and the batched call give the same
    bits (same kernel, same tiles; only the addressing differs)."""
    import torch

    B, H, N, d = 3, 4, 320, 128
    st = {t: synthetic.full_storage(1995, t, B, H, N, d, "bf16") for t in ("q", "k", "v")}
    q, k, v = (to_device(st[t], "bf16") for t in ("q", "k", "v"))
    o, lse = fa.fwd(q, k, v, causal=True)
    pack = lambda x: x.permute(1, 0, 2, 3).reshape(H, B * N, d).contiguous()
    cu = torch.arange(0, (B + 1) * N, N, dtype=torch.int32, device="cuda")
    o2, l2 = fa.fwd_varlen(pack(q), pack(k), pack(v), cu, N, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(pack(o).view(torch.int16), o2.view(torch.int16))
    assert torch.equal(lse.permute(1, 0, 2).reshape(H, B * N), l2)


def test_long_sequence_sampled(fa):
    """B1 H2 N131072 d128 causal (twice the longest workload): 64 seeded
    rows plus edge rows, last row included, in each head."""
    rows = synthetic.sample_rows(1990, 131072, 64)
    assert 131071 in set(int(r) for r in rows)
    assert_close(run_case(fa, 1990, 1, 2, 131072, 128, "bf16", True, rows=rows), "bf16")
