"""GPU parity of the 8-bit forward (fa_fwd_fp8) against the fp64 oracle.

Inputs: seeded N(0, 1) draws times 32, encoded as OCP FP8 E4M3 codes
(synthetic.e4m3_round_bits), dequantisation factor 1/32 per tensor.  The
oracle is the exact attention of the decoded, dequantised tensors
(oracle.attention_fp8).  The kernel's products of two e4m3 values are exact
and V widens exactly to bf16, so its error sources are those of the bf16
kernels (fp32 sums, P rounded to bf16, bf16 output), and the bf16 bounds
apply: max |dO| <= 2e-2, max |dL| <= 1e-2.
"""
import math

import numpy as np
import pytest

import oracle
import synthetic

pytestmark = pytest.mark.gpu

TOL_O, TOL_L = 2e-2, 1e-2
DS = synthetic.E4M3_DESCALE


@pytest.fixture(scope="module")
def fa():
    import aware_softmax_amd

    return aware_softmax_amd


def run_case(fa, cid, B, H, Hkv, N, d, causal, scale=None, heads=None, rows=None, descales=(DS, DS, DS)):
    import torch

    scale = 1.0 / math.sqrt(d) if scale is None else scale
    st = {"q": synthetic.full_storage(cid, "q", B, H, N, d, "e4m3"),
          "k": synthetic.full_storage(cid, "k", B, Hkv, N, d, "e4m3"),
          "v": synthetic.full_storage(cid, "v", B, Hkv, N, d, "e4m3")}
    q, k, v = (torch.from_numpy(st[t]).cuda() for t in ("q", "k", "v"))
    o, lse = fa.fwd_fp8(q, k, v, *descales, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16 and o.shape == (B, H, N, d)
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    g = H // Hkv
    err_o = err_l = 0.0
    for b, h in heads:
        ref_o, ref_l = oracle.attention_fp8(st["q"][b, h], st["k"][b, h // g], st["v"][b, h // g], *descales,
                                            causal, scale, rows=rows)
        sel = slice(None) if rows is None else rows
        ob = o[b, h].float().cpu().numpy().astype(np.float64)[sel]
        lb = lse[b, h].cpu().numpy().astype(np.float64)[sel]
        err_o = max(err_o, float(np.max(np.abs(ob - ref_o))))
        err_l = max(err_l, float(np.max(np.abs(lb - ref_l))))
    # O is linear in V: with a V factor other than 1/32 the dequantised V,
    # O and every rounding error of O scale by v_descale / (1/32), and so
    # does the bound (the scores, and so L, depend only on q_descale k_descale).
    tol_o = TOL_O * max(1.0, descales[2] / DS)
    assert err_o <= tol_o, f"max |O - oracle| = {err_o:.3e} > {tol_o:.3e}"
    assert err_l <= TOL_L, f"max |L - oracle| = {err_l:.3e}"


@pytest.mark.parametrize("n", [1, 7, 63, 64, 65, 129, 333, 1000])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_ragged(fa, n, d, causal):
    run_case(fa, 9500 + n * 4 + (d == 128) * 2 + causal, 2, 3, 3, n, d, causal)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_large_grid_single_group(fa, d, causal):
    """B8 H32 N1000: 2048 workgroups (the one-group variant); 4 seeded heads."""
    cid = 9700 + d + causal
    run_case(fa, cid, 8, 32, 32, 1000, d, causal, heads=synthetic.sample_heads(cid, 8, 32, 4))


def test_fp8_throughput_shape_sampled(fa):
    """B8 H32 N8192 d128 causal (the bench's fp8 leg): 3 seeded heads x 256
    seeded rows plus edge rows."""
    rows = synthetic.sample_rows(9800, 8192, 256)
    run_case(fa, 9800, 8, 32, 32, 8192, 128, True, heads=synthetic.sample_heads(9800, 8, 32, 3), rows=rows)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("variant", ["plain", "grouped", "negative_scale", "zero_scale", "descales"])
def test_fp8_two_waves_per_simd(fa, d, causal, variant):
    """B4 H16 N4096 (1024 blocks of 256 rows): the two-waves-per-SIMD
    kernel, persistent, with e4m3 Q.K and V widened to bf16 in LDS; 3
    seeded heads x 256 rows plus edge rows, with grouped key/value heads
    (Hkv 4), scales -0.2 and 0, or distinct factors per tensor."""
    cid = 9760 + causal + 2 * ["plain", "grouped", "negative_scale", "zero_scale", "descales"].index(variant)
    cid += 20 * (d == 64)
    hkv = 4 if variant == "grouped" else 16
    scale = {"negative_scale": -0.2, "zero_scale": 0.0}.get(variant)
    descales = (1 / 16, 1 / 64, 1 / 8) if variant == "descales" else (DS, DS, DS)
    rows = synthetic.sample_rows(cid, 4096, 256)
    run_case(fa, cid, 4, 16, hkv, 4096, d, causal, scale=scale, heads=synthetic.sample_heads(cid, 4, 16, 3),
             rows=rows, descales=descales)


@pytest.mark.parametrize("shape", [(1, 8, 2, 333, 128), (2, 6, 3, 200, 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_grouped_heads(fa, shape, causal):
    B, H, Hkv, N, d = shape
    run_case(fa, 9850 + H + Hkv + causal, B, H, Hkv, N, d, causal)


@pytest.mark.parametrize("scale", [-0.2, 0.0, 0.4])
def test_fp8_other_scales(fa, scale):
    run_case(fa, 9900 + int(scale * 10), 1, 2, 2, 300, 128, True, scale=scale)


def test_fp8_other_descales(fa):
    """Distinct factors per tensor (the codes stay those of the draws times
    32): the Q and K factors join the softmax scale, the V factor the output."""
    run_case(fa, 9950, 1, 2, 2, 257, 128, True, descales=(1 / 16, 1 / 64, 1 / 8))
