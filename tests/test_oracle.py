"""Pins for the fp64 oracle (CPU only).

Each pin checks the oracle against something other than itself: a closed
form, an invariant of softmax attention, a library routine (torch's fp64 CPU
attention and autograd, scipy's logsumexp), brute force on tiny inputs, the
page's own tiled-versus-naive experiment, or finite differences.  The
mutation tests at the end plant plausible mistakes in copies of the naive
oracle and check that at least one pin catches each of them.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from synthetic import random_values

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(seed, shape):
    return random_values(seed, shape).astype(np.float64)


def qkv(seed, n, d, n_k=None):
    n_k = n if n_k is None else n_k
    return rnd(seed, (n, d)), rnd(seed + 1, (n_k, d)), rnd(seed + 2, (n_k, d))


# ---------------------------------------------------------------- pins
# Each pin takes an attention callable with the signature of
# oracle.naive_attention and raises AssertionError when it is violated.


def pin_rows_sum_to_one(attn):
    for causal in (False, True):
        q, k, v = qkv(10, 33, 8)
        _, _, p = attn(q, k, v, causal, 0.7, return_p=True)
        assert np.all(p >= 0)
        assert np.max(np.abs(p.sum(axis=1) - 1.0)) < 1e-14


def pin_scale_zero_means(attn):
    """scale = 0 makes every visible score equal: O is the mean of the
    visible V rows and L = log(#visible)."""
    n, d = 17, 5
    q, k, v = qkv(20, n, d)
    o, lse = attn(q, k, v, False, 0.0)
    assert np.max(np.abs(o - v.mean(axis=0)[None, :])) < 1e-14
    assert np.max(np.abs(lse - math.log(n))) < 1e-14
    o, lse = attn(q, k, v, True, 0.0)
    prefix_mean = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    assert np.max(np.abs(o - prefix_mean)) < 1e-14
    assert np.max(np.abs(lse - np.log(np.arange(1, n + 1)))) < 1e-14


def pin_shift_invariance(attn):
    """Adding c_i to every score of row i leaves O unchanged and shifts L by
    c_i.  Realised by appending a column c_i / scale to Q and 1 to K."""
    n, d, scale = 23, 6, 0.4
    q, k, v = qkv(30, n, d)
    c = rnd(33, (n,)) * 3.0
    q2 = np.concatenate([q, (c / scale)[:, None]], axis=1)
    k2 = np.concatenate([k, np.ones((n, 1))], axis=1)
    for causal in (False, True):
        o1, l1 = attn(q, k, v, causal, scale)
        o2, l2 = attn(q2, k2, v, causal, scale)
        assert np.max(np.abs(o1 - o2)) < 1e-12
        assert np.max(np.abs((l1 + c) - l2)) < 1e-12


def pin_causal_first_row(attn):
    """Causal query 0 sees only key 0: O_0 = V_0 and L_0 = scale q_0 . k_0."""
    q, k, v = qkv(40, 9, 4)
    o, lse = attn(q, k, v, True, 0.3)
    assert np.max(np.abs(o[0] - v[0])) < 1e-15
    assert abs(lse[0] - 0.3 * float(q[0] @ k[0])) < 1e-14


def pin_single_key(attn):
    q, k, v = qkv(50, 1, 7)
    for causal in (False, True):
        o, lse = attn(q, k, v, causal, 1.3)
        assert np.max(np.abs(o - v)) < 1e-15
        assert abs(lse[0] - 1.3 * float(q[0] @ k[0])) < 1e-14


def pin_hardmax_limit(attn):
    """With a huge scale and a unique largest score, softmax becomes one-hot
    on the argmax: O_i = V_argmax, L_i = scale * max_j s_ij."""
    n, d = 12, 4
    q, k, v = qkv(60, n, d)
    scale = 1e4
    o, lse = attn(q, k, v, False, scale)
    s = q @ k.T
    am = np.argmax(s, axis=1)
    assert np.max(np.abs(o - v[am])) < 1e-9
    assert np.max(np.abs(lse - scale * s.max(axis=1))) < 1e-6


def pin_permutation(attn):
    """Non-causal: permuting the key/value rows together leaves O, L
    unchanged; permuting query rows permutes O and L."""
    n, d = 19, 5
    q, k, v = qkv(70, n, d)
    o, lse = attn(q, k, v, False, 0.5)
    perm = np.random.default_rng(3).permutation(n)
    o2, l2 = attn(q, k[perm], v[perm], False, 0.5)
    assert np.max(np.abs(o - o2)) < 1e-13 and np.max(np.abs(lse - l2)) < 1e-13
    o3, l3 = attn(q[perm], k, v, False, 0.5)
    assert np.max(np.abs(o[perm] - o3)) < 1e-13 and np.max(np.abs(lse[perm] - l3)) < 1e-13


def pin_lse_consistency(attn):
    """exp(S_ij - L_i) = P_ij, with S the scaled masked scores."""
    q, k, v = qkv(80, 15, 3)
    for causal in (False, True):
        _, lse, p = attn(q, k, v, causal, 0.9, return_p=True)
        s = 0.9 * (q @ k.T)
        if causal:
            s = np.where(np.triu(np.ones_like(s, dtype=bool), 1), -np.inf, s)
        assert np.max(np.abs(np.exp(s - lse[:, None]) - p)) < 1e-14
        assert np.max(np.abs(lse - scipy.special.logsumexp(s, axis=1))) < 1e-13


def pin_torch_sdpa(attn):
    """Library cross-check: torch's math attention in fp64 on the CPU."""
    for n, n_k, d, causal, scale in [(31, 31, 16, False, 0.25), (40, 40, 8, True, 0.35), (7, 29, 3, False, 1.1)]:
        q, k, v = qkv(90 + n, n, d, n_k)
        o, lse = attn(q, k, v, causal, scale)
        tq, tk, tv = (torch.from_numpy(x)[None] for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)[0].numpy()
        assert np.max(np.abs(o - ref)) < 1e-13
        s = scale * (tq[0] @ tk[0].T)
        if causal:
            s = s.masked_fill(torch.triu(torch.ones_like(s, dtype=torch.bool), 1), -math.inf)
        assert np.max(np.abs(lse - torch.logsumexp(s, dim=1).numpy())) < 1e-13


def pin_brute_force(attn):
    """Scalar loops with math.exp on a tiny problem, no arrays."""
    n, d, scale = 5, 3, 0.8
    q, k, v = qkv(100, n, d)
    for causal in (False, True):
        o, lse = attn(q, k, v, causal, scale)
        for i in range(n):
            keys = range(i + 1) if causal else range(n)
            w = {j: math.exp(scale * sum(q[i][c] * k[j][c] for c in range(d))) for j in keys}
            z = sum(w.values())
            for c in range(d):
                assert abs(o[i][c] - sum(w[j] * v[j][c] for j in keys) / z) < 1e-14
            assert abs(lse[i] - math.log(z)) < 1e-14


PINS = [
    pin_rows_sum_to_one,
    pin_scale_zero_means,
    pin_shift_invariance,
    pin_causal_first_row,
    pin_single_key,
    pin_hardmax_limit,
    pin_permutation,
    pin_lse_consistency,
    pin_torch_sdpa,
    pin_brute_force,
]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_naive_oracle_pins(pin):
    pin(oracle.naive_attention)


def test_scores_brute_force_and_row_selection():
    """oracle.scores against scalar loops: S_ij = scale * sum_c q_ic k_jc,
    -inf exactly where a causal key index exceeds the query index, and a
    row selection returns those rows of the full matrix (also for more keys
    than queries, where causal rows still see keys 0..i)."""
    for n, n_k in ((6, 6), (4, 7)):
        q, k, _ = qkv(110 + n_k, n, 3, n_k)
        for causal in (False, True):
            s = oracle.scores(q, k, causal, 0.6)
            assert s.shape == (n, n_k)
            for i in range(n):
                for j in range(n_k):
                    if causal and j > i:
                        assert s[i, j] == -math.inf
                    else:
                        assert abs(s[i, j] - 0.6 * sum(q[i][c] * k[j][c] for c in range(3))) < 1e-14
            rows = np.array([3, 0, 2])
            assert np.array_equal(oracle.scores(q, k, causal, 0.6, rows=rows), s[rows])


def test_every_oracle_function_has_a_pin():
    """Every function the oracle exports is called by a test in this file
    (no oracle function is left unpinned)."""
    import inspect

    text = open(__file__).read()
    exported = [name for name, obj in vars(oracle).items()
                if inspect.isfunction(obj) and not name.startswith("_")]
    assert len(exported) >= 13
    for name in exported:
        assert f"oracle.{name}(" in text, f"oracle.{name} is not exercised by a pin"


def test_attention_from_scores_shift():
    """The score-level entry point: S + c_i per row leaves P, O unchanged."""
    s = rnd(110, (6, 9)) * 2
    v = rnd(111, (9, 4))
    c = rnd(112, (6,))
    o1, l1, p1 = oracle.attention_from_scores(s, v, return_p=True)
    o2, l2, p2 = oracle.attention_from_scores(s + c[:, None], v, return_p=True)
    assert np.max(np.abs(p1 - p2)) < 1e-15
    assert np.max(np.abs(o1 - o2)) < 1e-14
    assert np.max(np.abs(l1 + c - l2)) < 1e-14
    assert np.max(np.abs(p1 - scipy.special.softmax(s, axis=1))) < 1e-15


def test_fully_masked_row_reading():
    s = np.array([[-np.inf, -np.inf], [0.0, 1.0]])
    o, lse = oracle.attention_from_scores(s, np.ones((2, 3)))
    assert np.all(o[0] == 0) and lse[0] == -np.inf
    assert np.allclose(o[1], 1.0)


# ---------------------------------------------------------------- tiled


@pytest.mark.parametrize("n", [1, 7, 64, 257])
@pytest.mark.parametrize("d", [1, 8, 64])
@pytest.mark.parametrize("blocks", [(1, 1), (7, 5), (64, 64), (128, 32)])
@pytest.mark.parametrize("causal", [False, True])
def test_tiled_matches_naive(n, d, blocks, causal):
    q, k, v = qkv(200 + n + d, n, d)
    scale = 1.0 / math.sqrt(d)
    o1, l1 = oracle.naive_attention(q, k, v, causal, scale)
    o2, l2 = oracle.tiled_attention(q, k, v, causal, scale, *blocks)
    assert np.max(np.abs(o1 - o2)) <= 1e-12
    assert np.max(np.abs(l1 - l2)) <= 1e-12


def test_tiled_page_experiment():
    """The page's check: blocked versus textbook at 2048x64, blocks 128,
    causal, scale 1/sqrt(d), prints a max-abs difference of about 1e-15."""
    with open(os.path.join(GOLDEN, "page_tiled_vs_naive.json")) as f:
        g = json.load(f)
    n, d = g["N"], g["d"]
    q, k, v = qkv(300, n, d)
    scale = 1.0 / math.sqrt(d)
    o1, _ = oracle.naive_attention(q, k, v, g["causal"], scale)
    o2, _ = oracle.tiled_attention(q, k, v, g["causal"], scale, g["block_q"], g["block_k"])
    diff = float(np.max(np.abs(o1 - o2)))
    # same order of magnitude as the printed value (rounding-order noise only)
    assert diff < 100 * g["printed_max_abs_diff"]


def test_tiled_hardmax_and_large_scores():
    """Scores far beyond exp's range: the running max keeps every exp finite."""
    q, k, v = qkv(310, 50, 4)
    o1, l1 = oracle.naive_attention(q, k, v, True, 300.0)
    o2, l2 = oracle.tiled_attention(q, k, v, True, 300.0, 8, 3)
    assert np.all(np.isfinite(o2)) and np.max(np.abs(o1 - o2)) < 1e-12
    assert np.max(np.abs(l1 - l2)) / np.max(np.abs(l1)) < 1e-13


# ---------------------------------------------------------------- split-K merge


@pytest.mark.parametrize("causal", [False, True])
def test_split_partials_combine(causal):
    n, d = 37, 6
    q, k, v = qkv(400, n, d)
    o_ref, l_ref = oracle.naive_attention(q, k, v, causal, 0.45)
    for bounds in ([(0, n)], [(0, 10), (10, 11), (11, n)], [(j, min(j + 4, n)) for j in range(0, n, 4)]):
        m, l, o = oracle.split_kv_partials(q, k, v, causal, 0.45, bounds)
        o2, l2 = oracle.combine_partials(m, l, o)
        assert np.max(np.abs(o2 - o_ref)) < 1e-13
        assert np.max(np.abs(l2 - l_ref)) < 1e-13


def test_combine_two_halves_by_hand():
    """Two partials with maxima 0 and 2: weights exp(-2) and 1."""
    m = np.array([[0.0], [2.0]])
    l = np.array([[3.0], [1.5]])
    o = np.array([[[3.0]], [[6.0]]])
    out, lse = oracle.combine_partials(m, l, o)
    w0 = math.exp(-2.0)
    assert abs(out[0, 0] - (w0 * 3.0 + 6.0) / (w0 * 3.0 + 1.5)) < 1e-15
    assert abs(lse[0] - (2.0 + math.log(w0 * 3.0 + 1.5))) < 1e-15


# ---------------------------------------------------------------- backward


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_finite_differences(causal):
    """Central differences of f = <O, dO> at N=16, d=8 (fp64, step 1e-6)."""
    n, d = 16, 8
    q, k, v = qkv(500, n, d)
    do = rnd(504, (n, d))
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, causal, scale)

    def f(qq, kk, vv):
        o, _ = oracle.naive_attention(qq, kk, vv, causal, scale)
        return float(np.sum(o * do))

    h = 1e-6
    for grad, which in ((dq, 0), (dk, 1), (dv, 2)):
        num = np.zeros_like(grad)
        for i in range(n):
            for c in range(d):
                args = [q.copy(), k.copy(), v.copy()]
                args[which][i, c] += h
                fp = f(*args)
                args[which][i, c] -= 2 * h
                fm = f(*args)
                num[i, c] = (fp - fm) / (2 * h)
        assert np.max(np.abs(num - grad)) < 1e-7


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_torch_autograd(causal):
    n, d = 24, 8
    q, k, v = qkv(510, n, d)
    do = rnd(514, (n, d))
    scale = 0.3
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, causal, scale)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None], is_causal=causal, scale=scale)[0]
    out.backward(torch.from_numpy(do))
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.max(np.abs(mine - ref.numpy())) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_invariants(causal):
    """sum_j dV_j = sum_i dO_i (P rows sum to 1) and sum_j dK_j = 0
    (rows of dS sum to 0)."""
    n, d = 21, 5
    q, k, v = qkv(520, n, d)
    do = rnd(524, (n, d))
    _, dk, dv = oracle.attention_bwd(q, k, v, do, causal, 0.6)
    assert np.max(np.abs(dv.sum(axis=0) - do.sum(axis=0))) < 1e-13
    assert np.max(np.abs(dk.sum(axis=0))) < 1e-13


# ---------------------------------------------------------------- grouped heads


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_torch_repeated_heads(causal):
    """Library cross-check: torch fp64 SDPA with each key/value head
    repeated for its group (repeat_interleave), forward and autograd (which
    sums the gradient of a repeated tensor over its copies)."""
    H, Hkv, n, d = 6, 2, 13, 8
    q = rnd(600, (H, n, d))
    k = rnd(601, (Hkv, n, d))
    v = rnd(602, (Hkv, n, d))
    do = rnd(603, (H, n, d))
    scale = 0.45
    o, lse = oracle.attention_gqa(q, k, v, causal, scale)
    dq, dk, dv = oracle.attention_bwd_gqa(q, k, v, do, causal, scale)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    rk = tk.repeat_interleave(H // Hkv, dim=0)
    rv = tv.repeat_interleave(H // Hkv, dim=0)
    out = torch.nn.functional.scaled_dot_product_attention(tq[None], rk[None], rv[None], is_causal=causal,
                                                           scale=scale)[0]
    assert np.max(np.abs(o - out.detach().numpy())) < 1e-12
    s = scale * torch.einsum("hnd,hmd->hnm", tq.detach(), rk.detach())
    if causal:
        s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
    assert np.max(np.abs(lse - torch.logsumexp(s, dim=-1).numpy())) < 1e-12
    out.backward(torch.from_numpy(do))
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.max(np.abs(mine - ref.numpy())) < 1e-12


def test_gqa_finite_differences():
    """Central differences of f = sum_h <O_h, dO_h> through the shared K and
    V (H = 4 query heads on Hkv = 2 key/value heads, N = 9, d = 4)."""
    H, Hkv, n, d = 4, 2, 9, 4
    q = rnd(610, (H, n, d))
    k = rnd(611, (Hkv, n, d))
    v = rnd(612, (Hkv, n, d))
    do = rnd(613, (H, n, d))
    scale = 0.7
    dq, dk, dv = oracle.attention_bwd_gqa(q, k, v, do, True, scale)

    def f(qq, kk, vv):
        o, _ = oracle.attention_gqa(qq, kk, vv, True, scale)
        return float(np.sum(o * do))

    h = 1e-6
    for grad, which in ((dq, 0), (dk, 1), (dv, 2)):
        num = np.zeros_like(grad)
        for idx in np.ndindex(*grad.shape):
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += h
            fp = f(*args)
            args[which][idx] -= 2 * h
            fm = f(*args)
            num[idx] = (fp - fm) / (2 * h)
        assert np.max(np.abs(num - grad)) < 1e-7


def test_gqa_one_group_is_multi_head():
    """Hkv = H: every query head has its own key/value head."""
    H, n, d = 3, 11, 8
    q, k, v, do = (rnd(620 + i, (H, n, d)) for i in range(4))
    o, lse = oracle.attention_gqa(q, k, v, True, 0.5)
    dq, dk, dv = oracle.attention_bwd_gqa(q, k, v, do, True, 0.5)
    for h in range(H):
        ro, rl = oracle.naive_attention(q[h], k[h], v[h], True, 0.5)
        assert np.array_equal(o[h], ro) and np.array_equal(lse[h], rl)
        for a, b in zip((dq[h], dk[h], dv[h]), oracle.attention_bwd(q[h], k[h], v[h], do[h], True, 0.5)):
            assert np.array_equal(a, b)


# ---------------------------------------------------------------- variable length


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_equal_lengths_is_batched(causal):
    """Equal lengths: the packed problem is the batched one with the batch
    axis folded into the rows (torch fp64 SDPA per sequence)."""
    H, B, n, d = 3, 4, 9, 8
    q = rnd(700, (H, B * n, d))
    k = rnd(701, (H, B * n, d))
    v = rnd(702, (H, B * n, d))
    cu = np.arange(B + 1) * n
    o, lse = oracle.attention_varlen(q, k, v, cu, causal, 0.4)
    for b in range(B):
        sl = slice(b * n, (b + 1) * n)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[:, sl]), torch.from_numpy(k[:, sl]), torch.from_numpy(v[:, sl]),
            is_causal=causal, scale=0.4).numpy()
        assert np.max(np.abs(o[:, sl] - ref)) < 1e-12


def test_varlen_sequences_are_independent():
    """Changing the keys and values of one sequence leaves every other
    sequence's output bit-identical; empty sequences are allowed."""
    H, d = 2, 4
    cu = np.array([0, 5, 5, 12, 13])
    total = cu[-1]
    q, k, v = (rnd(710 + i, (H, total, d)) for i in range(3))
    o1, l1 = oracle.attention_varlen(q, k, v, cu, True, 0.9)
    k2, v2 = k.copy(), v.copy()
    k2[:, 5:12] += 1.0
    v2[:, 5:12] -= 2.0
    o2, l2 = oracle.attention_varlen(q, k2, v2, cu, True, 0.9)
    for sl in (slice(0, 5), slice(12, 13)):
        assert np.array_equal(o1[:, sl], o2[:, sl]) and np.array_equal(l1[:, sl], l2[:, sl])
    assert np.max(np.abs(o1[:, 5:12] - o2[:, 5:12])) > 0.1
    # a sequence of one row sees only itself: o = v, L = scale q.k
    assert np.allclose(o1[:, 12], v[:, 12], atol=1e-15)
    assert np.allclose(l1[:, 12], 0.9 * np.sum(q[:, 12] * k[:, 12], axis=-1), atol=1e-14)


def test_varlen_bwd_finite_differences():
    """Central differences of f = sum <O, dO> over packed sequences (one of
    them empty): gradients stay inside each sequence."""
    H, Hkv, d = 2, 1, 3
    cu = np.array([0, 4, 4, 9])
    total = cu[-1]
    q = rnd(720, (H, total, d))
    k = rnd(721, (Hkv, total, d))
    v = rnd(722, (Hkv, total, d))
    do = rnd(723, (H, total, d))
    dq, dk, dv = oracle.attention_bwd_varlen(q, k, v, do, cu, True, 0.8)

    def f(qq, kk, vv):
        o, _ = oracle.attention_varlen(qq, kk, vv, cu, True, 0.8)
        return float(np.sum(o * do))

    h = 1e-6
    for grad, which in ((dq, 0), (dk, 1), (dv, 2)):
        num = np.zeros_like(grad)
        for idx in np.ndindex(*grad.shape):
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += h
            fp = f(*args)
            args[which][idx] -= 2 * h
            fm = f(*args)
            num[idx] = (fp - fm) / (2 * h)
        assert np.max(np.abs(num - grad)) < 1e-7


# ---------------------------------------------------------------- planted mistakes


def _mutant(kind):
    """A copy of the naive oracle with one planted mistake."""

    def attn(q, k, v, causal, scale, rows=None, return_p=False):
        q = np.asarray(q, np.float64)
        k = np.asarray(k, np.float64)
        v = np.asarray(v, np.float64)
        rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
        sc = 1.0 if kind == "scale_dropped" else scale
        s = sc * ((k @ q.T)[rows] if kind == "transposed_scores" and q.shape[0] == k.shape[0] else q[rows] @ k.T)
        if causal:
            kj = np.arange(k.shape[0])[None, :]
            ri = rows[:, None]
            bad = {"mask_flipped": kj < ri, "mask_off_by_one": kj >= ri}.get(kind, kj > ri)
            s = np.where(bad, -np.inf, s)
        m = np.max(s, axis=1, keepdims=True)
        if kind == "max_not_subtracted":
            m = np.zeros_like(m)
        m = np.where(np.isfinite(m), m, 0.0)
        e = np.exp(m - s) if kind == "exp_sign" else np.exp(s - m)
        e = np.where(np.isnan(e), 0.0, e)
        lsum = e.sum(axis=1, keepdims=True)
        p = e if kind == "no_normalisation" else e / lsum
        o = (p.T @ v) if kind == "pv_transposed" and p.shape[0] == p.shape[1] else p @ v
        lse = m[:, 0] + (np.log2(lsum[:, 0]) if kind == "lse_log2" else np.log(lsum[:, 0]))
        return (o, lse, p) if return_p else (o, lse)

    return attn


MUTANTS = [
    "scale_dropped",
    "transposed_scores",
    "mask_flipped",
    "mask_off_by_one",
    "max_not_subtracted",
    "exp_sign",
    "no_normalisation",
    "pv_transposed",
    "lse_log2",
]


def test_unmutated_copy_passes_pins():
    attn = _mutant("none")
    for pin in PINS:
        pin(attn)


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_catch_planted_mistake(kind):
    attn = _mutant(kind)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(attn)
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {kind}"


# ------------------------------------------------------------ 8-bit inputs

# OCP 8-bit floating point specification (OFP8), E4M3: (code, value).
E4M3_PINS = [(0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x30, 0.5),
             (0x38, 1.0), (0x39, 1.125), (0x3C, 1.5), (0x40, 2.0), (0x58, 16.0), (0x77, 240.0),
             (0x7E, 448.0), (0x80, -0.0), (0xB8, -1.0), (0xFE, -448.0)]


@pytest.mark.parametrize("code,value", E4M3_PINS)
def test_e4m3_decode_pins(code, value):
    got = float(oracle.e4m3_to_f64(np.array([code], dtype=np.uint8))[0])
    assert got == value and math.copysign(1.0, got) == math.copysign(1.0, value)


def test_e4m3_nan_codes_and_order():
    vals = oracle.e4m3_to_f64(np.arange(256, dtype=np.uint8))
    assert np.isnan(vals[0x7F]) and np.isnan(vals[0xFF]) and int(np.isnan(vals).sum()) == 2
    pos = vals[:0x7F]
    assert np.all(np.diff(pos) > 0)                     # codes 0x00..0x7E increase strictly
    assert np.array_equal(vals[0x80:0xFF], -pos)        # sign bit negates


def test_e4m3_values_are_bf16_values():
    """Every finite E4M3 value is a bfloat16 value: the 8-bit forward may
    widen V to bf16 without rounding."""
    vals = oracle.e4m3_to_f64(np.arange(256, dtype=np.uint8))
    fin = vals[np.isfinite(vals)]
    as_bf16 = torch.from_numpy(fin).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(as_bf16, fin)


def test_e4m3_codes_round_trip_through_the_input_encoder():
    import synthetic

    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    back = synthetic.e4m3_round_bits(oracle.e4m3_to_f64(codes))
    assert np.array_equal(back, codes)


def test_e4m3_encoder_rounds_to_nearest_even():
    import synthetic

    rng = np.random.default_rng(7)
    x = rng.standard_normal(20000) * 40
    codes = synthetic.e4m3_round_bits(x)
    dec = oracle.e4m3_to_f64(codes)
    grid = oracle.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))  # non-negative finite values
    a = np.minimum(np.abs(x), 448.0)
    nearest = grid[np.argmin(np.abs(grid[None, :] - a[:, None]), axis=1)]
    assert np.array_equal(np.abs(dec), nearest)  # no ties occur in continuous draws


def test_fp8_attention_constant_keys_give_mean_of_v():
    """All keys equal: every visible score of a row is the same, so O is the
    mean of the visible dequantised V rows (closed form), whatever the Q and
    K factors; the V factor scales it."""
    rng = np.random.default_rng(3)
    n, d = 37, 16
    q = rng.integers(0, 0x7F, size=(n, d)).astype(np.uint8)
    k = np.tile(rng.integers(0, 0x7F, size=(1, d)).astype(np.uint8), (n, 1))
    v = rng.integers(0, 0x7F, size=(n, d)).astype(np.uint8)
    vd = oracle.e4m3_to_f64(v) * 0.25
    for causal in (False, True):
        o, _ = oracle.attention_fp8(q, k, v, 0.5, 3.0, 0.25, causal, 0.125)
        for i in (0, 5, n - 1):
            ref = vd[: i + 1].mean(axis=0) if causal else vd.mean(axis=0)
            assert np.allclose(o[i], ref, rtol=1e-12, atol=1e-12)


def test_fp8_attention_q_factor_acts_as_scale():
    rng = np.random.default_rng(4)
    q, k, v = (rng.integers(0, 0x7F, size=(20, 8)).astype(np.uint8) for _ in range(3))
    o1, l1 = oracle.attention_fp8(q, k, v, 2.0, 0.5, 1.0, True, 0.1)
    o2, l2 = oracle.attention_fp8(q, k, v, 1.0, 1.0, 1.0, True, 0.1)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-14) and np.allclose(l1, l2, rtol=1e-12, atol=1e-12)
