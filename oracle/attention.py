"""CPU fp64 oracle for exact softmax attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and this module imports
nothing from the product path.

Sources, cited by page title and section:

[P1] "FlashAttention-2: Why the Attention Bottleneck Wasn't Where Everyone Was
     Looking": "The hook: softmax doesn't tile" (the four-line textbook
     attention), "FA2 change #1: Stop dividing so much" (unnormalised
     accumulator, rescale factor alpha, one divide at the end, saving
     L = m + log l), "FA2 change #2" (loop order: outer over query blocks),
     "The causal masking freebie" (mask entries with key > query).
[P2] "FlashAttention: Move Less, Not Compute Less": "The Multiplication May
     Not Be the Slow Part" (S = QK^T, P = softmax(S), O = PV),
     "Tiling Is Easy; Softmax Couples the Entire Row" (stable softmax
     m, l; online recurrences m', l', o' and O = o / l),
     "Why More Arithmetic Can Finish Sooner" (the backward rebuilds S, P
     from saved per-row statistics),
     "What It Changes--and What It Does Not" (GQA shrinks the number of
     key/value heads; the reference implementation has GQA/MQA and
     variable-length paths).
[P3] "PidokuInfra 10 -- FlashAttention": section 1 (softmax(QK^T/sqrt(d))V,
     exact), section 4 "Tiny example -- the algorithm" (block loop with a
     causal per-row key bound, online update, normalise at the end),
     section 5 "The decode variant: FlashDecoding" (partials (m, l, o)
     merged with the same rescaling).

Readings where the pages leave a step open:
  * scale multiplies QK^T before the mask, the max and the exponential
    ([P3] s1 and s4 scale the dot product before taking the max);
  * the causal mask is additive -inf for key index j > query index i
    (top-left aligned, [P3] s4: query i sees keys 0..i);
  * "log" in L = m + log(l) is the natural logarithm, so L is the row
    logsumexp of the scaled, masked scores ([P1] change #1);
  * a row with no visible key (only possible when the caller passes
    such a score matrix) has O = 0 and L = -inf;
  * grouped heads: of H query heads and Hkv key/value heads, query head h
    uses key/value head h // (H // Hkv) (consecutive query heads share one).

Parity pins live in ``tests/test_oracle.py``: closed forms, invariants,
library cross-checks (torch's fp64 CPU attention, scipy's logsumexp),
brute force on tiny inputs, the page's own tiled-versus-naive experiment
and finite differences for the backward.  Every function here is pinned by
at least one of them.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "scores",
    "attention_from_scores",
    "naive_attention",
    "tiled_attention",
    "attention_bwd",
    "split_kv_partials",
    "combine_partials",
    "attention_gqa",
    "attention_bwd_gqa",
    "attention_varlen",
    "attention_bwd_varlen",
]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def scores(q, k, causal, scale, rows=None):
    """Scaled, masked score rows S_r = scale * q_r . K^T, masked to -inf.

    [P2] "The Multiplication May Not Be the Slow Part": S = Q K^T per head;
    [P3] s1/s4: the product is scaled (1/sqrt(d) there, a parameter here);
    [P1] "The causal masking freebie" and [P3] s4: with a causal mask query
    i sees keys 0..i, so S_ij = -inf for j > i.

    q: (N, d), k: (N, d) (any float dtype, upcast exactly to fp64).
    rows: optional 1-D int array of query indices; default all rows.
    Returns S with shape (len(rows), N), fp64.
    """
    q = _f64(q)
    k = _f64(k)
    n_q = q.shape[0]
    if rows is None:
        rows = np.arange(n_q)
    rows = np.asarray(rows, dtype=np.int64)
    s = scale * (q[rows] @ k.T)
    if causal:
        key_idx = np.arange(k.shape[0])[None, :]
        s = np.where(key_idx > rows[:, None], -np.inf, s)
    return s


def attention_from_scores(s, v, return_p=False):
    """Numerically stable softmax of each score row, then P V and L.

    [P2] "Tiling Is Easy; Softmax Couples the Entire Row": m = max_i x_i,
    l = sum_i exp(x_i - m), softmax(x)_i = exp(x_i - m) / l;
    [P2] "The Multiplication May Not Be the Slow Part": O = P V;
    [P1] "FA2 change #1": the saved per-row statistic is L = m + log(l).

    s: (R, N) scores (fp64, -inf for masked entries); v: (N, dv).
    Returns (O (R, dv), L (R,)) and P (R, N) when return_p.
    """
    s = _f64(s)
    v = _f64(v)
    m = np.max(s, axis=1, keepdims=True)
    empty = ~np.isfinite(m)  # all entries masked (-inf)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe)  # exp(-inf) = 0 for masked entries
    l = np.sum(e, axis=1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        p = np.where(empty, 0.0, e / np.where(empty, 1.0, l))
        lse = np.where(empty[:, 0], -np.inf, m_safe[:, 0] + np.log(np.where(empty[:, 0], 1.0, l[:, 0])))
    o = p @ v
    if return_p:
        return o, lse, p
    return o, lse


def naive_attention(q, k, v, causal, scale, rows=None, return_p=False):
    """Textbook attention that materialises S and P for the requested rows.

    [P1] "The hook": S = Q K^T, S = S + mask, P = softmax(S), O = P V; the
    scale and mask readings are in the module header.  This is the
    definition the fused method reaches up to rounding ([P2] "Tiling Is
    Easy", last paragraph; [P3] s1 "EXACT").

    q, k, v: (N, d) arrays for one (batch, head).  Returns (O, L[, P]) in
    fp64 for rows (default: all rows).
    """
    s = scores(q, k, causal, scale, rows)
    return attention_from_scores(s, v, return_p=return_p)


def tiled_attention(q, k, v, causal, scale, block_q, block_k):
    """Exact attention by the blocked online-softmax recurrence, in fp64.

    Follows the loop order of [P1] "FA2 change #2" (outer loop over query
    blocks, running state kept per block, inner loop streams key/value
    blocks) and the per-row update of [P2] "Tiling Is Easy":
        m'  = max(m, max_j x_j)
        l'  = exp(m - m') l + sum_j exp(x_j - m')
        o'  = exp(m - m') o + sum_j exp(x_j - m') v_j
    with the single final division O = o / l of [P1] "FA2 change #1".
    The causal key bound follows [P3] s4: for a query block ending at row
    i1 - 1 only key blocks starting below i1 are visited, and inside a
    block a row skips the update when none of the block's keys is visible
    to it (so exp(-inf - (-inf)) never arises).
    Returns (O (N, dv), L (N,)), L = m + log(l) ([P1] change #1).
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    n, n_k = q.shape[0], k.shape[0]
    dv = v.shape[1]
    out = np.zeros((n, dv))
    lse = np.zeros(n)
    for i0 in range(0, n, block_q):
        i1 = min(i0 + block_q, n)
        rows = np.arange(i0, i1)
        m = np.full(i1 - i0, -np.inf)
        l = np.zeros(i1 - i0)
        acc = np.zeros((i1 - i0, dv))
        key_end = min(i1, n_k) if causal else n_k
        for j0 in range(0, key_end, block_k):
            j1 = min(j0 + block_k, n_k)
            x = scale * (q[i0:i1] @ k[j0:j1].T)
            if causal:
                keys = np.arange(j0, j1)[None, :]
                x = np.where(keys > rows[:, None], -np.inf, x)
            x_max = np.max(x, axis=1)
            live = np.isfinite(x_max)  # rows with at least one visible key here
            m_new = np.where(live, np.maximum(m, x_max), m)
            m_use = np.where(live, m_new, 0.0)
            with np.errstate(over="ignore", invalid="ignore"):
                alpha = np.where(live, np.exp(m - m_use), 1.0)
                p = np.where(live[:, None], np.exp(x - m_use[:, None]), 0.0)
            l = alpha * l + np.sum(p, axis=1)
            acc = alpha[:, None] * acc + p @ v[j0:j1]
            m = m_new
        out[i0:i1] = acc / l[:, None]
        lse[i0:i1] = m + np.log(l)
    return out, lse


def attention_bwd(q, k, v, do, causal, scale):
    """Analytic gradients of O = softmax(scale Q K^T + mask) V, in fp64.

    The pages fix what the backward reuses -- S and P rebuilt from Q, K and
    the saved per-row statistic rather than stored ([P2] "Why More
    Arithmetic Can Finish Sooner") -- but print no formulas; these are the
    chain rule through the definition in ``naive_attention``:
        P = exp(S - L),  dV = P^T dO,  dP = dO V^T,
        D_i = sum_j P_ij dP_ij,  dS = P * (dP - D),
        dQ = scale dS K,  dK = scale dS^T Q.
    Pinned against central finite differences and torch's fp64 autograd.
    Returns (dQ, dK, dV).
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    do = _f64(do)
    s = scores(q, k, causal, scale)
    _, lse = attention_from_scores(s, v)
    p = np.exp(s - lse[:, None])  # masked entries: exp(-inf) = 0
    dv = p.T @ do
    dp = do @ v.T
    d_row = np.sum(p * dp, axis=1, keepdims=True)
    ds = p * (dp - d_row)
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def split_kv_partials(q, k, v, causal, scale, split_bounds):
    """Per-split unnormalised partials (m, l, o) over key ranges.

    [P3] s5 "The decode variant: FlashDecoding": the key dimension is split
    across workers, each producing an unnormalised output with its own
    (m, l).  split_bounds is a list of (j0, j1) key ranges covering 0..N.
    Returns arrays m (S, R), l (S, R), o (S, R, dv) where R = number of
    query rows; a split with no visible key for a row has m = -inf, l = 0,
    o = 0.
    """
    s_full = scores(q, k, causal, scale)
    v = _f64(v)
    ms, ls, os_ = [], [], []
    for j0, j1 in split_bounds:
        x = s_full[:, j0:j1]
        m = np.max(x, axis=1) if j1 > j0 else np.full(x.shape[0], -np.inf)
        live = np.isfinite(m)
        m_use = np.where(live, m, 0.0)
        e = np.where(live[:, None], np.exp(x - m_use[:, None]), 0.0)
        ms.append(m)
        ls.append(np.sum(e, axis=1))
        os_.append(e @ v[j0:j1])
    return np.stack(ms), np.stack(ls), np.stack(os_)


def combine_partials(m, l, o):
    """Merge split partials with the online-softmax rescale, then divide once.

    [P3] s5 "FlashDecoding": a second step combines the partials with the
    same rescaling as online softmax; [P2] "Tiling Is Easy": each partial is
    brought to the global max M by exp(m_s - M) before summing.
    m, l: (S, R); o: (S, R, dv).  Returns (O (R, dv), L (R,)).
    """
    m = _f64(m)
    l = _f64(l)
    o = _f64(o)
    big_m = np.max(m, axis=0)
    w = np.where(np.isfinite(m), np.exp(m - big_m[None, :]), 0.0)
    l_tot = np.sum(w * l, axis=0)
    o_tot = np.sum(w[:, :, None] * o, axis=0)
    return o_tot / l_tot[:, None], big_m + np.log(l_tot)


def attention_gqa(q, k, v, causal, scale):
    """Attention with grouped key/value heads for one batch entry.

    [P2] "What It Changes--and What It Does Not": GQA keeps fewer key/value
    heads than query heads; each query head computes ordinary attention
    (``naive_attention``) against the K and V of its group, head
    h // (H // Hkv).  q: (H, N, d); k, v: (Hkv, N, d) with H a multiple of
    Hkv.  Returns (O (H, N, d), L (H, N)) in fp64.
    """
    n_h, n_kv = q.shape[0], k.shape[0]
    group = n_h // n_kv
    outs = [naive_attention(q[h], k[h // group], v[h // group], causal, scale) for h in range(n_h)]
    return np.stack([o for o, _ in outs]), np.stack([l for _, l in outs])


def attention_bwd_gqa(q, k, v, do, causal, scale):
    """Gradients of ``attention_gqa`` for one batch entry, in fp64.

    Each query head's dQ is that of its own attention (``attention_bwd``);
    a key/value head enters the attention of every query head of its group,
    so by the chain rule its dK and dV are the sums of those heads'
    contributions.  Pinned against central finite differences through the
    shared K, V and torch's fp64 autograd through repeated key/value heads.
    Returns (dQ (H, N, d), dK (Hkv, N, d), dV (Hkv, N, d)).
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    do = _f64(do)
    n_h, n_kv = q.shape[0], k.shape[0]
    group = n_h // n_kv
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for h in range(n_h):
        gq, gk, gv = attention_bwd(q[h], k[h // group], v[h // group], do[h], causal, scale)
        dq[h] = gq
        dk[h // group] += gk
        dv[h // group] += gv
    return dq, dk, dv


def attention_varlen(q, k, v, cu_seqlens, causal, scale):
    """Attention over packed sequences of different lengths.

    [P2] "What It Changes--and What It Does Not" (variable-length paths) and
    [P3] sections 8-9 (pack sequences instead of padding them): sequence b
    is rows cu_seqlens[b] .. cu_seqlens[b + 1] - 1 of every head and attends
    only within itself -- ``attention_gqa`` applied to each sequence's rows.
    q: (H, total, d); k, v: (Hkv, total, d); cu_seqlens: B + 1 offsets.
    Returns (O (H, total, d), L (H, total)) in fp64.
    """
    q = _f64(q)
    n_h, total, _ = q.shape
    out = np.zeros(q.shape[:2] + (v.shape[2],))
    lse = np.zeros((n_h, total))
    for b in range(len(cu_seqlens) - 1):
        r0, r1 = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        if r1 > r0:
            o_b, l_b = attention_gqa(q[:, r0:r1], k[:, r0:r1], v[:, r0:r1], causal, scale)
            out[:, r0:r1] = o_b
            lse[:, r0:r1] = l_b
    return out, lse


def attention_bwd_varlen(q, k, v, do, cu_seqlens, causal, scale):
    """Gradients of ``attention_varlen``: each sequence's rows get the
    gradients of their own attention (``attention_bwd_gqa``); rows of
    different sequences never interact.  Returns (dQ, dK, dV) in fp64 with
    the shapes of q, k, v."""
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    do = _f64(do)
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for b in range(len(cu_seqlens) - 1):
        r0, r1 = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        if r1 > r0:
            gq, gk, gv = attention_bwd_gqa(q[:, r0:r1], k[:, r0:r1], v[:, r0:r1], do[:, r0:r1], causal, scale)
            dq[:, r0:r1] = gq
            dk[:, r0:r1] = gk
            dv[:, r0:r1] = gv
    return dq, dk, dv
