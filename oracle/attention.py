"""Dense masked softmax attention and the prefill masks (float64, CPU).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, and from where:

* Scaled dot-product attention, attention glossary "Self-Attentionの計算原理":
  logits are q.k / sqrt(d_k), a softmax over the allowed keys normalises
  them, and the output is the weighted sum of the values.  The oracle also
  returns the natural-log log-sum-exp of the scaled logits (the softmax
  normaliser), which a split computation needs to merge partial results.
* GQA, attention glossary FAQ Q2: several query heads share one K/V head;
  query head h reads K/V head h // (Hq / Hkv).
* The causal band of sliding-window attention, SWA glossary "概要と動作原理":
  each token sees itself and the w-1 tokens before it (the attention matrix
  is a band matrix, zero outside the window).  The reading taken for
  "the w tokens up to itself" is: the query itself plus the w-1 previous
  tokens, i.e. 0 <= i - j <= w - 1.  Through the general mask below this is
  window_left = w - 1, window_right = 0, causal = True.
* The bidirectional local window plus global tokens, local-global glossary
  "ローカルアテンションの仕組み" and "グローバルアテンションの仕組み":
  token i sees j when |i - j| is within the window, and a global token sees
  and is seen by every token.  Reading: "window 512 (+-256)" means
  -256 <= j - i <= 256 (both ends included), and a pair allowed by both the
  band and a global token is one pair (the mask is a boolean union).
* Dilated SWA, SWA glossary "SWAの拡張手法": the positions inside the window
  are thinned out (dilation) so the same amount of computation covers a wider
  range.  Reading: with dilation s the window's keys are every s-th position
  counted from the query, i.e. j is allowed for row i when the band above
  allows it and i - j is a multiple of s (s = 1 is the plain band).  A causal
  window of w keys at spacing s is window_left = (w - 1) s.  Global tokens are
  not combined with dilation here.

A row with no allowed key has output 0 and log-sum-exp -inf (never happens
for the masks above: the diagonal is always allowed).
"""

from __future__ import annotations

import numpy as np


def prefill_allowed(rows, cols, window_left, window_right, causal, global_pos=(), dilation=1):
    """Boolean mask allowed[r, c] for query positions ``rows`` and key positions ``cols``.

    allowed(i, j) = (i - window_left <= j <= i + window_right [and j <= i if causal]
                     [and (i - j) % dilation == 0])
                    or i in G or j in G.
    A negative ``window_left`` / ``window_right`` means no limit on that side.
    Global tokens are bidirectional only (local-global glossary, global attention
    section: they attend to and from all tokens); with ``causal`` they are refused,
    and so they are with a dilation above 1.
    """
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    diff = cols[None, :] - rows[:, None]  # j - i
    ok = np.ones(diff.shape, dtype=bool)
    if window_left >= 0:
        ok &= diff >= -window_left
    if window_right >= 0:
        ok &= diff <= window_right
    if causal:
        ok &= diff <= 0
    if dilation < 1:
        raise ValueError("dilation must be >= 1")
    if dilation > 1:
        ok &= diff % dilation == 0
    g = np.asarray(global_pos, dtype=np.int64)
    if g.size:
        if causal:
            raise ValueError("global tokens are bidirectional; causal masks take none")
        if dilation > 1:
            raise ValueError("global tokens are not combined with a dilated window")
        ok |= np.isin(rows, g)[:, None]
        ok |= np.isin(cols, g)[None, :]
    return ok


def masked_attention_rows(q, k, v, allowed, scale):
    """Softmax attention of query rows ``q`` [R, d] over keys ``k``/values ``v`` [N, d].

    ``allowed`` [R, N] selects the keys each row may see.  Returns (o [R, dv], lse [R])
    in float64: o = sum_j p_ij v_j with p_ij = exp(l_ij - lse_i) over allowed j,
    l_ij = scale * q_i . k_j, lse_i = log sum_j exp(l_ij).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    logits = scale * (q @ k.T)
    logits = np.where(allowed, logits, -np.inf)
    m = logits.max(axis=1)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    p = np.exp(logits - m_safe[:, None])  # exp(-inf) = 0 on masked keys
    l = p.sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        o = (p @ v) / l[:, None]
        lse = m_safe + np.log(l)
    o[empty] = 0.0
    lse[empty] = -np.inf
    return o, lse


def prefill(Q, K, V, window_left, window_right, causal, global_pos=(), scale=None,
            rows=None, batches=None, heads=None, tile=512, dilation=1):
    """Masked attention for every (or a sample of) query row of a prefill.

    Q [B, Hq, N, d]; K, V [B, Hkv, N, d] (any float dtype; upcast to float64).
    ``rows`` / ``batches`` / ``heads`` restrict the output to those indices (default all).
    ``scale`` defaults to 1/sqrt(d) (attention glossary, step 2).
    ``dilation`` thins the window to every s-th key counted from the query (SWA
    glossary, dilated SWA).
    Returns O [nb, nh, nr, d] and lse [nb, nh, nr] in float64.
    """
    B, Hq, N, d = Q.shape
    Hkv = K.shape[1]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of K/V heads")
    group = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    batches = range(B) if batches is None else batches
    heads = range(Hq) if heads is None else heads
    batches, heads = list(batches), list(heads)
    cols = np.arange(N)
    O = np.zeros((len(batches), len(heads), len(rows), V.shape[-1]))
    L = np.zeros((len(batches), len(heads), len(rows)))
    for bi, b in enumerate(batches):
        for hi, h in enumerate(heads):
            kv = h // group
            kb = np.asarray(K[b, kv], dtype=np.float64)
            vb = np.asarray(V[b, kv], dtype=np.float64)
            for r0 in range(0, len(rows), tile):
                r = rows[r0:r0 + tile]
                allowed = prefill_allowed(r, cols, window_left, window_right, causal, global_pos, dilation)
                o, lse = masked_attention_rows(Q[b, h, r], kb, vb, allowed, scale)
                O[bi, hi, r0:r0 + tile] = o
                L[bi, hi, r0:r0 + tile] = lse
    return O, L
