"""Sparse decode over the selected blocks plus window, sink and global tokens (float64, CPU).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Given a selected block set, the method attends exactly: one softmax over the
token set T = forced tokens (sink, window, globals) union the tokens of every
selected block.  Reading: T is a set, so a token reached two ways (a global
token inside a selected block, a window that overlaps a block) counts once, and
the branches share a single softmax (the pages give NSA's separate gated
branches only as learned components, which are out of scope).  Sources: COBS
explainer technical summary sections 1 and 2.1 (read only the chosen blocks),
SWA glossary "SWAの拡張手法" (sink tokens) and the comparison table
(O(n (w+s) d) for window plus sinks), local-global glossary (global tokens).
"""

from __future__ import annotations

import numpy as np

from .attention import masked_attention_rows
from .selector import (block_summaries, candidate_blocks, forced_token_mask,
                       group_scores, head_scores, top_k_blocks)


def decode_token_set(n, S, forced, sel):
    """Sorted token indices of T = forced tokens union the selected blocks' tokens."""
    inT = np.array(forced[:n], dtype=bool, copy=True)
    for b in np.asarray(sel):
        if b >= 0:
            inT[b * S:(b + 1) * S] = True
    return np.nonzero(inT)[0]


def sparse_decode_group(q, K, V, tokens, scale):
    """Attention of the query heads ``q`` [G, d] over ``tokens`` of K, V [n, d].

    Returns (o [G, d], lse [G]) in float64.
    """
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    allowed = np.zeros((q.shape[0], K.shape[0]), dtype=bool)
    allowed[:, tokens] = True
    return masked_attention_rows(q, K, V, allowed, scale)


def decode_step(Q, K, V, n, S, rank, top_k, window, n_sink, global_pos=(), scale=None,
                pairs=None, summaries=None, mean_bf16=False, factor_fp4=False, basis=None):
    """One decode step for the query token t = n - 1 of every (batch, K/V head) pair.

    Q [B, Hq, d]; K, V [B, Hkv, >= n, d].  ``pairs`` restricts the work to a list of
    (b, kv_head); ``summaries`` may map (b, kv_head) -> (mean, factor) already built;
    ``mean_bf16`` / ``factor_fp4`` store the block means in bfloat16 / the factor rows
    in FP4 (see ``block_summaries``); ``basis`` [Hkv, s, d] holds each K/V head's
    query-subspace rows (factor rows then live in that subspace).
    Returns a dict keyed by (b, kv_head) with:
      'scores'  [NB] group scores of all complete blocks,
      'cand'    candidate block indices,
      'sel'     [top_k] selected blocks, ascending, -1 padded,
      'tokens'  the attended token set T,
      'o'       [G, d] output of the group's query heads, 'lse' [G].
    """
    B, Hq, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    forced = forced_token_mask(n, n_sink, window, global_pos)
    cand = candidate_blocks(n, S, forced)
    if pairs is None:
        pairs = [(b, g) for b in range(B) for g in range(Hkv)]
    out = {}
    for (b, g) in pairs:
        Kbg = np.asarray(K[b, g, :n], dtype=np.float64)
        Vbg = np.asarray(V[b, g, :n], dtype=np.float64)
        if summaries is not None and (b, g) in summaries:
            mean, factor = summaries[(b, g)]
        else:
            mean, factor = block_summaries(Kbg, S, rank, mean_bf16=mean_bf16, factor_fp4=factor_fp4,
                                           basis=None if basis is None else basis[g])
        q = np.asarray(Q[b, g * G:(g + 1) * G], dtype=np.float64)
        qs = scale * q
        s = group_scores(head_scores(qs, mean, factor if rank > 0 else None,
                                     basis=None if basis is None or rank == 0 else basis[g]))
        sel = top_k_blocks(s, cand, top_k)
        tokens = decode_token_set(n, S, forced, sel)
        o, lse = sparse_decode_group(q, Kbg, Vbg, tokens, scale)
        out[(b, g)] = dict(scores=s, cand=cand, sel=sel, tokens=tokens, o=o, lse=lse)
    return out
