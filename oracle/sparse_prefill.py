"""Block-sparse causal prefill: query tiles share one selected block set (float64, CPU).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, and from where.  The sparse-attention overview describes NSA's
data flow (coarse compression of the tokens, then a fine-grained selection of the
important ones) and block-wise sparse attention that splits the sequence into
blocks; the COBS explainer builds on NSA's compression, selection and sliding
window branches (technical summary 2.3) and scores blocks from their summaries
(2.2).  The pages give no prefill-specific rule, so these are readings:

* Selection unit: the T = 128 consecutive query rows of a tile share one block
  set per (batch, K/V head); the group's query heads share it as in decode.
* Score of block j for a tile: ln sum over the tile's rows r and the group's
  heads h of exp(q~_{r,h} . mean_j), q~ = scale * q (first order: the log of the
  tile's summed estimated mass).
* Forced keys of row i: its causal window [max(0, i - wl), i] and the sinks
  [0, min(n_sink, i + 1)).  Candidates of a tile: complete blocks with a key
  before the window of the tile's last row (so outside some row's forced set),
  other than blocks wholly inside the sinks; the top-k by (score descending,
  index ascending), ascending, -1 padded.  Selecting every candidate therefore
  gives every row all its causal keys in complete blocks.
* Row i attends the union of its forced keys and the keys <= i of its tile's
  selected blocks, one softmax, a key reached twice counted once.
"""

import numpy as np

from .attention import masked_attention_rows
from .selector import block_summaries, group_scores, head_scores, top_k_blocks

TILE = 128


def tile_candidates(i0, n, S, window_left, n_sink, tile=TILE):
    """Candidate blocks of the query tile starting at row i0 (see the module docstring)."""
    i_last = min(n, i0 + tile) - 1
    klo = max(0, i_last - window_left)
    return np.array([j for j in range(n // S) if j * S < klo and (j + 1) * S > n_sink], dtype=np.int64)


def sparse_prefill_selection(Q, K, n, S, top_k, window_left, n_sink, scale=None, mean_bf16=False,
                             tile=TILE, pairs=None):
    """Per (b, K/V head): tile scores [n_tiles, NB] and selections [n_tiles, top_k].

    Q [B, Hq, >= n, d]; K [B, Hkv, >= n, d].  The block means come from
    ``block_summaries`` (bfloat16-rounded with ``mean_bf16``).
    """
    B, Hq, _, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    n_tiles = (n + tile - 1) // tile
    if pairs is None:
        pairs = [(b, g) for b in range(B) for g in range(Hkv)]
    out = {}
    for (b, g) in pairs:
        mean, _ = block_summaries(np.asarray(K[b, g, :n], dtype=np.float64), S, 0, mean_bf16=mean_bf16)
        scores = np.zeros((n_tiles, n // S))
        sel = np.full((n_tiles, top_k), -1, dtype=np.int64)
        for t in range(n_tiles):
            i0, i1 = t * tile, min(n, (t + 1) * tile)
            q = scale * np.asarray(Q[b, g * G:(g + 1) * G, i0:i1], dtype=np.float64).reshape(-1, d)
            if n // S:
                scores[t] = group_scores(head_scores(q, mean))
            sel[t] = top_k_blocks(scores[t], tile_candidates(i0, n, S, window_left, n_sink, tile), top_k)
        out[(b, g)] = dict(scores=scores, sel=sel)
    return out


def sparse_prefill_allowed(rows, n, S, window_left, n_sink, sel_rows):
    """allowed[r, c]: key c for query row rows[r], whose tile selected the blocks sel_rows[r]."""
    cols = np.arange(n)
    allowed = np.zeros((len(rows), n), dtype=bool)
    for r, i in enumerate(rows):
        keys = set(range(max(0, i - window_left), i + 1)) | set(range(min(n_sink, i + 1)))
        for j in sel_rows[r]:
            if j >= 0:
                keys |= set(range(j * S, min((j + 1) * S, i + 1)))
        allowed[r, sorted(keys)] = True
    assert not allowed[cols[None, :] > np.asarray(rows)[:, None]].any()  # causal
    return allowed


def sparse_prefill(Q, K, V, n, S, window_left, n_sink, selection, scale=None, rows=None, tile=TILE,
                   pairs=None):
    """Outputs of the block-sparse prefill for the rows ``rows`` (default all) of every
    query head of the pairs in ``selection`` ((b, g) -> dict with 'sel' [n_tiles, k]).
    Returns (b, g) -> (O [G, R, d], lse [G, R])."""
    B, Hq, _, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    out = {}
    for (b, g), s in (selection.items() if pairs is None else [(p, selection[p]) for p in pairs]):
        allowed = sparse_prefill_allowed(rows, n, S, window_left, n_sink, [s["sel"][i // tile] for i in rows])
        O = np.zeros((G, len(rows), V.shape[-1]))
        L = np.zeros((G, len(rows)))
        for hh in range(G):
            q = np.asarray(Q[b, g * G + hh], dtype=np.float64)[rows]
            O[hh], L[hh] = masked_attention_rows(q, K[b, g, :n], V[b, g, :n], allowed, scale)
        out[(b, g)] = (O, L)
    return out
