"""Pins of the block-sparse prefill oracle (query tiles sharing a selected block set)
against closed forms, a dense reduction and an independent mask formula."""

import numpy as np
import pytest

import oracle
from oracle import (sparse_prefill, sparse_prefill_allowed, sparse_prefill_selection, tile_candidates)


def _inputs(seed, B, Hq, Hkv, N, d):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, Hq, N, d)), rng.standard_normal((B, Hkv, N, d)),
            rng.standard_normal((B, Hkv, N, d)))


def test_candidates_worked_example():
    """n = 1024, S = 64, window 100 back, 64 sinks, tiles of 128.  Tile 0 (rows 0..127):
    the last row's window starts at 27, so only block 0 has a key before it, and block 0
    is all sinks: no candidate.  Tile 3 (rows 384..511): window of row 511 starts at 411,
    blocks 0..6 start before it; block 0 is all sinks: candidates 1..6."""
    assert tile_candidates(0, 1024, 64, 100, 64).tolist() == []
    assert tile_candidates(384, 1024, 64, 100, 64).tolist() == [1, 2, 3, 4, 5, 6]
    assert tile_candidates(384, 1024, 64, 100, 0).tolist() == [0, 1, 2, 3, 4, 5, 6]
    # the last, short tile of a 1000-token sequence: rows 896..999, window of 999 from 899;
    # the complete blocks are 0..14 (15 x 64 = 960 <= 1000) and all start before 899
    assert tile_candidates(896, 1000, 64, 100, 0).tolist() == list(range(15))


def test_every_candidate_selected_is_dense_causal():
    """With top_k >= the number of blocks, every row sees all its causal keys."""
    Q, K, V = _inputs(50, 1, 4, 2, 512, 16)
    sel = sparse_prefill_selection(Q, K, 512, 64, 8, 37, 0)
    got = sparse_prefill(Q, K, V, 512, 64, 37, 0, sel)
    ref_o, ref_l = oracle.prefill(Q, K, V, -1, 0, True)
    for (b, g), (O, L) in got.items():
        np.testing.assert_allclose(O, ref_o[b, 2 * g:2 * g + 2], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(L, ref_l[b, 2 * g:2 * g + 2], rtol=1e-12, atol=1e-12)


def test_window_covering_the_tile_is_the_band():
    """A window reaching back past every row's start leaves no candidate: the prefill is the
    causal band (here the whole causal triangle)."""
    Q, K, V = _inputs(51, 1, 2, 1, 256, 16)
    sel = sparse_prefill_selection(Q, K, 256, 64, 3, 300, 0)
    assert all((s["sel"] == -1).all() for s in sel.values())
    (O, L), = sparse_prefill(Q, K, V, 256, 64, 300, 0, sel).values()
    ref_o, ref_l = oracle.prefill(Q, K, V, 300, 0, True)
    np.testing.assert_allclose(O, ref_o[0], rtol=1e-12, atol=1e-12)


def test_allowed_mask_matches_an_independent_formula():
    """allowed(i, c) = c <= i and (c >= i - wl or c < n_sink or c // S in sel[tile(i)])."""
    rng = np.random.default_rng(52)
    n, S, wl, ns, T = 700, 64, 90, 20, 128
    sel = {t: np.sort(rng.choice(10, 3, replace=False)) for t in range(6)}
    rows = np.arange(n)
    got = sparse_prefill_allowed(rows, n, S, wl, ns, [sel[i // T] for i in rows])
    c = np.arange(n)[None, :]
    i = rows[:, None]
    blocks = np.stack([np.isin(np.arange(n) // S, sel[t // T]) for t in rows])
    ref = (c <= i) & ((c >= i - wl) | (c < ns) | blocks)
    assert np.array_equal(got, ref)


def test_tile_score_closed_forms():
    """A tile of R identical rows and G identical heads scores q~.mean + ln(R G); a one-row,
    one-head tile scores q~.mean."""
    rng = np.random.default_rng(53)
    d, S = 8, 64
    K = rng.standard_normal((1, 1, 256, d))
    q = rng.standard_normal(d)
    Q = np.tile(q, (1, 3, 128, 1))  # B 1, G 3 heads, 128 rows
    mean, _ = oracle.block_summaries(K[0, 0], S, 0)
    sel = sparse_prefill_selection(Q, K, 128, S, 1, 0, 0, scale=1.0)
    s = sel[(0, 0)]["scores"][0]
    np.testing.assert_allclose(s, mean[:2] @ q + np.log(3 * 128), rtol=1e-12)
    sel1 = sparse_prefill_selection(Q[:, :1], K, 128, S, 1, 0, 0, scale=0.5, tile=1)
    np.testing.assert_allclose(sel1[(0, 0)]["scores"][5], 0.5 * mean[:2] @ q, rtol=1e-12)


def test_selection_takes_the_tile_mass_top_k():
    """The selected blocks are the candidates of largest tile score (ties to the lower index)."""
    Q, K, V = _inputs(54, 1, 4, 1, 640, 16)
    K[0, 0, 5 * 64:6 * 64] += 2.0 * Q[0, :, 600:].mean(axis=(0, 1))  # block 5 aligned with tile 4
    sel = sparse_prefill_selection(Q, K, 640, 64, 2, 50, 0)[(0, 0)]
    assert 5 in sel["sel"][4].tolist()
    cand = tile_candidates(512, 640, 64, 50, 0)
    order = sorted(cand.tolist(), key=lambda j: (-sel["scores"][4][j], j))
    assert sel["sel"][4].tolist() == sorted(order[:2])
