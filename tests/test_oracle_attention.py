"""Pins of the oracle's dense masked attention and its prefill masks (CPU only).

Each check compares the oracle with something other than itself: torch's own
scaled_dot_product_attention / logsumexp in float64, closed forms, exact pair
counts, or graph facts printed on the local-global and SWA glossary pages.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import masked_attention_rows, prefill, prefill_allowed


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _torch_ref(Q, K, V, allowed, scale):
    """torch SDPA in float64 on the CPU with an explicit boolean mask."""
    q = torch.from_numpy(Q)[None, None]
    k = torch.from_numpy(K)[None, None]
    v = torch.from_numpy(V)[None, None]
    m = torch.from_numpy(allowed)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=scale)
    logits = scale * (torch.from_numpy(Q) @ torch.from_numpy(K).T)
    lse = torch.logsumexp(logits.masked_fill(~torch.from_numpy(allowed), -math.inf), dim=1)
    return o[0, 0].numpy(), lse.numpy()


MASKS = [
    dict(window_left=0, window_right=0, causal=True, global_pos=()),
    dict(window_left=6, window_right=0, causal=True, global_pos=()),
    dict(window_left=-1, window_right=0, causal=True, global_pos=()),
    dict(window_left=5, window_right=5, causal=False, global_pos=()),
    dict(window_left=4, window_right=4, causal=False, global_pos=(0, 17, 30)),
    dict(window_left=2, window_right=7, causal=False, global_pos=(9,)),
    dict(window_left=-1, window_right=-1, causal=False, global_pos=()),
]


@pytest.mark.parametrize("mask", MASKS)
def test_masked_attention_matches_torch_sdpa(mask):
    rng = np.random.default_rng(11)
    n, d = 37, 8
    Q, K, V = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    allowed = prefill_allowed(np.arange(n), np.arange(n), **mask)
    o, lse = masked_attention_rows(Q, K, V, allowed, 0.3)
    o_ref, lse_ref = _torch_ref(Q, K, V, allowed, 0.3)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def test_prefill_gqa_head_mapping_matches_torch():
    """Query head h reads K/V head h // (Hq/Hkv) (attention glossary FAQ Q2)."""
    rng = np.random.default_rng(5)
    B, Hq, Hkv, N, d = 2, 6, 2, 19, 4
    Q, K, V = _rand(rng, B, Hq, N, d), _rand(rng, B, Hkv, N, d), _rand(rng, B, Hkv, N, d)
    O, L = prefill(Q, K, V, 3, 0, True)
    allowed = prefill_allowed(np.arange(N), np.arange(N), 3, 0, True)
    for b in range(B):
        for h in range(Hq):
            o_ref, lse_ref = _torch_ref(Q[b, h], K[b, h // 3], V[b, h // 3], allowed, 1 / math.sqrt(d))
            np.testing.assert_allclose(O[b, h], o_ref, atol=1e-12)
            np.testing.assert_allclose(L[b, h], lse_ref, atol=1e-12)


def test_window_one_returns_values():
    """w = 1 (itself only): every output row is its own value row, exactly."""
    rng = np.random.default_rng(1)
    Q, K, V = _rand(rng, 1, 2, 23, 8), _rand(rng, 1, 1, 23, 8), _rand(rng, 1, 1, 23, 8)
    O, L = prefill(Q, K, V, 0, 0, True)
    np.testing.assert_array_equal(O[0, 0], V[0, 0])
    np.testing.assert_array_equal(O[0, 1], V[0, 0])


def test_zero_keys_give_window_running_mean():
    """K = 0 makes every allowed logit equal: o_i is the plain mean of V over the window."""
    rng = np.random.default_rng(2)
    n, d, w = 50, 6, 7
    Q, V = _rand(rng, 1, 1, n, d), _rand(rng, 1, 1, n, d)
    K = np.zeros((1, 1, n, d))
    O, L = prefill(Q, K, V, w - 1, 0, True)
    csum = np.vstack([np.zeros((1, d)), np.cumsum(V[0, 0], axis=0)])
    for i in range(n):
        lo = max(0, i - w + 1)
        np.testing.assert_allclose(O[0, 0, i], (csum[i + 1] - csum[lo]) / (i + 1 - lo), atol=1e-12)
        assert abs(L[0, 0, i] - math.log(i + 1 - lo)) < 1e-12


def test_constant_and_shifted_values():
    rng = np.random.default_rng(3)
    Q, K = _rand(rng, 1, 1, 31, 5), _rand(rng, 1, 1, 31, 5)
    V = np.full((1, 1, 31, 5), 0.75)
    O, _ = prefill(Q, K, V, 3, 3, False, (0, 20))
    np.testing.assert_allclose(O, 0.75, atol=1e-14)
    V2 = _rand(rng, 1, 1, 31, 5)
    O1, _ = prefill(Q, K, V2, 3, 3, False, (0, 20))
    O2, _ = prefill(Q, K, V2 + 2.5, 3, 3, False, (0, 20))
    np.testing.assert_allclose(O2, O1 + 2.5, atol=1e-12)


def _pair_count(n, tile=1024, **mask):
    total = 0
    rows_out = []
    for r0 in range(0, n, tile):
        r = np.arange(r0, min(n, r0 + tile))
        c = prefill_allowed(r, np.arange(n), **mask).sum(axis=1)
        rows_out.append(c)
        total += int(c.sum())
    return total, np.concatenate(rows_out)


def test_swa_band_pair_count_closed_form():
    """Causal band, self + 4095 previous, n = 8192: sum_i min(i+1, 4096) pairs per head."""
    n, w = 8192, 4096
    total, per_row = _pair_count(n, window_left=w - 1, window_right=0, causal=True)
    assert total == w * (w + 1) // 2 + (n - w) * w == 25_167_872
    np.testing.assert_array_equal(per_row, np.minimum(np.arange(n) + 1, w))


def test_local_global_pair_count_closed_form():
    """+-256 band plus 16 globals (every 1024th token), n = 16384: 8,847,344 pairs per head.

    band: 16384 rows x 513 minus the clipped triangles 2 * (256*257/2);
    globals: each adds its full row and column (2n) minus the pairs already in the band,
    minus the global-global pairs counted twice.
    """
    n, half = 16384, 256
    G = np.arange(0, n, 1024)
    band = n * (2 * half + 1) - 2 * (half * (half + 1) // 2)
    assert band == 8_339_200
    total, per_row = _pair_count(n, window_left=half, window_right=half, causal=False,
                                 global_pos=G)
    band_rows = np.minimum(np.arange(n) + half, n - 1) - np.maximum(np.arange(n) - half, 0) + 1
    in_band = lambda g: int(band_rows[g])  # noqa: E731  keys of row g already in the band
    extra = 0
    for g in G:
        extra += (n - in_band(g)) * 2  # row g and column g beyond the band
    # global-global pairs outside the band were added twice (row of g1, column of g2)
    gg_outside = sum(1 for a in G for b in G if abs(a - b) > half)
    expect = band + extra - gg_outside
    assert total == expect == 8_847_344
    assert per_row[G].tolist() == [n] * len(G)


def test_bidirectional_mask_is_symmetric_and_reaches_in_two_hops(golden_dir):
    facts = json.load(open(os.path.join(golden_dir, "pages_printed.json")))
    n = 200
    G = np.arange(0, n, 64)
    M = prefill_allowed(np.arange(n), np.arange(n), 8, 8, False, G).astype(np.int64)
    np.testing.assert_array_equal(M, M.T)
    hops = facts["two_hop_reach"]["max_hops"]
    reach = np.linalg.matrix_power(M, hops)
    assert (reach > 0).all()
    band_only = prefill_allowed(np.arange(n), np.arange(n), 8, 8, False).astype(np.int64)
    assert not (np.linalg.matrix_power(band_only, hops) > 0).all()


def test_global_token_added_cost_is_about_2n(golden_dir):
    facts = json.load(open(os.path.join(golden_dir, "pages_printed.json")))
    per_global = facts["global_token_cost"]["added_pairs_per_global_over_n"]
    n = 3000
    base, _ = _pair_count(n, window_left=16, window_right=16, causal=False)
    for g in ([0], [0, 1500]):
        with_g, _ = _pair_count(n, window_left=16, window_right=16, causal=False, global_pos=g)
        added = with_g - base
        assert added <= per_global * n * len(g)
        assert added >= per_global * n * len(g) - len(g) * (2 * 33 + len(g))


def test_no_window_is_dense_and_matches_printed_matrix_size(golden_dir):
    facts = json.load(open(os.path.join(golden_dir, "pages_printed.json")))["dense_matrix_128k"]
    n = 300
    total, _ = _pair_count(n, window_left=-1, window_right=-1, causal=False)
    assert total == n * n
    assert abs(facts["n"] ** 2 - facts["entries_approx"]) <= facts["relative_rounding"] * facts["entries_approx"]


def test_window_at_least_n_is_full_causal():
    rng = np.random.default_rng(4)
    n = 40
    Q, K, V = _rand(rng, 1, 1, n, 4), _rand(rng, 1, 1, n, 4), _rand(rng, 1, 1, n, 4)
    O1, L1 = prefill(Q, K, V, n + 5, 0, True)
    O2, L2 = prefill(Q, K, V, -1, 0, True)
    np.testing.assert_array_equal(O1, O2)
    o_ref, lse_ref = _torch_ref(Q[0, 0], K[0, 0], V[0, 0], np.tril(np.ones((n, n), bool)), 0.5)
    np.testing.assert_allclose(O1[0, 0], o_ref, atol=1e-12)


def test_swa_window_cost_shape(golden_dir):
    """Band pair count grows like n*w, not n^2 (SWA glossary comparison table)."""
    w = json.load(open(os.path.join(golden_dir, "pages_printed.json")))["swa_cost_shape"]["mistral_window"]
    for n in (2 * w, 4 * w):
        total, _ = _pair_count(n, tile=2048, window_left=w - 1, window_right=0, causal=True)
        assert n * w - w * w / 2 <= total <= n * w


def test_causal_with_globals_is_refused():
    with pytest.raises(ValueError):
        prefill_allowed(np.arange(4), np.arange(4), 2, 0, True, (1,))


def test_dilated_causal_pair_count_closed_form():
    """Dilated SWA (SWA glossary, SWAの拡張手法): w keys at spacing s counted from the
    query.  Row i sees the multiples of s in [i - (w-1)s, i] that are >= 0, i.e.
    min(w, i // s + 1) keys; over n >= s w rows the total is s w (w+1)/2 + (n - s w) w
    (each value q = i // s < w repeats s times)."""
    for n, w, s in ((1000, 7, 3), (4096, 64, 2), (777, 5, 11)):
        total, per_row = _pair_count(n, window_left=(w - 1) * s, window_right=0, causal=True, dilation=s)
        np.testing.assert_array_equal(per_row, np.minimum(w, np.arange(n) // s + 1))
        assert n >= s * w
        assert total == s * w * (w + 1) // 2 + (n - s * w) * w


def test_dilation_one_is_the_plain_band_and_dilated_rows_split_by_residue():
    """Dilation 1 is the plain mask.  With dilation s, rows and keys of one residue
    mod s form a plain band over that subsequence with window floor(wl / s) (and
    floor(wr / s)): i - j = s (i' - j') for i = r + s i', j = r + s j'."""
    rng = np.random.default_rng(5)
    n, d = 203, 16
    q, k, v = (rng.standard_normal((1, 1, n, d)) for _ in range(3))
    for wl, wr, causal in ((60, 0, True), (37, 22, False)):
        a = prefill(q, k, v, wl, wr, causal)
        b = prefill(q, k, v, wl, wr, causal, dilation=1)
        np.testing.assert_array_equal(a[0], b[0])
        s = 4
        O, L = prefill(q, k, v, wl, wr, causal, dilation=s)
        for r in range(s):
            sub = slice(r, None, s)
            Or, Lr = prefill(q[:, :, sub], k[:, :, sub], v[:, :, sub], wl // s, wr // s, causal,
                             scale=1.0 / np.sqrt(d))
            np.testing.assert_allclose(O[0, 0, sub], Or[0, 0], rtol=0, atol=1e-12)
            np.testing.assert_allclose(L[0, 0, sub], Lr[0, 0], rtol=0, atol=1e-12)


def test_dilated_mask_matches_brute_force_and_sdpa():
    """Tiny case: the mask from explicit loops over (i, j), and torch SDPA (float64,
    CPU) under that mask."""
    import torch
    rng = np.random.default_rng(6)
    n, d, wl, s = 40, 8, 14, 3
    allowed = prefill_allowed(np.arange(n), np.arange(n), wl, 0, True, dilation=s)
    brute = np.zeros((n, n), dtype=bool)
    for i in range(n):
        for j in range(n):
            brute[i, j] = j <= i and i - j <= wl and (i - j) % s == 0
    np.testing.assert_array_equal(allowed, brute)
    q, k, v = (rng.standard_normal((1, 1, n, d)) for _ in range(3))
    O, _ = prefill(q, k, v, wl, 0, True, dilation=s)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=torch.from_numpy(brute))
    np.testing.assert_allclose(O, ref.numpy(), rtol=0, atol=1e-12)


def test_dilation_with_globals_is_refused():
    with pytest.raises(ValueError):
        prefill_allowed(np.arange(8), np.arange(8), 4, 4, False, global_pos=(3,), dilation=2)
