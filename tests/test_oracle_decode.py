"""Pins of the oracle's sparse decode (CPU only).

A sparse decode whose token set is everything must equal dense causal
attention (torch SDPA, float64); with any selection it must equal torch SDPA
under a mask built independently from Python sets; permuting tokens inside a
block leaves summaries, scores and outputs unchanged.
"""

import math

import numpy as np
import pytest
import torch

from oracle import block_summaries, decode_step, forced_token_mask, head_scores
from synthetic import WORKLOADS, bf16_bits_to_f32, make_decode_inputs


def _sdpa(q, K, V, allowed_tokens, scale):
    n = K.shape[0]
    mask = torch.zeros(q.shape[0], n, dtype=torch.bool)
    mask[:, list(allowed_tokens)] = True
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(K)[None], torch.from_numpy(V)[None],
        attn_mask=mask[None], scale=scale)
    lse = torch.logsumexp((scale * torch.from_numpy(q) @ torch.from_numpy(K).T).masked_fill(~mask, -math.inf), 1)
    return o[0].numpy(), lse.numpy()


def _inputs(seed, B=2, Hq=4, Hkv=2, n=200, d=8):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((B, Hq, d)), rng.standard_normal((B, Hkv, n, d)), rng.standard_normal((B, Hkv, n, d))


@pytest.mark.parametrize("rank", [0, 2])
def test_k_covering_every_candidate_is_dense_causal(rank):
    Q, K, V = _inputs(0)
    n, S = 200, 16
    res = decode_step(Q, K, V, n, S, rank, top_k=100, window=20, n_sink=4)
    for (b, g), r in res.items():
        assert (r["sel"][r["sel"] >= 0] == r["cand"]).all()
        o, lse = _sdpa(Q[b, 2 * g:2 * g + 2], K[b, g], V[b, g], range(n), 1 / math.sqrt(8))
        # tail tokens 192..199 are in the window, so T is all of [0, n)
        np.testing.assert_allclose(r["o"], o, atol=1e-12)
        np.testing.assert_allclose(r["lse"], lse, atol=1e-12)


def test_window_at_least_n_is_dense_causal():
    Q, K, V = _inputs(1)
    res = decode_step(Q, K, V, 200, 16, 0, top_k=2, window=500, n_sink=0)
    for (b, g), r in res.items():
        assert (r["sel"] == -1).all() and len(r["cand"]) == 0
        o, _ = _sdpa(Q[b, 2 * g:2 * g + 2], K[b, g], V[b, g], range(200), 1 / math.sqrt(8))
        np.testing.assert_allclose(r["o"], o, atol=1e-12)


@pytest.mark.parametrize("globals_", [(), (3, 50, 51, 130, 199)])
def test_sparse_decode_matches_sdpa_on_the_set_union(globals_):
    Q, K, V = _inputs(2)
    n, S, W, ns = 200, 16, 24, 5
    res = decode_step(Q, K, V, n, S, 1, top_k=3, window=W, n_sink=ns, global_pos=globals_)
    for (b, g), r in res.items():
        T = set(range(ns)) | set(range(n - W, n)) | set(globals_)
        for blk in r["sel"]:
            if blk >= 0:
                T |= set(range(blk * S, blk * S + S))
        assert sorted(T) == r["tokens"].tolist()
        o, lse = _sdpa(Q[b, 2 * g:2 * g + 2], K[b, g], V[b, g], sorted(T), 1 / math.sqrt(8))
        np.testing.assert_allclose(r["o"], o, atol=1e-12)
        np.testing.assert_allclose(r["lse"], lse, atol=1e-12)


def test_permuting_tokens_inside_blocks_changes_nothing():
    Q, K, V = _inputs(3, B=1, Hkv=1, Hq=2)
    n, S = 200, 16
    rng = np.random.default_rng(0)
    perm = np.arange(n)
    for b0 in range(0, (n // S) * S, S):
        perm[b0:b0 + S] = b0 + rng.permutation(S)
    K2, V2 = K[:, :, perm], V[:, :, perm]
    kw = dict(n=n, S=S, rank=3, top_k=4, window=8, n_sink=0)
    # window 8 only covers the tail block; permuting inside complete blocks keeps
    # the token set of every block, so T maps onto itself
    r1 = decode_step(Q, K, V, **kw)[(0, 0)]
    r2 = decode_step(Q, K2, V2, **kw)[(0, 0)]
    np.testing.assert_allclose(r1["scores"], r2["scores"], atol=1e-12)
    assert r1["sel"].tolist() == r2["sel"].tolist()
    np.testing.assert_allclose(r1["o"], r2["o"], atol=1e-12)
    m1, f1 = block_summaries(K[0, 0], S, 3)
    m2, f2 = block_summaries(K2[0, 0], S, 3)
    np.testing.assert_allclose(m1, m2, atol=1e-13)
    np.testing.assert_allclose(np.abs(f1), np.abs(f2), atol=1e-10)


def test_tiny_workload_selects_four_of_fourteen():
    w = WORKLOADS["tiny_decode_1k"]
    x = make_decode_inputs(w)
    assert x["Q"].dtype == np.float32 and x["K"].shape == (1, 1, 1024, 64)
    res = decode_step(x["Q"], x["K"], x["V"], w.n_ctx, w.block_size, w.rank, w.top_k, w.window, w.n_sink)
    r = res[(0, 0)]
    assert len(r["cand"]) == 14 and (r["sel"] >= 1).all() and (r["sel"] <= 14).all()
    assert len(r["tokens"]) == 64 * 6
    # the chosen blocks are the four best by group score among blocks 1..14
    best = np.argsort(-r["scores"][1:15], kind="stable")[:4] + 1
    assert sorted(best.tolist()) == r["sel"].tolist()


def test_needles_are_found_by_the_intended_selector():
    """Workload realism, not parity: shifted needles lift the mean score; spread needles
    keep the mean and lift only the second-order term."""
    w = WORKLOADS["first_order_decode_32k"].scaled(batch=1, n_kv_heads=2, n_q_heads=8, n_ctx=4096,
                                                 top_k=4)
    x = make_decode_inputs(w)
    Q, K = bf16_bits_to_f32(x["Q"]), bf16_bits_to_f32(x["K"])
    res = decode_step(Q, K, K, w.n_ctx, 64, 0, w.top_k, w.window, w.n_sink)
    hits = [len(set(res[(0, g)]["sel"].tolist()) & set(x["needles"][0].tolist())) for g in range(2)]
    assert sum(hits) >= 4  # chance level is about 0.6 of 8
    w2 = WORKLOADS["cobs_decode_128k"].scaled(batch=1, n_kv_heads=1, n_q_heads=8, n_ctx=8192, top_k=4)
    x2 = make_decode_inputs(w2)
    Q2, K2 = bf16_bits_to_f32(x2["Q"]), bf16_bits_to_f32(x2["K"])
    r2 = decode_step(Q2, K2, K2, w2.n_ctx, 64, 4, w2.top_k, w2.window, w2.n_sink)[(0, 0)]
    r1 = decode_step(Q2, K2, K2, w2.n_ctx, 64, 0, w2.top_k, w2.window, w2.n_sink)[(0, 0)]
    needles = set(x2["needles"][0].tolist())
    assert len(set(r2["sel"].tolist()) & needles) >= 3
    assert len(set(r1["sel"].tolist()) & needles) <= 1
