"""Pins of the oracle's block summaries, scores, candidates and top-k (CPU only).

The pins come from outside the oracle's own code: exact identities of the
cumulant expansion (single-token blocks, a two-point block in closed form,
the O(eps^3) remainder), numpy's covariance routine, torch's softmax, planted
spectra with known eigenpairs, and brute force over all subsets.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (E2M1_MAGNITUDES, block_summaries, candidate_blocks, dequantize_e2m1_rows,
                    exact_mass_scores, forced_token_mask, group_scores, head_scores,
                    quantize_e2m1_rows, round_to_bf16, top_k_blocks, query_subspace_basis)
from synthetic import WORKLOADS


# ---------------------------------------------------------------- bf16 storage of the mean


def test_bf16_rounding_worked_cases():
    """bfloat16 keeps 8 significant bits: near 1 the spacing is 2^-7.  Halfway cases go
    to the even last bit: 1 + 2^-8 -> 1 (even), 1 + 3 * 2^-8 -> 1 + 2^-6 (even), and a
    hair above a halfway point rounds up."""
    x = np.array([1.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -30,
                  -(1 + 2.0 ** -8), 0.0, 3.0, 2.0 ** -20 * (1 + 2.0 ** -9), 255.5, 256.5])
    want = np.array([1.0, 1.0, 1 + 2.0 ** -6, 1 + 2.0 ** -7, -1.0, 0.0, 3.0, 2.0 ** -20,
                     256.0, 256.0])
    assert np.array_equal(round_to_bf16(x), want)


def test_bf16_rounding_matches_torch_on_float32_values():
    """On values that float32 holds exactly, rounding float64 straight to bfloat16 is
    torch's float32 -> bfloat16 conversion (round to nearest, ties to even)."""
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, 20000),
                        (rng.integers(-2 ** 15, 2 ** 15, 5000) + 0.5) * 2.0 ** -7]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(round_to_bf16(x.astype(np.float64)), want)


def test_bf16_mean_is_the_rounded_mean_and_leaves_the_factor():
    rng = np.random.default_rng(4)
    K = rng.standard_normal((4 * 16, 8))
    m32, f32 = block_summaries(K, 16, 3)
    m16, f16 = block_summaries(K, 16, 3, mean_bf16=True)
    assert np.array_equal(m16, round_to_bf16(m32))
    assert np.array_equal(f16, f32)
    assert np.all(np.abs(m16 - m32) <= np.abs(m32) * 2.0 ** -8)
    assert not np.array_equal(m16, m32)


# ---------------------------------------------------------------- FP4 (E2M1) storage of the factor


def test_e2m1_magnitudes_follow_the_format():
    """E2M1: 2 exponent bits with bias 1 and 1 mantissa bit; exponent 0 is subnormal
    (0.5 * m), otherwise 2^(e-1) * (1 + m/2)."""
    want = []
    for code in range(8):
        e, m = code >> 1, code & 1
        want.append(0.5 * m if e == 0 else 2.0 ** (e - 1) * (1 + m / 2))
    assert np.array_equal(E2M1_MAGNITUDES, np.array(want))


def test_e2m1_worked_cases():
    """Scale 1 (the row's largest magnitude is 6).  Midpoints go to the even code:
    0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4."""
    row = np.array([[6.0, 0.25, 0.75, 1.25, -1.75, 2.5, 3.5, 5.0, -5.0001, 0.0, -0.1, 0.26]])
    codes, scale = quantize_e2m1_rows(row)
    assert scale[0] == np.float32(1.0)
    assert codes[0].tolist() == [7, 0, 2, 2, 8 | 4, 4, 6, 6, 8 | 7, 0, 0, 1]
    assert np.array_equal(dequantize_e2m1_rows(codes, scale)[0],
                          [6, 0, 1, 1, -2, 2, 4, 4, -6, 0, 0, 0.5])


def test_e2m1_matches_the_midpoint_rule_on_random_rows():
    """An independent statement of the same rounding: the magnitude code counts the
    midpoints below |v| (k even: strictly below; k odd: at or below, so a tie lands
    on the even code)."""
    rng = np.random.default_rng(7)
    rows = rng.standard_normal((200, 128)) * rng.gamma(1.0, 1.0, (200, 1))
    rows[:20, :8] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0]) * (np.abs(rows[:20, 8:]).max(axis=1, keepdims=True) / 6.0)
    codes, scale = quantize_e2m1_rows(rows)
    x32 = rows.astype(np.float32)
    v = (x32 / scale[:, None]).astype(np.float32).astype(np.float64)
    a = np.abs(v)
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    mag = sum(((a > m) if k % 2 == 0 else (a >= m)).astype(int) for k, m in enumerate(mids))
    assert np.array_equal(codes & 7, mag)
    assert np.array_equal((codes >> 3).astype(bool), (v < 0) & (mag > 0))


def test_e2m1_rows_keep_their_maximum_and_half_a_step():
    rng = np.random.default_rng(8)
    rows = rng.standard_normal((50, 64)) * 3.0
    codes, scale = quantize_e2m1_rows(rows)
    deq = dequantize_e2m1_rows(codes, scale)
    big = np.argmax(np.abs(rows), axis=1)
    assert np.all((codes[np.arange(50), big] & 7) == 7)  # the largest entry is +-6 * scale
    # error at most half the spacing around the value (spacing 0.5, 1 or 2 times the scale)
    spacing = np.where(np.abs(deq) < 2 * scale[:, None], 0.5, np.where(np.abs(deq) < 4 * scale[:, None], 1.0, 2.0))
    assert np.all(np.abs(deq - rows) <= (0.5 * spacing + 1e-6) * scale[:, None])
    c2, s2 = quantize_e2m1_rows(-rows)
    assert np.array_equal(s2, scale) and np.array_equal(c2 & 7, codes & 7)
    zero_c, zero_s = quantize_e2m1_rows(np.zeros((2, 8)))
    assert np.all(zero_c == 0) and np.all(zero_s == 0)


def test_fp4_factor_is_the_dequantized_factor():
    rng = np.random.default_rng(9)
    K = rng.standard_normal((4 * 16, 8))
    m0, f0 = block_summaries(K, 16, 3)
    m1, f1 = block_summaries(K, 16, 3, factor_fp4=True)
    assert np.array_equal(m0, m1)
    assert np.array_equal(f1, dequantize_e2m1_rows(*quantize_e2m1_rows(f0)))


# ---------------------------------------------------------------- summaries


def test_factor_rows_are_eigenpairs_of_the_population_covariance():
    rng = np.random.default_rng(0)
    S, d, r = 16, 8, 4
    K = rng.standard_normal((3 * S, d))
    mean, factor = block_summaries(K, S, r)
    for b in range(3):
        X = K[b * S:(b + 1) * S]
        np.testing.assert_allclose(mean[b], X.mean(axis=0), atol=1e-15)
        cov = np.cov(X, rowvar=False, bias=True)  # 1/L normalisation
        lam = np.einsum("id,id->i", factor[b], factor[b])
        assert np.all(np.diff(lam) <= 1e-12), "eigenvalues must be descending"
        for i in range(r):
            v = factor[b, i] / math.sqrt(lam[i])
            np.testing.assert_allclose(cov @ v, lam[i] * v, atol=1e-12)
            assert abs(np.linalg.norm(v) - 1) < 1e-12
            assert factor[b, i][np.argmax(np.abs(factor[b, i]))] > 0
        gram = factor[b] @ factor[b].T
        np.testing.assert_allclose(gram - np.diag(np.diag(gram)), 0, atol=1e-12)
        # the top-r eigenvalues of numpy's covariance, from a separate routine
        ref = np.sort(np.linalg.eigvalsh(cov))[::-1][:r]
        np.testing.assert_allclose(lam, ref, atol=1e-12)


def test_full_rank_factor_reproduces_the_trace_and_matrix():
    rng = np.random.default_rng(1)
    S, d = 16, 6
    K = rng.standard_normal((S, d))
    _, factor = block_summaries(K, S, d)
    cov = np.cov(K, rowvar=False, bias=True)
    np.testing.assert_allclose(factor[0].T @ factor[0], cov, atol=1e-12)
    assert abs((factor[0] ** 2).sum() - np.trace(cov)) < 1e-12


def test_planted_spike_closed_form():
    """Keys mu + a_r u: mean mu + mean(a) u, one eigenpair (var(a), u), the rest zero."""
    rng = np.random.default_rng(2)
    S, d = 64, 16
    mu = rng.standard_normal(d)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    a = rng.standard_normal(S) * 3
    K = mu[None, :] + a[:, None] * u[None, :]
    mean, factor = block_summaries(K, S, 3)
    np.testing.assert_allclose(mean[0], mu + a.mean() * u, atol=1e-13)
    var = ((a - a.mean()) ** 2).mean()
    expect = math.sqrt(var) * u * np.sign(u[np.argmax(np.abs(u))])
    np.testing.assert_allclose(factor[0, 0], expect, atol=1e-12)
    np.testing.assert_allclose(factor[0, 1:], 0, atol=1e-7)


def test_rank_is_at_most_block_length_minus_one():
    rng = np.random.default_rng(3)
    S, d = 4, 10
    K = rng.standard_normal((S, d))
    _, factor = block_summaries(K, S, 8)
    lam = (factor[0] ** 2).sum(axis=1)
    assert (lam[: S - 1] > 1e-6).all()
    np.testing.assert_allclose(lam[S - 1:], 0, atol=1e-12)


# ---------------------------------------------------------------- scores


def test_single_token_blocks_make_every_score_the_exact_log_mass():
    """S = 1: mean = k, covariance 0, so first order = second order = ln exp(q.k) exactly,
    and the group score is torch's logsumexp of the group's scaled logits."""
    rng = np.random.default_rng(4)
    G, n, d = 4, 9, 8
    q = rng.standard_normal((G, d)) / math.sqrt(d)
    K = rng.standard_normal((n, d))
    mean, factor = block_summaries(K, 1, 3)
    s1 = head_scores(q, mean)
    s2 = head_scores(q, mean, factor)
    s_star = exact_mass_scores(q, K, 1)
    np.testing.assert_allclose(s2, s1, atol=1e-15)
    np.testing.assert_allclose(s_star, s1, atol=1e-14)
    ref = torch.logsumexp(torch.from_numpy(q) @ torch.from_numpy(K).T, dim=0).numpy()
    np.testing.assert_allclose(group_scores(s2), ref, atol=1e-13)


def test_exact_mass_matches_torch_softmax_block_sums():
    """exp(s*_b) / sum_b' exp(s*_b') is the softmax weight landing in block b."""
    rng = np.random.default_rng(5)
    n, d, S = 256, 16, 32
    q = rng.standard_normal((1, d)) / 4
    K = rng.standard_normal((n, d))
    s_star = exact_mass_scores(q, K, S)[0]
    p = torch.softmax(torch.from_numpy(q[0]) @ torch.from_numpy(K).T, dim=0).numpy()
    block_mass = p.reshape(-1, S).sum(axis=1)
    frac = np.exp(s_star - s_star.max())
    np.testing.assert_allclose(frac / frac.sum(), block_mass, atol=1e-14)


@pytest.mark.parametrize("delta", [1e-3, 0.05, 0.3, 1.0])
def test_two_point_block_closed_forms(delta):
    """Keys mu +- delta u.  Exact: s* - ln 2 - q.mu = ln cosh(delta q.u).
    COBS second order: s2 - q.mu = 1/2 (delta q.u)^2 (covariance delta^2 u u^T with 1/L)."""
    rng = np.random.default_rng(6)
    d = 8
    mu, u = rng.standard_normal(d), rng.standard_normal(d)
    u /= np.linalg.norm(u)
    q = rng.standard_normal((1, d))
    K = np.vstack([mu + delta * u, mu - delta * u])
    mean, factor = block_summaries(K, 2, 1)
    x = delta * float(q[0] @ u)
    qmu = float(q[0] @ mu)
    s_star = exact_mass_scores(q, K, 2)[0, 0]
    s2 = head_scores(q, mean, factor)[0, 0]
    assert abs((s_star - math.log(2) - qmu) - math.log(math.cosh(x))) < 1e-12
    assert abs((s2 - qmu) - 0.5 * x * x) < 1e-12
    # both agree to leading order: ln cosh x = x^2/2 - x^4/12 + ...
    assert abs((s_star - math.log(2)) - s2) <= x ** 4 / 12 + 1e-12


def test_full_rank_second_order_equals_the_quadratic_form():
    rng = np.random.default_rng(7)
    S, d, G = 32, 8, 3
    K = rng.standard_normal((2 * S, d))
    q = rng.standard_normal((G, d)) / math.sqrt(d)
    mean, factor = block_summaries(K, S, d)
    s2 = head_scores(q, mean, factor)
    for b in range(2):
        cov = np.cov(K[b * S:(b + 1) * S], rowvar=False, bias=True)
        expect = q @ K[b * S:(b + 1) * S].mean(axis=0) + 0.5 * np.einsum("hd,de,he->h", q, cov, q)
        np.testing.assert_allclose(s2[:, b], expect, atol=1e-12)


def test_second_order_remainder_is_third_order_in_the_spread():
    """Keys mu + eps z: s* - ln L - s2 = O(eps^3) (cumulant expansion, COBS explainer 2.2),
    while the first-order remainder is O(eps^2)."""
    rng = np.random.default_rng(8)
    S, d = 64, 8
    mu, Z = rng.standard_normal(d), rng.standard_normal((S, d))
    Z -= Z.mean(axis=0)
    Z[:, 0] += 0.8 * (Z[:, 1] ** 2 - (Z[:, 1] ** 2).mean())  # some skew, so the cubic term is nonzero
    q = rng.standard_normal((1, d))
    res2, res1 = [], []
    for eps in (0.02, 0.01):
        K = mu + eps * Z
        mean, factor = block_summaries(K, S, d)
        s_star = exact_mass_scores(q, K, S)[0, 0]
        res2.append(abs(s_star - math.log(S) - head_scores(q, mean, factor)[0, 0]))
        res1.append(abs(s_star - math.log(S) - head_scores(q, mean)[0, 0]))
    assert 6.0 < res2[0] / res2[1] < 10.0
    assert 3.0 < res1[0] / res1[1] < 5.0


def test_group_score_of_identical_heads_adds_log_g():
    s = np.array([[0.3, -1.0, 2.0]] * 4)
    np.testing.assert_allclose(group_scores(s), s[0] + math.log(4), atol=1e-15)
    np.testing.assert_array_equal(group_scores(s[:1]), s[0])


def test_group_score_is_the_log_of_the_group_exact_mass():
    """With exact masses the group score is the log of the group's total softmax numerator
    over the block: torch logsumexp over (head, token) pairs."""
    rng = np.random.default_rng(9)
    G, n, d, S = 4, 128, 8, 16
    q = rng.standard_normal((G, d)) / math.sqrt(d)
    K = rng.standard_normal((n, d))
    gs = group_scores(exact_mass_scores(q, K, S))
    logits = (torch.from_numpy(q) @ torch.from_numpy(K).T).reshape(G, n // S, S)
    ref = torch.logsumexp(logits.permute(1, 0, 2).reshape(n // S, -1), dim=1).numpy()
    np.testing.assert_allclose(gs, ref, atol=1e-13)


# ---------------------------------------------------------------- forced set and candidates


@pytest.mark.parametrize("name,first,last", [
    ("tiny_decode_1k", 1, 14), ("first_order_decode_32k", 1, 503), ("cobs_decode_128k", 1, 2031)])
def test_candidates_of_the_workloads(name, first, last):
    w = WORKLOADS[name]
    forced = forced_token_mask(w.n_ctx, w.n_sink, w.window)
    cand = candidate_blocks(w.n_ctx, w.block_size, forced)
    np.testing.assert_array_equal(cand, np.arange(first, last + 1))


def test_forced_set_edges():
    f = forced_token_mask(10, 3, 4, (5,))
    assert f.tolist() == [1, 1, 1, 0, 0, 1, 1, 1, 1, 1]
    assert forced_token_mask(5, 100, 0).all()
    assert forced_token_mask(5, 0, 100).all()
    assert not forced_token_mask(5, 0, 0).any()
    with pytest.raises(ValueError):
        forced_token_mask(5, 0, 0, (5,))


def test_candidates_skip_tail_and_fully_forced_blocks():
    S = 4
    # n = 18: blocks 0..3 complete, tokens 16, 17 form a tail block
    forced = forced_token_mask(18, 4, 3, (8, 9, 10, 11, 13))
    # block 0 = sinks (forced), block 2 = globals 8..11 (forced), block 3 has 13 forced only
    assert candidate_blocks(18, S, forced).tolist() == [1, 3]
    assert candidate_blocks(3, S, forced_token_mask(3, 0, 1)).tolist() == []


# ---------------------------------------------------------------- top-k


def _brute_top_k(score, cand, k):
    best = None
    for sub in itertools.combinations(cand, min(k, len(cand))):
        key = (sum(score[b] for b in sub), -sum(sub))
        if best is None or key > best[0]:
            best = (key, sub)
    return sorted(best[1])


@pytest.mark.parametrize("seed", range(6))
def test_top_k_brute_force(seed):
    rng = np.random.default_rng(seed)
    nb = 10
    score = np.round(rng.standard_normal(nb), 1)  # coarse values: ties happen
    cand = np.sort(rng.choice(nb, size=8, replace=False))
    for k in (1, 3, 5, 8, 12):
        got = top_k_blocks(score, cand, k)
        ref = _brute_top_k(score, cand.tolist(), k)
        assert got[: len(ref)].tolist() == ref
        assert (got[len(ref):] == -1).all()


def test_top_k_ties_prefer_lower_index_and_output_ascends():
    score = np.array([1.0, 5.0, 5.0, 5.0, 0.0])
    assert top_k_blocks(score, np.arange(5), 2).tolist() == [1, 2]
    assert top_k_blocks(score, np.array([4, 3, 2]), 2).tolist() == [2, 3]


def test_top_k_with_exact_mass_captures_the_most_attention():
    """Ranking by exact mass (COBS explainer 2.1) maximises the softmax mass kept."""
    rng = np.random.default_rng(12)
    n, d, S = 96, 8, 8
    q = rng.standard_normal((1, d)) / 2
    K = rng.standard_normal((n, d))
    s_star = exact_mass_scores(q, K, S)[0]
    p = torch.softmax(torch.from_numpy(q[0]) @ torch.from_numpy(K).T, dim=0).numpy().reshape(-1, S).sum(1)
    cand = np.arange(n // S)
    got = top_k_blocks(s_star, cand, 3)
    best = max(itertools.combinations(cand, 3), key=lambda sub: p[list(sub)].sum())
    assert got.tolist() == sorted(best)


def test_rank_guidance_of_the_page(golden_dir):
    facts = json.load(open(os.path.join(golden_dir, "pages_printed.json")))
    assert WORKLOADS["cobs_decode_128k"].rank <= facts["cobs_rank_guidance"]["max_rank"]


# --- query-subspace projection (COBS explainer 2.3, covariance compression) ---

def _orthonormal_rows(rng, s, d):
    q, _ = np.linalg.qr(rng.standard_normal((d, s)))
    return q.T  # [s, d]


def test_identity_basis_reproduces_the_unprojected_summaries():
    rng = np.random.default_rng(40)
    K = rng.standard_normal((5 * 16, 12)) * rng.uniform(0.2, 3.0, 12)
    m0, f0 = block_summaries(K, 16, 3)
    m1, f1 = block_summaries(K, 16, 3, basis=np.eye(12))
    np.testing.assert_allclose(m1, m0, rtol=0, atol=0)
    np.testing.assert_allclose(f1, f0, rtol=1e-12, atol=1e-12)
    q = rng.standard_normal((3, 12))
    np.testing.assert_allclose(head_scores(q, m1, f1, basis=np.eye(12)), head_scores(q, m0, f0),
                               rtol=1e-12, atol=1e-12)


def test_permutation_basis_permutes_the_factor_entries():
    """Basis rows e_{pi(0)}, e_{pi(1)}, ...: the projected key has entries k[pi(j)], so
    factor entry j is the unprojected entry pi(j).  A transposed projection (keys times
    P instead of P^T) would apply the inverse permutation and fail."""
    rng = np.random.default_rng(41)
    d = 10
    perm = np.array([3, 7, 0, 9, 1, 5, 2, 8, 4, 6])
    assert not np.array_equal(np.argsort(perm), perm)
    P = np.eye(d)[perm]
    K = rng.standard_normal((4 * 16, d)) * np.linspace(0.5, 2.5, d)
    _, f0 = block_summaries(K, 16, 4)
    _, f1 = block_summaries(K, 16, 4, basis=P)
    np.testing.assert_allclose(f1, f0[:, :, perm], rtol=1e-12, atol=1e-12)


def test_projected_second_order_term_equals_the_key_average_in_the_subspace():
    """For a query inside the subspace (q = P^T z) and rank = s, the projected term
    1/2 sum_i (factor_i . P q)^2 is 1/2 q^T Sigma q = 1/2 mean_r (q . (k_r - mean))^2,
    computed here straight from the keys."""
    rng = np.random.default_rng(42)
    d, s, S = 16, 6, 32
    P = _orthonormal_rows(rng, s, d)
    K = rng.standard_normal((3 * S, d)) * np.linspace(0.3, 2.0, d)
    mean, factor = block_summaries(K, S, s, basis=P)
    z = rng.standard_normal((2, s))
    q = z @ P
    got = head_scores(q, mean, factor, basis=P)
    for b in range(3):
        X = K[b * S:(b + 1) * S]
        mu = X.sum(0) / S
        for h in range(2):
            quad = sum(float(np.dot(q[h], x - mu)) ** 2 for x in X) / S
            assert got[h, b] == pytest.approx(float(q[h] @ mu) + 0.5 * quad, rel=1e-10, abs=1e-12)
    # a query outside the subspace only sees its component inside it
    q_out = q + rng.standard_normal((2, d)) @ (np.eye(d) - P.T @ P)
    np.testing.assert_allclose(head_scores(q_out, mean, factor, basis=P) - q_out @ mean.T,
                               got - q @ mean.T, rtol=1e-10, atol=1e-12)


def test_query_subspace_basis_recovers_a_planted_subspace():
    """Queries q = U z with orthonormal U [d, s0] and independent z_j of variances
    9 > 4 > 1: the basis spans U, in variance order, with orthonormal rows."""
    rng = np.random.default_rng(43)
    d, s0, N = 12, 3, 4000
    U = _orthonormal_rows(rng, s0, d).T
    z = rng.standard_normal((N, s0)) * np.array([3.0, 2.0, 1.0])
    z -= z.mean(0)
    z = z @ np.linalg.inv(np.linalg.cholesky(z.T @ z / N)).T * np.array([3.0, 2.0, 1.0])
    Q = z @ U.T
    P = query_subspace_basis(Q, s0)
    np.testing.assert_allclose(P @ P.T, np.eye(s0), atol=1e-12)
    np.testing.assert_allclose(P.T @ P, U @ U.T, atol=1e-10)
    for j in range(s0):
        assert abs(float(P[j] @ U[:, j])) == pytest.approx(1.0, abs=1e-10)
        assert P[j, np.argmax(np.abs(P[j]))] > 0
    # a wider basis keeps the planted rows first
    P5 = query_subspace_basis(Q + 1e-3 * rng.standard_normal((N, d)), 5)
    np.testing.assert_allclose(P5[:s0].T @ P5[:s0], U @ U.T, atol=2e-4)  # noise 1e-3: measured 2.8e-5


def test_projected_fp4_factor_rows_have_s_entries():
    rng = np.random.default_rng(44)
    d, s, S = 16, 8, 32
    P = _orthonormal_rows(rng, s, d)
    K = rng.standard_normal((2 * S, d))
    _, f = block_summaries(K, S, 3, basis=P)
    _, f4 = block_summaries(K, S, 3, basis=P, factor_fp4=True)
    assert f.shape == f4.shape == (2, 3, s)
    codes, scale = quantize_e2m1_rows(f)
    np.testing.assert_allclose(f4, dequantize_e2m1_rows(codes, scale), rtol=0, atol=0)
