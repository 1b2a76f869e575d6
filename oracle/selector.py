"""Block summaries, block scores, candidates and top-k selection (float64, CPU).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The method, as the COBS explainer states it:

* Keys are grouped into contiguous, non-overlapping blocks (technical summary
  section 1; section 5 names "non-overlapping blocks").  Block b holds tokens
  [b*S, (b+1)*S).  Only complete blocks have a summary; the reading is that a
  partly filled tail block is never a candidate and its tokens are reached only
  through the window.
* Selection oracle (section 2.1): the ideal ranking orders blocks by their
  attention mass m_b = sum over the block's keys of exp(q.k).  The explainer
  prints the exponent without the softmax scale; the reading taken is that the
  mass is the one of the attention actually run, so q is scaled by 1/sqrt(d)
  first (attention glossary, step 2).  ``exact_mass_scores`` is this ranking.
* Cumulant expansion (section 2.2): ln m_b = ln L + q.kappa1 + 1/2 q^T kappa2 q + ...
  with kappa1 the block's mean key and kappa2 its key covariance.  The
  reading of L is the number of keys in the block (the expansion is that of
  the log of a sum of L exponentials); it is the same for every complete
  block, so it is dropped from the score, as the COBS score drops it.  kappa2
  is the second cumulant of the block's empirical key distribution, so it is
  normalised by 1/L (not 1/(L-1)).
* First-order score (section 2.2): q.mean.  Second-order COBS score
  (section 2.3): q.mean + 1/2 q^T Sigma q, with Sigma replaced by its top-r
  eigenpairs (low-rank factorisation, section 2.3): 1/2 sum_i lambda_i (v_i.q)^2.
  The factor is stored as rows sqrt(lambda_i) v_i; r <= 8 (section 4.3).
* Grouped heads (attention glossary FAQ Q2: query heads share a K/V head).
  Reading: one block set per K/V head, ranked by the log of the group's summed
  mass, ln sum_h m_{b,h}; each m_{b,h} is estimated by exp(score_{b,h}).
* Forced tokens (SWA glossary "SWAの拡張手法": sink tokens always attended;
  sliding window; local-global glossary: global tokens).  The decode query is
  the last cached token t = n - 1 and the window [t-W+1, t] contains it.
  Candidates are complete blocks with at least one token outside the forced
  set; the top-k are chosen among them, in addition to the forced tokens.
* Top-k: largest group score first, equal scores broken by the lower block
  index; the chosen indices are returned in ascending order, padded with -1
  when there are fewer than k candidates.
* Stored summary precision (section 2.3, compression): the explainer keeps the
  block mean in BF16.  ``block_summaries(..., mean_bf16=True)`` returns the
  mean rounded to the nearest BF16 value (ties to even); the covariance is
  still that of the block's keys about their exact mean (the rounding is a
  storage step, applied after the summary is computed).
* The same section stores the eigenvectors in FP4 (E2M1) with a scale.  Reading:
  one float32 scale per factor row (the row's largest magnitude over 6, the
  largest E2M1 value) and each entry stored as the E2M1 value nearest to
  entry / scale (ties to the even code); the arithmetic of that decision is
  float32.  ``quantize_e2m1_rows`` / ``dequantize_e2m1_rows``;
  ``block_summaries(..., factor_fp4=True)`` returns the dequantized factor.
* Subspace projection (same section): the covariance is projected onto the
  subspace spanned by the leading eigenvectors of the queries' second moment,
  so a factor row holds s numbers instead of d.  Readings: the second moment is
  the uncentred M = (1/N) sum q q^T of a calibration sample of the group's
  queries (one subspace per K/V head; the explainer's s is chosen per layer),
  taken offline; its s leading eigenvectors are the rows of an orthonormal
  basis P [s, d] (``query_subspace_basis``).  The projected covariance is
  P Sigma P^T, i.e. the covariance of the projected centred keys P (k - mean);
  the factor rows are its top-r eigenpairs sqrt(lambda_i) v_i (s numbers, the
  same sign rule), and the score's second-order term uses the projected query
  P q: 1/2 sum_i (factor_i . P q)^2.  The mean stays d-dimensional.
"""

from __future__ import annotations

import numpy as np


# E2M1 (FP4): sign bit, 2 exponent bits (bias 1), 1 mantissa bit.  Magnitude
# codes 0..7 in order: 0, 0.5 (subnormal), 1, 1.5, 2, 3, 4, 6.
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def quantize_e2m1_rows(rows):
    """FP4 E2M1 codes of factor rows with one scale per row.

    rows [..., d] (float64).  In float32, as the stored factor is float32:
    amax = max |x| over the row, scale = amax / 6, v = x / scale.  The code's
    magnitude is the E2M1 value nearest to |v| (on a tie, the even code: the one
    whose mantissa bit is 0), its sign bit (8) is set when v < 0 and the magnitude
    is not 0.  A row of zeros gets scale 0 and codes 0.  Returns (codes uint8
    [..., d] in 0..15, scale float32 [...]).
    """
    x = np.asarray(rows, dtype=np.float64).astype(np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = (amax / np.float32(6.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    v = np.where(scale[..., None] > 0, x / safe[..., None], np.float32(0.0)).astype(np.float32)
    a = np.abs(v.astype(np.float64))
    # nearest magnitude, written out: distance to each of the 8 values, ties to even
    dist = np.abs(a[..., None] - E2M1_MAGNITUDES)
    best = dist.min(axis=-1, keepdims=True)
    near = dist == best
    even = near & (np.arange(8) % 2 == 0)
    idx = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(near, axis=-1))
    sign = ((v < 0) & (idx > 0)).astype(np.uint8)
    return (idx.astype(np.uint8) | (sign << 3)), scale


def dequantize_e2m1_rows(codes, scale):
    """Float64 values of E2M1 codes [..., d] with their row scales [...]."""
    codes = np.asarray(codes, dtype=np.uint8)
    mag = E2M1_MAGNITUDES[codes & 7]
    val = np.where(codes & 8, -mag, mag)
    return val * np.asarray(scale, dtype=np.float64)[..., None]


def round_to_bf16(x):
    """Nearest bfloat16 value of each entry of ``x`` (as float64), ties to even.

    bfloat16 keeps 8 significant bits (1 implicit + 7 stored) and float32's
    exponent range.  With x = m * 2^e, 0.5 <= |m| < 1 (frexp), the nearest value
    with 8 significant bits is rint(m * 2^8) * 2^(e - 8); numpy's rint rounds
    halves to even, which is the ties-to-even rule on the last kept bit.  Inputs
    here are finite and far from the float32 overflow and subnormal range.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def query_subspace_basis(Q_sample, s):
    """Orthonormal rows P [s, d] spanning the query subspace of a calibration sample.

    The s leading eigenvectors (eigenvalue descending) of the uncentred second
    moment M = (1/N) sum_n q_n q_n^T of ``Q_sample`` [N, d] (COBS explainer section
    2.3, subspace projection).  Each row's sign is fixed as for factor rows: its entry
    of largest magnitude (first on ties) is positive.
    """
    Q = np.asarray(Q_sample, dtype=np.float64)
    d = Q.shape[1]
    if not 0 < s <= d:
        raise ValueError("s must be in [1, d]")
    M = Q.T @ Q / Q.shape[0]
    _, vec = np.linalg.eigh(M)  # ascending
    P = vec[:, ::-1][:, :s].T
    big = np.argmax(np.abs(P), axis=1)
    sign = np.sign(P[np.arange(s), big])
    sign[sign == 0] = 1.0
    return P * sign[:, None]


def block_summaries(K, S, rank, mean_bf16=False, factor_fp4=False, basis=None):
    """Per complete block of ``K`` [n, d]: mean [NB, d] and low-rank factor [NB, rank, d].

    factor[b, i] = sqrt(lambda_i) * v_i for the i-th largest eigenpair of the block's
    covariance Sigma_b = (1/L) sum_r (k_r - mean)(k_r - mean)^T, L = S.  Eigenvalues below
    zero (rounding) are clamped to 0.  Each row's sign is fixed so that its entry of
    largest magnitude (first such entry on ties) is positive; the sign never changes a
    score because the score only uses squares of projections.  With ``mean_bf16`` the
    returned mean is rounded to bfloat16 (``round_to_bf16``); with ``factor_fp4`` the
    returned factor is its FP4 storage, dequantized (``quantize_e2m1_rows``).  With a
    ``basis`` P [s, d] the covariance is the projected P Sigma_b P^T (that of the
    projected centred keys P (k - mean)) and the factor is [NB, rank, s].
    """
    K = np.asarray(K, dtype=np.float64)
    n, d = K.shape
    nb = n // S
    X = K[: nb * S].reshape(nb, S, d)
    mean = X.mean(axis=1)
    stored = round_to_bf16(mean) if mean_bf16 else mean
    if rank == 0:
        return stored, np.zeros((nb, 0, d))
    C = X - mean[:, None, :]
    if basis is not None:
        P = np.asarray(basis, dtype=np.float64)
        if P.ndim != 2 or P.shape[1] != d:
            raise ValueError("basis must be [s, d]")
        C = C @ P.T  # projected centred keys, [nb, S, s]
    if not 0 < rank <= C.shape[2]:
        raise ValueError("rank must be in [0, d] (or [0, s] with a basis)")
    sigma = np.einsum("brd,bre->bde", C, C) / S
    lam, vec = np.linalg.eigh(sigma)  # ascending; vec[:, :, i] is the i-th eigenvector
    lam = lam[:, ::-1][:, :rank]
    vec = vec[:, :, ::-1][:, :, :rank]
    lam = np.clip(lam, 0.0, None)
    rows = np.transpose(vec, (0, 2, 1)) * np.sqrt(lam)[:, :, None]  # [nb, rank, d]
    big = np.argmax(np.abs(rows), axis=2)
    sign = np.sign(np.take_along_axis(rows, big[:, :, None], axis=2))
    sign[sign == 0] = 1.0
    factor = rows * sign
    if factor_fp4:
        factor = dequantize_e2m1_rows(*quantize_e2m1_rows(factor))
    return stored, factor


def head_scores(q_scaled, mean, factor=None, basis=None):
    """Per-head block scores s[h, b] for scaled queries ``q_scaled`` [G, d].

    First order: q.mean.  With a factor [NB, r, d] (r > 0) the COBS second-order term
    1/2 sum_i (factor_i . q)^2 = 1/2 q^T (sum_i lambda_i v_i v_i^T) q is added.  With a
    ``basis`` P [s, d] the factor rows are s-dimensional and meet the projected query
    P q.
    """
    q = np.asarray(q_scaled, dtype=np.float64)
    s = q @ np.asarray(mean, dtype=np.float64).T
    if factor is not None and factor.shape[1] > 0:
        qf = q if basis is None else q @ np.asarray(basis, dtype=np.float64).T
        proj = np.einsum("hd,brd->hbr", qf, np.asarray(factor, dtype=np.float64))
        s = s + 0.5 * (proj ** 2).sum(axis=2)
    return s


def exact_mass_scores(q_scaled, K, S):
    """Log attention mass of every complete block: s*[h, b] = ln sum_{j in b} exp(q_h.k_j).

    This is the selection oracle's ranking (COBS explainer section 2.1), which reads every
    key; it serves as a reference ranking and a diagnostic, not as a selector on the path.
    """
    q = np.asarray(q_scaled, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    nb = K.shape[0] // S
    logits = (q @ K[: nb * S].T).reshape(q.shape[0], nb, S)
    m = logits.max(axis=2, keepdims=True)
    return (m + np.log(np.exp(logits - m).sum(axis=2, keepdims=True)))[:, :, 0]


def group_scores(s):
    """Group score per block: ln sum_h exp(s[h, b]) over the query heads sharing a K/V head."""
    s = np.asarray(s, dtype=np.float64)
    m = s.max(axis=0)
    return m + np.log(np.exp(s - m).sum(axis=0))


def forced_token_mask(n, n_sink, window, global_pos=()):
    """Tokens every decode step attends: sinks [0, n_sink), window [t-W+1, t], globals.

    t = n - 1 is the query's own position.  Sizes past n are clamped; ``window`` <= 0
    means no window.
    """
    forced = np.zeros(n, dtype=bool)
    forced[: max(0, min(n_sink, n))] = True
    if window > 0:
        t = n - 1
        forced[max(0, t - window + 1): t + 1] = True
    g = np.asarray(global_pos, dtype=np.int64)
    if g.size:
        if g.min() < 0 or g.max() >= n:
            raise ValueError("global position out of range")
        forced[g] = True
    return forced


def candidate_blocks(n, S, forced):
    """Complete blocks ((b+1)*S <= n) holding at least one token outside ``forced``."""
    nb = n // S
    if nb == 0:
        return np.zeros(0, dtype=np.int64)
    not_forced = ~np.asarray(forced[: nb * S]).reshape(nb, S)
    return np.nonzero(not_forced.any(axis=1))[0]


def top_k_blocks(score, cand, k):
    """The k best candidates by (score descending, block index ascending), in ascending order.

    Returns an int64 array of length k padded with -1 when fewer than k candidates exist.
    """
    cand = np.asarray(cand, dtype=np.int64)
    score = np.asarray(score, dtype=np.float64)
    order = sorted(cand.tolist(), key=lambda b: (-score[b], b))
    chosen = sorted(order[:k])
    out = np.full(k, -1, dtype=np.int64)
    out[: len(chosen)] = chosen
    return out
