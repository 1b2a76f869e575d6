"""Helpers for the GPU parity tests: device copies, a full decode step through the
C ABI, and the comparison rules (selected sets with the near-tie allowance,
outputs at max-abs 2e-3)."""

from __future__ import annotations

import math

import numpy as np

import oracle
from synthetic import bf16_bits_to_f32, make_decode_inputs

OUT_TOL = 2e-3       # max-abs on outputs, compared in fp32
TIE_REL = 1e-4       # relative gap of the oracle's k-th and (k+1)-th scores


def torch_mod():
    import torch
    return torch


def to_dev(arr):
    """numpy float32 -> cuda float32; numpy uint16 (bf16 bits) -> cuda bfloat16."""
    torch = torch_mod()
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


def as_f64(arr):
    return (bf16_bits_to_f32(arr) if arr.dtype == np.uint16 else np.asarray(arr, np.float32)).astype(np.float64)


def paged_pools(K, V, page_tokens, seed, spare=5):
    """Scatter contiguous caches K, V [B, Hkv, cap, d] (device tensors, cap a multiple
    of page_tokens) into page pools [n_pages, Hkv, P, d] under a random assignment of
    distinct pages; pages no token maps to hold NaN.  Returns Kp, Vp, the int32 block
    table [B, cap / P] and n_pages."""
    torch = torch_mod()
    B, Hkv, cap, d = K.shape
    P = page_tokens
    mp = cap // P
    n_pages = B * mp + spare
    perm = np.random.default_rng(seed).permutation(n_pages)[:B * mp].reshape(B, mp)
    table = torch.from_numpy(perm.astype(np.int32)).cuda()
    idx = torch.from_numpy(perm.reshape(-1)).cuda().long()
    out = []
    for X in (K, V):
        pool = torch.full((n_pages, Hkv, P, d), float("nan"), dtype=X.dtype, device="cuda")
        pool[idx] = X.reshape(B, Hkv, mp, P, d).permute(0, 2, 1, 3, 4).reshape(B * mp, Hkv, P, d)
        out.append(pool)
    return out[0], out[1], table, n_pages


def gpu_decode_step(api, x, w, kv_capacity=None, nblk_capacity=None, global_pos=(), dev=None,
                    one_call=False, mean_dtype="f32", factor_fp4=False, basis=None, page_tokens=None,
                    page_seed=0):
    """Run summaries -> select/top-k -> decode on the GPU through the binding.

    ``x`` holds Q, K, V numpy arrays (float32 or bf16 bits) of workload ``w``.
    With ``one_call`` the step is bsattn_decode_step (selection and decode in one
    call); otherwise bsattn_select_topk, then bsattn_decode.  ``mean_dtype`` "bf16"
    stores the block means in bfloat16; ``factor_fp4`` the factor rows as FP4 codes
    (returned as ``factor`` uint8 codes plus ``factor_scale``).  ``basis`` [Hkv, s, d]
    (numpy float32) projects the factor rows onto each K/V head's query subspace.
    ``page_tokens`` runs every call on page pools (``paged_pools``) through a block table.
    Returns numpy copies of mean (as float32), factor, scores, sel, O, lse.
    """
    torch = torch_mod()
    B, Hq, Hkv, d, n = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_ctx
    cap = x["K"].shape[2] if kv_capacity is None else kv_capacity
    nb = n // w.block_size
    nbcap = nb if nblk_capacity is None else nblk_capacity
    dev = dev or {}
    Q = dev["Q"] if "Q" in dev else to_dev(x["Q"])
    K = dev["K"] if "K" in dev else to_dev(x["K"])
    V = dev["V"] if "V" in dev else to_dev(x["V"])
    shape = api.make_shape(B, Hq, Hkv, d, n, kv_capacity=cap, dtype=w.dtype)
    pg = None
    if page_tokens is not None:
        K, V, table, n_pages = paged_pools(K, V, page_tokens, page_seed)
        pg = api.paged_kv(table, page_tokens, n_pages)
    mean = torch.full((B, Hkv, max(nbcap, 1), d), float("nan"), device="cuda",
                      dtype=torch.bfloat16 if mean_dtype == "bf16" else torch.float32)
    factor = fscale = bdev = None
    e = d if basis is None else basis.shape[1]
    if basis is not None:
        bdev = torch.from_numpy(np.ascontiguousarray(basis, dtype=np.float32)).cuda()
    if w.rank > 0 and factor_fp4:
        factor = torch.full((B, Hkv, max(nbcap, 1), w.rank, e // 2), 255, dtype=torch.uint8, device="cuda")
        fscale = torch.full((B, Hkv, max(nbcap, 1), w.rank), float("nan"), device="cuda")
    elif w.rank > 0:
        factor = torch.full((B, Hkv, max(nbcap, 1), w.rank, e), float("nan"), device="cuda")
    api.bsattn_build_summaries(shape, K, w.rank, 0, nb, max(nbcap, 1), mean, factor, factor_scale=fscale,
                               basis=bdev, paged=pg)
    scores = torch.full((B, Hkv, max(nbcap, 1)), float("nan"), device="cuda")
    sel = torch.full((B, Hkv, w.top_k), -7, dtype=torch.int32, device="cuda")
    O = torch.full((B, Hq, d), float("nan"), device="cuda")
    lse = torch.full((B, Hq), float("nan"), device="cuda")
    gp = list(global_pos)
    nbytes = api.bsattn_decode_workspace_bytes(shape, w.top_k, w.window, w.n_sink, len(gp))
    ws = torch.full((nbytes,), 255, dtype=torch.uint8, device="cuda")  # garbage contents
    if one_call:
        api.bsattn_decode_step(shape, Q, K, V, mean, factor, w.rank, max(nbcap, 1), w.top_k, w.window,
                               w.n_sink, gp, sel, scores, O, lse, ws, factor_scale=fscale, basis=bdev, paged=pg)
    else:
        api.bsattn_select_topk(shape, Q, mean, factor, w.rank, max(nbcap, 1), w.top_k, w.window,
                               w.n_sink, gp, sel, scores, factor_scale=fscale, basis=bdev)
        api.bsattn_decode(shape, Q, K, V, sel, w.top_k, w.window, w.n_sink, gp, O, lse, ws, paged=pg)
    torch.cuda.synchronize()
    return dict(mean=mean.float().cpu().numpy(), factor=None if factor is None else factor.cpu().numpy(),
                factor_scale=None if fscale is None else fscale.cpu().numpy(),
                scores=scores.cpu().numpy(), sel=sel.cpu().numpy(), O=O.cpu().numpy(),
                lse=lse.cpu().numpy())


def compare_selection(sel_gpu, scores_oracle, cand, k):
    """True/False for a (b, kv head) pair, plus whether the oracle has a near tie at k.

    Sets must be identical, except at a near tie (relative gap of the oracle's k-th and
    (k+1)-th candidate scores < 1e-4), where only blocks whose oracle scores lie in the
    tie band may differ.
    """
    ref = oracle.top_k_blocks(scores_oracle, cand, k)
    got = np.asarray(sel_gpu)
    valid = got[got >= 0]
    if len(valid) and (np.any(np.diff(valid) <= 0) or np.any(got[len(valid):] >= 0)):
        return False, False  # not ascending / padding not at the end
    if np.array_equal(got, ref):
        return True, False
    if len(cand) <= k:
        return False, False
    cs = np.sort(scores_oracle[cand])[::-1]
    sk, sk1 = cs[k - 1], cs[k]
    scale = max(abs(sk), abs(sk1))
    near = abs(sk - sk1) <= TIE_REL * scale
    if not near:
        return False, False
    diff = set(valid.tolist()) ^ set(ref[ref >= 0].tolist())
    lo, hi = sk1 - TIE_REL * scale, sk + TIE_REL * scale
    ok = all(lo <= scores_oracle[b] <= hi for b in diff) and len(valid) == len(ref[ref >= 0])
    return ok, True


def oracle_decode_with_sel(q, Kbg, Vbg, n, S, window, n_sink, global_pos, sel, scale):
    """Oracle output for a given selected set (the output is unique given the set)."""
    forced = oracle.forced_token_mask(n, n_sink, window, global_pos)
    tokens = oracle.decode_token_set(n, S, forced, sel)
    return oracle.sparse_decode_group(q, Kbg[:n], Vbg[:n], tokens, scale)


def bf16_ulp(x):
    """Spacing of bfloat16 values at |x| (8 significant bits)."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(np.where(x > 0, x, 1.0))
    return np.ldexp(1.0, e - 8)


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)))) if np.size(a) else 0.0


def default_scale(d):
    return 1.0 / math.sqrt(d)


# ----------------------------------------------------------------------------- summaries
# A block's rank-r factor is unique (up to the row signs the sign rule fixes) only
# when its top r + 1 eigenvalues are separated.  Where neighbouring eigenvalues
# nearly coincide, every rotation inside their eigenspace is a correct result
# (several correct factors), and where such a cluster straddles the cut between
# rank r and r + 1 the choice also changes the score.  The checks below accept
# exactly the correct results: a factor row of a separated eigenvalue must match
# the oracle's row; a row of a cluster must lie in the cluster's eigenspace with a
# norm between the cluster's extreme sqrt(lambda); and each block's group score
# must lie in the interval of scores that the correct factors give.

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
# half-width of the values that round to each E2M1 magnitude code (in scale
# units): 0 <- [0, .25], 0.5 <- [.25, .75], ..., 4 <- [3.5, 5], 6 <- [5, 6]
E2M1_HALF = np.array([0.25, 0.25, 0.25, 0.25, 0.5, 0.5, 1.0, 1.0])
CLUSTER_TAU = 1e-4   # neighbouring eigenvalues closer than this (relative to lambda_1) form a cluster


def unpack_fp4(codes, scale):
    """Packed FP4 codes [..., e/2] (entry 2i in the low nibble) with row scales [...]:
    float64 values [..., e] and the 4-bit codes [..., e]."""
    codes = np.asarray(codes)
    c = np.stack([codes & 15, codes >> 4], axis=-1).reshape(*codes.shape[:-1], -1)
    val = np.where(c & 8, -E2M1[c & 7], E2M1[c & 7]) * np.asarray(scale, np.float64)[..., None]
    return val, c


def block_spectra(Kbg, nb, S, basis=None):
    """Full spectrum of every complete block's covariance (projected onto ``basis``
    [s, d] when given), from the S x S Gram of the centred keys: eigenvalues
    lam [nb, S] descending and unit eigenvectors vec [nb, e, S] (columns; zero
    for a zero eigenvalue).  Float64; an independent route to the oracle's eigh."""
    X = np.asarray(Kbg[:nb * S], np.float64).reshape(nb, S, -1)
    C = X - X.mean(axis=1, keepdims=True)
    if basis is not None:
        C = C @ np.asarray(basis, np.float64).T
    Gm = np.einsum("brd,bsd->brs", C, C) / S
    lam, w = np.linalg.eigh(Gm)
    lam, w = np.clip(lam[:, ::-1], 0.0, None), w[:, :, ::-1]
    vec = np.einsum("brd,brj->bdj", C, w) / np.sqrt(S)
    norm = np.sqrt(np.maximum(lam, 0.0))
    vec = np.where(norm[:, None, :] > 1e-150, vec / np.where(norm > 1e-150, norm, 1.0)[:, None, :], 0.0)
    return lam, vec


def eig_cluster(lam_row, i, tau=CLUSTER_TAU):
    """Index range [a, c) of the run of neighbouring eigenvalues, each within
    tau * lam[0] of the next, that holds eigenvalue i."""
    eps = tau * max(lam_row[0], 1e-300)
    a = i
    while a > 0 and lam_row[a - 1] - lam_row[a] < eps:
        a -= 1
    c = i + 1
    while c < len(lam_row) and lam_row[c - 1] - lam_row[c] < eps:
        c += 1
    return a, c


def score_intervals(qs, mean, lam, vec, r, basis=None, row_err=None, tau=CLUSTER_TAU):
    """Interval [lo, hi] of the group score of every block over all correct rank-r
    factors, for scaled queries ``qs`` [G, d] and stored means [nb, d].

    Per head: q.mean + sum over eigenvalue clusters C = [a, c) that meet the top r
    of the range of 1/2 sum_{rows in C} lambda' (v'.q)^2: a cluster wholly inside the
    top r gives [1/2 lam_{c-1} |V_C^T q|^2, 1/2 lam_a |V_C^T q|^2] (a singleton: the
    exact 1/2 lam (v.q)^2); a cluster that straddles rank r keeps m < c - a rows and
    gives [0, 1/2 lam_a |V_C^T q|^2].  ``row_err`` [nb, r, G] widens each row's
    projection by a bound on its storage error e (FP4): |(p+e)^2 - p^2| / 2 <=
    (|p| + |e|/2) |e| with |p| <= sqrt(lam_a) |V_C^T q|.  The group interval is the
    log-sum-exp of the per-head ends (monotone in every head's score).
    """
    qf = qs if basis is None else qs @ np.asarray(basis, np.float64).T
    s1 = qs @ np.asarray(mean, np.float64).T          # [G, nb]
    nb = s1.shape[1]
    lo, hi = s1.copy(), s1.copy()
    proj = np.einsum("hd,bdj->hbj", qf, vec[:, :, :r + 1])   # [G, nb, r + 1]
    gaps = (lam[:, :r] - lam[:, 1:r + 1]) / np.maximum(lam[:, :1], 1e-300)
    clean = np.all(gaps >= tau, axis=1)
    exact = 0.5 * np.sum(lam[None, :, :r] * proj[:, :, :r] ** 2, axis=2)
    lo[:, clean] += exact[:, clean]
    hi[:, clean] += exact[:, clean]
    pmax = np.sqrt(lam[None, :, :r]) * np.abs(proj[:, :, :r])   # [G, nb, r]
    for j in np.nonzero(~clean)[0]:
        i = 0
        while i < r:
            a, c = eig_cluster(lam[j], i, tau)
            z2 = np.sum(np.einsum("hd,dj->hj", qf, vec[j][:, a:c]) ** 2, axis=1)   # [G]
            if c <= r:
                lo[:, j] += 0.5 * lam[j, c - 1] * z2
                hi[:, j] += 0.5 * lam[j, a] * z2
            else:
                hi[:, j] += 0.5 * lam[j, a] * z2
            pmax[:, j, i:min(c, r)] = np.sqrt(lam[j, a] * z2)[:, None]
            i = c
    if row_err is not None:
        e = np.transpose(row_err, (2, 0, 1))                       # [G, nb, r]
        widen = np.sum((pmax + e / 2) * e, axis=2)
        lo -= widen
        hi += widen
    return group_scores_np(lo), group_scores_np(hi), clean


def group_scores_np(s):
    m = s.max(axis=0)
    return m + np.log(np.exp(s - m).sum(axis=0))


def check_factor_rows(f_gpu, f_ref, lam, vec, r, slack, tau=CLUSTER_TAU):
    """Validity of the GPU's factor rows [nb, r, e] (float64; FP4 rows dequantized).

    Row i of a block whose eigenvalue i is separated from its neighbours must equal
    the oracle's row within ``slack`` [nb, r] (either sign when the oracle row's two
    largest magnitudes nearly tie, as the sign rule is then decided by rounding).  A
    row of a cluster C = [a, c) must lie within ``slack`` of C's eigenspace and have
    a norm in [sqrt(lam_{c-1}) - slack, sqrt(lam_a) + slack].  Returns (number of
    rows checked against the oracle's row, number checked as cluster rows); asserts.
    """
    nb = f_gpu.shape[0]
    n_single = n_cluster = 0
    for j in range(nb):
        i = 0
        while i < r:
            a, c = eig_cluster(lam[j], i, tau)
            if c - a == 1:
                d = np.linalg.norm(f_gpu[j, i] - f_ref[j, i])
                if d > slack[j, i]:
                    mags = np.sort(np.abs(f_ref[j, i]))[::-1]
                    near_tie = mags[0] - mags[1] <= 1e-4 * mags[0]
                    assert near_tie and np.linalg.norm(f_gpu[j, i] + f_ref[j, i]) <= slack[j, i], \
                        f"factor row {i} of block {j}: distance {d:.3e} > {slack[j, i]:.3e}"
                n_single += 1
            else:
                V = vec[j][:, a:c]
                for t in range(i, min(c, r)):
                    x = f_gpu[j, t]
                    out = np.linalg.norm(x - V @ (V.T @ x))
                    nrm = np.linalg.norm(x)
                    assert out <= slack[j, t], f"cluster row {t} of block {j} leaves the eigenspace: {out:.3e}"
                    assert np.sqrt(lam[j, c - 1]) - slack[j, t] <= nrm <= np.sqrt(lam[j, a]) + slack[j, t], \
                        f"cluster row {t} of block {j}: norm {nrm:.4e}"
                    n_cluster += 1
            i = max(c, i + 1) if c - a > 1 else i + 1
    return n_single, n_cluster


def check_selection_in_intervals(sel_row, lo, hi, cand, k):
    """The selection is a top-k of some scores inside the intervals: no candidate
    left out is certainly better than one taken (min hi of the taken >= max lo of
    the rest), and it has min(k, |cand|) distinct ascending candidates."""
    got = np.asarray(sel_row)
    valid = got[got >= 0]
    assert len(valid) == min(k, len(cand)) and np.all(np.diff(valid) > 0) and np.all(got[len(valid):] < 0)
    cs = set(np.asarray(cand).tolist())
    assert all(v in cs for v in valid.tolist())
    rest = np.array(sorted(cs - set(valid.tolist())), dtype=np.int64)
    if len(valid) and len(rest):
        assert hi[valid].min() >= lo[rest].max() - 1e-9 * (1 + abs(lo[rest].max())), \
            f"a block left out ({rest[np.argmax(lo[rest])]}) is certainly better than one taken"


EIG_REL = 1e-5   # fp32 eigensolver: |error of a unit eigenvector| <= EIG_REL * lam_1 / gap (Davis-Kahan with |dG| <= EIG_REL lam_1)


def eig_error(lam, r):
    """Bound on the distance of the GPU's factor row sqrt(lam_i) v_i from an exact one
    [nb, r]: sqrt(lam_i) * EIG_REL * lam_1 / gap_i (gap_i: distance of lam_i to its
    nearest other eigenvalue), plus EIG_REL sqrt(lam_1) for the rounding of lam."""
    l1 = np.maximum(lam[:, :1], 1e-300)
    up = np.concatenate([np.full((lam.shape[0], 1), np.inf), lam[:, :r] - lam[:, 1:r + 1]], axis=1)[:, :r]
    down = lam[:, :r] - lam[:, 1:r + 1]
    gap = np.maximum(np.minimum(up, down), 1e-300)
    return np.sqrt(lam[:, :r]) * np.minimum(EIG_REL * l1 / gap, 2.0) + EIG_REL * np.sqrt(l1)


def check_pair(got, b, g, Q, K, V, w, globals_, mean_dtype="f32", factor_fp4=False, basis=None,
               stats=None):
    """Every stage of one (b, K/V head) pair of a GPU decode step against the oracle.

    * means: within 1e-5 (fp32) or one bfloat16 step of the oracle's (both sides
      round once, from an fp32 and an fp64 mean);
    * factor rows (rank > 0): ``check_factor_rows`` against the oracle's eigenpairs
      (every block, no exemption); FP4 rows additionally code by code on separated
      eigenvalues: a code may differ from the oracle's only by one E2M1 step, where
      the oracle's value lies within the eigensolver's error of the midpoint, and a
      scale only by that error; at most 1% of codes differ;
    * scores: the oracle's scorer applied to the GPU's stored summaries (exact
      arithmetic check, 3e-5 rank 0 / 2e-4 relative otherwise), and every block's
      score inside the interval of scores the correct factors give (``score_intervals``);
    * selection: identical to the oracle's top-k of those scores except at near ties,
      and a top-k of scores inside the intervals;
    * O and lse: within 2e-3 of the oracle's attention over the GPU's token set.
    Returns 1 when the pair has a near tie at k, else 0.
    """
    S, n, G, d, r = w.block_size, w.n_ctx, w.n_q_heads // w.n_kv_heads, w.head_dim, w.rank
    nb = n // S
    scale = default_scale(d)
    mb = mean_dtype == "bf16"
    P = None if basis is None else np.asarray(basis[g], np.float64)
    forced = oracle.forced_token_mask(n, w.n_sink, w.window, globals_)
    cand = oracle.candidate_blocks(n, S, forced)
    mean, f = oracle.block_summaries(K[b, g, :n], S, r, mean_bf16=mb, basis=P)
    mean_gpu = got["mean"][b, g, :nb].astype(np.float64)
    if mb:
        assert np.all(np.abs(mean_gpu - mean) <= bf16_ulp(mean) + 1e-30), f"bf16 mean at ({b}, {g})"
    else:
        assert max_abs(mean_gpu, mean) < 1e-5, f"mean at ({b}, {g})"
    qs = scale * Q[b, g * G:(g + 1) * G]
    f_gpu = None
    row_err = None
    if r > 0 and nb > 0:
        lam, vec = block_spectra(K[b, g, :n], nb, S, basis=P)
        ee = eig_error(lam, r)                                            # [nb, r]
        qf = qs if P is None else qs @ P.T
        if factor_fp4:
            f_gpu, codes_gpu = unpack_fp4(got["factor"][b, g, :nb], got["factor_scale"][b, g, :nb])
            sc_gpu = got["factor_scale"][b, g, :nb].astype(np.float64)
            half = E2M1_HALF[codes_gpu & 7] * sc_gpu[..., None]           # |fp32 row - stored| per entry
            slack = ee + np.linalg.norm(half, axis=2) + 1e-7 * np.sqrt(lam[:, :1])
            row_err = np.einsum("hd,brd->brh", np.abs(qf), half) + ee[..., None] * np.linalg.norm(qf, axis=1)
            # code by code on the rows of separated eigenvalues
            codes_or, sc_or = oracle.quantize_e2m1_rows(f)
            sing = np.zeros((nb, r), bool)
            for j in range(nb):
                for i in range(r):
                    a, c = eig_cluster(lam[j], i)
                    sing[j, i] = c - a == 1
            sc_or64 = sc_or.astype(np.float64)
            assert np.all(np.abs(sc_gpu - sc_or64)[sing] <= (ee / 6 + 1e-6 * sc_or64)[sing]), f"scales at ({b}, {g})"
            v_or = f / np.where(sc_or64 > 0, sc_or64, 1.0)[..., None]
            sv = lambda c: np.where(c & 8, -E2M1[c & 7], E2M1[c & 7])      # noqa: E731
            va, vb = sv(codes_or), sv(codes_gpu)
            flip = (codes_or != codes_gpu) & ~((va == 0) & (vb == 0)) & sing[..., None]
            if flip.any():
                lo_v, hi_v = np.minimum(va, vb), np.maximum(va, vb)
                idx_lo = np.searchsorted(np.concatenate([-E2M1[::-1], E2M1[1:]]), lo_v)
                adjacent = np.concatenate([-E2M1[::-1], E2M1[1:]])[np.minimum(idx_lo + 1, 14)] == hi_v
                mid = (lo_v + hi_v) / 2
                delta = (2 * ee / np.where(sc_gpu > 0, sc_gpu, 1.0))[..., None] + 1e-6
                assert np.all(adjacent[flip]) and np.all((np.abs(v_or - mid) <= delta)[flip]), \
                    f"FP4 code beyond a midpoint flip at ({b}, {g})"
            if stats is not None:
                stats["codes"] = stats.get("codes", 0) + int(sing.sum()) * f.shape[2]
                stats["flips"] = stats.get("flips", 0) + int(flip.sum())
        else:
            f_gpu = got["factor"][b, g, :nb].astype(np.float64)
            slack = ee + 1e-6 * np.sqrt(lam[:, :1])
            row_err = ee[..., None] * np.linalg.norm(qf, axis=1)
        n1, n2 = check_factor_rows(f_gpu, f, lam, vec, r, slack)
        if stats is not None:
            stats["cluster_rows"] = stats.get("cluster_rows", 0) + n2
    if nb == 0:
        s_rows = np.zeros(0)
    else:
        s_rows = oracle.group_scores(oracle.head_scores(qs, mean_gpu, f_gpu if r else None,
                                                        basis=P if r else None))
        tol = 3e-5 if r == 0 else 2e-4 * (1 + np.abs(s_rows))
        assert np.all(np.abs(got["scores"][b, g, :nb] - s_rows) <= tol), f"scores at ({b}, {g})"
    ok, tie = compare_selection(got["sel"][b, g], s_rows, cand, w.top_k)
    assert ok, f"selection at ({b}, {g}): gpu {got['sel'][b, g]} vs {oracle.top_k_blocks(s_rows, cand, w.top_k)}"
    if r > 0 and nb > 0:
        lo, hi, _ = score_intervals(qs, mean_gpu, lam, vec, r, basis=P, row_err=row_err)
        slack_s = 2e-4 * (1 + np.abs(s_rows))
        sg = got["scores"][b, g, :nb]
        assert np.all(sg >= lo - slack_s) and np.all(sg <= hi + slack_s), f"score outside its interval at ({b}, {g})"
        check_selection_in_intervals(got["sel"][b, g], lo - slack_s, hi + slack_s, cand, w.top_k)
    o_ref, lse_ref = oracle_decode_with_sel(Q[b, g * G:(g + 1) * G], K[b, g], V[b, g], n, S, w.window,
                                            w.n_sink, globals_, got["sel"][b, g], scale)
    assert max_abs(got["O"][b, g * G:(g + 1) * G], o_ref) < OUT_TOL, f"O at ({b}, {g})"
    assert max_abs(got["lse"][b, g * G:(g + 1) * G], lse_ref) < OUT_TOL, f"lse at ({b}, {g})"
    return int(tie)


# ----------------------------------------------------------------------------- whole cases
def check_decode_case(api, w, globals_, extra_cap, one_call=False, mean_dtype="f32", page_tokens=None):
    """One seeded decode case through the GPU (fp32 factor rows or none), every pair
    checked with ``check_pair``; returns the near-tie count."""
    x = make_decode_inputs(w, kv_capacity=w.n_ctx + extra_cap)
    print(f"[decode parity] {w.name} one_call={one_call} mean={mean_dtype} pages={page_tokens}", flush=True)
    got = gpu_decode_step(api, x, w, global_pos=globals_, one_call=one_call, mean_dtype=mean_dtype,
                          page_tokens=page_tokens)
    Q, K, V = as_f64(x["Q"]), as_f64(x["K"]), as_f64(x["V"])
    stats = {}
    ties = sum(check_pair(got, b, g, Q, K, V, w, globals_, mean_dtype=mean_dtype, stats=stats)
               for b in range(w.batch) for g in range(w.n_kv_heads))
    print(f"[decode parity] {w.name}: near ties {ties}, cluster rows {stats.get('cluster_rows', 0)}", flush=True)
    return ties


def check_fp4_case(api, w, globals_, pairs=None, one_call=True, mean_dtype="bf16", basis=None, x=None, got=None,
                   page_tokens=None):
    """FP4 factor rows (bf16 or fp32 means, optional query subspace): ``check_pair`` on
    every block of the given pairs (all pairs when None).  The GPU quantises its fp32
    eigensolver's rows and the oracle its fp64 rows: a code may differ only by one
    E2M1 step at a rounding midpoint (within the eigensolver's error), and at most 1%
    of codes may; rows of nearly equal eigenvalues are checked against their
    eigenspace (several correct results).  With a query-subspace ``basis`` [Hkv, s, d]
    the rows are the projected covariance's and meet the projected query (the GPU
    multiplies the basis, split into two bfloat16 parts, with the bf16 query, and
    splits the projected query into two bfloat16 parts: 2^-17 relative each, inside
    the scores' 2e-4 slack)."""
    x = make_decode_inputs(w) if x is None else x
    sd = None if basis is None else basis.shape[1]
    print(f"[decode fp4] {w.name} one_call={one_call} mean={mean_dtype} sub_dim={sd}", flush=True)
    if got is None:
        got = gpu_decode_step(api, x, w, global_pos=globals_, one_call=one_call, mean_dtype=mean_dtype,
                              factor_fp4=True, basis=basis, page_tokens=page_tokens)
    Q = as_f64(x["Q"])
    if pairs is None:
        pairs = [(b, g) for b in range(w.batch) for g in range(w.n_kv_heads)]
    stats = {}
    ties = 0
    for (b, g) in pairs:
        Kb = {(b, g): as_f64(x["K"][b, g])}
        Vb = {(b, g): as_f64(x["V"][b, g])}
        ties += check_pair(got, b, g, Q, PairView(Kb), PairView(Vb), w, globals_, mean_dtype=mean_dtype,
                           factor_fp4=True, basis=basis, stats=stats)
    n_codes, n_flips = stats.get("codes", 0), stats.get("flips", 0)
    print(f"[decode fp4] {w.name}: {n_flips} of {n_codes} codes one step from the oracle's, "
          f"{stats.get('cluster_rows', 0)} rows checked against a cluster eigenspace, near ties {ties}", flush=True)
    if n_codes:
        assert n_flips <= 0.01 * n_codes


class PairView:
    """K or V of selected pairs as float64, indexed [b, g] (the pairs a check reads)."""

    def __init__(self, rows):
        self.rows = rows

    def __getitem__(self, key):
        b, g = key[:2]
        out = self.rows[(b, g)]
        return out[key[2:]] if len(key) > 2 else out


