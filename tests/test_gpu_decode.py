"""GPU parity of the decode path (summaries -> select/top-k -> sparse decode) against
the fp64 oracle, through the C ABI.

Bar: selected sets identical per (b, K/V head) except at the oracle's near ties
(relative gap < 1e-4 between its k-th and (k+1)-th scores); outputs and lse within
max-abs 2e-3 of the oracle's attention over the GPU's selected set; summaries and
scores within fp32 rounding of the oracle's float64 values.
"""

import numpy as np
import pytest

import oracle
from synthetic import WORKLOADS, DecodeWorkload, make_decode_inputs

from gpu_util import (OUT_TOL, as_f64, bf16_ulp, compare_selection, default_scale, gpu_decode_step,
                      max_abs, oracle_decode_with_sel)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    import torch
    assert torch.cuda.is_available(), "GPU tests need the GPU"
    import sliding_window_attention_block_amd as m
    m.library()
    return m


def _w(name, B, Hq, Hkv, d, n, rank, k, W, ns, dtype, seed):
    return DecodeWorkload(name=name, batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, n_ctx=n,
                          block_size=64, rank=rank, top_k=k, window=W, n_sink=ns, dtype=dtype,
                          seed=seed)


SMALL = [
    # name                    B  Hq Hkv  d    n     r  k   W    ns  dtype  seed  globals           extra cap
    (_w("bf16_g4_d128_r0", 2, 8, 2, 128, 1000, 0, 3, 100, 5, "bf16", 10), (), 0),
    (_w("bf16_g8_d128_r4", 1, 16, 2, 128, 2065, 4, 5, 130, 64, "bf16", 11), (), 0),
    (_w("bf16_g16_d64_r2", 1, 16, 1, 64, 777, 2, 4, 64, 0, "bf16", 12), (3, 200, 201, 500, 776), 0),
    (_w("bf16_g1_d64_r8", 2, 2, 2, 64, 1500, 8, 6, 1, 1, "bf16", 13), (), 100),
    (_w("f32_g8_d128_r4", 1, 8, 1, 128, 640, 4, 2, 64, 64, "f32", 14), (70,), 0),
    (_w("f32_g2_d64_r0", 3, 4, 2, 64, 129, 0, 1, 3, 2, "f32", 15), (), 7),
    (_w("k_exceeds_candidates", 1, 4, 1, 64, 600, 0, 50, 64, 64, "bf16", 16), (), 0),
    (_w("window_covers_all", 1, 4, 1, 64, 300, 0, 4, 1000, 0, "bf16", 17), (), 0),
    (_w("short_context", 1, 8, 1, 128, 40, 1, 2, 16, 4, "bf16", 18), (), 0),
    # groups that end inside a 4-head lane group (MFMA scorer: 3 of 4, 12 of 16 heads)
    (_w("bf16_g3_d64_r0", 2, 6, 2, 64, 2000, 0, 9, 128, 16, "bf16", 40), (50, 1300), 0),
    (_w("bf16_g12_d128_r3", 1, 24, 2, 128, 1900, 3, 7, 200, 64, "bf16", 41), (), 0),
    # fp32 rank-8 factor rows with 16 query heads at d = 128: the VALU scorer keeps
    # one unit of summary rows in flight instead of two (the second would spill)
    (_w("bf16_g16_d128_r8", 1, 16, 1, 128, 1300, 8, 5, 100, 16, "bf16", 42), (), 0),
    (_w("f32_g13_d128_r6", 2, 26, 2, 128, 700, 6, 3, 64, 8, "f32", 43), (40,), 0),
]


def _check_case(api, w, globals_, extra_cap, one_call=False, mean_dtype="f32"):
    x = make_decode_inputs(w, kv_capacity=w.n_ctx + extra_cap)
    print(f"[decode parity] {w.name} one_call={one_call} mean={mean_dtype}", flush=True)
    got = gpu_decode_step(api, x, w, global_pos=globals_, one_call=one_call, mean_dtype=mean_dtype)
    mb = mean_dtype == "bf16"
    Q, K, V = as_f64(x["Q"]), as_f64(x["K"]), as_f64(x["V"])
    S, n, G, d = w.block_size, w.n_ctx, w.n_q_heads // w.n_kv_heads, w.head_dim
    scale = default_scale(d)
    nb = n // S
    forced = oracle.forced_token_mask(n, w.n_sink, w.window, globals_)
    cand = oracle.candidate_blocks(n, S, forced)
    ties = 0
    for b in range(w.batch):
        for g in range(w.n_kv_heads):
            mean, factor = oracle.block_summaries(K[b, g, :n], S, w.rank, mean_bf16=mb)
            if mb:
                # both sides round once (from an fp32 and an fp64 mean): at most one step apart
                err = np.abs(got["mean"][b, g, :nb].astype(np.float64) - mean)
                assert np.all(err <= bf16_ulp(mean) + 1e-30)
            else:
                assert max_abs(got["mean"][b, g, :nb], mean) < 1e-5
            if w.rank > 0:
                proj_gpu = np.einsum("bid,bie->bde", got["factor"][b, g, :nb].astype(np.float64),
                                     got["factor"][b, g, :nb].astype(np.float64))
                proj_ref = np.einsum("bid,bie->bde", factor, factor)
                lam = (factor ** 2).sum(axis=2)
                full = np.linalg.eigvalsh(np.einsum("brd,bre->bde",
                                                    K[b, g, :nb * S].reshape(nb, S, d) - mean[:, None],
                                                    K[b, g, :nb * S].reshape(nb, S, d) - mean[:, None]) / S)
                full = full[:, ::-1]
                gap = (full[:, w.rank - 1] - full[:, w.rank]) / np.maximum(full[:, 0], 1e-30)
                ok = gap > 1e-3
                err = np.abs(proj_gpu - proj_ref).max(axis=(1, 2)) / np.maximum(lam[:, 0], 1e-30)
                assert np.all(err[ok] < 1e-3), f"rank-{w.rank} projector error {err[ok].max()}"
            qs = scale * Q[b, g * G:(g + 1) * G]
            s_ref = oracle.group_scores(oracle.head_scores(qs, mean, factor if w.rank else None))
            if nb:
                assert max_abs(got["scores"][b, g, :nb], s_ref) < (2e-4 if w.rank else 3e-5)
            ok, tie = compare_selection(got["sel"][b, g], s_ref, cand, w.top_k)
            ties += tie
            assert ok, f"selection mismatch at (b={b}, g={g}): gpu {got['sel'][b, g]} vs " \
                       f"oracle {oracle.top_k_blocks(s_ref, cand, w.top_k)}"
            o_ref, lse_ref = oracle_decode_with_sel(Q[b, g * G:(g + 1) * G], K[b, g], V[b, g], n, S,
                                                    w.window, w.n_sink, globals_, got["sel"][b, g],
                                                    scale)
            assert max_abs(got["O"][b, g * G:(g + 1) * G], o_ref) < OUT_TOL
            assert max_abs(got["lse"][b, g * G:(g + 1) * G], lse_ref) < OUT_TOL
    return ties


@pytest.mark.parametrize("case", SMALL, ids=[c[0].name for c in SMALL])
def test_decode_small_cases(api, case):
    w, globals_, extra = case
    _check_case(api, w, globals_, extra)


NO_FORCED = _w("no_forced_tokens", 2, 8, 2, 128, 1200, 0, 4, 0, 0, "bf16", 19)
# bsattn_decode_step selects inside the decode waves for bf16 with <= 512 blocks and
# top_k <= 256, else it runs the two calls' kernels
ONE_CALL_EXTRA = [
    (NO_FORCED, (), 0),
    (_w("fused_512_blocks_k256_g8_d64", 1, 8, 1, 64, 512 * 64, 2, 256, 700, 64, "bf16", 25), (5, 64, 65), 0),
    (_w("fused_500_blocks_tail_d128", 2, 4, 1, 128, 500 * 64 + 17, 0, 24, 64, 64, "bf16", 26), (), 0),
    (_w("fallback_513_blocks", 1, 4, 1, 64, 513 * 64, 0, 8, 64, 64, "bf16", 28), (), 0),
    (_w("fallback_k257", 1, 4, 1, 64, 600 * 64, 0, 257, 64, 64, "bf16", 29), (), 0),
]


@pytest.mark.parametrize("case", SMALL + ONE_CALL_EXTRA,
                         ids=[c[0].name for c in SMALL + ONE_CALL_EXTRA])
def test_one_call_step_small_cases(api, case):
    """bsattn_decode_step: the same oracle bar as the two calls, on every small case."""
    w, globals_, extra = case
    _check_case(api, w, globals_, extra, one_call=True)


def test_one_call_step_breaks_ties_by_index(api):
    """Every block holds the same keys, so every candidate's score ties exactly: both
    selection paths must take the lowest-index candidates (the sink block is forced)."""
    w = _w("all_ties", 1, 4, 1, 64, 64 * 300, 0, 7, 64, 64, "bf16", 27)
    x = make_decode_inputs(w)
    K = x["K"].copy()
    K[:, :, :] = np.tile(K[:, :, :64], (1, 1, 300, 1))
    x = dict(x, K=K)
    two = gpu_decode_step(api, x, w)
    one = gpu_decode_step(api, x, w, one_call=True)
    assert np.array_equal(one["sel"][0, 0], np.arange(1, 8)), one["sel"][0, 0]
    assert np.array_equal(two["sel"], one["sel"])
    assert max_abs(two["O"], one["O"]) < 1e-5


@pytest.mark.parametrize("name", ["first_order_decode_32k", "cobs_decode_128k"])
def test_one_call_step_equals_two_calls(api, name):
    """Full-size workloads: bsattn_decode_step selects exactly the blocks of
    bsattn_select_topk and gives the decode's outputs up to rounding order."""
    w = WORKLOADS[name]
    x = make_decode_inputs(w)
    print(f"[decode one call vs two] {name}", flush=True)
    two = gpu_decode_step(api, x, w)
    one = gpu_decode_step(api, x, w, one_call=True)
    assert np.array_equal(two["sel"], one["sel"])
    assert np.array_equal(two["scores"], one["scores"])
    assert max_abs(two["O"], one["O"]) < 1e-5
    assert max_abs(two["lse"], one["lse"]) < 1e-5


def test_tiny_decode_workload(api):
    """The 1K-token fp32 workload end to end: G = 4, d = 64, top-4 + sink block + last block."""
    _check_case(api, WORKLOADS["tiny_decode_1k"], (), 0)


def test_k_covering_all_candidates_equals_dense_causal(api):
    w = _w("dense", 2, 8, 2, 128, 900, 0, 64, 32, 0, "bf16", 21)
    x = make_decode_inputs(w)
    got = gpu_decode_step(api, x, w)
    Q, K, V = as_f64(x["Q"]), as_f64(x["K"]), as_f64(x["V"])
    for b in range(2):
        for g in range(2):
            o, lse = oracle.masked_attention_rows(Q[b, 4 * g:4 * g + 4], K[b, g], V[b, g],
                                                  np.ones((4, 900), bool), default_scale(128))
            assert max_abs(got["O"][b, 4 * g:4 * g + 4], o) < OUT_TOL
            assert max_abs(got["lse"][b, 4 * g:4 * g + 4], lse) < OUT_TOL


def _full_size(api, name, pairs, one_call=False, mean_dtype="f32"):
    import torch
    w = WORKLOADS[name]
    print(f"[decode full size] {name}: generating inputs", flush=True)
    x = make_decode_inputs(w)
    print(f"[decode full size] {name}: running on the GPU", flush=True)
    got = gpu_decode_step(api, x, w, one_call=one_call, mean_dtype=mean_dtype)
    torch.cuda.empty_cache()
    mb = mean_dtype == "bf16"
    # properties over every pair
    S, n = w.block_size, w.n_ctx
    forced = oracle.forced_token_mask(n, w.n_sink, w.window)
    cand = oracle.candidate_blocks(n, S, forced)
    candset = set(cand.tolist())
    for b in range(w.batch):
        for g in range(w.n_kv_heads):
            s = got["sel"][b, g]
            assert len(set(s.tolist())) == w.top_k and all(v in candset for v in s.tolist())
            assert np.all(np.diff(s) > 0)
    assert np.isfinite(got["O"]).all() and np.isfinite(got["lse"]).all()
    # oracle on sampled pairs
    Q = as_f64(x["Q"])
    G, d = w.n_q_heads // w.n_kv_heads, w.head_dim
    scale = default_scale(d)
    ties = 0
    for (b, g) in pairs:
        print(f"[decode full size] {name}: oracle for pair ({b}, {g})", flush=True)
        Kbg, Vbg = as_f64(x["K"][b, g]), as_f64(x["V"][b, g])
        mean, factor = oracle.block_summaries(Kbg, S, w.rank, mean_bf16=mb)
        if mb:
            assert np.all(np.abs(got["mean"][b, g].astype(np.float64) - mean) <= bf16_ulp(mean) + 1e-30)
        else:
            assert max_abs(got["mean"][b, g], mean) < 1e-5
        s_ref = oracle.group_scores(oracle.head_scores(scale * Q[b, g * G:(g + 1) * G], mean,
                                                       factor if w.rank else None))
        assert max_abs(got["scores"][b, g], s_ref) < (2e-4 if w.rank else 3e-5)
        ok, tie = compare_selection(got["sel"][b, g], s_ref, cand, w.top_k)
        ties += tie
        assert ok, f"selection mismatch at ({b}, {g})"
        o_ref, lse_ref = oracle_decode_with_sel(Q[b, g * G:(g + 1) * G], Kbg, Vbg, n, S, w.window,
                                                w.n_sink, (), got["sel"][b, g], scale)
        assert max_abs(got["O"][b, g * G:(g + 1) * G], o_ref) < OUT_TOL
        assert max_abs(got["lse"][b, g * G:(g + 1) * G], lse_ref) < OUT_TOL
    print(f"[decode full size] {name}: near ties among sampled pairs: {ties}", flush=True)


def test_first_order_decode_32k_full_size(api):
    _full_size(api, "first_order_decode_32k", [(0, 0), (5, 3), (15, 7)])


def test_cobs_decode_128k_full_size(api):
    _full_size(api, "cobs_decode_128k", [(0, 0), (3, 7)])


@pytest.mark.parametrize("case", SMALL, ids=[c[0].name for c in SMALL])
def test_bf16_means_small_cases(api, case):
    """Block means stored in bfloat16 (the COBS explainer's storage), one-call step:
    means within one bfloat16 step of the oracle's rounded means, selection and
    outputs to the same bar against the oracle using those means."""
    w, globals_, extra = case
    _check_case(api, w, globals_, extra, one_call=True, mean_dtype="bf16")


@pytest.mark.parametrize("name,pairs", [("first_order_decode_32k", [(0, 0), (15, 7)]),
                                        ("cobs_decode_128k", [(2, 5)])])
def test_bf16_means_full_size(api, name, pairs):
    _full_size(api, name, pairs, one_call=True, mean_dtype="bf16")


E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _unpack_fp4(codes, scale):
    """Test-side decoding of packed FP4 codes [..., d/2] (entry 2i in the low nibble)
    with row scales [...]: values [..., d] and the 4-bit codes."""
    c = np.stack([codes & 15, codes >> 4], axis=-1).reshape(*codes.shape[:-1], -1)
    val = np.where(c & 8, -E2M1[c & 7], E2M1[c & 7]) * scale.astype(np.float64)[..., None]
    return val, c


def _check_fp4(api, w, globals_, pairs=None, one_call=True, mean_dtype="bf16", basis=None):
    """FP4 factor rows.  The GPU quantises its fp32 eigensolver's rows, the oracle its
    fp64 rows, so a code can differ where the exact value sits at a rounding midpoint:
    codes must match the oracle's except for at most 1% of entries, each one E2M1 step
    away; scales to 1e-3.  Scores are compared with the oracle's (from its own FP4
    rows) within a per-block bound computed here from how the two sets of codes differ
    (1/2 |(p + e)^2 - p^2| <= (|p| + |e|/2) |e| per row, p the oracle's projection, e
    bounded by |q| . |row difference|), and the selections may differ only within that
    bound of the k-th score.  Outputs: the usual bar over the GPU's selection.  With a
    query-subspace ``basis`` [Hkv, s, d] the rows are the projected covariance's and
    meet the projected query (the GPU multiplies the basis, split into two bfloat16
    parts, with the bf16 query, and splits the projected query into two bfloat16
    parts: 2^-17 relative each, inside the 2e-4 slack of the bound)."""
    x = make_decode_inputs(w)
    sd = None if basis is None else basis.shape[1]
    print(f"[decode fp4] {w.name} one_call={one_call} mean={mean_dtype} sub_dim={sd}", flush=True)
    got = gpu_decode_step(api, x, w, global_pos=globals_, one_call=one_call, mean_dtype=mean_dtype,
                          factor_fp4=True, basis=basis)
    Q, K, V = as_f64(x["Q"]), as_f64(x["K"]), as_f64(x["V"])
    S, n, G, d, r = w.block_size, w.n_ctx, w.n_q_heads // w.n_kv_heads, w.head_dim, w.rank
    nb = n // S
    scale = default_scale(d)
    forced = oracle.forced_token_mask(n, w.n_sink, w.window, globals_)
    cand = oracle.candidate_blocks(n, S, forced)
    if pairs is None:
        pairs = [(b, g) for b in range(w.batch) for g in range(w.n_kv_heads)]
    n_codes = n_flips = 0
    for (b, g) in pairs:
        P = None if basis is None else basis[g].astype(np.float64)
        mean, f = oracle.block_summaries(K[b, g, :n], S, r, mean_bf16=mean_dtype == "bf16", basis=P)
        if nb == 0:
            continue
        codes_or, sc_or = oracle.quantize_e2m1_rows(f)
        deq_or = oracle.dequantize_e2m1_rows(codes_or, sc_or)
        deq_gpu, codes_gpu = _unpack_fp4(got["factor"][b, g, :nb], got["factor_scale"][b, g, :nb])
        # blocks whose top r+1 eigenvalues are separated: rows defined up to sign (fixed)
        X = K[b, g, :nb * S].reshape(nb, S, d)
        Xc = X - X.mean(axis=1, keepdims=True)
        if P is not None:
            Xc = Xc @ P.T
        lam = np.sort(np.linalg.eigvalsh(np.einsum("brd,bre->bde", Xc, Xc) / S), axis=1)[:, ::-1]
        gaps = np.min(np.abs(np.diff(lam[:, :r + 1], axis=1)), axis=1) / np.maximum(lam[:, 0], 1e-30)
        ok = gaps > 1e-3
        assert np.all(np.abs(got["factor_scale"][b, g, :nb][ok] / np.where(sc_or[ok] > 0, sc_or[ok], 1) - 1) < 1e-3)
        diff = codes_gpu[ok] != codes_or[ok]
        n_codes += diff.size
        n_flips += int(diff.sum())
        assert np.all(np.abs(deq_gpu[ok] - deq_or[ok])[diff] <= 2.0 * np.max(sc_or[ok]) * 1.001)
        qs = scale * Q[b, g * G:(g + 1) * G]
        s_ref = oracle.group_scores(oracle.head_scores(qs, mean, deq_or, basis=P))
        qp = qs if P is None else qs @ P.T
        p = np.einsum("hd,brd->hbr", qp, deq_or)
        e = np.einsum("hd,brd->hbr", np.abs(qp), np.abs(deq_gpu - deq_or))
        bound = np.max(np.sum((np.abs(p) + e / 2) * e, axis=2), axis=0) + 2e-4 * (1 + np.abs(s_ref))
        assert np.all(np.abs(got["scores"][b, g, :nb] - s_ref)[ok] <= bound[ok])
        # selection within the quantisation band of the k-th score
        ref = oracle.top_k_blocks(s_ref, cand, w.top_k)
        gsel = got["sel"][b, g]
        assert len(gsel[gsel >= 0]) == len(ref[ref >= 0])
        odd = set(gsel[gsel >= 0].tolist()) ^ set(ref[ref >= 0].tolist())
        if odd:
            ks = np.sort(s_ref[cand])[::-1][min(w.top_k, len(cand)) - 1]
            band = 2 * np.max(bound[cand][ok[cand]]) + 1e-4 * abs(ks)
            assert all((not ok[j]) or abs(s_ref[j] - ks) <= band for j in odd), f"selection at ({b}, {g})"
        o_ref, lse_ref = oracle_decode_with_sel(Q[b, g * G:(g + 1) * G], K[b, g], V[b, g], n, S, w.window,
                                                w.n_sink, globals_, gsel, scale)
        assert max_abs(got["O"][b, g * G:(g + 1) * G], o_ref) < OUT_TOL
        assert max_abs(got["lse"][b, g * G:(g + 1) * G], lse_ref) < OUT_TOL
    if n_codes:
        print(f"[decode fp4] {w.name}: {n_flips} of {n_codes} codes one step from the oracle's", flush=True)
        assert n_flips <= 0.01 * n_codes


FP4_CASES = [c for c in SMALL if c[0].rank > 0]


@pytest.mark.parametrize("case", FP4_CASES, ids=[c[0].name for c in FP4_CASES])
@pytest.mark.parametrize("one_call", [False, True])
def test_fp4_factors_small_cases(api, case, one_call):
    w, globals_, _ = case
    _check_fp4(api, w, globals_, one_call=one_call, mean_dtype="bf16" if one_call else "f32")


def test_fp4_factors_cobs_128k(api):
    _check_fp4(api, WORKLOADS["cobs_decode_128k"], (), pairs=[(0, 0), (3, 6)])


def calibration_basis(w, s, seed):
    """Per K/V head, the oracle's query-subspace basis [s, d] of a seeded calibration
    sample: 512 Gaussian queries with a decaying spectrum in a random orientation (the
    concentrated query distribution the subspace projection assumes)."""
    rng = np.random.default_rng(seed)
    d = w.head_dim
    out = []
    for _ in range(w.n_kv_heads):
        R, _ = np.linalg.qr(rng.standard_normal((d, d)))
        Qc = (rng.standard_normal((512, d)) * np.exp(-np.arange(d) / 24.0)) @ R.T
        out.append(oracle.query_subspace_basis(Qc, s))
    return np.stack(out).astype(np.float32)


# sub_dim per bf16 case: 96, 32, 64, 32, 128 (every projected scorer variant)
SUBSPACE_CASES = [(c, s) for c, s in zip([c for c in FP4_CASES if c[0].dtype == "bf16"], (96, 32, 64, 32, 128))]


@pytest.mark.parametrize("case,sub_dim", SUBSPACE_CASES,
                         ids=[f"{c[0].name}_s{s}" for c, s in SUBSPACE_CASES])
@pytest.mark.parametrize("one_call", [False, True])
def test_subspace_projection_small_cases(api, case, sub_dim, one_call):
    w, globals_, _ = case
    _check_fp4(api, w, globals_, one_call=one_call, basis=calibration_basis(w, sub_dim, 50 + sub_dim))


def test_subspace_projection_cobs_128k(api):
    w = WORKLOADS["cobs_decode_128k"]
    _check_fp4(api, w, (), pairs=[(0, 0), (2, 5)], basis=calibration_basis(w, 96, 60))


def test_repeated_calls_reuse_the_workspace(api):
    """The workspace only holds split partials: it needs no initialisation, and
    repeated calls (and a smaller call after a larger one) on one workspace give
    identical results."""
    import torch
    w = _w("reuse", 2, 16, 2, 128, 3000, 2, 8, 256, 64, "bf16", 22)
    x = make_decode_inputs(w)
    ref = gpu_decode_step(api, x, w)
    Q, K, V = (torch.from_numpy(np.ascontiguousarray(x[k]).view(np.int16)).view(torch.bfloat16).cuda()
               for k in ("Q", "K", "V"))
    shape = api.make_shape(2, 16, 2, 128, 3000)
    sel = torch.from_numpy(ref["sel"]).cuda()
    nbytes = api.bsattn_decode_workspace_bytes(shape, w.top_k, w.window, w.n_sink, 0)
    ws = torch.full((nbytes,), 255, dtype=torch.uint8, device="cuda")  # garbage contents
    for rep in range(3):
        O = torch.full((2, 16, 128), float("nan"), device="cuda")
        lse = torch.full((2, 16), float("nan"), device="cuda")
        api.bsattn_decode(shape, Q, K, V, sel, w.top_k, w.window, w.n_sink, None, O, lse, ws)
        torch.cuda.synchronize()
        assert np.array_equal(O.cpu().numpy(), ref["O"]), rep
        assert np.array_equal(lse.cpu().numpy(), ref["lse"]), rep
    # a smaller problem on the same workspace
    small = _w("reuse_small", 1, 4, 1, 128, 700, 0, 2, 64, 0, "bf16", 23)
    xs = make_decode_inputs(small)
    got = gpu_decode_step(api, xs, small)
    Qs, Ks, Vs = (torch.from_numpy(np.ascontiguousarray(xs[k]).view(np.int16)).view(torch.bfloat16).cuda()
                  for k in ("Q", "K", "V"))
    O = torch.empty((1, 4, 128), device="cuda")
    api.bsattn_decode(api.make_shape(1, 4, 1, 128, 700), Qs, Ks, Vs, torch.from_numpy(got["sel"]).cuda(),
                      2, 64, 0, None, O, None, ws)
    torch.cuda.synchronize()
    assert np.array_equal(O.cpu().numpy(), got["O"])


def test_maximum_sizes(api):
    """Every limit of the ABI at once: 65,536 complete blocks, top_k = 1024, 16 query
    heads per K/V head and 256 global positions (d = 64, first-order selector)."""
    n = 65536 * 64
    w = _w("max_sizes", 1, 16, 1, 64, n, 0, 1024, 64, 64, "bf16", 24)
    rng = np.random.default_rng(5)
    globals_ = tuple(int(p) for p in np.sort(rng.choice(n, size=256, replace=False)))
    ties = _check_case(api, w, globals_, 0)
    print(f"[decode max sizes] near ties: {ties}", flush=True)


def test_dilated_window_as_forced_positions(api):
    """A dilated sliding window (the SWA glossary's extension: every delta-th token
    back from the query) expressed as forced positions: the window argument 0 and the
    positions t, t - 4, ..., t - 4 * 39 given as global positions; checked against the
    oracle with the same forced set."""
    w = _w("dilated_window", 1, 8, 2, 128, 3000, 0, 6, 0, 16, "bf16", 45)
    t = w.n_ctx - 1
    globals_ = tuple(sorted(t - 4 * m for m in range(40)))
    _check_case(api, w, globals_, 0, one_call=True, mean_dtype="bf16")
