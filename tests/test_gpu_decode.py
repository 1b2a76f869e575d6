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

from gpu_util import (OUT_TOL, PairView, as_f64, check_decode_case, check_fp4_case, check_pair, default_scale,
                      gpu_decode_step, max_abs)

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


@pytest.mark.parametrize("case", SMALL, ids=[c[0].name for c in SMALL])
def test_decode_small_cases(api, case):
    w, globals_, extra = case
    check_decode_case(api, w, globals_, extra)


NO_FORCED = _w("no_forced_tokens", 2, 8, 2, 128, 1200, 0, 4, 0, 0, "bf16", 19)
# bsattn_decode_step selects inside the decode kernel for bf16 with top_k <= 256: each
# wave alone up to 512 blocks, each workgroup together up to 2048 blocks; else it runs
# the two calls' kernels
ONE_CALL_EXTRA = [
    (NO_FORCED, (), 0),
    (_w("fused_512_blocks_k256_g8_d64", 1, 8, 1, 64, 512 * 64, 2, 256, 700, 64, "bf16", 25), (5, 64, 65), 0),
    (_w("fused_500_blocks_tail_d128", 2, 4, 1, 128, 500 * 64 + 17, 0, 24, 64, 64, "bf16", 26), (), 0),
    (_w("wg_select_513_blocks", 1, 4, 1, 64, 513 * 64, 0, 8, 64, 64, "bf16", 28), (), 0),
    (_w("wg_select_2048_blocks_g8_d128_r2", 1, 8, 1, 128, 2048 * 64, 2, 40, 300, 10, "bf16", 30),
     (7, 5000, 90000), 0),
    (_w("wg_select_1500_blocks_tail_k256_d64", 2, 4, 2, 64, 1500 * 64 + 33, 0, 256, 64, 64, "bf16", 31), (), 0),
    (_w("fallback_2049_blocks", 1, 4, 1, 64, 2049 * 64, 0, 8, 64, 64, "bf16", 32), (), 0),
    (_w("fallback_k257", 1, 4, 1, 64, 600 * 64, 0, 257, 64, 64, "bf16", 29), (), 0),
    # fp32, first order, fp32 means: up to 256 complete blocks and 16 items per pair the
    # step is one decode workgroup per pair that scores, selects and attends
    (WORKLOADS["tiny_decode_1k"], (), 0),
    (_w("f32_fused_256_blocks_tail_g16_d128", 1, 16, 1, 128, 256 * 64 + 40, 0, 8, 64, 64, "f32", 33), (), 0),
    (_w("f32_fused_globals_g8_d64", 2, 16, 2, 64, 5000, 0, 5, 100, 3, "f32", 34), (10, 2500, 4999), 0),
    (_w("f32_fallback_257_blocks", 1, 4, 1, 64, 257 * 64, 0, 4, 64, 64, "f32", 35), (), 0),
    (_w("f32_fallback_17_items", 1, 4, 1, 64, 3000, 0, 14, 64, 64, "f32", 36), (), 0),
]


@pytest.mark.parametrize("case", SMALL + ONE_CALL_EXTRA,
                         ids=[c[0].name for c in SMALL + ONE_CALL_EXTRA])
def test_one_call_step_small_cases(api, case):
    """bsattn_decode_step: the same oracle bar as the two calls, on every small case."""
    w, globals_, extra = case
    check_decode_case(api, w, globals_, extra, one_call=True)


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


def test_fp32_one_call_step_breaks_ties_by_index(api):
    """The fused fp32 step (one workgroup per pair scores and selects): with every
    candidate's score tied it takes the lowest-index candidates, as the top-k kernel."""
    w = _w("all_ties_f32", 1, 4, 1, 64, 64 * 200, 0, 7, 64, 64, "f32", 37)
    x = make_decode_inputs(w)
    K = x["K"].copy()
    K[:, :, :] = np.tile(K[:, :, :64], (1, 1, 200, 1))
    x = dict(x, K=K)
    two = gpu_decode_step(api, x, w)
    one = gpu_decode_step(api, x, w, one_call=True)
    assert np.array_equal(one["sel"][0, 0], np.arange(1, 8)), one["sel"][0, 0]
    assert np.array_equal(two["sel"], one["sel"])
    assert max_abs(two["O"], one["O"]) < 1e-5


def test_workgroup_select_breaks_ties_by_index(api):
    """1000 blocks (the workgroup-wide selection): every candidate's score ties
    exactly, so the lowest-index candidates are taken, as by the two calls."""
    w = _w("all_ties_wg", 1, 4, 1, 64, 64 * 1000, 0, 11, 64, 64, "bf16", 33)
    x = make_decode_inputs(w)
    K = x["K"].copy()
    K[:, :, :] = np.tile(K[:, :, :64], (1, 1, 1000, 1))
    x = dict(x, K=K)
    two = gpu_decode_step(api, x, w)
    one = gpu_decode_step(api, x, w, one_call=True)
    assert np.array_equal(one["sel"][0, 0], np.arange(1, 12)), one["sel"][0, 0]
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
    check_decode_case(api, WORKLOADS["tiny_decode_1k"], (), 0)


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


def _full_size(api, name, pairs=None, one_call=False, mean_dtype="f32"):
    """Full-size workload against the oracle, every stage, on ``pairs`` (all pairs
    when None)."""
    import torch
    w = WORKLOADS[name]
    print(f"[decode full size] {name}: generating inputs", flush=True)
    x = make_decode_inputs(w)
    print(f"[decode full size] {name}: running on the GPU", flush=True)
    got = gpu_decode_step(api, x, w, one_call=one_call, mean_dtype=mean_dtype)
    torch.cuda.empty_cache()
    assert np.isfinite(got["O"]).all() and np.isfinite(got["lse"]).all()
    if pairs is None:
        pairs = [(b, g) for b in range(w.batch) for g in range(w.n_kv_heads)]
    Q = as_f64(x["Q"])
    ties = 0
    stats = {}
    for (b, g) in pairs:
        Kb, Vb = PairView({(b, g): as_f64(x["K"][b, g])}), PairView({(b, g): as_f64(x["V"][b, g])})
        ties += check_pair(got, b, g, Q, Kb, Vb, w, (), mean_dtype=mean_dtype, stats=stats)
    print(f"[decode full size] {name}: {len(pairs)} pairs checked, near ties {ties}, "
          f"cluster rows {stats.get('cluster_rows', 0)}", flush=True)


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
    check_decode_case(api, w, globals_, extra, one_call=True, mean_dtype="bf16")


def test_headline_step_full_size_every_pair(api):
    """The headline configuration as measured (32K first-order workload, one-call
    step, bfloat16 means): every one of its 128 (b, K/V head) pairs against the
    oracle, every stage."""
    _full_size(api, "first_order_decode_32k", None, one_call=True, mean_dtype="bf16")


def test_bf16_means_full_size_cobs(api):
    _full_size(api, "cobs_decode_128k", [(2, 5)], one_call=True, mean_dtype="bf16")


FP4_CASES = [c for c in SMALL if c[0].rank > 0]


@pytest.mark.parametrize("case", FP4_CASES, ids=[c[0].name for c in FP4_CASES])
@pytest.mark.parametrize("one_call", [False, True])
def test_fp4_factors_small_cases(api, case, one_call):
    w, globals_, _ = case
    check_fp4_case(api, w, globals_, one_call=one_call, mean_dtype="bf16" if one_call else "f32")


def test_fp4_factors_cobs_128k(api):
    check_fp4_case(api, WORKLOADS["cobs_decode_128k"], (), pairs=[(0, 0), (3, 6)])


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
    check_fp4_case(api, w, globals_, one_call=one_call, basis=calibration_basis(w, sub_dim, 50 + sub_dim))


_COBS = {}


def _cobs_compressed(api):
    """The COBS 128K workload as measured (one-call step, bf16 means, FP4 rows in a
    96-dim query subspace), run once on the GPU and kept for the pair checks."""
    if not _COBS:
        w = WORKLOADS["cobs_decode_128k"]
        x = make_decode_inputs(w)
        basis = calibration_basis(w, 96, 60)
        print("[decode fp4] cobs_decode_128k compressed: running on the GPU", flush=True)
        got = gpu_decode_step(api, x, w, one_call=True, mean_dtype="bf16", factor_fp4=True, basis=basis)
        _COBS.update(w=w, x=x, basis=basis, got=got)
    return _COBS


@pytest.mark.parametrize("pairs", [[(0, 0), (0, 7), (1, 2), (1, 5)], [(2, 1), (2, 5), (3, 3), (3, 6)]],
                         ids=["pairs_0_1", "pairs_2_3"])
def test_subspace_projection_cobs_128k(api, pairs):
    """Eight of the 32 (b, K/V head) pairs, two in every sequence, every block."""
    c = _cobs_compressed(api)
    check_fp4_case(api, c["w"], (), pairs=pairs, basis=c["basis"], x=c["x"], got=c["got"])
    if pairs[-1] == (3, 6):
        _COBS.clear()


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
    ties = check_decode_case(api, w, globals_, 0)
    print(f"[decode max sizes] near ties: {ties}", flush=True)


def test_dilated_window_as_forced_positions(api):
    """A dilated sliding window (the SWA glossary's extension: every delta-th token
    back from the query) expressed as forced positions: the window argument 0 and the
    positions t, t - 4, ..., t - 4 * 39 given as global positions; checked against the
    oracle with the same forced set."""
    w = _w("dilated_window", 1, 8, 2, 128, 3000, 0, 6, 0, 16, "bf16", 45)
    t = w.n_ctx - 1
    globals_ = tuple(sorted(t - 4 * m for m in range(40)))
    check_decode_case(api, w, globals_, 0, one_call=True, mean_dtype="bf16")
