"""GPU parity of the exact-mass selector (the selection oracle of the COBS explainer,
section 2.1, on the GPU) against the fp64 oracle, through the C ABI.

Bar: group scores ln sum_h sum_{t in block} exp(q~_h . k_t) within 1e-4 relative
(bf16 keys and queries: exact products; fp32 sums against fp64); the selected sets
equal to the oracle's except at near ties; the decode over that selection within
max-abs 2e-3 of the oracle's.
"""

import numpy as np
import pytest

import oracle
from synthetic import WORKLOADS, DecodeWorkload, make_decode_inputs

from gpu_util import OUT_TOL, as_f64, compare_selection, default_scale, max_abs, oracle_decode_with_sel, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    import torch
    assert torch.cuda.is_available(), "GPU tests need the GPU"
    import sliding_window_attention_block_amd as m
    m.library()
    return m


def _w(name, B, Hq, Hkv, d, n, k, W, ns, seed):
    return DecodeWorkload(name=name, batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, n_ctx=n,
                          block_size=64, rank=0, top_k=k, window=W, n_sink=ns, dtype="bf16", seed=seed)


def _check(api, w, globals_=(), pairs=None):
    import torch
    x = make_decode_inputs(w)
    B, Hq, Hkv, d, n = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_ctx
    nb = n // 64
    print(f"[exact select] {w.name}", flush=True)
    Q, K, V = to_dev(x["Q"]), to_dev(x["K"]), to_dev(x["V"])
    shape = api.make_shape(B, Hq, Hkv, d, n, kv_capacity=x["K"].shape[2], dtype="bf16")
    scores = torch.full((B, Hkv, max(nb, 1)), float("nan"), device="cuda")
    sel = torch.full((B, Hkv, w.top_k), -7, dtype=torch.int32, device="cuda")
    api.bsattn_select_exact(shape, Q, K, max(nb, 1), w.top_k, w.window, w.n_sink, list(globals_), sel, scores)
    O = torch.full((B, Hq, d), float("nan"), device="cuda")
    lse = torch.full((B, Hq), float("nan"), device="cuda")
    ws = torch.zeros(api.bsattn_decode_workspace_bytes(shape, w.top_k, w.window, w.n_sink, len(globals_)),
                     dtype=torch.uint8, device="cuda")
    api.bsattn_decode(shape, Q, K, V, sel, w.top_k, w.window, w.n_sink, list(globals_), O, lse, ws)
    torch.cuda.synchronize()
    got_s, got_sel, got_O, got_l = scores.cpu().numpy(), sel.cpu().numpy(), O.cpu().numpy(), lse.cpu().numpy()
    Qf, Kf, Vf = as_f64(x["Q"]), as_f64(x["K"]), as_f64(x["V"])
    G, scale = Hq // Hkv, default_scale(d)
    forced = oracle.forced_token_mask(n, w.n_sink, w.window, globals_)
    cand = oracle.candidate_blocks(n, 64, forced)
    for (b, g) in (pairs or [(b, g) for b in range(B) for g in range(Hkv)]):
        q = Qf[b, g * G:(g + 1) * G]
        s_ref = oracle.group_scores(oracle.exact_mass_scores(scale * q, Kf[b, g, :n], 64))
        if nb:
            assert np.all(np.abs(got_s[b, g, :nb] - s_ref) <= 1e-4 * (1 + np.abs(s_ref))), f"scores ({b}, {g})"
        ok, _ = compare_selection(got_sel[b, g], s_ref, cand, w.top_k)
        assert ok, f"selection ({b}, {g}): {got_sel[b, g]} vs {oracle.top_k_blocks(s_ref, cand, w.top_k)}"
        o_ref, l_ref = oracle_decode_with_sel(q, Kf[b, g], Vf[b, g], n, 64, w.window, w.n_sink, globals_,
                                              got_sel[b, g], scale)
        assert max_abs(got_O[b, g * G:(g + 1) * G], o_ref) < OUT_TOL
        assert max_abs(got_l[b, g * G:(g + 1) * G], l_ref) < OUT_TOL


SMALL = [
    (_w("ex_g4_d128", 2, 8, 2, 128, 1000, 3, 100, 5, 60), ()),
    (_w("ex_g8_d64_globals", 1, 16, 2, 64, 2065, 5, 130, 64, 61), (3, 200, 201, 1500)),
    (_w("ex_g1_tail", 2, 2, 2, 128, 64 * 20 + 33, 4, 1, 1, 62), ()),
    (_w("ex_g16_k_exceeds", 1, 16, 1, 64, 640, 20, 64, 64, 63), ()),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0].name for c in SMALL])
def test_exact_select_small_cases(api, case):
    w, globals_ = case
    _check(api, w, globals_)


def test_exact_select_first_order_32k(api):
    """The 32K workload: every key of 128 (b, K/V head) pairs is read; two pairs
    checked against the oracle."""
    _check(api, WORKLOADS["first_order_decode_32k"], pairs=[(0, 0), (11, 6)])
