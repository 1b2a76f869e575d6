"""GPU parity of the dilated sliding-window prefill (SWA glossary, SWAの拡張手法:
dilated SWA) against the fp64 oracle, through the C ABI.  Query i sees key j when
the band allows it and i - j is a multiple of the dilation s.  Bar: O and lse within
max-abs 2e-3 of the oracle (compared in fp32); every output on the small cases,
sampled rows on the 8K case.
"""

import numpy as np
import pytest

import oracle
from synthetic import PrefillWorkload, make_prefill_inputs

from gpu_util import OUT_TOL, as_f64, max_abs, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    import torch
    assert torch.cuda.is_available(), "GPU tests need the GPU"
    import sliding_window_attention_block_amd as m
    m.library()
    return m


def _pw(name, B, Hq, Hkv, N, d, wl, wr, causal, seed, scale_in=1.0):
    return PrefillWorkload(name=name, batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, seq_len=N,
                           window_left=wl, window_right=wr, causal=causal, seed=seed, input_scale=scale_in)


def _run(api, w, x, s, extra_cap=0, plain=False):
    import torch
    B, Hq, Hkv, N, d = w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len, w.head_dim
    Q = to_dev(x["Q"])
    K, V = x["K"], x["V"]
    if extra_cap:
        pad = ((0, 0), (0, 0), (0, extra_cap), (0, 0))
        K, V = np.pad(K, pad), np.pad(V, pad)
    K, V = to_dev(K), to_dev(V)
    shape = api.make_shape(B, Hq, Hkv, d, N, kv_capacity=N + extra_cap, dtype="bf16")
    O = torch.full((B, Hq, N, d), float("nan"), device="cuda")
    lse = torch.full((B, Hq, N), float("nan"), device="cuda")
    if plain:
        api.bsattn_prefill(shape, Q, K, V, w.window_left, w.window_right, w.causal, [], O, lse, None)
    else:
        api.bsattn_prefill_dilated(shape, Q, K, V, w.window_left, w.window_right, w.causal, s, O, lse)
    torch.cuda.synchronize()
    return O.cpu().numpy(), lse.cpu().numpy()


#        case                                                                              dilation  extra cap
SMALL = [
    # 200 keys at spacing 2, GQA, d = 128 (several 64-key stages per residue class)
    (_pw("causal_d128_gqa_s2", 1, 8, 2, 1000, 128, 2 * 199, 0, True, 60, 0.5), 2, 0),
    # a ragged length and a window that is not a multiple of the spacing
    (_pw("causal_d64_s3_ragged", 2, 2, 1, 777, 64, 3 * 149 + 2, 0, True, 61), 3, 0),
    (_pw("causal_d64_s7_wide", 1, 4, 4, 2000, 64, 7 * 300, 0, True, 62), 7, 16),
    (_pw("bidir_d64_s2", 1, 3, 1, 900, 64, 120, 61, False, 63), 2, 0),
    (_pw("bidir_d128_s5", 1, 4, 2, 1300, 128, 400, 400, False, 64, 0.5), 5, 8),
    # no window limit: every s-th earlier key
    (_pw("causal_unlimited_s4", 1, 2, 1, 600, 64, -1, 0, True, 65), 4, 0),
    # a spacing above the length: every residue class is one row (itself)
    (_pw("spacing_above_length", 1, 2, 1, 300, 64, 5000, 0, True, 66), 1000, 0),
    # residue classes shorter than one 128-row tile
    (_pw("short_classes_s9", 1, 2, 1, 250, 128, 90, 0, True, 67, 0.5), 9, 0),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0].name for c in SMALL])
def test_dilated_prefill_small_cases(api, case):
    w, s, extra = case
    print(f"[dilated prefill] {w.name} s={s}", flush=True)
    x = make_prefill_inputs(w)
    O, lse = _run(api, w, x, s, extra)
    Oref, Lref = oracle.prefill(as_f64(x["Q"]), as_f64(x["K"]), as_f64(x["V"]), w.window_left,
                                w.window_right, w.causal, dilation=s)
    assert max_abs(O, Oref) < OUT_TOL
    assert max_abs(lse, Lref) < OUT_TOL


def test_dilation_one_is_the_plain_prefill(api):
    """Dilation 1 runs the plain band kernel: bit for bit bsattn_prefill's output."""
    w = _pw("dilation_one", 1, 4, 1, 700, 128, 255, 0, True, 68, 0.5)
    x = make_prefill_inputs(w)
    O1, L1 = _run(api, w, x, 1)
    O0, L0 = _run(api, w, x, 1, plain=True)
    assert np.array_equal(O1, O0) and np.array_equal(L1, L0)


def test_dilated_prefill_8k_sampled_rows(api):
    """The 8K Mistral-shaped prefill (32 query / 8 K/V heads, d = 128) with 2048 keys
    at spacing 2 (window_left = 4094): the same number of attended pairs per row as
    the plain w = 2048 band, spread over 4095 positions."""
    w = _pw("dilated_swa_8k", 1, 32, 8, 8192, 128, 2 * 2047, 0, True, 69, 0.5)
    print("[dilated prefill] 8K: inputs", flush=True)
    x = make_prefill_inputs(w)
    print("[dilated prefill] 8K: GPU", flush=True)
    O, lse = _run(api, w, x, 2)
    assert np.isfinite(O).all() and np.isfinite(lse).all()
    rows = np.array(sorted(set(list(range(0, 40)) + list(range(4070, 4130)) + list(range(8150, 8192)) +
                               [int(r) for r in np.random.default_rng(7).integers(0, 8192, 40)])))
    heads = [0, 9, 31]
    print(f"[dilated prefill] 8K: oracle on {len(rows)} rows x {len(heads)} heads", flush=True)
    Oref, Lref = oracle.prefill(as_f64(x["Q"]), as_f64(x["K"]), as_f64(x["V"]), w.window_left,
                                w.window_right, w.causal, rows=rows, heads=heads, dilation=2)
    for hi, h in enumerate(heads):
        assert max_abs(O[0, h][rows], Oref[0, hi]) < OUT_TOL, h
        assert max_abs(lse[0, h][rows], Lref[0, hi]) < OUT_TOL, h
