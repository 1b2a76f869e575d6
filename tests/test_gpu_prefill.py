"""GPU parity of the MFMA prefill (causal band and local+global masks) against the fp64
oracle, through the C ABI.  Bar: O and lse within max-abs 2e-3 (compared in fp32).

Small cases compare every output; the full-size workloads compare sampled rows
(first rows, band edges, global rows and their neighbours, the last rows) in
the exact launch configuration the benchmark times.
"""

import numpy as np
import pytest

import oracle
from synthetic import WORKLOADS, PrefillWorkload, make_prefill_inputs

from gpu_util import OUT_TOL, as_f64, max_abs, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    import torch
    assert torch.cuda.is_available(), "GPU tests need the GPU"
    import sliding_window_attention_block_amd as m
    m.library()
    return m


def _run(api, w, x, extra_cap=0):
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
    nbytes = api.bsattn_prefill_workspace_bytes(shape, len(w.global_pos))
    # garbage contents: the workspace needs no initialisation
    ws = torch.full((nbytes,), 255, dtype=torch.uint8, device="cuda") if nbytes else None
    api.bsattn_prefill(shape, Q, K, V, w.window_left, w.window_right, w.causal, list(w.global_pos),
                       O, lse, ws)
    torch.cuda.synchronize()
    return O.cpu().numpy(), lse.cpu().numpy()


def _pw(name, B, Hq, Hkv, N, d, wl, wr, causal, globals_=(), seed=0, scale_in=1.0):
    return PrefillWorkload(name=name, batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, seq_len=N,
                           window_left=wl, window_right=wr, causal=causal, seed=seed,
                           input_scale=scale_in, global_pos=tuple(globals_))


SMALL = [
    (_pw("band_d128_gqa", 1, 8, 2, 700, 128, 99, 0, True, seed=30, scale_in=0.5), 0),
    (_pw("band_d64_w1", 1, 2, 1, 300, 64, 0, 0, True, seed=31), 0),
    (_pw("full_causal_d64", 2, 4, 4, 333, 64, -1, 0, True, seed=32), 16),
    (_pw("band_d128_wide", 1, 4, 1, 1100, 128, 700, 0, True, seed=33, scale_in=0.5), 0),
    (_pw("lg_d64", 1, 3, 3, 1500, 64, 40, 40, False, (0, 130, 131, 700, 1499), seed=34), 0),
    (_pw("lg_d128_gqa", 2, 4, 2, 900, 128, 64, 64, False, (0, 512), seed=35), 8),
    (_pw("lg_many_globals", 1, 2, 1, 1200, 64, 16, 16, False, tuple(range(3, 1200, 37)), seed=36), 0),
    (_pw("bidir_asym", 1, 2, 2, 500, 64, 5, 60, False, seed=37), 0),
    (_pw("dense_bidir", 1, 2, 1, 260, 128, -1, -1, False, seed=38), 0),
    (_pw("tiny_seq", 1, 2, 1, 7, 64, 3, 0, True, seed=39), 0),
    (_pw("lg_short_seq", 1, 2, 1, 100, 128, 8, 8, False, (5, 50, 99), seed=40), 3),
    # the global-position limit (256: eight 32-row global tiles; most key tiles
    # hold globals outside the band), and a d = 128 GQA case with 100 globals
    (_pw("lg_max_globals", 1, 2, 1, 2048, 64, 32, 32, False,
         tuple(int(p) for p in np.sort(np.random.default_rng(42).choice(2048, 256, replace=False))), seed=41), 0),
    (_pw("lg_d128_100_globals", 1, 4, 2, 1600, 128, 48, 20, False,
         tuple(int(p) for p in np.sort(np.random.default_rng(43).choice(1600, 100, replace=False))), seed=42,
         scale_in=0.5), 5),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0].name for c in SMALL])
def test_prefill_small_cases(api, case):
    w, extra = case
    print(f"[prefill parity] {w.name}", flush=True)
    x = make_prefill_inputs(w)
    O, lse = _run(api, w, x, extra)
    Oref, Lref = oracle.prefill(as_f64(x["Q"]), as_f64(x["K"]), as_f64(x["V"]), w.window_left,
                                w.window_right, w.causal, w.global_pos)
    assert max_abs(O, Oref) < OUT_TOL
    assert max_abs(lse, Lref) < OUT_TOL


def _sampled(api, name, rows, heads, batches=(0,)):
    w = WORKLOADS[name]
    print(f"[prefill full size] {name}: generating inputs", flush=True)
    x = make_prefill_inputs(w)
    print(f"[prefill full size] {name}: running on the GPU", flush=True)
    O, lse = _run(api, w, x)
    assert np.isfinite(O).all() and np.isfinite(lse).all()
    rows = np.array(sorted(set(r for r in rows if 0 <= r < w.seq_len)))
    print(f"[prefill full size] {name}: oracle on {len(rows)} rows x {len(heads)} heads", flush=True)
    Oref, Lref = oracle.prefill(as_f64(x["Q"]), as_f64(x["K"]), as_f64(x["V"]), w.window_left,
                                w.window_right, w.causal, w.global_pos, rows=rows,
                                batches=batches, heads=heads)
    for bi, b in enumerate(batches):
        for hi, h in enumerate(heads):
            assert max_abs(O[b, h][rows], Oref[bi, hi]) < OUT_TOL, (b, h)
            assert max_abs(lse[b, h][rows], Lref[bi, hi]) < OUT_TOL, (b, h)


def test_swa_prefill_8k_full_size(api):
    rows = (list(range(0, 70)) + list(range(4030, 4160)) + list(range(8100, 8192)) +
            list(np.random.default_rng(0).integers(0, 8192, 60)))
    _sampled(api, "swa_prefill_8k", rows, heads=[0, 5, 31])


def test_local_global_prefill_16k_full_size(api):
    g = list(range(0, 16384, 1024))
    rows = (g + [p + o for p in g for o in (-257, -256, -1, 1, 255, 256, 257)] +
            list(range(0, 40)) + list(range(16340, 16384)) +
            list(np.random.default_rng(1).integers(0, 16384, 60)))
    _sampled(api, "local_global_prefill_16k", rows, heads=[0, 11], batches=(0, 1))
