"""GPU parity of the block-sparse causal prefill (query tiles of 128 rows sharing a
selected block set) against the fp64 oracle, through the C ABI.

Bar: the tile scores of candidate blocks within 1e-4 (both sides score bf16 means;
the GPU rounds its fp32 block mean, the oracle its fp64 mean); per (b, K/V head,
tile) the selected set equal to the oracle's except at near ties (relative gap
< 1e-4 between the k-th and (k+1)-th scores); outputs and lse within max-abs 2e-3
of the oracle's attention over the GPU's selection.
"""

import numpy as np
import pytest

import oracle
from synthetic import PrefillWorkload, make_prefill_inputs

from gpu_util import OUT_TOL, as_f64, compare_selection, max_abs, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    import torch
    assert torch.cuda.is_available(), "GPU tests need the GPU"
    import sliding_window_attention_block_amd as m
    m.library()
    return m


def _pw(name, B, Hq, Hkv, d, N, seed):
    return PrefillWorkload(name=name, batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, seq_len=N,
                           window_left=-1, window_right=0, causal=True, seed=seed)


def _run(api, x, w, wl, ns, k):
    import torch
    B, Hq, Hkv, d, N = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.seq_len
    nb = N // 64
    nbcap = max(nb, 1)
    n_tiles = (N + 127) // 128
    Q, K, V = to_dev(x["Q"]), to_dev(x["K"]), to_dev(x["V"])
    shape = api.make_shape(B, Hq, Hkv, d, N, dtype="bf16")
    mean = torch.full((B, Hkv, nbcap, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    api.bsattn_build_summaries(shape, K, 0, 0, nb, nbcap, mean)
    scores = torch.full((B, Hkv, n_tiles, nbcap), float("nan"), device="cuda")
    sel = torch.full((B, Hkv, n_tiles, k), -7, dtype=torch.int32, device="cuda")
    api.bsattn_select_prefill(shape, Q, mean, nbcap, k, wl, ns, sel, scores)
    O = torch.full((B, Hq, N, d), float("nan"), device="cuda")
    lse = torch.full((B, Hq, N), float("nan"), device="cuda")
    api.bsattn_sparse_prefill(shape, Q, K, V, sel, k, wl, ns, O, lse)
    torch.cuda.synchronize()
    return dict(scores=scores.cpu().numpy(), sel=sel.cpu().numpy(), O=O.cpu().numpy(), lse=lse.cpu().numpy())


def _check(api, w, wl, ns, k, rows=None, pairs=None):
    x = make_prefill_inputs(w)
    print(f"[sparse prefill] {w.name}: N={w.seq_len} d={w.head_dim} wl={wl} sinks={ns} k={k}", flush=True)
    got = _run(api, x, w, wl, ns, k)
    Q, K, V = as_f64(x["Q"]), as_f64(x["K"]), as_f64(x["V"])
    N, G = w.seq_len, w.n_q_heads // w.n_kv_heads
    if pairs is None:
        pairs = [(b, g) for b in range(w.batch) for g in range(w.n_kv_heads)]
    ref = oracle.sparse_prefill_selection(Q, K, N, 64, k, wl, ns, mean_bf16=True, pairs=pairs)
    n_tiles = (N + 127) // 128
    for (b, g) in pairs:
        for t in range(n_tiles):
            cand = oracle.tile_candidates(128 * t, N, 64, wl, ns)
            s_ref = ref[(b, g)]["scores"][t]
            if len(cand):
                err = np.abs(got["scores"][b, g, t, cand] - s_ref[cand])
                assert np.all(err <= 1e-4 * (1 + np.abs(s_ref[cand]))), f"scores (b={b}, g={g}, tile {t})"
            ok, _ = compare_selection(got["sel"][b, g, t], s_ref, cand, k)
            assert ok, f"selection (b={b}, g={g}, tile {t}): {got['sel'][b, g, t]} vs " \
                       f"{oracle.top_k_blocks(s_ref, cand, k)}"
    # outputs over the GPU's selection
    gsel = {(b, g): dict(sel=got["sel"][b, g]) for (b, g) in pairs}
    out = oracle.sparse_prefill(Q, K, V, N, 64, wl, ns, gsel, rows=rows)
    r = np.arange(N) if rows is None else np.asarray(rows)
    for (b, g), (O, L) in out.items():
        for hh in range(G):
            h = g * G + hh
            assert max_abs(got["O"][b, h, r], O[hh]) < OUT_TOL, f"O (b={b}, h={h})"
            assert max_abs(got["lse"][b, h, r], L[hh]) < OUT_TOL, f"lse (b={b}, h={h})"


SMALL = [
    # workload, window_left, sinks, k
    (_pw("sp_tail_d128", 1, 8, 2, 128, 1000, 90), 127, 64, 3),
    (_pw("sp_d64_g4", 2, 8, 2, 64, 1536, 91), 300, 0, 5),
    (_pw("sp_sink_past_end", 1, 4, 1, 64, 100, 92), 20, 90, 2),   # sink block 1 runs past N
    (_pw("sp_k_exceeds", 1, 4, 2, 128, 777, 93), 64, 16, 64),     # k above the candidates
    (_pw("sp_short_window", 1, 2, 1, 128, 640, 94), 0, 1, 4),     # window: the row itself
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0].name for c in SMALL])
def test_sparse_prefill_small_cases(api, case):
    w, wl, ns, k = case
    _check(api, w, wl, ns, k)


def test_sparse_prefill_8k_sampled_rows(api):
    """The Mistral-shaped 8K GQA prefill with a 1024-token window, 64 sinks and 16
    selected blocks per 128-row tile; oracle on sampled rows of two K/V heads."""
    w = _pw("sparse_prefill_8k", 1, 32, 8, 128, 8192, 95)
    rows = np.array([0, 127, 128, 1000, 1023, 1024, 2047, 4096, 5000, 8064, 8191])
    _check(api, w, 1023, 64, 16, rows=rows, pairs=[(0, 0), (0, 5)])


def test_random_blocks_bigbird_style(api):
    """Random attention (the SWA glossary's BigBird extension), block-wise: each
    query tile attends r seeded random earlier blocks besides its causal window and
    sinks.  The blocks are an input (drawn here, not selected), passed as the tile
    selection; outputs against the oracle with the same blocks."""
    import torch
    w = _pw("sp_bigbird", 1, 8, 2, 128, 1280, 96)
    wl, ns, r = 127, 32, 3
    N, G = w.seq_len, w.n_q_heads // w.n_kv_heads
    n_tiles = (N + 127) // 128
    rng = np.random.default_rng(97)
    sel = np.full((w.batch, w.n_kv_heads, n_tiles, r), -1, dtype=np.int32)
    for b in range(w.batch):
        for g in range(w.n_kv_heads):
            for t in range(n_tiles):
                earlier = np.arange((128 * t) // 64)
                if len(earlier):
                    pick = np.sort(rng.choice(earlier, min(r, len(earlier)), replace=False))
                    sel[b, g, t, :len(pick)] = pick
    x = make_prefill_inputs(w)
    Q, K, V = to_dev(x["Q"]), to_dev(x["K"]), to_dev(x["V"])
    shape = api.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, N, dtype="bf16")
    O = torch.full((w.batch, w.n_q_heads, N, w.head_dim), float("nan"), device="cuda")
    lse = torch.full((w.batch, w.n_q_heads, N), float("nan"), device="cuda")
    api.bsattn_sparse_prefill(shape, Q, K, V, torch.from_numpy(sel).cuda(), r, wl, ns, O, lse)
    torch.cuda.synchronize()
    Of, Lf = O.cpu().numpy(), lse.cpu().numpy()
    selection = {(b, g): dict(sel=sel[b, g]) for b in range(w.batch) for g in range(w.n_kv_heads)}
    ref = oracle.sparse_prefill(as_f64(x["Q"]), as_f64(x["K"]), as_f64(x["V"]), N, 64, wl, ns, selection)
    for (b, g), (Or, Lr) in ref.items():
        for hh in range(G):
            assert max_abs(Of[b, g * G + hh], Or[hh]) < OUT_TOL
            assert max_abs(Lf[b, g * G + hh], Lr[hh]) < OUT_TOL


def test_sparse_prefill_maximum_sizes(api):
    """top_k = 256 and n_sink = 256 (the limits): late tiles of a 300-block sequence
    have more than 256 candidates, and their extra-stage list holds 256 selected plus
    4 sink blocks; oracle on sampled rows."""
    w = _pw("sp_max", 1, 4, 1, 64, 64 * 300, 98)
    rows = np.array([0, 255, 256, 4000, 16383, 17000, 19100, 64 * 300 - 1])
    _check(api, w, 127, 256, 256, rows=rows)
