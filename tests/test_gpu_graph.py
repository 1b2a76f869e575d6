"""The library's calls inside a captured HIP graph: every replay gives the same
bits as the eager calls.  The kernels allocate nothing, clear nothing with
memset and keep no state, so a graph replays them as recorded; this checks it
on several replays with eager work and synchronisations between them."""

import numpy as np
import pytest

from synthetic import DecodeWorkload, PrefillWorkload, make_decode_inputs, make_prefill_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_api():
    import torch
    assert torch.cuda.is_available(), "GPU tests need the GPU"
    import sliding_window_attention_block_amd as m
    m.library()
    return torch, m


def _dev(torch, a):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def test_decode_step_replays_bit_exactly(torch_api):
    torch, api = torch_api
    w = DecodeWorkload(name="graph_decode", batch=2, n_q_heads=16, n_kv_heads=2, head_dim=128,
                       n_ctx=4100, block_size=64, rank=2, top_k=6, window=200, n_sink=64,
                       dtype="bf16", seed=41)
    x = make_decode_inputs(w)
    Q, K, V = _dev(torch, x["Q"]), _dev(torch, x["K"]), _dev(torch, x["V"])
    B, Hq, Hkv, d, n, nb = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_ctx, w.n_ctx // 64
    shape = api.make_shape(B, Hq, Hkv, d, n)
    mean = torch.empty((B, Hkv, nb, d), device="cuda")
    factor = torch.empty((B, Hkv, nb, w.rank, d), device="cuda")
    api.bsattn_build_summaries(shape, K, w.rank, 0, nb, nb, mean, factor)
    scores = torch.empty((B, Hkv, nb), device="cuda")
    sel = torch.empty((B, Hkv, w.top_k), dtype=torch.int32, device="cuda")
    ws = torch.empty(api.bsattn_decode_workspace_bytes(shape, w.top_k, w.window, w.n_sink, 0),
                     dtype=torch.uint8, device="cuda")
    O = torch.empty((B, Hq, d), device="cuda")
    lse = torch.empty((B, Hq), device="cuda")

    def step():
        api.bsattn_select_topk(shape, Q, mean, factor, w.rank, nb, w.top_k, w.window, w.n_sink, None,
                               sel, scores)
        api.bsattn_decode(shape, Q, K, V, sel, w.top_k, w.window, w.n_sink, None, O, lse, ws)

    step()
    torch.cuda.synchronize()
    ref = [t.cpu().numpy().copy() for t in (sel, O, lse)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in (O, lse):
            t.fill_(float("nan"))
        sel.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((sel, O, lse), ref):
            assert np.array_equal(got.cpu().numpy(), want), f"replay {rep}"
        step()  # eager work between replays
        torch.cuda.synchronize()


def test_local_global_prefill_replays_bit_exactly(torch_api):
    torch, api = torch_api
    w = PrefillWorkload(name="graph_prefill", batch=1, n_q_heads=2, n_kv_heads=1, head_dim=64,
                        seq_len=1500, window_left=64, window_right=64, causal=False, seed=42,
                        global_pos=(0, 700, 1499))
    x = make_prefill_inputs(w)
    Q, K, V = _dev(torch, x["Q"]), _dev(torch, x["K"]), _dev(torch, x["V"])
    shape = api.make_shape(1, 2, 1, 64, 1500)
    ws = torch.empty(api.bsattn_prefill_workspace_bytes(shape, 3), dtype=torch.uint8, device="cuda")
    O = torch.empty((1, 2, 1500, 64), device="cuda")
    lse = torch.empty((1, 2, 1500), device="cuda")

    def run():
        api.bsattn_prefill(shape, Q, K, V, 64, 64, 0, [0, 700, 1499], O, lse, ws)

    run()
    torch.cuda.synchronize()
    ref = [t.cpu().numpy().copy() for t in (O, lse)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        O.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((O, lse), ref):
            assert np.array_equal(got.cpu().numpy(), want), f"replay {rep}"
        run()
        torch.cuda.synchronize()


def test_one_call_decode_step_replays_bit_exactly(torch_api):
    """bsattn_decode_step (scores, then the decode kernel that selects in its waves,
    then the merge) captured as one graph."""
    torch, api = torch_api
    w = DecodeWorkload(name="graph_one_call", batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128,
                       n_ctx=5000, block_size=64, rank=0, top_k=5, window=300, n_sink=64,
                       dtype="bf16", seed=43)
    x = make_decode_inputs(w)
    Q, K, V = _dev(torch, x["Q"]), _dev(torch, x["K"]), _dev(torch, x["V"])
    B, Hq, Hkv, d, n, nb = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_ctx, w.n_ctx // 64
    shape = api.make_shape(B, Hq, Hkv, d, n)
    mean = torch.empty((B, Hkv, nb, d), device="cuda")
    api.bsattn_build_summaries(shape, K, 0, 0, nb, nb, mean, None)
    scores = torch.empty((B, Hkv, nb), device="cuda")
    sel = torch.empty((B, Hkv, w.top_k), dtype=torch.int32, device="cuda")
    ws = torch.empty(api.bsattn_decode_workspace_bytes(shape, w.top_k, w.window, w.n_sink, 0),
                     dtype=torch.uint8, device="cuda")
    O = torch.empty((B, Hq, d), device="cuda")
    lse = torch.empty((B, Hq), device="cuda")

    def step():
        api.bsattn_decode_step(shape, Q, K, V, mean, None, 0, nb, w.top_k, w.window, w.n_sink, None,
                               sel, scores, O, lse, ws)

    step()
    torch.cuda.synchronize()
    ref = [t.cpu().numpy().copy() for t in (sel, O, lse)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in (O, lse):
            t.fill_(float("nan"))
        sel.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((sel, O, lse), ref):
            assert np.array_equal(got.cpu().numpy(), want), f"replay {rep}"
        step()
        torch.cuda.synchronize()


def _replay_check(torch, step, outs, fill):
    """Eager step, capture, then four replays (outputs refilled before each, eager
    work between them), each bit-equal to the eager result."""
    step()
    torch.cuda.synchronize()
    ref = [t.cpu().numpy().copy() for t in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        fill()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip(outs, ref):
            assert np.array_equal(got.cpu().numpy(), want), f"replay {rep}"
        step()
        torch.cuda.synchronize()


def test_paged_one_call_step_replays_bit_exactly(torch_api):
    """The one-call step on 16-token pages (compressed summary: bf16 means, FP4 rows)."""
    torch, api = torch_api
    w = DecodeWorkload(name="graph_paged", batch=2, n_q_heads=16, n_kv_heads=2, head_dim=128,
                       n_ctx=3000, block_size=64, rank=4, top_k=5, window=200, n_sink=64,
                       dtype="bf16", seed=44)
    x = make_decode_inputs(w, kv_capacity=3008)
    Q, K, V = _dev(torch, x["Q"]), _dev(torch, x["K"]), _dev(torch, x["V"])
    B, Hq, Hkv, d, n, nb, P = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_ctx, w.n_ctx // 64, 16
    mp = 3008 // P
    perm = np.random.default_rng(45).permutation(B * mp).reshape(B, mp).astype(np.int32)
    idx = torch.from_numpy(perm.reshape(-1)).cuda().long()
    pools = []
    for X in (K, V):
        pool = torch.empty((B * mp, Hkv, P, d), dtype=X.dtype, device="cuda")
        pool[idx] = X.reshape(B, Hkv, mp, P, d).permute(0, 2, 1, 3, 4).reshape(B * mp, Hkv, P, d)
        pools.append(pool)
    table = torch.from_numpy(perm).cuda()
    pg = api.paged_kv(table, P, B * mp)
    shape = api.make_shape(B, Hq, Hkv, d, n, kv_capacity=3008)
    mean = torch.empty((B, Hkv, nb, d), dtype=torch.bfloat16, device="cuda")
    factor = torch.empty((B, Hkv, nb, w.rank, d // 2), dtype=torch.uint8, device="cuda")
    fscale = torch.empty((B, Hkv, nb, w.rank), device="cuda")
    api.bsattn_build_summaries(shape, pools[0], w.rank, 0, nb, nb, mean, factor, factor_scale=fscale, paged=pg)
    scores = torch.empty((B, Hkv, nb), device="cuda")
    sel = torch.empty((B, Hkv, w.top_k), dtype=torch.int32, device="cuda")
    ws = torch.empty(api.bsattn_decode_workspace_bytes(shape, w.top_k, w.window, w.n_sink, 0),
                     dtype=torch.uint8, device="cuda")
    O = torch.empty((B, Hq, d), device="cuda")
    lse = torch.empty((B, Hq), device="cuda")

    def step():
        api.bsattn_decode_step(shape, Q, pools[0], pools[1], mean, factor, w.rank, nb, w.top_k, w.window,
                               w.n_sink, None, sel, scores, O, lse, ws, factor_scale=fscale, paged=pg)

    def fill():
        O.fill_(float("nan"))
        lse.fill_(float("nan"))
        sel.fill_(-7)

    _replay_check(torch, step, (sel, O, lse), fill)


def test_sparse_prefill_chain_replays_bit_exactly(torch_api):
    """Block means, tile selection and sparse attention captured as one graph."""
    torch, api = torch_api
    w = PrefillWorkload(name="graph_sparse", batch=1, n_q_heads=8, n_kv_heads=2, head_dim=128,
                        seq_len=1200, window_left=-1, window_right=0, causal=True, seed=46)
    x = make_prefill_inputs(w)
    Q, K, V = _dev(torch, x["Q"]), _dev(torch, x["K"]), _dev(torch, x["V"])
    N, nb, nt, k = 1200, 18, 10, 4
    shape = api.make_shape(1, 8, 2, 128, N)
    mean = torch.empty((1, 2, nb, 128), dtype=torch.bfloat16, device="cuda")
    scores = torch.empty((1, 2, nt, nb), device="cuda")
    sel = torch.empty((1, 2, nt, k), dtype=torch.int32, device="cuda")
    O = torch.empty((1, 8, N, 128), device="cuda")
    lse = torch.empty((1, 8, N), device="cuda")

    def step():
        api.bsattn_build_summaries(shape, K, 0, 0, nb, nb, mean)
        api.bsattn_select_prefill(shape, Q, mean, nb, k, 150, 32, sel, scores)
        api.bsattn_sparse_prefill(shape, Q, K, V, sel, k, 150, 32, O, lse)

    def fill():
        O.fill_(float("nan"))
        lse.fill_(float("nan"))
        sel.fill_(-7)

    _replay_check(torch, step, (sel, O, lse), fill)
