"""Paged K/V caches on the GPU, through the C ABI (the attention glossary's KV-cache
section: PagedAttention keeps the cache in fixed-size pages).  K and V are
scattered into page pools under a random page assignment (a block table per batch
entry); rows past n_ctx and pages no token maps to hold NaN, so a read of a wrong
row shows.  Checks: paged decode steps and summaries against the fp64 oracle, every
stage, and equal, bit for bit, to the contiguous run (only addresses change); the
paged append loop's cache rows and summaries, and a decode step after it, against
the oracle.
"""

import numpy as np
import pytest

from synthetic import DecodeWorkload, make_decode_inputs

from gpu_util import (as_f64, check_decode_case, check_fp4_case, check_pair, gpu_decode_step, paged_pools,
                      to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    import torch
    assert torch.cuda.is_available(), "GPU tests need the GPU"
    import sliding_window_attention_block_amd as m
    m.library()
    return m


def _w(name, B, Hq, Hkv, d, n, rank, k, W, ns, seed):
    return DecodeWorkload(name=name, batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, n_ctx=n,
                          block_size=64, rank=rank, top_k=k, window=W, n_sink=ns, dtype="bf16", seed=seed)


def _poison_tail(x, n):
    """Rows at and past n hold NaN (bf16 0x7FC0)."""
    K, V = x["K"].copy(), x["V"].copy()
    K[:, :, n:] = 0x7FC0
    V[:, :, n:] = 0x7FC0
    return dict(x, K=K, V=V)


CASES = [
    # name, workload, globals, page tokens, one call, summaries
    ("fused_p16_globals_tail", _w("pg_a", 2, 8, 2, 128, 64 * 9 + 37, 0, 4, 100, 16, 80), (5, 300), 16, True,
     dict(mean_dtype="bf16")),
    ("unfused_601_blocks_p32", _w("pg_b", 1, 16, 2, 64, 64 * 601 + 5, 2, 8, 64, 64, 81), (), 32, True,
     dict(mean_dtype="f32")),
    ("compressed_p64", _w("pg_c", 1, 16, 2, 128, 64 * 20 + 10, 4, 5, 130, 64, 82), (), 64, True,
     dict(mean_dtype="bf16", factor_fp4=True, sub_dim=64)),
    ("two_calls_p64", _w("pg_d", 2, 8, 2, 128, 64 * 9 + 37, 0, 4, 100, 16, 83), (7,), 64, False,
     dict(mean_dtype="bf16")),
    ("two_calls_p16_rank2", _w("pg_e", 1, 4, 1, 64, 64 * 7 + 63, 2, 3, 40, 8, 84), (), 16, False,
     dict(mean_dtype="f32")),
]


@pytest.mark.parametrize("name,w,globals_,P,one_call,summ", CASES, ids=[c[0] for c in CASES])
def test_paged_step_equals_contiguous(api, name, w, globals_, P, one_call, summ):
    cap = (w.n_ctx + P - 1) // P * P + P  # a multiple of the page size, one spare page
    x = _poison_tail(make_decode_inputs(w, kv_capacity=cap), w.n_ctx)
    summ = dict(summ)
    basis = None
    if summ.pop("sub_dim", 0):
        rng = np.random.default_rng(85)
        basis = np.stack([np.linalg.qr(rng.standard_normal((w.head_dim, 64)))[0].T
                          for _ in range(w.n_kv_heads)]).astype(np.float32)
    print(f"[paged] {name}: contiguous", flush=True)
    ref = gpu_decode_step(api, x, w, global_pos=globals_, one_call=one_call, basis=basis, **summ)
    print(f"[paged] {name}: {P}-token pages", flush=True)
    got = gpu_decode_step(api, x, w, global_pos=globals_, one_call=one_call, basis=basis, page_tokens=P,
                          page_seed=86, **summ)
    nb = w.n_ctx // 64
    for key in ("mean", "factor", "factor_scale"):
        if ref[key] is not None:
            assert np.array_equal(got[key][:, :, :nb], ref[key][:, :, :nb]), key
    assert np.array_equal(got["scores"][:, :, :nb], ref["scores"][:, :, :nb])
    assert np.array_equal(got["sel"], ref["sel"])
    assert np.all(np.isfinite(got["O"])) and np.all(np.isfinite(got["lse"]))
    assert np.array_equal(got["O"], ref["O"]) and np.array_equal(got["lse"], ref["lse"])


@pytest.mark.parametrize("P", [16, 64])
def test_paged_append_writes_the_page_rows(api, P):
    """20 appends into page pools (from 430 tokens: token 448 completes block 6) leave
    the pools holding the contiguous cache's rows and build the same summaries."""
    import torch
    w = _w("pg_append", 2, 8, 2, 128, 450, 2, 4, 64, 16, 87)
    n0, T = 430, 20
    cap = 512
    x = make_decode_inputs(w, kv_capacity=cap)
    K_all, V_all = to_dev(x["K"]), to_dev(x["V"])
    Kc = K_all.clone()
    Vc = V_all.clone()
    Kc[:, :, n0:] = float("nan")
    Vc[:, :, n0:] = float("nan")
    Kp, Vp, table, n_pages = paged_pools(Kc, Vc, P, 88)
    pg = api.paged_kv(table, P, n_pages)
    B, Hkv, d, nbcap = w.batch, w.n_kv_heads, w.head_dim, cap // 64
    sums = []
    for paged in (False, True):
        mean = torch.full((B, Hkv, nbcap, d), float("nan"), device="cuda")
        factor = torch.full((B, Hkv, nbcap, w.rank, d), float("nan"), device="cuda")
        shape0 = api.make_shape(B, w.n_q_heads, Hkv, d, n0, kv_capacity=cap, dtype="bf16")
        api.bsattn_build_summaries(shape0, Kp if paged else Kc, w.rank, 0, n0 // 64, nbcap, mean, factor,
                                   paged=pg if paged else None)
        for t in range(T):
            n = n0 + t + 1
            shape = api.make_shape(B, w.n_q_heads, Hkv, d, n, kv_capacity=cap, dtype="bf16")
            api.bsattn_append_kv(shape, K_all[:, :, n - 1].contiguous(), V_all[:, :, n - 1].contiguous(),
                                 Kp if paged else Kc, Vp if paged else Vc, w.rank, nbcap, mean, factor,
                                 paged=pg if paged else None)
        torch.cuda.synchronize()
        sums.append((mean.cpu().numpy(), factor.cpu().numpy()))
    # gather the pools back in token order and compare with the contiguous cache
    mp = cap // P
    idx = table.long().reshape(-1)
    for pool, cont in ((Kp, Kc), (Vp, Vc)):
        back = pool[idx].reshape(B, mp, Hkv, P, d).permute(0, 2, 1, 3, 4).reshape(B, Hkv, cap, d)
        n = n0 + T
        assert torch.equal(back[:, :, :n], cont[:, :, :n])
        assert torch.equal(back[:, :, :n], K_all[:, :, :n] if pool is Kp else V_all[:, :, :n])
    nb = (n0 + T) // 64
    assert np.array_equal(sums[0][0][:, :, :nb], sums[1][0][:, :, :nb])
    assert np.array_equal(sums[0][1][:, :, :nb], sums[1][1][:, :, :nb])


ORACLE_CASES = [
    # (workload, globals, page tokens, one call, mean dtype); kv_capacity = n + extra, a
    # multiple of the page size
    ("p16_fused_globals", _w("pgo_a", 2, 8, 2, 128, 64 * 9 + 37, 0, 4, 100, 16, 90), (5, 300), 16, True, "bf16"),
    ("p32_two_calls_rank2_f32", _w("pgo_b", 1, 4, 1, 64, 64 * 7 + 63, 2, 3, 40, 8, 91), (), 32, False, "f32"),
    ("p64_unfused_601_blocks", _w("pgo_c", 1, 16, 2, 64, 64 * 601 + 5, 0, 8, 64, 64, 92), (), 64, True, "bf16"),
]


@pytest.mark.parametrize("name,w,globals_,P,one_call,mean_dtype", ORACLE_CASES, ids=[c[0] for c in ORACLE_CASES])
def test_paged_step_against_the_oracle(api, name, w, globals_, P, one_call, mean_dtype):
    extra = (w.n_ctx + P - 1) // P * P + P - w.n_ctx
    check_decode_case(api, w, globals_, extra, one_call=one_call, mean_dtype=mean_dtype, page_tokens=P)


def test_paged_compressed_step_against_the_oracle(api):
    """bf16 means and FP4 rows in a 64-dim query subspace, 64-token pages."""
    w = _w("pgo_d", 1, 16, 2, 128, 64 * 20, 4, 5, 130, 64, 93)
    rng = np.random.default_rng(94)
    basis = np.stack([np.linalg.qr(rng.standard_normal((128, 64)))[0].T for _ in range(2)]).astype(np.float32)
    x = make_decode_inputs(w, kv_capacity=64 * 21)
    check_fp4_case(api, w, (), basis=basis, x=x, page_tokens=64)


@pytest.mark.parametrize("P", [16, 64])
def test_paged_append_loop_against_the_oracle(api, P):
    """Appends into page pools from 430 tokens to 450 (token 448 completes block 6),
    then one decode step on the pools: the pools' rows are the appended tokens, the
    summaries (fp32 rank 2) and the step are checked against the oracle at n = 450."""
    import torch
    w = _w("pgo_append", 2, 8, 2, 128, 450, 2, 4, 64, 16, 95)
    n0, n1, cap = 430, 450, 512
    x = make_decode_inputs(w, kv_capacity=cap)
    K_all, V_all = to_dev(x["K"]), to_dev(x["V"])
    Kc, Vc = K_all.clone(), V_all.clone()
    Kc[:, :, n0:] = float("nan")
    Vc[:, :, n0:] = float("nan")
    Kp, Vp, table, n_pages = paged_pools(Kc, Vc, P, 96)
    pg = api.paged_kv(table, P, n_pages)
    B, Hq, Hkv, d, nbcap = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, cap // 64
    mean = torch.full((B, Hkv, nbcap, d), float("nan"), device="cuda")
    factor = torch.full((B, Hkv, nbcap, w.rank, d), float("nan"), device="cuda")
    api.bsattn_build_summaries(api.make_shape(B, Hq, Hkv, d, n0, kv_capacity=cap), Kp, w.rank, 0, n0 // 64, nbcap,
                               mean, factor, paged=pg)
    for n in range(n0 + 1, n1 + 1):
        api.bsattn_append_kv(api.make_shape(B, Hq, Hkv, d, n, kv_capacity=cap), K_all[:, :, n - 1].contiguous(),
                             V_all[:, :, n - 1].contiguous(), Kp, Vp, w.rank, nbcap, mean, factor, paged=pg)
    shape = api.make_shape(B, Hq, Hkv, d, n1, kv_capacity=cap)
    Q = to_dev(x["Q"])
    sel = torch.full((B, Hkv, w.top_k), -7, dtype=torch.int32, device="cuda")
    scores = torch.full((B, Hkv, nbcap), float("nan"), device="cuda")
    O = torch.full((B, Hq, d), float("nan"), device="cuda")
    lse = torch.full((B, Hq), float("nan"), device="cuda")
    ws = torch.full((api.bsattn_decode_workspace_bytes(shape, w.top_k, w.window, w.n_sink, 0),), 255,
                    dtype=torch.uint8, device="cuda")
    api.bsattn_decode_step(shape, Q, Kp, Vp, mean, factor, w.rank, nbcap, w.top_k, w.window, w.n_sink, (), sel,
                           scores, O, lse, ws, paged=pg)
    torch.cuda.synchronize()
    # the pools, gathered back in token order, hold the appended tokens
    mp = cap // P
    idx = table.long().reshape(-1)
    for pool, ref in ((Kp, K_all), (Vp, V_all)):
        back = pool[idx].reshape(B, mp, Hkv, P, d).permute(0, 2, 1, 3, 4).reshape(B, Hkv, cap, d)
        assert torch.equal(back[:, :, :n1], ref[:, :, :n1])
    got = dict(mean=mean.cpu().numpy(), factor=factor.cpu().numpy(), scores=scores.cpu().numpy(),
               sel=sel.cpu().numpy(), O=O.cpu().numpy(), lse=lse.cpu().numpy())
    Qf, Kf, Vf = as_f64(x["Q"]), as_f64(x["K"]), as_f64(x["V"])
    ties = sum(check_pair(got, b, g, Qf, Kf, Vf, w, (), mean_dtype="f32") for b in range(B) for g in range(Hkv))
    print(f"[paged append] P={P}: near ties {ties}", flush=True)


def test_append_through_an_unallocated_page_writes_nothing(api):
    """A block-table entry outside [0, n_pages) (here -1 and n_pages) for the new
    token's page: the append writes no pool row (reads clamp such an entry; a write
    through it would land in another sequence's page)."""
    import torch
    w = _w("pg_unalloc", 2, 4, 2, 64, 40, 0, 2, 16, 0, 97)
    cap, P = 64, 16
    x = make_decode_inputs(w, kv_capacity=cap)
    K, V = to_dev(x["K"]), to_dev(x["V"])
    Kp, Vp, table, n_pages = paged_pools(K, V, P, 98)
    table[0, 40 // P] = -1
    table[1, 40 // P] = n_pages
    Kp0, Vp0 = Kp.clone(), Vp.clone()
    shape = api.make_shape(2, 4, 2, 64, 41, kv_capacity=cap)
    Knew = torch.zeros((2, 2, 64), dtype=torch.bfloat16, device="cuda")
    api.bsattn_append_kv(shape, Knew, Knew, Kp, Vp, 0, 1, torch.empty((2, 2, 1, 64), device="cuda"), None,
                         paged=api.paged_kv(table, P, n_pages))
    torch.cuda.synchronize()
    assert torch.equal(Kp.view(torch.int16), Kp0.view(torch.int16))
    assert torch.equal(Vp.view(torch.int16), Vp0.view(torch.int16))
