"""The incremental decode loop on the GPU, through the C ABI: per step, the new
token's K/V row is appended (bsattn_append_kv, which builds the summary of a block
the token completes), then one decode step runs on the grown cache.

Checks: every step against the fp64 oracle at that step's length (rank 0 and an
fp32 rank-2 loop; the bar of the decode parity tests), and, for the compressed
summary (bf16 means, FP4 rows, query subspace), the loop's summaries and outputs
equal, bit for bit, a from-scratch build and step at the same length.  Cache rows
past the current length hold NaN, so a read past n_ctx would show in the outputs.
"""

import numpy as np
import pytest

import oracle
from synthetic import DecodeWorkload, make_decode_inputs, normal_f32

from gpu_util import (OUT_TOL, as_f64, bf16_ulp, compare_selection, default_scale, gpu_decode_step,
                      max_abs, oracle_decode_with_sel, to_dev)

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
                          block_size=64, rank=rank, top_k=k, window=W, n_sink=ns, dtype=dtype, seed=seed)


def _loop(api, w, n0, T, mean_dtype="f32", factor_fp4=False, basis=None, one_call=True, seed=70):
    """Run T appends + steps from a cache of n0 tokens; returns the inputs, the step
    queries and per step (sel, scores, O, lse), plus the final summaries."""
    import torch
    B, Hq, Hkv, d = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
    cap = n0 + T
    nbcap = cap // 64
    x = make_decode_inputs(w.scaled(n_ctx=cap))
    bf = w.dtype == "bf16"
    Qs = normal_f32(np.random.default_rng(seed), (T, B, Hq, d), out_bf16=bf)
    K_all, V_all = to_dev(x["K"]), to_dev(x["V"])
    K = torch.full_like(K_all, float("nan"))
    V = torch.full_like(V_all, float("nan"))
    K[:, :, :n0] = K_all[:, :, :n0]
    V[:, :, :n0] = V_all[:, :, :n0]
    mean = torch.full((B, Hkv, nbcap, d), float("nan"), device="cuda",
                      dtype=torch.bfloat16 if mean_dtype == "bf16" else torch.float32)
    e = d if basis is None else basis.shape[1]
    factor = fscale = bdev = None
    if basis is not None:
        bdev = torch.from_numpy(np.ascontiguousarray(basis, dtype=np.float32)).cuda()
    if w.rank > 0 and factor_fp4:
        factor = torch.full((B, Hkv, nbcap, w.rank, e // 2), 255, dtype=torch.uint8, device="cuda")
        fscale = torch.full((B, Hkv, nbcap, w.rank), float("nan"), device="cuda")
    elif w.rank > 0:
        factor = torch.full((B, Hkv, nbcap, w.rank, e), float("nan"), device="cuda")
    shape0 = api.make_shape(B, Hq, Hkv, d, n0, kv_capacity=cap, dtype=w.dtype)
    api.bsattn_build_summaries(shape0, K, w.rank, 0, n0 // 64, nbcap, mean, factor, factor_scale=fscale,
                               basis=bdev)
    steps = []
    for t in range(T):
        n = n0 + t + 1
        shape = api.make_shape(B, Hq, Hkv, d, n, kv_capacity=cap, dtype=w.dtype)
        api.bsattn_append_kv(shape, K_all[:, :, n - 1].contiguous(), V_all[:, :, n - 1].contiguous(), K, V,
                             w.rank, nbcap, mean, factor, factor_scale=fscale, basis=bdev)
        Q = to_dev(Qs[t])
        sel = torch.full((B, Hkv, w.top_k), -7, dtype=torch.int32, device="cuda")
        scores = torch.full((B, Hkv, nbcap), float("nan"), device="cuda")
        O = torch.full((B, Hq, d), float("nan"), device="cuda")
        lse = torch.full((B, Hq), float("nan"), device="cuda")
        ws = torch.full((api.bsattn_decode_workspace_bytes(shape, w.top_k, w.window, w.n_sink, 0),), 255,
                        dtype=torch.uint8, device="cuda")
        if one_call:
            api.bsattn_decode_step(shape, Q, K, V, mean, factor, w.rank, nbcap, w.top_k, w.window, w.n_sink,
                                   (), sel, scores, O, lse, ws, factor_scale=fscale, basis=bdev)
        else:
            api.bsattn_select_topk(shape, Q, mean, factor, w.rank, nbcap, w.top_k, w.window, w.n_sink, (),
                                   sel, scores, factor_scale=fscale, basis=bdev)
            api.bsattn_decode(shape, Q, K, V, sel, w.top_k, w.window, w.n_sink, (), O, lse, ws)
        torch.cuda.synchronize()
        steps.append(dict(n=n, sel=sel.cpu().numpy(), scores=scores.cpu().numpy()[:, :, :n // 64],
                          O=O.cpu().numpy(), lse=lse.cpu().numpy()))
    summ = dict(mean=mean.float().cpu().numpy(), factor=None if factor is None else factor.cpu().numpy(),
                factor_scale=None if fscale is None else fscale.cpu().numpy())
    return x, Qs, steps, summ


def _check_against_oracle(w, x, Qs, steps, mean_dtype):
    K, V = as_f64(x["K"]), as_f64(x["V"])
    S, G, d = 64, w.n_q_heads // w.n_kv_heads, w.head_dim
    scale = default_scale(d)
    mb = mean_dtype == "bf16"
    for t, st in enumerate(steps):
        n = st["n"]
        Q = as_f64(Qs[t])
        forced = oracle.forced_token_mask(n, w.n_sink, w.window, ())
        cand = oracle.candidate_blocks(n, S, forced)
        for b in range(w.batch):
            for g in range(w.n_kv_heads):
                mean, factor = oracle.block_summaries(K[b, g, :n], S, w.rank, mean_bf16=mb)
                qs = scale * Q[b, g * G:(g + 1) * G]
                s_ref = oracle.group_scores(oracle.head_scores(qs, mean, factor if w.rank else None))
                if n // S:
                    assert max_abs(st["scores"][b, g], s_ref) < (2e-4 if w.rank else 3e-5), f"scores, n={n}"
                ok, _ = compare_selection(st["sel"][b, g], s_ref, cand, w.top_k)
                assert ok, f"selection at n={n} (b={b}, g={g})"
                o_ref, lse_ref = oracle_decode_with_sel(Q[b, g * G:(g + 1) * G], K[b, g], V[b, g], n, S,
                                                        w.window, w.n_sink, (), st["sel"][b, g], scale)
                assert max_abs(st["O"][b, g * G:(g + 1) * G], o_ref) < OUT_TOL, f"O at n={n}"
                assert max_abs(st["lse"][b, g * G:(g + 1) * G], lse_ref) < OUT_TOL, f"lse at n={n}"


def test_loop_first_order_bf16_means_every_step_against_the_oracle(api):
    """90 steps from 306 tokens: blocks 4 and 5 complete during the loop (tokens 320
    and 384); the partial tail block is reached only through the window."""
    w = _w("loop_first_order", 2, 8, 2, 128, 306, 0, 6, 100, 16, "bf16", 71)
    print("[decode loop] first order, bf16 means, 90 steps", flush=True)
    x, Qs, steps, summ = _loop(api, w, 306, 90, mean_dtype="bf16")
    _check_against_oracle(w, x, Qs, steps, "bf16")
    # the summaries the loop built equal the oracle's (one bfloat16 step)
    K = as_f64(x["K"])
    for b in range(w.batch):
        for g in range(w.n_kv_heads):
            mean, _ = oracle.block_summaries(K[b, g, :396], 64, 0, mean_bf16=True)
            err = np.abs(summ["mean"][b, g, :6].astype(np.float64) - mean)
            assert np.all(err <= bf16_ulp(mean) + 1e-30)


def test_loop_fp32_rank2_two_calls_every_step_against_the_oracle(api):
    w = _w("loop_fp32_r2", 1, 4, 2, 64, 120, 2, 3, 40, 8, "f32", 72)
    print("[decode loop] fp32 rank 2, two calls, 80 steps", flush=True)
    x, Qs, steps, _ = _loop(api, w, 120, 80, one_call=False)
    _check_against_oracle(w, x, Qs, steps, "f32")


def test_loop_compressed_summary_equals_a_from_scratch_build(api):
    """bf16 means, FP4 rows in a 64-dim query subspace: after 20 appends (token 448
    completes block 6) the loop's summaries, and its steps, equal a fresh build and
    step at the same length bit for bit."""
    w = _w("loop_compressed", 1, 16, 2, 128, 446, 4, 5, 130, 64, "bf16", 73)
    rng = np.random.default_rng(74)
    basis = np.stack([np.linalg.qr(rng.standard_normal((128, 64)))[0].T for _ in range(2)]).astype(np.float32)
    print("[decode loop] compressed summary, 20 steps", flush=True)
    x, Qs, steps, summ = _loop(api, w, 446, 20, mean_dtype="bf16", factor_fp4=True, basis=basis)
    for t in (0, 1, 2, 19):  # before, at and after the completion of block 6
        n = steps[t]["n"]
        ws = w.scaled(n_ctx=n)
        xs = dict(Q=Qs[t], K=x["K"], V=x["V"])
        ref = gpu_decode_step(api, xs, ws, kv_capacity=x["K"].shape[2], nblk_capacity=x["K"].shape[2] // 64,
                              one_call=True, mean_dtype="bf16", factor_fp4=True, basis=basis)
        assert np.array_equal(steps[t]["sel"], ref["sel"]), f"sel at n={n}"
        assert np.array_equal(steps[t]["O"], ref["O"]) and np.array_equal(steps[t]["lse"], ref["lse"]), n
        if t == 19:
            nb = n // 64
            assert np.array_equal(summ["mean"][:, :, :nb], ref["mean"][:, :, :nb])
            assert np.array_equal(summ["factor"][:, :, :nb], ref["factor"][:, :, :nb])
            assert np.array_equal(summ["factor_scale"][:, :, :nb], ref["factor_scale"][:, :, :nb])
