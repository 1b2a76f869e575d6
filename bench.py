#!/usr/bin/env python3
"""Throughput of the block-sparse attention hot path on one MI355X.

Step (the timed unit): one decode step of the first-order 32K workload (batch
16, 32 query / 8 K/V heads, d 128, 64-token blocks, top-16 + sink block + 512-
token window), one bsattn_decode_step call: the sparse decode kernel, whose
workgroups score their pair's blocks and whose waves take the top-k
themselves, then the log-sum-exp merge.
`value` is tokens/s = batch / step time.  Summaries are built once
before timing (as the method builds them when blocks fill), with the block
means stored in bfloat16 as the COBS explainer stores them (the same step with
fp32 means is reported beside it); their build time is reported separately,
as are the COBS 128K decode step and the two prefills.

Every timed loop cycles through R device-resident replicas of its inputs so the
reuse distance exceeds the 256 MB Infinity Cache: each step reads HBM, not
cache.  Decode steps are timed as one captured HIP graph of K steps (the step
is a few short kernels; launching them one at a time from Python would time the
host); warmup is W eager steps plus one untimed replay.  Durations come from
HIP events on the stream the library launches on (torch's current stream).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME] [--no-cpu-baseline]
                      [--no-context] [--calibrate-copy]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # B/s, MI355X HBM3E
CALIB_BYTES = 512 << 20    # the plain device copy --calibrate-copy runs (bytes read = bytes written)

# HBM bytes per decode step (the launches of bsattn_decode_step), from
# rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE runs of `bench.py --only <workload>
# --calibrate-copy`, each scaled by CALIB_BYTES / (the same counter for the
# calibration copy: FETCH x 1.9999, WRITE x 1.0), summed over the step's
# launches.  Valid only for the sources they were taken on (their SHA-256);
# otherwise traffic is null.
STEP_TRAFFIC = {"sources_sha256": "3dcfc467e2774249af4dde74abdf60aad24f754f555b1cce8b7f87124472b791",
                "bytes_per_step": {"first_order_decode_32k": 124015919,
                                   "cobs_decode_128k": 91442392}}
STEP_SOURCES = ("sliding_window_attention_block_amd/csrc/decode.hip",
                "sliding_window_attention_block_amd/csrc/select.hip",
                "sliding_window_attention_block_amd/csrc/bsattn.cpp",
                "sliding_window_attention_block_amd/csrc/device.hpp",
                "sliding_window_attention_block_amd/csrc/launch.hpp")


def sources_sha256(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def step_traffic(name=None):
    if STEP_TRAFFIC["sources_sha256"] == sources_sha256(STEP_SOURCES):
        return STEP_TRAFFIC["bytes_per_step"].get(name or HEADLINE)
    return None
# HBM bytes per call of the prefill kernels (rocprofv3 --pmc FETCH_SIZE and
# WRITE_SIZE, calibrated as above, summed over the call's launches), keyed by
# workload; valid only for the sources they were taken on, otherwise null.
PREFILL_TRAFFIC = {"sources_sha256": "5673afc19e58880636df07ec08e5d27dac4c02920cd92005ae02d3cda8437953",
                   "bytes_per_call": {"swa_prefill_8k": 280444601,
                                      "local_global_prefill_16k": 562533642,
                                      "sparse_prefill_8k": 285985836}}
PREFILL_SOURCES = ("sliding_window_attention_block_amd/csrc/prefill.hip",
                   "sliding_window_attention_block_amd/csrc/select.hip",
                   "sliding_window_attention_block_amd/csrc/summaries.hip",
                   "sliding_window_attention_block_amd/csrc/bsattn.cpp",
                   "sliding_window_attention_block_amd/csrc/device.hpp",
                   "sliding_window_attention_block_amd/csrc/launch.hpp")


def prefill_traffic(name):
    if PREFILL_TRAFFIC["sources_sha256"] == sources_sha256(PREFILL_SOURCES):
        return PREFILL_TRAFFIC["bytes_per_call"].get(name)
    return None
BF16_PEAK = 2.5e15         # flop/s, MI355X dense bf16 MFMA
MALL_BYTES = 256 << 20
METRIC = "sparse-decode tokens/s and gathered-KV GB/s (% HBM peak); prefill % MFMA peak"
HEADLINE = "first_order_decode_32k"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dist(samples):
    """Median and 10th / 90th percentiles of a list of durations (ms)."""
    a = np.asarray(samples, dtype=np.float64)
    return dict(median=float(np.median(a)), p10=float(np.percentile(a, 10)), p90=float(np.percentile(a, 90)),
                n=int(a.size))


def gpu_state():
    """Power cap and graphics clocks as the driver reports them (amd-smi / rocm-smi),
    read right after a timed region so the clock is the one the work ran at."""
    import re
    import subprocess
    out = {}
    if "rocprof" in os.environ.get("LD_PRELOAD", ""):
        # under rocprofv3 the smi tools (python scripts) would start with the
        # profiler's library preloaded; the profile has its own clock counters
        return {"skipped": "run under rocprofv3"}

    def run(cmd):
        try:
            return subprocess.run(cmd, capture_output=True, text=True, timeout=20).stdout
        except Exception:  # noqa: BLE001
            return ""
    try:
        m = json.loads(run(["amd-smi", "metric", "-p", "-c", "--json"]) or "null")
        g = m[0] if isinstance(m, list) else (m.get("gpu_data", [m])[0] if isinstance(m, dict) else None)
        if g:
            clk = g.get("clock", {})
            gfx = [v for k, v in clk.items() if k.lower().startswith("gfx")]
            cur = [float(v["clk"]["value"]) for v in gfx if isinstance(v.get("clk"), dict)]
            mx = [float(v["max_clk"]["value"]) for v in gfx if isinstance(v.get("max_clk"), dict)]
            if cur:
                out["gfx_clk_MHz_now"] = dict(min=min(cur), max=max(cur))
            if mx:
                out["gfx_clk_MHz_max"] = max(mx)
            pw = g.get("power", {})
            sp = pw.get("socket_power")
            if isinstance(sp, dict):
                out["socket_power_W_now"] = float(sp["value"])
    except Exception:  # noqa: BLE001
        pass
    txt = run(["rocm-smi", "--showmaxpower"])
    mm = re.search(r"Max Graphics Package Power \(W\):\s*([0-9.]+)", txt)
    if mm:
        out["power_cap_W"] = float(mm.group(1))
    return out


# ----------------------------------------------------------------------------- models
def attended_tokens(n, S, window, n_sink, global_pos, sel_row):
    """Size of the decode token set: forced tokens union the selected blocks' tokens."""
    inT = np.zeros(n, dtype=bool)
    inT[: min(n_sink, n)] = True
    if window > 0:
        inT[max(0, n - window):] = True
    if len(global_pos):
        inT[np.asarray(global_pos)] = True
    for b in sel_row:
        if b >= 0:
            inT[b * S:(b + 1) * S] = True
    return int(inT.sum())


def prefill_pairs(N, wl, wr, causal, global_pos, dilation=1):
    """Allowed (query, key) pairs per (b, h) of the prefill mask, by per-row closed form
    (with a dilation s: the multiples of s between the window ends and the row)."""
    i = np.arange(N, dtype=np.int64)
    lo = np.zeros(N, np.int64) if wl < 0 else np.maximum(0, i - wl)
    right = 0 if causal else wr
    hi = np.full(N, N - 1, np.int64) if right < 0 else np.minimum(N - 1, i + right)
    cnt = (i - lo) // dilation + (hi - i) // dilation + 1
    g = np.asarray(sorted(global_pos), dtype=np.int64)
    if g.size:
        inside = np.searchsorted(g, hi, side="right") - np.searchsorted(g, lo, side="left")
        cnt = cnt + (g.size - inside)
        cnt[g] = N
    return int(cnt.sum())


def replicas_for(step_bytes):
    # at most 64: a step that small (the tiny workload) is bound by latency, not by
    # where its bytes come from
    return min(64, max(2, int(np.ceil(2 * MALL_BYTES / max(step_bytes, 1))) + 1))


# ----------------------------------------------------------------------------- decode
def to_dev(torch, a):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_pages(torch, X, page_tokens, perm):
    """Contiguous cache [B, Hkv, cap, d] -> page pool [n_pages, Hkv, P, d] under the
    page assignment perm [B, cap / P] (distinct page numbers)."""
    B, Hkv, cap, d = X.shape
    P, mp = page_tokens, cap // page_tokens
    pool = torch.empty((int(perm.max()) + 1, Hkv, P, d), dtype=X.dtype, device="cuda")
    idx = torch.from_numpy(perm.reshape(-1)).cuda().long()
    pool[idx] = X.reshape(B, Hkv, mp, P, d).permute(0, 2, 1, 3, 4).reshape(B * mp, Hkv, P, d)
    return pool


def bench_append(api, torch, w, rp, shape_step, mean_dtype, fp4, basis, steps):
    """bsattn_append_kv latency: the token that completes a block for every (b, K/V
    head) pair (the copy, then that block's summary: mean, and rank-r factor when
    r > 0), and a token that completes none (the copy alone).  Per-call HIP events."""
    B, Hq, Hkv, d, n = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_ctx
    nb = n // 64
    assert n % 64 == 0
    Knew = rp["K"][:, :, n - 1].contiguous() if rp["pg"] is None else rp["K"][0, :, 0].expand(B, Hkv, d).contiguous()
    Vnew = Knew.clone()
    out = {}
    for label, m in (("completes_block", n), ("no_block", n - 1)):
        shape = api.make_shape(B, Hq, Hkv, d, m, dtype=w.dtype)
        def call():
            api.bsattn_append_kv(shape, Knew, Vnew, rp["K"], rp["V"], w.rank, nb, rp["mean"], rp["factor"],
                                 factor_scale=rp["fscale"], basis=basis, paged=rp["pg"])
        for _ in range(3):
            call()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(max(10, min(steps, 50)))]
        torch.cuda.synchronize()
        for e0, e1 in evs:
            e0.record()
            call()
            e1.record()
        torch.cuda.synchronize()
        out[label] = dist([a.elapsed_time(b) for a, b in evs])
    out["pairs"] = B * Hkv
    return out


def bench_gather_probe(api, torch, w, reps, shape, steps, R):
    """The loads-only gather ceiling for this step's own token set (bsattn_probe_gather):
    the same K/V blocks (sink, window and selected blocks of every pair) read from the
    same rotating replicas with the decode's placement of two workgroups per pair,
    nothing computed, as one captured graph of `steps` calls per setting."""
    B, Hkv, n, S = w.batch, w.n_kv_heads, w.n_ctx, w.block_size
    forced = sorted(set(range(0, (min(w.n_sink, n) + S - 1) // S)) | set(range(max(0, n - w.window) // S, n // S)))
    sel_h = reps[0]["sel"].cpu().numpy().reshape(B * Hkv, -1)
    rows = [forced + sorted(int(j) for j in r if j >= 0 and j not in forced) for r in sel_h]
    nbl = min(len(r) for r in rows)
    blocks = torch.from_numpy(np.asarray([r[:nbl] for r in rows], dtype=np.int32)).cuda()
    nbytes = B * Hkv * nbl * S * w.head_dim * 2 * 2
    out = {"blocks_per_pair": nbl, "bytes": nbytes}
    for wg, depth in ((2, 2), (2, 4), (1, 4)):
        cks = torch.empty((B * Hkv * wg * 256,), dtype=torch.int32, device="cuda")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                rp = reps[i % R]
                api.bsattn_probe_gather(shape, rp["K"], rp["V"], blocks, wg, depth, cks)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        out[f"wg{wg}_depth{depth}"] = dict(ms=ms, GBps=nbytes / (ms * 1e-3) / 1e9,
                                           frac_hbm=nbytes / (ms * 1e-3) / HBM_PEAK)
        del g
    return out


def gather_chunk_sweep(api, torch, w, steps):
    """The gather probe's rate against the contiguous chunk size and against the
    waves per pair: 24 blocks per (b, K/V head) pair of the workload's shape
    listed as runs of 1, 2, 4 or 8 adjacent blocks at random places (16 to 128
    KB contiguous K and V reads at d = 128), then single blocks read by 1 to 16
    workgroups per pair; over 6 rotating replicas of N(0,1) bf16 caches, each
    setting one captured graph of `steps` launches timed with HIP events."""
    B, Hq, Hkv, d, n = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_ctx
    R, nbl, nb = 6, 24, n // 64
    shape = api.make_shape(B, Hq, Hkv, d, n, dtype="bf16")
    reps = [(torch.randn(B, Hkv, n, d, device="cuda").to(torch.bfloat16),
             torch.randn(B, Hkv, n, d, device="cuda").to(torch.bfloat16)) for _ in range(R)]
    rng = np.random.default_rng(0)
    nbytes = B * Hkv * nbl * 64 * d * 2 * 2
    out = {"bytes_per_launch": nbytes}
    settings = [(run, wg, depth) for run in (1, 2, 4, 8) for wg, depth in ((2, 2), (2, 4))]
    settings += [(1, wg, 2) for wg in (1, 4, 6, 12, 16)]
    for run in (1, 2, 4, 8):
        rows = []
        for _ in range(B * Hkv):
            starts = rng.choice(nb // run, size=nbl // run, replace=False) * run
            rows.append(np.concatenate([np.arange(st, st + run) for st in sorted(starts)]))
        blocks = torch.from_numpy(np.asarray(rows, dtype=np.int32)).cuda()
        for wg, depth in [(wg, dp) for r, wg, dp in settings if r == run]:
            cks = torch.empty(B * Hkv * wg * 256, dtype=torch.int32, device="cuda")
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(steps):
                    api.bsattn_probe_gather(shape, reps[i % R][0], reps[i % R][1], blocks, wg, depth, cks)
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / steps
            out[f"chunk_{16 * run}KB_wg{wg}_depth{depth}"] = dict(us=ms * 1e3, GBps=nbytes / (ms * 1e-3) / 1e9)
            del g
    return out


def bench_decode(api, torch, w, x, steps, warmup, mean_dtype="bf16", factor_fp4=True, subspace=True,
                 page_tokens=None, append_rows=False, replicas=None, gather_probe=False):
    B, Hq, Hkv, d, n, S = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_ctx, w.block_size
    nb = n // S
    shape = api.make_shape(B, Hq, Hkv, d, n, dtype=w.dtype)
    ws_bytes = api.bsattn_decode_workspace_bytes(shape, w.top_k, w.window, w.n_sink, 0)
    elem = 2 if w.dtype == "bf16" else 4
    mean_elem = 2 if mean_dtype == "bf16" else 4
    fp4 = factor_fp4 and w.rank > 0
    # the page's compressed summary: bf16 mean, FP4 rows in the query subspace
    sub = w.sub_dim if (subspace and fp4 and mean_dtype == "bf16" and w.sub_dim > 0) else 0
    e = sub or d
    factor_row_bytes = (e // 2 + 4) if fp4 else 4 * d  # FP4 codes + float32 scale, or fp32
    basis_bytes = Hkv * sub * d * 4
    summ_bytes = B * Hkv * nb * (d * mean_elem + w.rank * factor_row_bytes)
    kv_est = B * Hkv * (w.top_k * S + w.n_sink + w.window) * d * 2 * elem
    # replicas: enough that the working set exceeds the 256 MB Infinity Cache
    # (every step reads HBM), or the caller's count (1: the warm context row)
    R = replicas or replicas_for(summ_bytes + kv_est)
    log(f"[bench] {w.name}: {R} replicas, {2 * x['K'].nbytes * R / 2**30:.1f} GiB of K/V")
    K0, V0, Q0 = to_dev(torch, x["K"]), to_dev(torch, x["V"]), to_dev(torch, x["Q"])
    basis = None
    if sub:  # a random orthonormal frame per K/V head: its values do not change the timing
        from synthetic import orthonormal_rows
        basis = torch.from_numpy(orthonormal_rows(np.random.default_rng(w.seed + 1000), Hkv, sub, d)).cuda()
    reps = []
    for r in range(R):
        K = K0 if r == 0 else K0.clone()
        V = V0 if r == 0 else V0.clone()
        Q = Q0 if r == 0 else Q0.clone()
        pg = table = None
        if page_tokens:  # pages of every replica in a random order (a fragmented pool)
            mp = K.shape[2] // page_tokens
            perm = np.random.default_rng(w.seed + 2000 + r).permutation(B * mp).reshape(B, mp).astype(np.int32)
            K, V = to_pages(torch, K, page_tokens, perm), to_pages(torch, V, page_tokens, perm)
            table = torch.from_numpy(perm).cuda()
            pg = api.paged_kv(table, page_tokens, B * mp)
        mean = torch.empty((B, Hkv, nb, d), device="cuda",
                           dtype=torch.bfloat16 if mean_dtype == "bf16" else torch.float32)
        fscale = None
        if fp4:
            factor = torch.empty((B, Hkv, nb, w.rank, e // 2), dtype=torch.uint8, device="cuda")
            fscale = torch.empty((B, Hkv, nb, w.rank), device="cuda")
        else:
            factor = torch.empty((B, Hkv, nb, w.rank, d), device="cuda") if w.rank else None
        scores = torch.empty((B, Hkv, nb), device="cuda")
        sel = torch.empty((B, Hkv, w.top_k), dtype=torch.int32, device="cuda")
        ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
        O = torch.empty((B, Hq, d), device="cuda")
        lse = torch.empty((B, Hq), device="cuda")
        reps.append(dict(K=K, V=V, Q=Q, mean=mean, factor=factor, fscale=fscale, scores=scores, sel=sel,
                         ws=ws, O=O, lse=lse, pg=pg, table=table))
    del K0, V0, Q0
    # A1: summaries (built once per block; timed on every replica)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    build_ms = []
    for rp in reps:
        ev[0].record()
        api.bsattn_build_summaries(shape, rp["K"], w.rank, 0, nb, nb, rp["mean"], rp["factor"],
                                   factor_scale=rp["fscale"], basis=basis, paged=rp["pg"])
        ev[1].record()
        torch.cuda.synchronize()
        build_ms.append(ev[0].elapsed_time(ev[1]))

    def select(rp):
        api.bsattn_select_topk(shape, rp["Q"], rp["mean"], rp["factor"], w.rank, nb, w.top_k,
                               w.window, w.n_sink, None, rp["sel"], rp["scores"], factor_scale=rp["fscale"],
                               basis=basis)

    def decode(rp):
        api.bsattn_decode(shape, rp["Q"], rp["K"], rp["V"], rp["sel"], w.top_k, w.window, w.n_sink,
                          None, rp["O"], rp["lse"], rp["ws"], paged=rp["pg"])

    def step(rp):
        api.bsattn_decode_step(shape, rp["Q"], rp["K"], rp["V"], rp["mean"], rp["factor"], w.rank, nb,
                               w.top_k, w.window, w.n_sink, None, rp["sel"], rp["scores"], rp["O"],
                               rp["lse"], rp["ws"], factor_scale=rp["fscale"], basis=basis, paged=rp["pg"])

    for i in range(warmup):
        rp = reps[i % R]
        step(rp)
        select(rp)
        decode(rp)
    torch.cuda.synchronize()
    # token-set size from the actual selection (identical on every replica)
    sel_h = reps[0]["sel"].cpu().numpy()
    tokens = sum(attended_tokens(n, S, w.window, w.n_sink, (), sel_h[b, g])
                 for b in range(B) for g in range(Hkv))
    kv_bytes = tokens * d * 2 * elem
    io_bytes = B * Hq * d * elem + B * Hq * (d + 1) * 4 + B * Hkv * w.top_k * 4  # Q in, O + lse out, sel
    sel_bytes = summ_bytes + basis_bytes + B * Hq * d * elem + B * Hkv * w.top_k * 4

    # The timed steps run as one HIP graph of `steps` steps (replica i % R at step i):
    # a decode step is a handful of short kernels, and launching them one by one
    # from Python would time the host, not the GPU.  Separate graphs give the
    # context figures: the same step as two calls (bsattn_select_topk, then
    # bsattn_decode), and each of those calls alone.
    def capture(fns):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                for f in fns:
                    f(reps[i % R])
        return g

    def timed_replay(g):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps, (time.perf_counter() - t0) * 1e3 / steps

    g_step = capture((step,))
    g_two, g_sel, g_dec = capture((select, decode)), capture((select,)), capture((decode,))
    for g in (g_step, g_two, g_sel, g_dec):
        g.replay()  # untimed: the first replay of a graph uploads it
    torch.cuda.synchronize()
    ms_step, wall_step = timed_replay(g_step)
    # distribution: further replays of the same K-step graph (per-step mean of each)
    step_dist = dist([timed_replay(g_step)[0] for _ in range(10)])
    state = gpu_state()
    two_ms, _ = timed_replay(g_two)
    sel_ms, _ = timed_replay(g_sel)
    dec_ms, _ = timed_replay(g_dec)
    del g_step, g_two, g_sel, g_dec
    # the same steps launched one call at a time from Python (context only)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(reps[i % R])
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / steps
    probe = None
    if gather_probe:
        probe = bench_gather_probe(api, torch, w, reps, shape, steps, R)
    append = None
    if append_rows:
        append = bench_append(api, torch, w, reps[0], shape, mean_dtype, fp4, basis, steps)
    res = dict(
        workload=w.name, mean_dtype=mean_dtype, factor="fp4" if fp4 else ("f32" if w.rank else None),
        sub_dim=sub or None, page_tokens=page_tokens,
        ms_per_step=ms_step, wall_ms_per_step=wall_step, step_ms_dist=step_dist, gpu_state=state,
        tokens_per_s=B / (ms_step * 1e-3),
        eager_ms_per_step=eager_ms, two_call_ms_per_step=two_ms, replicas=R, attended_tokens=tokens,
        gathered_kv_bytes=kv_bytes, select_ms=sel_ms, decode_ms=dec_ms,
        select_bytes=sel_bytes, decode_bytes=kv_bytes + io_bytes,
        summary_build_ms=float(np.median(build_ms)),
        summary_build_bytes=B * Hkv * nb * S * d * elem + summ_bytes,
        append=append,
        gather_probe=probe,
    )
    res["gathered_kv_GBps"] = kv_bytes / (dec_ms * 1e-3) / 1e9
    res["gathered_kv_frac_hbm"] = res["gathered_kv_GBps"] * 1e9 / HBM_PEAK
    res["decode_GBps"] = (kv_bytes + io_bytes) / (dec_ms * 1e-3) / 1e9
    res["select_GBps"] = sel_bytes / (sel_ms * 1e-3) / 1e9
    # algorithmic bytes of a step: summaries, Q, the gathered K/V rows, and the
    # outputs (scores, sel, O, lse), each once
    res["step_bytes"] = summ_bytes + basis_bytes + kv_bytes + io_bytes + B * Hkv * nb * 4
    res["step_GBps"] = res["step_bytes"] / (ms_step * 1e-3) / 1e9
    # measured HBM bytes of the step (counters; the workload's default row only)
    default_row = mean_dtype == "bf16" and factor_fp4 and subspace and not page_tokens
    res["traffic_bytes"] = step_traffic(w.name) if default_row else None
    del reps
    torch.cuda.empty_cache()
    return res


def bench_exact_select(api, torch, w, x, steps, warmup):
    """The exact-mass selector (every key of the context read) on the decode workload:
    a reference for the summary-based selection, reported as context."""
    B, Hq, Hkv, d, n = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_ctx
    nb = n // 64
    shape = api.make_shape(B, Hq, Hkv, d, n, dtype=w.dtype)
    K, Q = to_dev(torch, x["K"]), to_dev(torch, x["Q"])
    scores = torch.empty((B, Hkv, nb), device="cuda")
    sel = torch.empty((B, Hkv, w.top_k), dtype=torch.int32, device="cuda")

    def run():
        api.bsattn_select_exact(shape, Q, K, nb, w.top_k, w.window, w.n_sink, None, sel, scores)

    for _ in range(warmup):
        run()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    key_bytes = B * Hkv * nb * 64 * d * 2
    del K, Q
    torch.cuda.empty_cache()
    return dict(workload=w.name, selector="exact block mass", ms_per_call=ms, key_bytes=key_bytes,
                GBps=key_bytes / (ms * 1e-3) / 1e9, frac_hbm=key_bytes / (ms * 1e-3) / HBM_PEAK)


# ----------------------------------------------------------------------------- prefill
def sparse_prefill_keys(sel, N, wl, ns, tile=128, S=64):
    """Keys each row attends in the block-sparse prefill, from a selection
    [n_tiles, k] (window, sinks before the window, selected keys before the window
    and past the sinks: disjoint by construction)."""
    i = np.arange(N)
    cnt = np.minimum(i, wl) + 1 + np.maximum(0, np.minimum(np.minimum(ns, i + 1), i - wl))
    lim = i - wl  # keys below the window
    for t in range(sel.shape[0]):
        r = slice(t * tile, min(N, (t + 1) * tile))
        for j in sel[t]:
            if j >= 0:
                lo, hi = max(S * j, ns), np.minimum(S * j + S, lim[r])
                cnt[r] += np.maximum(0, hi - lo)
    return cnt


def bench_sparse_prefill(api, torch, w, x, steps, warmup):
    """One call chain of the block-sparse prefill on resident inputs: block means
    (bsattn_build_summaries), tile selection (bsattn_select_prefill) and the sparse
    attention (bsattn_sparse_prefill)."""
    B, Hq, Hkv, N, d = w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len, w.head_dim
    wl, ns, k = w.window_left, w.n_sink, w.top_k
    shape = api.make_shape(B, Hq, Hkv, d, N, dtype="bf16")
    nb, n_tiles = N // 64, (N + 127) // 128
    io = (x["Q"].nbytes + x["K"].nbytes + x["V"].nbytes) + B * Hq * N * (d + 1) * 4
    R = replicas_for(io)
    reps = []
    for r in range(R):
        reps.append(dict(Q=to_dev(torch, x["Q"]), K=to_dev(torch, x["K"]), V=to_dev(torch, x["V"]),
                         mean=torch.empty((B, Hkv, nb, d), dtype=torch.bfloat16, device="cuda"),
                         scores=torch.empty((B, Hkv, n_tiles, nb), device="cuda"),
                         sel=torch.empty((B, Hkv, n_tiles, k), dtype=torch.int32, device="cuda"),
                         O=torch.empty((B, Hq, N, d), device="cuda"), lse=torch.empty((B, Hq, N), device="cuda")))

    def summaries(rp):
        api.bsattn_build_summaries(shape, rp["K"], 0, 0, nb, nb, rp["mean"])

    def select(rp):
        api.bsattn_select_prefill(shape, rp["Q"], rp["mean"], nb, k, wl, ns, rp["sel"], rp["scores"])

    def attend(rp):
        api.bsattn_sparse_prefill(shape, rp["Q"], rp["K"], rp["V"], rp["sel"], k, wl, ns, rp["O"], rp["lse"])

    def step(rp):
        summaries(rp)
        select(rp)
        attend(rp)

    for i in range(warmup):
        step(reps[i % R])
    torch.cuda.synchronize()
    sel_h = reps[0]["sel"].cpu().numpy()
    keys = sum(int(sparse_prefill_keys(sel_h[b, g], N, wl, ns).sum()) * (Hq // Hkv)
               for b in range(B) for g in range(Hkv))
    flops = 4.0 * d * keys  # QK and PV over the attended (query, key) pairs

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(steps):
            fn(reps[i % R])
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    step_ms = timed(step)
    attend_samples = []
    for i in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        attend(reps[i % R])
        e1.record()
        attend_samples.append((e0, e1))
    torch.cuda.synchronize()
    attend_dist = dist([a.elapsed_time(b) for a, b in attend_samples])
    attend_ms = timed(attend)
    select_ms = timed(select)
    summ_ms = timed(summaries)
    res = dict(workload=w.name, ms_per_call=step_ms, attend_ms=attend_ms, select_ms=select_ms,
               summaries_ms=summ_ms, attended_pairs=keys, gflop=flops / 1e9,
               tflops=flops / (step_ms * 1e-3) / 1e12, attend_tflops=flops / (attend_ms * 1e-3) / 1e12,
               attend_frac_mfma=flops / (attend_ms * 1e-3) / BF16_PEAK, replicas=R,
               window=wl + 1, sinks=ns, top_k=k, attend_ms_dist=attend_dist,
               roofline=dict(bound="mfma", kernel="the sparse attention launch (prefill_kernel, block-sparse)",
                             achieved=flops / (attend_ms * 1e-3) / 1e12, peak=BF16_PEAK / 1e12, unit="TFLOP/s",
                             frac=flops / (attend_ms * 1e-3) / BF16_PEAK, traffic=prefill_traffic(w.name),
                             flop_per_launch=flops, avg_launch_ms=attend_ms))
    del reps
    torch.cuda.empty_cache()
    return res


def bench_prefill(api, torch, w, x, steps, warmup):
    B, Hq, Hkv, N, d = w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len, w.head_dim
    shape = api.make_shape(B, Hq, Hkv, d, N, dtype="bf16")
    io = (x["Q"].nbytes + x["K"].nbytes + x["V"].nbytes) + B * Hq * N * (d + 1) * 4
    R = replicas_for(io)
    Q0, K0, V0 = to_dev(torch, x["Q"]), to_dev(torch, x["K"]), to_dev(torch, x["V"])
    reps = []
    for r in range(R):
        reps.append(dict(Q=Q0 if r == 0 else Q0.clone(), K=K0 if r == 0 else K0.clone(),
                         V=V0 if r == 0 else V0.clone(),
                         O=torch.empty((B, Hq, N, d), device="cuda"),
                         lse=torch.empty((B, Hq, N), device="cuda")))
    g = list(w.global_pos)
    ws_bytes = api.bsattn_prefill_workspace_bytes(shape, len(g))
    for rp in reps:
        rp["ws"] = torch.empty((ws_bytes,), dtype=torch.uint8, device="cuda") if ws_bytes else None

    def run(rp):
        if w.dilation > 1:
            api.bsattn_prefill_dilated(shape, rp["Q"], rp["K"], rp["V"], w.window_left, w.window_right,
                                       w.causal, w.dilation, rp["O"], rp["lse"])
        else:
            api.bsattn_prefill(shape, rp["Q"], rp["K"], rp["V"], w.window_left, w.window_right,
                               w.causal, g, rp["O"], rp["lse"], rp["ws"])

    for i in range(warmup):
        run(reps[i % R])
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        evs[i][0].record()
        run(reps[i % R])
        evs[i][1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    per_call = [a.elapsed_time(b) for a, b in evs]
    # the timed figure: the same calls captured as one HIP graph of `steps` calls
    # (replica i % R at call i), replayed once untimed, then timed with events on
    # the launch stream; the per-call events above (each call launched from
    # Python, its launches' gaps included) are reported beside it
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        for i in range(steps):
            run(reps[i % R])
    gr.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    graph_ms = []
    for _ in range(3):
        e0.record()
        gr.replay()
        e1.record()
        torch.cuda.synchronize()
        graph_ms.append(e0.elapsed_time(e1) / steps)
    del gr
    k_ms = float(np.median(graph_ms))
    state = gpu_state()
    pairs = prefill_pairs(N, w.window_left, w.window_right, w.causal, g, w.dilation)
    flops = 4.0 * d * pairs * B * Hq
    del reps
    torch.cuda.empty_cache()
    res = dict(workload=w.name, kernel_ms=k_ms, graph_replays_ms=graph_ms, eager_call_ms=float(np.mean(per_call)),
               eager_call_ms_dist=dist(per_call), wall_ms_per_call=(t1 - t0) * 1e3 / steps,
               pairs_per_head=pairs, gflop=flops / 1e9, tflops=flops / (k_ms * 1e-3) / 1e12,
               frac_mfma=flops / (k_ms * 1e-3) / BF16_PEAK, io_bytes=io,
               hbm_GBps=io / (k_ms * 1e-3) / 1e9, frac_hbm=io / (k_ms * 1e-3) / HBM_PEAK,
               replicas=R, gpu_state=state)
    # the bound is the larger of the two ideal times: MFMA flops at the bf16 peak, or
    # the inputs and fp32 outputs at the HBM peak
    if flops / BF16_PEAK >= io / HBM_PEAK:
        res["roofline"] = dict(bound="mfma", achieved=flops / (k_ms * 1e-3) / 1e12, peak=BF16_PEAK / 1e12,
                               unit="TFLOP/s", frac=flops / (k_ms * 1e-3) / BF16_PEAK,
                               traffic=prefill_traffic(w.name), flop_per_launch=flops, avg_launch_ms=k_ms)
    else:
        res["roofline"] = dict(bound="hbm", achieved=io / (k_ms * 1e-3) / 1e9, peak=HBM_PEAK / 1e9, unit="GB/s",
                               frac=io / (k_ms * 1e-3) / HBM_PEAK, traffic=prefill_traffic(w.name),
                               bytes_per_launch=io, avg_launch_ms=k_ms,
                               mfma_frac=flops / (k_ms * 1e-3) / BF16_PEAK)
    return res


def traffic_ratios(results):
    """The COBS explainer's traffic comparison (technical summary 4.1: COBS reads
    about 1.21x the first-order selector's bytes and dense attention 15.15x COBS's)
    computed from this byte model at the 128K shape: per decode step, the summaries
    read by the selector plus the K/V rows gathered, with the COBS workload's own
    token set (the same k, window and sinks for both selectors).  First order: bf16
    means; COBS: bf16 means + FP4 rank-4 rows in the 96-dim query subspace (scales
    included) + the basis; dense: every K/V row of the context.  The pages' numbers
    come from a trained model on RULER; these are the same ratios for our shapes."""
    c = results.get("cobs_decode_128k")
    if not c:
        return None
    from synthetic import WORKLOADS
    w = WORKLOADS["cobs_decode_128k"]
    B, Hkv, Hq, d, n, r = w.batch, w.n_kv_heads, w.n_q_heads, w.head_dim, w.n_ctx, w.rank
    nb = n // w.block_size
    s = w.sub_dim
    mean_b = B * Hkv * nb * d * 2
    fac_b = B * Hkv * nb * r * (s // 2 + 4) + Hkv * s * d * 4
    kv = c["gathered_kv_bytes"]
    q_o = B * Hq * d * 2 + B * Hq * (d + 1) * 4
    first = mean_b + kv + q_o
    cobs = mean_b + fac_b + kv + q_o
    dense = B * Hkv * n * d * 2 * 2 + q_o
    out = dict(shape="cobs_decode_128k", first_order_bytes=first, cobs_bytes=cobs, dense_bytes=dense,
               cobs_over_first_order=cobs / first, dense_over_cobs=dense / cobs,
               pages=dict(cobs_over_first_order=1.21, dense_over_cobs=15.15))
    h = results.get(HEADLINE)
    if h:
        wh = WORKLOADS[HEADLINE]
        dense_h = wh.batch * wh.n_kv_heads * wh.n_ctx * wh.head_dim * 2 * 2
        out["first_order_32k_dense_over_step"] = dense_h / h["step_bytes"]
    return out


# ----------------------------------------------------------------------------- CPU baseline
def cpu_baseline(w, x):
    """The oracle's decode step (score + top-k + attention over the token set) on the
    host cores, on the whole batch of one step; summaries are built before timing."""
    import oracle
    from synthetic import bf16_bits_to_f32
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = len(os.sched_getaffinity(0))
    Q = bf16_bits_to_f32(x["Q"]) if x["Q"].dtype == np.uint16 else x["Q"]
    pairs = [(b, g) for b in range(w.batch) for g in range(w.n_kv_heads)]
    summaries = {}
    Kf = {}
    Vf = {}
    for (b, g) in pairs:
        Kf[(b, g)] = bf16_bits_to_f32(x["K"][b, g]) if x["K"].dtype == np.uint16 else x["K"][b, g]
        Vf[(b, g)] = bf16_bits_to_f32(x["V"][b, g]) if x["V"].dtype == np.uint16 else x["V"][b, g]
        summaries[(b, g)] = oracle.block_summaries(Kf[(b, g)].astype(np.float64), w.block_size, w.rank,
                                                   mean_bf16=True)
    # whole decode steps (every (b, K/V head) pair) until about 10 s of CPU work
    steps = 0
    t0 = time.perf_counter()
    while True:
        for (b, g) in pairs:
            Kb = np.zeros((1, 1) + Kf[(b, g)].shape, np.float32)
            Kb[0, 0] = Kf[(b, g)]
            Vb = np.zeros_like(Kb)
            Vb[0, 0] = Vf[(b, g)]
            qb = Q[b:b + 1, g * (w.n_q_heads // w.n_kv_heads):(g + 1) * (w.n_q_heads // w.n_kv_heads)]
            oracle.decode_step(qb, Kb, Vb, w.n_ctx, w.block_size, w.rank, w.top_k, w.window, w.n_sink,
                               summaries={(0, 0): summaries[(b, g)]})
        steps += 1
        if time.perf_counter() - t0 > 10.0:
            break
    dt = time.perf_counter() - t0
    step_s = dt / steps
    return dict(value=w.batch / step_s, unit="tokens/s", cores=int(threads), kind="oracle",
                sample=f"{steps} full decode steps of {w.name} (all {len(pairs)} (batch, K/V head) "
                       f"pairs each), numpy float64 oracle, summaries prebuilt and untimed ({dt:.1f} s)")


# ----------------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--only", default=None,
                    help="run one workload only (first_order_decode_32k, cobs_decode_128k, "
                         "swa_prefill_8k, local_global_prefill_16k, sparse_prefill_8k); prints its result")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true",
                    help="time each workload's own row only (no fp32, paged, exact-selector or append "
                         "context rows): for profiler runs")
    ap.add_argument("--gather-chunks", action="store_true",
                    help="only the gather probe's rate against the contiguous chunk size on the headline "
                         "workload's shape (runs of 1, 2, 4, 8 adjacent blocks); prints its result")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 512 MiB device-to-device copy three times (the "
                         "reference dispatch for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the block-sparse attention path here has no "
              "multi-GPU part (each GPU would hold whole (batch, K/V head) pairs and run this "
              "same path on its share); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import sliding_window_attention_block_amd as api
    from synthetic import WORKLOADS, DecodeWorkload, make_decode_inputs, make_prefill_inputs

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    api.library()
    if args.gather_chunks:
        print(json.dumps({"workload": HEADLINE, "gather_chunk_sweep":
                          gather_chunk_sweep(api, torch, WORKLOADS[HEADLINE], args.steps)}))
        return
    if args.calibrate_copy:
        src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copies done: 3 x {CALIB_BYTES} bytes")
        del src, dst
    names = [args.only] if args.only else [HEADLINE, "cobs_decode_128k", "tiny_decode_1k", "swa_prefill_8k",
                                            "local_global_prefill_16k", "sparse_prefill_8k"]
    results = {}
    inputs = {}
    for name in names:
        w = WORKLOADS[name]
        decode = isinstance(w, DecodeWorkload)
        t = time.perf_counter()
        x = make_decode_inputs(w) if decode else make_prefill_inputs(w)
        log(f"[bench] {name}: inputs generated in {time.perf_counter() - t:.1f} s")
        if decode and w.dtype == "f32":  # the tiny fp32 workload: latency only
            results[name] = bench_decode(api, torch, w, x, args.steps, args.warmup, mean_dtype="f32")
        elif decode and args.no_context:
            results[name] = bench_decode(api, torch, w, x, args.steps, args.warmup, gather_probe=name == HEADLINE)
        elif decode:
            results[name] = bench_decode(api, torch, w, x, args.steps, args.warmup, append_rows=True,
                                         gather_probe=name == HEADLINE)
            if name == HEADLINE:  # context: fp32 block means; paged caches of 4 to 16 KB pages
                results[name + "/fp32_means"] = bench_decode(api, torch, w, x, args.steps, args.warmup,
                                                             mean_dtype="f32")
                for pt in (16, 32, 64):  # 4, 8 and 16 KB pages of one K/V head
                    results[name + f"/paged{pt}"] = bench_decode(api, torch, w, x, args.steps, args.warmup,
                                                                 page_tokens=pt)
                # warm: one input replica, so the Infinity Cache keeps most of a step's bytes
                results[name + "/warm_one_replica"] = bench_decode(api, torch, w, x, args.steps, args.warmup,
                                                                   replicas=1)
                results[name + "/exact_select"] = bench_exact_select(api, torch, w, x, min(args.steps, 10),
                                                                     min(args.warmup, 2))
            elif w.rank > 0:  # context: FP4 rows without the subspace projection; fp32 rows
                if w.sub_dim > 0:
                    results[name + "/no_subspace"] = bench_decode(api, torch, w, x, args.steps, args.warmup,
                                                                  subspace=False)
                results[name + "/fp32_factors"] = bench_decode(api, torch, w, x, args.steps, args.warmup,
                                                               factor_fp4=False)
                # the configuration's own fp32 summaries (fp32 mean and fp32 rank-r rows)
                results[name + "/fp32_summaries"] = bench_decode(api, torch, w, x, args.steps, args.warmup,
                                                                 mean_dtype="f32", factor_fp4=False,
                                                                 append_rows=True)
        elif w.top_k > 0:
            results[name] = bench_sparse_prefill(api, torch, w, x, args.steps, args.warmup)
        else:
            results[name] = bench_prefill(api, torch, w, x, args.steps, args.warmup)
            if name == "swa_prefill_8k" and not args.no_context:
                # context: the SWA glossary's dilated window on the same inputs, 4096
                # keys at spacing 2 (every other key over 8191 positions)
                wd = w.scaled(name="swa_prefill_8k_dilated2", window_left=2 * 4095, dilation=2)
                results[name + "/dilated2"] = bench_prefill(api, torch, wd, x, args.steps, args.warmup)
        log(f"[bench] {name}: {json.dumps(results[name])}")
        if name == HEADLINE:
            inputs[name] = x
        del x

    if args.only and args.only != HEADLINE:
        print(json.dumps({"workload": args.only, **results[args.only]}))
        return

    h = results[HEADLINE]
    w = WORKLOADS[HEADLINE]
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) ...")
        cpu = cpu_baseline(w, inputs[HEADLINE])
        log(f"[bench] cpu baseline: {cpu}")
    line = {
        "metric": METRIC,
        "value": h["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": HEADLINE, "batch": w.batch, "context": w.n_ctx,
                   "q_heads": w.n_q_heads, "kv_heads": w.n_kv_heads, "head_dim": w.head_dim,
                   "block": w.block_size, "top_k": w.top_k, "window": w.window, "sink": w.n_sink,
                   "rank": w.rank, "parallelism": "single GPU"},
        "gathered_kv_GBps": h.get("gathered_kv_GBps"),
        "gathered_kv_frac_hbm": h.get("gathered_kv_frac_hbm"),
        # the loads-only gather of the same blocks (bsattn_probe_gather), best setting
        "gather_ceiling_GBps": max((v["GBps"] for k, v in (h.get("gather_probe") or {}).items()
                                    if k.startswith("wg")), default=None),
        "roofline": {
            "kernel": "bsattn_decode_step: decode_bf16_kernel with in-kernel scoring and the in-wave "
                      "top-k, decode_merge_kernel (one call, two launches)",
            "bound": "hbm",
            "achieved": h["step_bytes"] / (h["ms_per_step"] * 1e-3) / 1e9,
            "peak": HBM_PEAK / 1e9,
            "unit": "GB/s",
            "frac": h["step_bytes"] / (h["ms_per_step"] * 1e-3) / HBM_PEAK,
            "traffic": step_traffic(),
            "bytes_per_launch": h["step_bytes"],
            "avg_launch_ms": h["ms_per_step"],
        },
        "cpu_baseline": cpu,
        "traffic_ratios": traffic_ratios(results),
        "rows": results,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
