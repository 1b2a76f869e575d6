"""Helpers for the GPU parity tests: device copies, a full decode step through the
C ABI, and the comparison rules (selected sets with the near-tie allowance,
outputs at max-abs 2e-3)."""

from __future__ import annotations

import math

import numpy as np

import oracle
from synthetic import bf16_bits_to_f32

OUT_TOL = 2e-3       # max-abs on outputs, compared in fp32
TIE_REL = 1e-4       # relative gap of the oracle's k-th and (k+1)-th scores


def torch_mod():
    import torch
    return torch


def to_dev(arr):
    """numpy float32 -> cuda float32; numpy uint16 (bf16 bits) -> cuda bfloat16."""
    torch = torch_mod()
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


def as_f64(arr):
    return (bf16_bits_to_f32(arr) if arr.dtype == np.uint16 else np.asarray(arr, np.float32)).astype(np.float64)


def paged_pools(K, V, page_tokens, seed, spare=5):
    """Scatter contiguous caches K, V [B, Hkv, cap, d] (device tensors, cap a multiple
    of page_tokens) into page pools [n_pages, Hkv, P, d] under a random assignment of
    distinct pages; pages no token maps to hold NaN.  Returns Kp, Vp, the int32 block
    table [B, cap / P] and n_pages."""
    torch = torch_mod()
    B, Hkv, cap, d = K.shape
    P = page_tokens
    mp = cap // P
    n_pages = B * mp + spare
    perm = np.random.default_rng(seed).permutation(n_pages)[:B * mp].reshape(B, mp)
    table = torch.from_numpy(perm.astype(np.int32)).cuda()
    idx = torch.from_numpy(perm.reshape(-1)).cuda().long()
    out = []
    for X in (K, V):
        pool = torch.full((n_pages, Hkv, P, d), float("nan"), dtype=X.dtype, device="cuda")
        pool[idx] = X.reshape(B, Hkv, mp, P, d).permute(0, 2, 1, 3, 4).reshape(B * mp, Hkv, P, d)
        out.append(pool)
    return out[0], out[1], table, n_pages


def gpu_decode_step(api, x, w, kv_capacity=None, nblk_capacity=None, global_pos=(), dev=None,
                    one_call=False, mean_dtype="f32", factor_fp4=False, basis=None, page_tokens=None,
                    page_seed=0):
    """Run summaries -> select/top-k -> decode on the GPU through the binding.

    ``x`` holds Q, K, V numpy arrays (float32 or bf16 bits) of workload ``w``.
    With ``one_call`` the step is bsattn_decode_step (selection and decode in one
    call); otherwise bsattn_select_topk, then bsattn_decode.  ``mean_dtype`` "bf16"
    stores the block means in bfloat16; ``factor_fp4`` the factor rows as FP4 codes
    (returned as ``factor`` uint8 codes plus ``factor_scale``).  ``basis`` [Hkv, s, d]
    (numpy float32) projects the factor rows onto each K/V head's query subspace.
    ``page_tokens`` runs every call on page pools (``paged_pools``) through a block table.
    Returns numpy copies of mean (as float32), factor, scores, sel, O, lse.
    """
    torch = torch_mod()
    B, Hq, Hkv, d, n = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_ctx
    cap = x["K"].shape[2] if kv_capacity is None else kv_capacity
    nb = n // w.block_size
    nbcap = nb if nblk_capacity is None else nblk_capacity
    dev = dev or {}
    Q = dev["Q"] if "Q" in dev else to_dev(x["Q"])
    K = dev["K"] if "K" in dev else to_dev(x["K"])
    V = dev["V"] if "V" in dev else to_dev(x["V"])
    shape = api.make_shape(B, Hq, Hkv, d, n, kv_capacity=cap, dtype=w.dtype)
    pg = None
    if page_tokens is not None:
        K, V, table, n_pages = paged_pools(K, V, page_tokens, page_seed)
        pg = api.paged_kv(table, page_tokens, n_pages)
    mean = torch.full((B, Hkv, max(nbcap, 1), d), float("nan"), device="cuda",
                      dtype=torch.bfloat16 if mean_dtype == "bf16" else torch.float32)
    factor = fscale = bdev = None
    e = d if basis is None else basis.shape[1]
    if basis is not None:
        bdev = torch.from_numpy(np.ascontiguousarray(basis, dtype=np.float32)).cuda()
    if w.rank > 0 and factor_fp4:
        factor = torch.full((B, Hkv, max(nbcap, 1), w.rank, e // 2), 255, dtype=torch.uint8, device="cuda")
        fscale = torch.full((B, Hkv, max(nbcap, 1), w.rank), float("nan"), device="cuda")
    elif w.rank > 0:
        factor = torch.full((B, Hkv, max(nbcap, 1), w.rank, e), float("nan"), device="cuda")
    api.bsattn_build_summaries(shape, K, w.rank, 0, nb, max(nbcap, 1), mean, factor, factor_scale=fscale,
                               basis=bdev, paged=pg)
    scores = torch.full((B, Hkv, max(nbcap, 1)), float("nan"), device="cuda")
    sel = torch.full((B, Hkv, w.top_k), -7, dtype=torch.int32, device="cuda")
    O = torch.full((B, Hq, d), float("nan"), device="cuda")
    lse = torch.full((B, Hq), float("nan"), device="cuda")
    gp = list(global_pos)
    nbytes = api.bsattn_decode_workspace_bytes(shape, w.top_k, w.window, w.n_sink, len(gp))
    ws = torch.full((nbytes,), 255, dtype=torch.uint8, device="cuda")  # garbage contents
    if one_call:
        api.bsattn_decode_step(shape, Q, K, V, mean, factor, w.rank, max(nbcap, 1), w.top_k, w.window,
                               w.n_sink, gp, sel, scores, O, lse, ws, factor_scale=fscale, basis=bdev, paged=pg)
    else:
        api.bsattn_select_topk(shape, Q, mean, factor, w.rank, max(nbcap, 1), w.top_k, w.window,
                               w.n_sink, gp, sel, scores, factor_scale=fscale, basis=bdev)
        api.bsattn_decode(shape, Q, K, V, sel, w.top_k, w.window, w.n_sink, gp, O, lse, ws, paged=pg)
    torch.cuda.synchronize()
    return dict(mean=mean.float().cpu().numpy(), factor=None if factor is None else factor.cpu().numpy(),
                factor_scale=None if fscale is None else fscale.cpu().numpy(),
                scores=scores.cpu().numpy(), sel=sel.cpu().numpy(), O=O.cpu().numpy(),
                lse=lse.cpu().numpy())


def compare_selection(sel_gpu, scores_oracle, cand, k):
    """True/False for a (b, kv head) pair, plus whether the oracle has a near tie at k.

    Sets must be identical, except at a near tie (relative gap of the oracle's k-th and
    (k+1)-th candidate scores < 1e-4), where only blocks whose oracle scores lie in the
    tie band may differ.
    """
    ref = oracle.top_k_blocks(scores_oracle, cand, k)
    got = np.asarray(sel_gpu)
    valid = got[got >= 0]
    if len(valid) and (np.any(np.diff(valid) <= 0) or np.any(got[len(valid):] >= 0)):
        return False, False  # not ascending / padding not at the end
    if np.array_equal(got, ref):
        return True, False
    if len(cand) <= k:
        return False, False
    cs = np.sort(scores_oracle[cand])[::-1]
    sk, sk1 = cs[k - 1], cs[k]
    scale = max(abs(sk), abs(sk1))
    near = abs(sk - sk1) <= TIE_REL * scale
    if not near:
        return False, False
    diff = set(valid.tolist()) ^ set(ref[ref >= 0].tolist())
    lo, hi = sk1 - TIE_REL * scale, sk + TIE_REL * scale
    ok = all(lo <= scores_oracle[b] <= hi for b in diff) and len(valid) == len(ref[ref >= 0])
    return ok, True


def oracle_decode_with_sel(q, Kbg, Vbg, n, S, window, n_sink, global_pos, sel, scale):
    """Oracle output for a given selected set (the output is unique given the set)."""
    forced = oracle.forced_token_mask(n, n_sink, window, global_pos)
    tokens = oracle.decode_token_set(n, S, forced, sel)
    return oracle.sparse_decode_group(q, Kbg[:n], Vbg[:n], tokens, scale)


def bf16_ulp(x):
    """Spacing of bfloat16 values at |x| (8 significant bits)."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(np.where(x > 0, x, 1.0))
    return np.ldexp(1.0, e - 8)


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)))) if np.size(a) else 0.0


def default_scale(d):
    return 1.0 / math.sqrt(d)
