"""The C-ABI library on the CPU: it loads, exports every function include/bsattn.h
declares, sizes the decode workspace, and rejects bad arguments before any launch
(every call below fails validation, so no GPU is touched)."""

import ctypes
import os
import re

import pytest

import sliding_window_attention_block_amd as api
from sliding_window_attention_block_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # a 256-byte aligned non-NULL address; never dereferenced on these paths


def _header_functions():
    text = open(os.path.join(ROOT, "include", "bsattn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsattn_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = api.library()
    declared = _header_functions()
    assert len(declared) == 17
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(_lib.EXPORTS)
    assert "gfx950" in api.bsattn_version()


def test_status_strings():
    for st in range(5):
        assert api.bsattn_status_string(st)
    assert api.bsattn_status_string(99) == "unknown status"


def test_workspace_size_matches_split_layout():
    s = api.make_shape(4, 64, 8, 128, 131072)
    # 32 selected + sink block + 16 window blocks = 49 items = 98 half items; the
    # 1024 resident waves give each of the 32 pairs 32 waves, 4 per workgroup ->
    # 8 partials per query head
    up = lambda x: -(-x // 256) * 256  # noqa: E731
    rows = 4 * 64 * 8
    expect = up(rows * 128 * 4) + up(rows * 8)
    assert api.bsattn_decode_workspace_bytes(s, 32, 1024, 64, 0) == expect
    # globals can only add blocks (the partials per head stay capped by the
    # resident waves here)
    assert api.bsattn_decode_workspace_bytes(s, 32, 1024, 64, 5) >= expect
    assert api.bsattn_decode_workspace_bytes(s, 32, 1024, 64, 40) >= expect
    # with one pair, each forced block adds waves until the cap: 49 items -> 100
    # waves (25 partials), 89 items -> 180 waves (45 partials)
    one = api.make_shape(1, 8, 1, 128, 131072)
    rows1 = lambda n: up(8 * n * 128 * 4) + up(8 * n * 8)  # noqa: E731
    assert api.bsattn_decode_workspace_bytes(one, 32, 1024, 64, 0) == rows1(25)
    assert api.bsattn_decode_workspace_bytes(one, 32, 1024, 64, 40) == rows1(45)
    small = api.make_shape(1, 4, 1, 64, 300)
    assert api.bsattn_decode_workspace_bytes(small, 2, 500, 10, 0) > 0
    assert api.bsattn_decode_workspace_bytes(small, 0, 10, 10, 0) == 0
    assert api.bsattn_decode_workspace_bytes(api.make_shape(1, 3, 2, 64, 10), 1, 1, 1, 0) == 0


def test_workspace_covers_globals_sharing_blocks():
    """Global tokens that share a block (or sit in the window) give fewer forced items
    than the bound; the size query covers every count, so such calls pass the check."""
    s = _shape(n_ctx=4096, kv_capacity=4096)
    lib = api.library()
    full = lib.bsattn_decode_workspace_bytes(s, 4, 64, 0, 3)
    for extra in range(4):
        assert full >= lib.bsattn_decode_workspace_bytes(s, 4, 64, 0, extra)


def _status(fn, *args):
    lib = api.library()
    st = getattr(lib, fn)(*args)
    return st, lib.bsattn_last_error().decode()


def _shape(**kw):
    base = dict(batch=1, n_q_heads=4, n_kv_heads=1, head_dim=64, n_ctx=256, kv_capacity=256,
                block_size=64, scale=0.0, dtype=1)
    base.update(kw)
    return ctypes.byref(_lib.Shape(*base.values()))


G3 = (ctypes.c_int32 * 3)


@pytest.mark.parametrize("shape_kw,code", [
    (dict(n_q_heads=6, n_kv_heads=4), 1),
    (dict(head_dim=96), 2),
    (dict(block_size=32), 2),
    (dict(kv_capacity=100), 1),
    (dict(dtype=7), 1),
    (dict(n_ctx=0), 1),
    (dict(scale=-1.0), 1),
    (dict(n_q_heads=32, n_kv_heads=1), 2),  # 32 query heads per K/V head
])
def test_decode_rejects_bad_shapes(shape_kw, code):
    st, msg = _status("bsattn_decode", _shape(**shape_kw), FAKE, FAKE, FAKE, FAKE, 4, 64, 0, None, 0,
                      FAKE, None, FAKE, 1 << 30, None, None)
    assert st == code and msg


def test_decode_rejects_bad_arguments():
    s = _shape()
    args = [s, FAKE, FAKE, FAKE, FAKE, 4, 64, 0, None, 0, FAKE, None, FAKE, 1 << 30, None, None]
    st, _ = _status("bsattn_decode", *args[:1], None, *args[2:])
    assert st == 1
    st, _ = _status("bsattn_decode", *args[:5], 0, *args[6:])            # top_k 0
    assert st == 1
    st, _ = _status("bsattn_decode", *args[:6], -1, *args[7:])           # negative window
    assert st == 1
    st, msg = _status("bsattn_decode", *args[:13], 16, None, None)       # workspace too small
    assert st == 4 and "workspace" in msg
    st, _ = _status("bsattn_decode", *args[:12], FAKE + 16, 1 << 30, None, None)  # misaligned workspace
    assert st == 1
    st, _ = _status("bsattn_decode", s, FAKE + 4, *args[2:])             # misaligned Q
    assert st == 1


STEP_ARGS = ("shape", "Q", "K", "V", "mean", "mean_dtype", "factor", "factor_dtype", "factor_scale",
             "basis", "sub_dim", "rank", "nblk", "top_k", "window", "n_sink", "gpos", "n_global", "sel", "scores", "O", "lse",
             "ws", "ws_bytes", "paged", "stream")
SELECT_ARGS = ("shape", "Q", "mean", "mean_dtype", "factor", "factor_dtype", "factor_scale", "basis",
               "sub_dim", "rank", "nblk",
               "top_k", "window", "n_sink", "gpos", "n_global", "sel", "scores", "stream")
SUMMARY_ARGS = ("shape", "K", "rank", "first_block", "n_blocks", "nblk", "mean", "mean_dtype", "factor",
                "factor_dtype", "factor_scale", "basis", "sub_dim", "paged", "stream")
GOOD = dict(Q=FAKE, K=FAKE, V=FAKE, mean=FAKE, mean_dtype=0, factor=None, factor_dtype=0, factor_scale=None,
            basis=None, sub_dim=0, rank=0, nblk=4, top_k=2, window=64, n_sink=0, gpos=None, n_global=0, sel=FAKE, scores=FAKE,
            O=FAKE, lse=None, ws=FAKE, ws_bytes=1 << 30, paged=None, stream=None, first_block=0, n_blocks=4)


def _call(fn, names, **over):
    kw = dict(GOOD, shape=_shape())
    kw.update(over)
    return _status(fn, *[kw[n] for n in names])


def test_decode_step_rejects_bad_arguments():
    f = "bsattn_decode_step"
    assert _call(f, STEP_ARGS, mean=None)[0] == 1
    assert _call(f, STEP_ARGS, mean_dtype=2)[0] == 1                      # mean neither fp32 nor bf16
    assert _call(f, STEP_ARGS, rank=1)[0] == 1                            # rank 1 without a factor
    assert _call(f, STEP_ARGS, rank=1, factor=FAKE, factor_dtype=2)[0] == 1  # FP4 without scales
    assert _call(f, STEP_ARGS, rank=1, factor=FAKE, factor_dtype=5)[0] == 1  # unknown factor dtype
    assert _call(f, STEP_ARGS, nblk=3)[0] == 1                            # nblk_capacity < 4 blocks
    assert _call(f, STEP_ARGS, top_k=0)[0] == 1
    assert _call(f, STEP_ARGS, sel=None)[0] == 1
    assert _call(f, STEP_ARGS, O=None)[0] == 1
    st, msg = _call(f, STEP_ARGS, ws_bytes=16)                            # workspace too small
    assert st == 4 and "workspace" in msg
    assert _call(f, STEP_ARGS, V=FAKE + 4)[0] == 1                        # misaligned V


@pytest.mark.parametrize("gpos", [(5, 3, 9), (1, 1, 2), (0, 10, 256), (-1, 2, 3)])
def test_global_positions_are_checked(gpos):
    st, msg = _call("bsattn_select_topk", SELECT_ARGS, gpos=G3(*gpos), n_global=3)
    assert st == 1 and "global" in msg


def test_select_rejects_bad_arguments():
    f = "bsattn_select_topk"
    assert _call(f, SELECT_ARGS, rank=2)[0] == 1                          # rank 2 without a factor
    assert _call(f, SELECT_ARGS, rank=9, factor=FAKE)[0] == 1             # rank above 8
    assert _call(f, SELECT_ARGS, nblk=3)[0] == 1                          # nblk_capacity below n_ctx / 64
    assert _call(f, SELECT_ARGS, scores=None)[0] == 1                     # scores is required
    assert _call(f, SELECT_ARGS, top_k=2000)[0] == 1                      # top_k above the maximum
    st, msg = _call(f, SELECT_ARGS, mean_dtype=7)
    assert st == 1 and "mean_dtype" in msg
    st, msg = _call(f, SELECT_ARGS, rank=4, factor=FAKE, factor_dtype=2, factor_scale=FAKE + 2)
    assert st == 1 and "factor_scale" in msg                              # misaligned scales
    assert _call(f, SELECT_ARGS, rank=4, factor=FAKE, factor_dtype=1)[0] == 1  # bf16 factors are not built
    big = _shape(n_ctx=64 * 65537, kv_capacity=64 * 65537)
    assert _call(f, SELECT_ARGS, shape=big, nblk=65537)[0] == 2


def test_summaries_reject_bad_ranges():
    f = "bsattn_build_summaries"
    assert _call(f, SUMMARY_ARGS, first_block=3, n_blocks=2, nblk=8)[0] == 1  # blocks 3..4 incomplete
    assert _call(f, SUMMARY_ARGS, nblk=3)[0] == 1                             # past nblk_capacity
    assert _call(f, SUMMARY_ARGS, rank=4)[0] == 1                             # rank 4 without a factor
    assert _call(f, SUMMARY_ARGS, mean_dtype=3)[0] == 1                       # unknown mean dtype
    assert _call(f, SUMMARY_ARGS, rank=4, factor=FAKE, factor_dtype=2)[0] == 1  # FP4 without scales
    assert _call(f, SUMMARY_ARGS, n_blocks=0, mean_dtype=1)[0] == 0           # empty range: no launch


FP4 = dict(rank=4, factor=FAKE, factor_dtype=2, factor_scale=FAKE, mean_dtype=1)


@pytest.mark.parametrize("f,names", [("bsattn_build_summaries", SUMMARY_ARGS),
                                     ("bsattn_select_topk", SELECT_ARGS),
                                     ("bsattn_decode_step", STEP_ARGS)])
def test_query_subspace_basis_is_checked(f, names):
    """sub_dim: 0 or a multiple of 32 in [32, d] with rank >= 1 and an aligned basis."""
    for bad in (48, 16, 96, -32):                              # d = 64 here
        st, msg = _call(f, names, basis=FAKE, sub_dim=bad, **FP4)
        assert st == 1 and "sub_dim" in msg
    st, msg = _call(f, names, basis=None, sub_dim=32, **FP4)
    assert st == 1 and "basis" in msg
    st, msg = _call(f, names, basis=FAKE + 4, sub_dim=32, **FP4)
    assert st == 1 and "basis" in msg
    st, msg = _call(f, names, basis=FAKE, sub_dim=32, rank=0)
    assert st == 1 and "rank" in msg
    if f != "bsattn_build_summaries":
        # the projected scorer takes the compressed summary only: bf16 means and FP4 rows
        st, msg = _call(f, names, basis=FAKE, sub_dim=32, **dict(FP4, factor_dtype=0))
        assert st == 2 and "basis" in msg
        st, msg = _call(f, names, basis=FAKE, sub_dim=32, **dict(FP4, mean_dtype=0))
        assert st == 2 and "basis" in msg
        st, msg = _call(f, names, basis=FAKE, sub_dim=32, shape=_shape(dtype=0), **FP4)
        assert st == 2 and "basis" in msg


def test_prefill_rejects_bad_arguments():
    P = (FAKE, FAKE, FAKE)
    st, _ = _status("bsattn_prefill", _shape(dtype=0), *P, 10, 0, 1, None, 0, FAKE, None, None, 0, None)
    assert st == 2  # fp32 prefill is not built
    st, msg = _status("bsattn_prefill", _shape(), *P, 10, 0, 1, G3(1, 2, 3), 3, FAKE, None, None, 0, None)
    assert st == 2 and "bidirectional" in msg
    st, _ = _status("bsattn_prefill", _shape(), *P, 10, 0, 2, None, 0, FAKE, None, None, 0, None)
    assert st == 1
    st, _ = _status("bsattn_prefill", _shape(), FAKE, None, FAKE, 10, 0, 1, None, 0, FAKE, None, None, 0, None)
    assert st == 1
    # globals need the workspace of the key-split global rows
    st, msg = _status("bsattn_prefill", _shape(), *P, 8, 8, 0, G3(1, 2, 3), 3, FAKE, None, None, 0, None)
    assert st == 4 and "workspace" in msg
    need = api.bsattn_prefill_workspace_bytes(api.make_shape(1, 4, 1, 64, 256), 3)
    st, _ = _status("bsattn_prefill", _shape(), *P, 8, 8, 0, G3(1, 2, 3), 3, FAKE, None, FAKE + 16, need,
                    None)
    assert st == 1  # misaligned workspace


def test_dilated_prefill_rejects_bad_arguments():
    P = (FAKE, FAKE, FAKE)
    st, _ = _status("bsattn_prefill_dilated", _shape(dtype=0), *P, 10, 0, 1, 2, FAKE, None, None)
    assert st == 2  # bf16 only
    for dil in (0, -3, 65537):
        st, msg = _status("bsattn_prefill_dilated", _shape(), *P, 10, 0, 1, dil, FAKE, None, None)
        assert st == 1 and "dilation" in msg
    st, _ = _status("bsattn_prefill_dilated", _shape(), *P, 10, 0, 2, 2, FAKE, None, None)
    assert st == 1  # causal must be 0 or 1
    st, _ = _status("bsattn_prefill_dilated", _shape(), FAKE, FAKE, FAKE, 10, 0, 1, 2, None, None, None)
    assert st == 1  # O must be non-NULL
    st, _ = _status("bsattn_prefill_dilated", _shape(), FAKE + 8, FAKE, FAKE, 10, 0, 1, 2, FAKE, None, None)
    assert st == 1  # misaligned


def test_prefill_workspace_size():
    up = lambda x: -(-x // 256) * 256  # noqa: E731
    s = api.make_shape(2, 12, 12, 64, 16384)
    # 16 global rows -> one 32-row tile; 16384 keys in ranges of 512 -> 32 splits
    rows = 2 * 12 * 1 * 32 * 32
    assert api.bsattn_prefill_workspace_bytes(s, 16) == up(rows * 64 * 4) + up(rows * 8)
    assert api.bsattn_prefill_workspace_bytes(s, 33) == 2 * up(rows * 64 * 4) + 2 * up(rows * 8)
    assert api.bsattn_prefill_workspace_bytes(s, 0) == 0
    assert api.bsattn_prefill_workspace_bytes(s, 257) == 0


def test_binding_raises_with_the_library_message():
    import torch
    with pytest.raises(ValueError):
        api.bsattn_prefill(api.make_shape(1, 1, 1, 64, 8), torch.zeros(1), torch.zeros(1),
                           torch.zeros(1), 1, 0, 1, None, torch.zeros(1))


APPEND_ARGS = ("shape", "K_new", "V_new", "K", "V", "rank", "nblk", "mean", "mean_dtype", "factor",
               "factor_dtype", "factor_scale", "basis", "sub_dim", "paged", "stream")


def test_append_rejects_bad_arguments():
    f = "bsattn_append_kv"
    kw = dict(K_new=FAKE, V_new=FAKE)
    assert _call(f, APPEND_ARGS, **dict(kw, K_new=None))[0] == 1
    assert _call(f, APPEND_ARGS, **dict(kw, V=FAKE + 8))[0] == 1                      # misaligned V
    assert _call(f, APPEND_ARGS, **kw, shape=_shape(n_ctx=300, kv_capacity=299))[0] == 1  # past capacity
    # token 256 completes block 3: the summary arguments are validated then, before any launch
    assert _call(f, APPEND_ARGS, **kw, shape=_shape(n_ctx=256), mean=None)[0] == 1
    assert _call(f, APPEND_ARGS, **kw, shape=_shape(n_ctx=256), nblk=3)[0] == 1      # block 3 past capacity
    assert _call(f, APPEND_ARGS, **kw, shape=_shape(n_ctx=256), rank=2)[0] == 1      # rank 2, no factor
    st, msg = _call(f, APPEND_ARGS, **kw, shape=_shape(n_ctx=256), basis=FAKE, sub_dim=48, **FP4)
    assert st == 1 and "sub_dim" in msg



def _pg(page_tokens=16, max_pages=16, n_pages=40, table=FAKE):
    return ctypes.byref(_lib.PagedKV(table, page_tokens, max_pages, n_pages))


@pytest.mark.parametrize("f,names", [("bsattn_build_summaries", SUMMARY_ARGS), ("bsattn_append_kv", APPEND_ARGS),
                                     ("bsattn_decode_step", STEP_ARGS)])
def test_paged_layout_is_checked(f, names):
    """page_tokens 16, 32 or 64; kv_capacity = max_pages * page_tokens; a non-NULL,
    aligned block table; at least one page."""
    kw = dict(K_new=FAKE, V_new=FAKE) if f == "bsattn_append_kv" else {}
    for bad in (_pg(page_tokens=8, max_pages=32), _pg(page_tokens=48), _pg(max_pages=8),
                _pg(table=None), _pg(table=FAKE + 2), _pg(n_pages=0)):
        st, msg = _call(f, names, paged=bad, **kw)
        assert st == 1 and "paged" in msg


def test_paged_decode_takes_bf16_only():
    st, msg = _call("bsattn_decode_step", STEP_ARGS, paged=_pg(), shape=_shape(dtype=0))
    assert st == 2 and "BF16" in msg


def test_sparse_prefill_rejects_bad_arguments():
    f, g = "bsattn_select_prefill", "bsattn_sparse_prefill"
    sel_args = lambda **o: [o.get("shape", _shape()), o.get("Q", FAKE), o.get("mean", FAKE), o.get("md", 1),
                            o.get("nblk", 4), o.get("k", 2), o.get("wl", 64), o.get("ns", 0), FAKE, FAKE, None]
    assert _status(f, *sel_args(md=0))[0] == 2                        # fp32 means
    assert _status(f, *sel_args(shape=_shape(dtype=0)))[0] == 2       # fp32 queries
    assert _status(f, *sel_args(k=0))[0] == 1
    assert _status(f, *sel_args(k=257))[0] == 1
    assert _status(f, *sel_args(wl=-1))[0] == 1
    assert _status(f, *sel_args(ns=300))[0] == 1
    assert _status(f, *sel_args(nblk=3))[0] == 1
    # 64K blocks (4M tokens): 32768 tiles x 1024 groups of 64 blocks per pair; 64 pairs overflow the grid
    big = _shape(batch=8, n_q_heads=64, n_kv_heads=8, n_ctx=64 * 65536, kv_capacity=64 * 65536)
    st, msg = _status(f, *sel_args(shape=big, nblk=65536))
    assert st == 2 and "grid" in msg
    pre = lambda **o: [o.get("shape", _shape()), FAKE, FAKE, FAKE, o.get("sel", FAKE), o.get("k", 2),
                       o.get("wl", 64), o.get("ns", 0), FAKE, None, None]
    assert _status(g, *pre(shape=_shape(dtype=0)))[0] == 2
    assert _status(g, *pre(sel=None))[0] == 1
    assert _status(g, *pre(wl=-5))[0] == 1
    assert _status(g, *pre(k=300))[0] == 1


def test_exact_selector_rejects_bad_arguments():
    f = "bsattn_select_exact"
    args = lambda **o: [o.get("shape", _shape()), FAKE, o.get("K", FAKE), o.get("nblk", 4), o.get("k", 2),
                        64, 0, None, 0, FAKE, FAKE, None]
    assert _status(f, *args(shape=_shape(dtype=0)))[0] == 2   # fp32
    assert _status(f, *args(K=None))[0] == 1
    assert _status(f, *args(K=FAKE + 8))[0] == 1              # misaligned
    assert _status(f, *args(k=0))[0] == 1
    assert _status(f, *args(nblk=3))[0] == 1


def test_gather_probe_rejects_bad_arguments():
    f = "bsattn_probe_gather"
    args = lambda **o: [o.get("shape", _shape()), o.get("K", FAKE), FAKE, o.get("blocks", FAKE), o.get("nb", 4),
                        o.get("wg", 2), o.get("depth", 2), o.get("out", FAKE), None]
    assert _status(f, *args(shape=_shape(dtype=0)))[0] == 2   # fp32 cache
    assert _status(f, *args(shape=_shape(head_dim=96)))[0] == 2
    assert _status(f, *args(K=None))[0] == 1
    assert _status(f, *args(blocks=None))[0] == 1
    assert _status(f, *args(out=None))[0] == 1
    assert _status(f, *args(nb=0))[0] == 1
    assert _status(f, *args(wg=0))[0] == 1
    assert _status(f, *args(wg=17))[0] == 1
    assert _status(f, *args(depth=0))[0] == 1
    st, msg = _status(f, *args(depth=5))
    assert st == 1 and "depth" in msg


def test_a_missing_library_raises_instead_of_falling_back(tmp_path, monkeypatch):
    """The binding has no CPU fallback: without the built library every entry
    point's loader raises, naming the missing file."""
    import sliding_window_attention_block_amd._lib as L
    missing = str(tmp_path / "libbsattn.so")
    monkeypatch.setattr(L, "LIB_PATH", missing)
    monkeypatch.setattr(L, "_lib", None)
    with pytest.raises(OSError, match="is missing"):
        L.load()


def test_noalloc_step_checks_its_arguments_and_the_scratch_limit():
    """bsattn_decode_step_noalloc: the decode step's argument checks, and a problem
    whose split partials pass the static scratch is refused (BSATTN_ERR_WORKSPACE)
    before any device call."""
    lib = _lib.load()
    assert _lib.BSATTN_NOALLOC_SCRATCH_BYTES == 16 << 20
    s = _lib.Shape(64, 1024, 64, 128, 4096 * 64, 4096 * 64, 64, 0.0, _lib.BSATTN_BF16)
    p = ctypes.c_void_p(16)
    assert lib.bsattn_decode_workspace_bytes(ctypes.byref(s), 1024, 512, 64, 0) > _lib.BSATTN_NOALLOC_SCRATCH_BYTES
    st = lib.bsattn_decode_step_noalloc(ctypes.byref(s), p, p, p, p, 1, None, 0, None, None, 0, 0, 4096, 1024, 512,
                                        64, None, 0, p, p, p, p, None, None)
    assert st == _lib.BSATTN_ERR_WORKSPACE
    assert b"static scratch" in lib.bsattn_last_error()
    bad = _lib.Shape(1, 3, 2, 128, 100, 100, 64, 0.0, _lib.BSATTN_BF16)  # Hq not a multiple of Hkv
    st = lib.bsattn_decode_step_noalloc(ctypes.byref(bad), p, p, p, p, 1, None, 0, None, None, 0, 0, 1, 4, 0,
                                        0, None, 0, p, p, p, p, None, None)
    assert st == _lib.BSATTN_ERR_INVALID
