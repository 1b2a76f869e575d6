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
    assert len(declared) == 10
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
    # 32 selected + sink block + 16 window blocks = 49 items = 98 half items (one per
    # wave); 4 waves per workgroup -> 25 partials
    up = lambda x: -(-x // 256) * 256  # noqa: E731
    rows = 4 * 64 * 25
    expect = up(rows * 128 * 4) + up(rows * 8)
    assert api.bsattn_decode_workspace_bytes(s, 32, 1024, 64, 0) == expect
    # globals can only add blocks
    assert api.bsattn_decode_workspace_bytes(s, 32, 1024, 64, 5) >= expect
    assert api.bsattn_decode_workspace_bytes(s, 32, 1024, 64, 40) > expect
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
                      FAKE, None, FAKE, 1 << 30, None)
    assert st == code and msg


def test_decode_rejects_bad_arguments():
    s = _shape()
    args = [s, FAKE, FAKE, FAKE, FAKE, 4, 64, 0, None, 0, FAKE, None, FAKE, 1 << 30, None]
    st, _ = _status("bsattn_decode", *args[:1], None, *args[2:])
    assert st == 1
    st, _ = _status("bsattn_decode", *args[:5], 0, *args[6:])            # top_k 0
    assert st == 1
    st, _ = _status("bsattn_decode", *args[:6], -1, *args[7:])           # negative window
    assert st == 1
    st, msg = _status("bsattn_decode", *args[:13], 16, None)             # workspace too small
    assert st == 4 and "workspace" in msg
    st, _ = _status("bsattn_decode", *args[:12], FAKE + 16, 1 << 30, None)  # misaligned workspace
    assert st == 1
    st, _ = _status("bsattn_decode", s, FAKE + 4, *args[2:])             # misaligned Q
    assert st == 1


def test_decode_step_rejects_bad_arguments():
    s = _shape()
    # shape Q K V mean mean_dtype factor rank nblk top_k window n_sink gpos n_global sel scores O lse
    # ws ws_bytes stream
    args = [s, FAKE, FAKE, FAKE, FAKE, 0, None, 0, 4, 2, 64, 0, None, 0, FAKE, FAKE, FAKE, None, FAKE,
            1 << 30, None]
    st, _ = _status("bsattn_decode_step", *args[:4], None, *args[5:])          # NULL mean
    assert st == 1
    st, _ = _status("bsattn_decode_step", *args[:5], 2, *args[6:])             # unknown mean dtype
    assert st == 1
    st, _ = _status("bsattn_decode_step", *args[:7], 1, *args[8:])             # rank 1, NULL factor
    assert st == 1
    st, _ = _status("bsattn_decode_step", *args[:8], 3, *args[9:])             # nblk_capacity < 4 blocks
    assert st == 1
    st, _ = _status("bsattn_decode_step", *args[:9], 0, *args[10:])            # top_k 0
    assert st == 1
    st, _ = _status("bsattn_decode_step", *args[:14], None, *args[15:])        # NULL sel
    assert st == 1
    st, _ = _status("bsattn_decode_step", *args[:16], None, *args[17:])        # NULL O
    assert st == 1
    st, msg = _status("bsattn_decode_step", *args[:19], 16, None)              # workspace too small
    assert st == 4 and "workspace" in msg
    st, _ = _status("bsattn_decode_step", *args[:3], FAKE + 4, *args[4:])      # misaligned V
    assert st == 1


@pytest.mark.parametrize("gpos", [(5, 3, 9), (1, 1, 2), (0, 10, 256), (-1, 2, 3)])
def test_global_positions_are_checked(gpos):
    st, msg = _status("bsattn_select_topk", _shape(), FAKE, FAKE, 0, None, 0, 4, 2, 64, 0, G3(*gpos), 3,
                      FAKE, FAKE, None)
    assert st == 1 and "global" in msg


def test_select_rejects_bad_arguments():
    s = _shape()
    # shape Q mean mean_dtype factor rank nblk top_k window n_sink gpos n_global sel scores stream
    st, _ = _status("bsattn_select_topk", s, FAKE, FAKE, 0, None, 2, 4, 2, 64, 0, None, 0, FAKE, FAKE, None)
    assert st == 1  # rank 2 without a factor
    st, _ = _status("bsattn_select_topk", s, FAKE, FAKE, 0, FAKE, 9, 4, 2, 64, 0, None, 0, FAKE, FAKE, None)
    assert st == 1  # rank above 8
    st, _ = _status("bsattn_select_topk", s, FAKE, FAKE, 0, None, 0, 3, 2, 64, 0, None, 0, FAKE, FAKE, None)
    assert st == 1  # nblk_capacity below n_ctx / 64
    st, _ = _status("bsattn_select_topk", s, FAKE, FAKE, 0, None, 0, 4, 2, 64, 0, None, 0, FAKE, None, None)
    assert st == 1  # scores is required
    st, _ = _status("bsattn_select_topk", s, FAKE, FAKE, 0, None, 0, 4, 2000, 64, 0, None, 0, FAKE, FAKE, None)
    assert st == 1  # top_k above the maximum
    st, msg = _status("bsattn_select_topk", s, FAKE, FAKE, 7, None, 0, 4, 2, 64, 0, None, 0, FAKE, FAKE, None)
    assert st == 1 and "mean_dtype" in msg  # mean stored as neither fp32 nor bf16
    big = _shape(n_ctx=64 * 65537, kv_capacity=64 * 65537)
    st, _ = _status("bsattn_select_topk", big, FAKE, FAKE, 1, None, 0, 65537, 2, 64, 0, None, 0, FAKE, FAKE,
                    None)
    assert st == 2


def test_summaries_reject_bad_ranges():
    s = _shape()
    # shape K rank first_block n_blocks nblk mean mean_dtype factor stream
    st, _ = _status("bsattn_build_summaries", s, FAKE, 0, 3, 2, 8, FAKE, 0, None, None)
    assert st == 1  # blocks 3..4 are not complete in 256 tokens
    st, _ = _status("bsattn_build_summaries", s, FAKE, 0, 0, 4, 3, FAKE, 0, None, None)
    assert st == 1  # past nblk_capacity
    st, _ = _status("bsattn_build_summaries", s, FAKE, 4, 0, 4, 4, FAKE, 0, None, None)
    assert st == 1  # rank 4 without a factor
    st, _ = _status("bsattn_build_summaries", s, FAKE, 0, 0, 4, 4, FAKE, 3, None, None)
    assert st == 1  # unknown mean dtype
    st, _ = _status("bsattn_build_summaries", s, FAKE, 0, 0, 0, 4, FAKE, 1, None, None)
    assert st == 0  # empty range: nothing to launch


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
