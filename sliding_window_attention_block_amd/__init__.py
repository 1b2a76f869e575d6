"""Python binding of the bsattn C ABI (include/bsattn.h).

Argument marshalling only: every function takes torch tensors that already live
on the GPU (PyTorch is used for device memory and streams), checks their dtype
and layout, and passes raw pointers to the same-named C entry point.  All the
work runs in the HIP kernels of libbsattn.so; there is no CPU path and no
fallback.  A non-OK status raises ``BsattnError``.
"""

from __future__ import annotations

import ctypes
import math

from . import _lib
from ._lib import BSATTN_BF16, BSATTN_F32, BSATTN_FP4_E2M1, BSATTN_NOALLOC_SCRATCH_BYTES, PagedKV, Shape

__all__ = [
    "BsattnError", "Shape", "PagedKV", "make_shape", "paged_kv", "library", "bsattn_build_summaries",
    "bsattn_append_kv", "bsattn_select_prefill", "bsattn_sparse_prefill", "bsattn_select_exact",
    "bsattn_select_topk", "bsattn_decode_workspace_bytes", "bsattn_decode",
    "bsattn_decode_step",
    "bsattn_decode_step_noalloc",
    "bsattn_prefill",
    "bsattn_prefill_dilated",
    "bsattn_prefill_workspace_bytes",
    "bsattn_probe_gather",
    "bsattn_status_string", "bsattn_version", "BSATTN_F32", "BSATTN_BF16", "BSATTN_FP4_E2M1",
    "BSATTN_NOALLOC_SCRATCH_BYTES",
]


class BsattnError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{message} (status {status})")
        self.status = status


def library():
    """The loaded ctypes library (raises OSError if it was never built)."""
    return _lib.load()


def make_shape(batch, n_q_heads, n_kv_heads, head_dim, n_ctx, kv_capacity=None, block_size=64,
               scale=0.0, dtype="bf16"):
    dt = {"bf16": BSATTN_BF16, "f32": BSATTN_F32}[dtype] if isinstance(dtype, str) else int(dtype)
    return Shape(batch, n_q_heads, n_kv_heads, head_dim, n_ctx,
                 n_ctx if kv_capacity is None else kv_capacity, block_size, float(scale), dt)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _globals(global_pos):
    g = [] if global_pos is None else [int(x) for x in global_pos]
    arr = (ctypes.c_int32 * max(1, len(g)))(*g)
    return (arr if g else None), len(g)


def _check(status):
    if status != 0:
        lib = library()
        msg = lib.bsattn_last_error().decode() or lib.bsattn_status_string(status).decode()
        raise BsattnError(status, msg)


def bsattn_status_string(status):
    return library().bsattn_status_string(status).decode()


def bsattn_version():
    return library().bsattn_version().decode()


def _mean_dtype(mean):
    """bsattn dtype code of a block-mean tensor: float32 or bfloat16."""
    import torch
    if mean.dtype == torch.float32:
        return BSATTN_F32
    if mean.dtype == torch.bfloat16:
        return BSATTN_BF16
    raise ValueError(f"block means must be float32 or bfloat16, not {mean.dtype}")


def _factor_dtype(factor, factor_scale):
    """bsattn dtype code of a factor tensor: float32 rows, or uint8 FP4 codes (with scales)."""
    import torch
    if factor is None or factor.dtype == torch.float32:
        return BSATTN_F32
    if factor.dtype == torch.uint8:
        if factor_scale is None:
            raise ValueError("FP4 factor codes need factor_scale")
        return BSATTN_FP4_E2M1
    raise ValueError(f"factor rows must be float32 or uint8 FP4 codes, not {factor.dtype}")


def paged_kv(block_table, page_tokens, n_pages):
    """bsattn_paged_kv for a block table tensor (int32 [B, max_pages] on the device) over
    K and V page pools of n_pages pages of page_tokens tokens.  Keep the tensor alive."""
    return PagedKV(block_table.data_ptr(), page_tokens, int(block_table.shape[1]), n_pages)


def _paged(paged):
    return None if paged is None else ctypes.byref(paged)


def _sub_dim(basis):
    """Subspace dimension of a query-subspace basis [Hkv, sub_dim, d] (0 without one)."""
    return 0 if basis is None else int(basis.shape[1])


def bsattn_build_summaries(shape, K, rank, first_block, n_blocks, nblk_capacity, mean, factor=None,
                           stream=None, factor_scale=None, basis=None, paged=None):
    _check(library().bsattn_build_summaries(ctypes.byref(shape), _ptr(K), rank, first_block,
                                            n_blocks, nblk_capacity, _ptr(mean), _mean_dtype(mean),
                                            _ptr(factor), _factor_dtype(factor, factor_scale),
                                            _ptr(factor_scale), _ptr(basis), _sub_dim(basis),
                                            _paged(paged), _stream(stream)))


def bsattn_append_kv(shape, K_new, V_new, K, V, rank, nblk_capacity, mean=None, factor=None, stream=None,
                     factor_scale=None, basis=None, paged=None):
    """Write token n_ctx - 1 of every (b, K/V head) and build the summary of the block
    it completes (summary buffers are only touched then)."""
    _check(library().bsattn_append_kv(ctypes.byref(shape), _ptr(K_new), _ptr(V_new), _ptr(K), _ptr(V), rank,
                                      nblk_capacity, _ptr(mean),
                                      BSATTN_F32 if mean is None else _mean_dtype(mean), _ptr(factor),
                                      _factor_dtype(factor, factor_scale), _ptr(factor_scale), _ptr(basis),
                                      _sub_dim(basis), _paged(paged), _stream(stream)))


def bsattn_select_exact(shape, Q, K, nblk_capacity, top_k, window, n_sink, global_pos, sel, scores, stream=None):
    """Top-k blocks by the group's exact attention mass, read from the keys (reference selector)."""
    g, ng = _globals(global_pos)
    _check(library().bsattn_select_exact(ctypes.byref(shape), _ptr(Q), _ptr(K), nblk_capacity, top_k, window,
                                         n_sink, g, ng, _ptr(sel), _ptr(scores), _stream(stream)))


def bsattn_select_prefill(shape, Q, mean, nblk_capacity, top_k, window_left, n_sink, sel, scores, stream=None):
    """Per query tile of 128 rows: block scores and the top-k selected blocks."""
    _check(library().bsattn_select_prefill(ctypes.byref(shape), _ptr(Q), _ptr(mean), _mean_dtype(mean),
                                           nblk_capacity, top_k, window_left, n_sink, _ptr(sel), _ptr(scores),
                                           _stream(stream)))


def bsattn_sparse_prefill(shape, Q, K, V, sel, top_k, window_left, n_sink, O, lse, stream=None):
    """Causal window + sinks + each tile's selected blocks, one softmax per row."""
    _check(library().bsattn_sparse_prefill(ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(V), _ptr(sel), top_k,
                                           window_left, n_sink, _ptr(O), _ptr(lse), _stream(stream)))


def bsattn_select_topk(shape, Q, mean, factor, rank, nblk_capacity, top_k, window, n_sink,
                       global_pos, sel, scores, stream=None, factor_scale=None, basis=None):
    g, ng = _globals(global_pos)
    _check(library().bsattn_select_topk(ctypes.byref(shape), _ptr(Q), _ptr(mean), _mean_dtype(mean),
                                        _ptr(factor), _factor_dtype(factor, factor_scale),
                                        _ptr(factor_scale), _ptr(basis), _sub_dim(basis), rank,
                                        nblk_capacity, top_k, window,
                                        n_sink, g, ng, _ptr(sel), _ptr(scores), _stream(stream)))


def bsattn_decode_workspace_bytes(shape, top_k, window, n_sink, n_global=0):
    return int(library().bsattn_decode_workspace_bytes(ctypes.byref(shape), top_k, window, n_sink,
                                                       n_global))


def bsattn_decode(shape, Q, K, V, sel, top_k, window, n_sink, global_pos, O, lse, workspace,
                  stream=None, paged=None):
    g, ng = _globals(global_pos)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(library().bsattn_decode(ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(V), _ptr(sel),
                                   top_k, window, n_sink, g, ng, _ptr(O), _ptr(lse),
                                   _ptr(workspace), ws_bytes, _paged(paged), _stream(stream)))


def bsattn_decode_step(shape, Q, K, V, mean, factor, rank, nblk_capacity, top_k, window, n_sink,
                       global_pos, sel, scores, O, lse, workspace, stream=None, factor_scale=None,
                       basis=None, paged=None):
    g, ng = _globals(global_pos)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(library().bsattn_decode_step(ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(V), _ptr(mean),
                                        _mean_dtype(mean), _ptr(factor),
                                        _factor_dtype(factor, factor_scale), _ptr(factor_scale),
                                        _ptr(basis), _sub_dim(basis), rank,
                                        nblk_capacity, top_k, window, n_sink, g, ng, _ptr(sel),
                                        _ptr(scores), _ptr(O), _ptr(lse), _ptr(workspace), ws_bytes,
                                        _paged(paged), _stream(stream)))


def bsattn_decode_step_noalloc(shape, Q, K, V, mean, factor, rank, nblk_capacity, top_k, window, n_sink,
                               global_pos, sel, scores, O, lse, stream=None, factor_scale=None, basis=None,
                               paged=None):
    """bsattn_decode_step with the split partials in the library's static device scratch
    (no workspace argument; the call allocates nothing)."""
    g, ng = _globals(global_pos)
    _check(library().bsattn_decode_step_noalloc(ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(V), _ptr(mean),
                                                _mean_dtype(mean), _ptr(factor),
                                                _factor_dtype(factor, factor_scale), _ptr(factor_scale),
                                                _ptr(basis), _sub_dim(basis), rank,
                                                nblk_capacity, top_k, window, n_sink, g, ng, _ptr(sel),
                                                _ptr(scores), _ptr(O), _ptr(lse), _paged(paged), _stream(stream)))


def bsattn_prefill_workspace_bytes(shape, n_global):
    return int(library().bsattn_prefill_workspace_bytes(ctypes.byref(shape), int(n_global)))


def bsattn_prefill(shape, Q, K, V, window_left, window_right, causal, global_pos, O, lse=None,
                   workspace=None, stream=None):
    g, ng = _globals(global_pos)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(library().bsattn_prefill(ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(V), window_left,
                                    window_right, int(bool(causal)), g, ng, _ptr(O), _ptr(lse),
                                    _ptr(workspace), ws_bytes, _stream(stream)))


def bsattn_prefill_dilated(shape, Q, K, V, window_left, window_right, causal, dilation, O, lse=None,
                           stream=None):
    _check(library().bsattn_prefill_dilated(ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(V), window_left,
                                            window_right, int(bool(causal)), int(dilation), _ptr(O), _ptr(lse),
                                            _stream(stream)))


def bsattn_probe_gather(shape, K, V, blocks, wg_per_pair, depth, checksum, stream=None):
    """Loads-only gather of the listed blocks' K/V rows (bandwidth ceiling; XOR per thread)."""
    _check(library().bsattn_probe_gather(ctypes.byref(shape), _ptr(K), _ptr(V), _ptr(blocks),
                                         int(blocks.shape[-1]), int(wg_per_pair), int(depth), _ptr(checksum),
                                         _stream(stream)))


def default_scale(head_dim):
    return 1.0 / math.sqrt(head_dim)
