"""The allocation-free decode step (bsattn_decode_step_noalloc) through the C ABI:
the same outputs as bsattn_decode_step with a caller workspace, bit for bit (the
same kernels), on two calls in a row, the second with a smaller problem (the
static scratch keeps the first call's partials; nothing may read them), plus the
size limit's error path."""

import numpy as np
import pytest

from synthetic import DecodeWorkload, make_decode_inputs

from gpu_util import to_dev

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


def _both(api, w, globals_=()):
    """The step through bsattn_decode_step (torch workspace) and through the
    allocation-free entry point, on the same inputs and summaries."""
    import torch
    B, Hq, Hkv, d, n = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_ctx
    nb = n // 64
    x = make_decode_inputs(w)
    Q, K, V = to_dev(x["Q"]), to_dev(x["K"]), to_dev(x["V"])
    shape = api.make_shape(B, Hq, Hkv, d, n)
    mean = torch.empty((B, Hkv, nb, d), dtype=torch.bfloat16, device="cuda")
    factor = torch.empty((B, Hkv, nb, w.rank, d), device="cuda") if w.rank else None
    api.bsattn_build_summaries(shape, K, w.rank, 0, nb, nb, mean, factor)
    out = []
    for noalloc in (False, True):
        sel = torch.full((B, Hkv, w.top_k), -7, dtype=torch.int32, device="cuda")
        scores = torch.full((B, Hkv, nb), float("nan"), device="cuda")
        O = torch.full((B, Hq, d), float("nan"), device="cuda")
        lse = torch.full((B, Hq), float("nan"), device="cuda")
        if noalloc:
            api.bsattn_decode_step_noalloc(shape, Q, K, V, mean, factor, w.rank, nb, w.top_k, w.window, w.n_sink,
                                           globals_, sel, scores, O, lse)
        else:
            ws = torch.full((api.bsattn_decode_workspace_bytes(shape, w.top_k, w.window, w.n_sink, len(globals_)),),
                            255, dtype=torch.uint8, device="cuda")
            api.bsattn_decode_step(shape, Q, K, V, mean, factor, w.rank, nb, w.top_k, w.window, w.n_sink, globals_,
                                   sel, scores, O, lse, ws)
        torch.cuda.synchronize()
        out.append(dict(sel=sel.cpu().numpy(), scores=scores.cpu().numpy(), O=O.cpu().numpy(),
                        lse=lse.cpu().numpy()))
    return out


def test_noalloc_step_equals_the_workspace_step_twice_in_a_row(api):
    # first a larger step (the fused in-wave top-k, 8 partials per pair) ...
    big = _w("noalloc_big", 4, 32, 8, 128, 300 * 64 + 17, 0, 16, 512, 64, 110)
    ref, got = _both(api, big, globals_=(5, 9000))
    for key in ("sel", "scores", "O", "lse"):
        assert np.array_equal(got[key], ref[key]), key
    assert np.isfinite(got["O"]).all()
    # ... then a smaller one (rank 2, the top-k kernel path, fewer partials)
    small = _w("noalloc_small", 1, 8, 2, 64, 700 * 64, 2, 5, 100, 16, 111)
    ref, got = _both(api, small)
    for key in ("sel", "scores", "O", "lse"):
        assert np.array_equal(got[key], ref[key]), key
    assert np.isfinite(got["O"]).all()


def test_noalloc_step_refuses_partials_past_the_scratch(api):
    """A problem whose split partials exceed the static scratch: BSATTN_ERR_WORKSPACE,
    raised by the binding, nothing launched."""
    import torch
    B, Hq, Hkv, d, n = 64, 1024, 64, 128, 4096 * 64
    shape = api.make_shape(B, Hq, Hkv, d, n)
    need = api.bsattn_decode_workspace_bytes(shape, 1024, 512, 64, 0)
    assert need > api.BSATTN_NOALLOC_SCRATCH_BYTES
    dummy = torch.empty(16, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError, match="static scratch"):
        api.bsattn_decode_step_noalloc(shape, dummy, dummy, dummy, dummy, None, 0, n // 64, 1024, 512, 64, (), dummy,
                                       dummy, dummy, dummy)
