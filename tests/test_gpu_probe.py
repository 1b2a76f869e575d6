"""GPU check of the gather probe (the loads-only bandwidth ceiling bench.py sets
beside the sparse decode's gather): it must read exactly the listed blocks' K and V
words, each once.  The XOR of every thread's checksum equals the XOR of those
words computed by numpy on the host; a block outside the cache is read clamped into
it.  No oracle is involved: the probe computes nothing of the method."""

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


def _host_xor(x, blocks, cap):
    """XOR of every 32-bit word of the listed blocks' K and V rows (clamped as the probe does)."""
    acc = np.uint32(0)
    nbc = cap // 64
    for p in range(blocks.shape[0]):
        b, g = divmod(p, x["K"].shape[1])
        for j in blocks[p]:
            j = min(max(int(j), 0), nbc - 1)
            for t in ("K", "V"):
                rows = np.ascontiguousarray(x[t][b, g, 64 * j:64 * (j + 1)])
                acc ^= np.bitwise_xor.reduce(rows.view(np.uint32).ravel())
    return acc


@pytest.mark.parametrize("d,wg,depth,nb", [(128, 2, 2, 25), (128, 1, 4, 7), (64, 3, 3, 11), (64, 16, 1, 5)])
def test_probe_reads_every_listed_word_once(api, d, wg, depth, nb):
    import torch
    w = DecodeWorkload(name="probe", batch=2, n_q_heads=4, n_kv_heads=2, head_dim=d, n_ctx=2048, block_size=64,
                       rank=0, top_k=4, window=64, n_sink=0, dtype="bf16", seed=11)
    x = make_decode_inputs(w)
    rng = np.random.default_rng(d + wg + depth)
    pairs = w.batch * w.n_kv_heads
    blocks = np.stack([rng.choice(2048 // 64, size=nb, replace=False) for _ in range(pairs)]).astype(np.int32)
    if nb >= 7:
        blocks[0, 1] = -3          # clamped to block 0
        blocks[1, 2] = 10_000      # clamped to the last block
    print(f"[probe] d={d} wg_per_pair={wg} depth={depth} blocks={nb}", flush=True)
    shape = api.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, d, 2048, dtype="bf16")
    out = torch.full((pairs * wg * 256,), 0xA5A5A5A5 - 2**32, dtype=torch.int32, device="cuda")
    api.bsattn_probe_gather(shape, to_dev(x["K"]), to_dev(x["V"]), torch.from_numpy(blocks).cuda(), wg, depth,
                            out)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert got == _host_xor(x, blocks, 2048)
