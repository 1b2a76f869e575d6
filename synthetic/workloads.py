"""The five synthetic workloads and their seeded input recipes.

Shapes follow the workloads the pages talk about: a tiny decode case, a
Mistral-shaped causal sliding-window prefill (w = 4096, GQA 32:8), a
Longformer-shaped local+global prefill (+-256 window, 16 global tokens), and
32K / 128K block-sparse decode with a first-order and a second-order (COBS)
selector.  No public dataset is involved: every tensor is a seeded draw.

Recipe (all draws from one ``Generator(PCG64(seed))`` per workload):

* decode: Q [B, Hq, d], then K [B, Hkv, n, d], then V [B, Hkv, n, d];
  N(0, 1) float32, rounded to bfloat16 unless the workload is float32.
* prefill: Q [B, Hq, N, d], then K, then V [B, Hkv, N, d]; N(0, 1) times
  ``input_scale``, rounded to bfloat16.
* "needle" blocks (decode workloads that ask for them), drawn after V.  For
  each sequence b, ``n_needles`` distinct blocks are chosen uniformly among the
  complete blocks that lie wholly after the sink tokens and wholly before the
  window (``rng.choice`` without replacement).  For each K/V head g the query
  direction is q_dir = normalise(sum of the group's query vectors), in
  float64 from the rounded queries.  For each needle block, in the order drawn:
    - "shifted": z ~ N(0, I) [S, d] and xi ~ N(0, 1) [S]; the keys are
      z - (z.q_dir) q_dir + (0.3 + 1.5 xi) q_dir: N(0.3, 1.5^2) along q_dir and
      N(0, 1) across it.
    - "spread": a unit direction u = normalise(rho q_dir + sqrt(1-rho^2) r),
      r a random unit vector orthogonal to q_dir (from one N(0, I) draw),
      rho = 0.8; z ~ N(0, I) [S, d]; the keys are z + 2 (z.u) u: mean 0 like the
      background, standard deviation 3 along u.
  The keys are rounded to bfloat16 and written over the block for every K/V
  head (same blocks for all heads); V is left as drawn.
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field

import numpy as np

from .generators import bf16_bits, normal_f32


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_ctx: int
    block_size: int
    rank: int
    top_k: int
    window: int
    n_sink: int
    dtype: str  # "f32" or "bf16"
    seed: int
    needle: str = "none"  # "none", "shifted" or "spread"
    n_needles: int = 4
    global_pos: tuple = ()
    sub_dim: int = 0  # query-subspace dimension of the factor rows (0: none)

    def scaled(self, **kw):
        return dataclasses.replace(self, **kw)


@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    seq_len: int
    window_left: int
    window_right: int
    causal: bool
    seed: int
    input_scale: float = 1.0
    global_pos: tuple = field(default_factory=tuple)
    top_k: int = 0   # block-sparse prefill: blocks selected per 128-row query tile (0: none)
    n_sink: int = 0
    dilation: int = 1  # dilated window: every dilation-th key counted from the query

    def scaled(self, **kw):
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny_decode_1k": DecodeWorkload(
        name="tiny_decode_1k", batch=1, n_q_heads=4, n_kv_heads=1, head_dim=64, n_ctx=1024,
        block_size=64, rank=0, top_k=4, window=64, n_sink=64, dtype="f32", seed=0),
    "swa_prefill_8k": PrefillWorkload(
        name="swa_prefill_8k", batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128, seq_len=8192,
        window_left=4095, window_right=0, causal=True, seed=1, input_scale=0.5),
    "local_global_prefill_16k": PrefillWorkload(
        name="local_global_prefill_16k", batch=2, n_q_heads=12, n_kv_heads=12, head_dim=64,
        seq_len=16384, window_left=256, window_right=256, causal=False, seed=2,
        global_pos=tuple(range(0, 16384, 1024))),
    "sparse_prefill_8k": PrefillWorkload(
        name="sparse_prefill_8k", batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128, seq_len=8192,
        window_left=1023, window_right=0, causal=True, seed=5, input_scale=0.5, top_k=16, n_sink=64),
    "first_order_decode_32k": DecodeWorkload(
        name="first_order_decode_32k", batch=16, n_q_heads=32, n_kv_heads=8, head_dim=128,
        n_ctx=32768, block_size=64, rank=0, top_k=16, window=512, n_sink=64, dtype="bf16",
        seed=3, needle="shifted"),
    "cobs_decode_128k": DecodeWorkload(
        name="cobs_decode_128k", batch=4, n_q_heads=64, n_kv_heads=8, head_dim=128,
        n_ctx=131072, block_size=64, rank=4, top_k=32, window=1024, n_sink=64, dtype="bf16",
        seed=4, needle="spread", sub_dim=96),
}


def _unit(x):
    return x / np.linalg.norm(x)


def _to_f32(bits_or_f32):
    a = np.asarray(bits_or_f32)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a.astype(np.float32)


def make_decode_inputs(w: DecodeWorkload, kv_capacity=None):
    """Q [B,Hq,d], K, V [B,Hkv,cap,d] as float32 (dtype f32) or uint16 bfloat16 bits.

    ``kv_capacity`` >= n_ctx pads the token axis (padding drawn after everything else
    is never read by the method; it is filled with zeros).  Returns a dict with the
    tensors and the needle block positions per sequence.
    """
    rng = np.random.Generator(np.random.PCG64(w.seed))
    bf = w.dtype == "bf16"
    B, Hq, Hkv, d, n, S = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_ctx, w.block_size
    Q = normal_f32(rng, (B, Hq, d), out_bf16=bf)
    K = normal_f32(rng, (B, Hkv, n, d), out_bf16=bf)
    V = normal_f32(rng, (B, Hkv, n, d), out_bf16=bf)
    needles = []
    if w.needle != "none":
        G = Hq // Hkv
        lo = -(-w.n_sink // S)
        hi = (n - w.window) // S
        pool = np.arange(lo, hi)
        qf = _to_f32(Q).astype(np.float64)
        for b in range(B):
            blocks = rng.choice(pool, size=w.n_needles, replace=False)
            needles.append(blocks)
            for g in range(Hkv):
                q_dir = _unit(qf[b, g * G:(g + 1) * G].sum(axis=0))
                for blk in blocks:
                    if w.needle == "shifted":
                        z = rng.standard_normal((S, d))
                        xi = rng.standard_normal(S)
                        keys = z - np.outer(z @ q_dir, q_dir) + np.outer(0.3 + 1.5 * xi, q_dir)
                    elif w.needle == "spread":
                        r = rng.standard_normal(d)
                        r = _unit(r - (r @ q_dir) * q_dir)
                        u = _unit(0.8 * q_dir + np.sqrt(1.0 - 0.8 ** 2) * r)
                        z = rng.standard_normal((S, d))
                        keys = z + 2.0 * np.outer(z @ u, u)
                    else:
                        raise ValueError(f"unknown needle kind {w.needle}")
                    keys = keys.astype(np.float32)
                    K[b, g, blk * S:(blk + 1) * S] = bf16_bits(keys) if bf else keys
    if kv_capacity is not None and kv_capacity > n:
        pad = ((0, 0), (0, 0), (0, kv_capacity - n), (0, 0))
        K = np.pad(K, pad)
        V = np.pad(V, pad)
    return dict(Q=Q, K=K, V=V, needles=needles)


def make_prefill_inputs(w: PrefillWorkload):
    """Q [B,Hq,N,d], K, V [B,Hkv,N,d] as uint16 bfloat16 bits."""
    rng = np.random.Generator(np.random.PCG64(w.seed))
    B, Hq, Hkv, N, d = w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len, w.head_dim
    Q = normal_f32(rng, (B, Hq, N, d), scale=w.input_scale, out_bf16=True)
    K = normal_f32(rng, (B, Hkv, N, d), scale=w.input_scale, out_bf16=True)
    V = normal_f32(rng, (B, Hkv, N, d), scale=w.input_scale, out_bf16=True)
    return dict(Q=Q, K=K, V=V)
