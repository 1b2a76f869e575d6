"""Random draws and bfloat16 rounding for the synthetic inputs.

Draws come from numpy's ``Generator(PCG64(seed))``: float32 standard normals,
drawn chunk by chunk in C order from one sequential stream per workload.
bfloat16 values are produced by round-to-nearest-even of the float32 draw and
are kept as raw uint16 bit patterns, so the GPU and the oracle read identical
bits.
"""

from __future__ import annotations

import hashlib

import numpy as np

CHUNK = 1 << 22


def bf16_bits(x):
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    nan = np.isnan(x)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    if nan.any():
        r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def bf16_bits_to_f32(bits):
    """Exact float32 value of bfloat16 bit patterns."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def normal_f32(rng, shape, scale=1.0, out_bf16=False, chunk=CHUNK):
    """float32 N(0, 1) draws times ``scale``, filled chunk-wise in C order.

    With ``out_bf16`` the result is the uint16 bfloat16 pattern of each scaled draw.
    """
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if out_bf16 else np.float32)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        x = rng.standard_normal(e - s, dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        out[s:e] = bf16_bits(x) if out_bf16 else x
    return out.reshape(shape)


def sha256_hex(arr):
    """SHA-256 of an array's raw bytes (C order), to record exactly which inputs ran."""
    return hashlib.sha256(np.ascontiguousarray(arr).tobytes()).hexdigest()


def orthonormal_rows(rng, n_sets, s, d):
    """``n_sets`` stacks of ``s`` orthonormal rows in R^d, float32 [n_sets, s, d]: the Q
    factor of a Gaussian d x s matrix's QR decomposition, transposed (a random frame)."""
    out = np.empty((n_sets, s, d), dtype=np.float32)
    for i in range(n_sets):
        q, _ = np.linalg.qr(rng.standard_normal((d, s)))
        out[i] = q.T
    return out
