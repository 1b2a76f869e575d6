"""The seeded input generators: reproducible, and bfloat16 rounding equal to torch's."""

import numpy as np
import torch

from synthetic import (WORKLOADS, bf16_bits, bf16_bits_to_f32, make_decode_inputs,
                       make_prefill_inputs, normal_f32, sha256_hex)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 3,
                        np.array([0.0, -0.0, np.inf, -np.inf, 1e-40, 3.3895314e38], np.float32)])
    ours = bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_draws_are_reproducible_and_chunk_independent():
    a = normal_f32(np.random.Generator(np.random.PCG64(5)), (3, 1000), chunk=64)
    b = normal_f32(np.random.Generator(np.random.PCG64(5)), (3, 1000), chunk=1 << 20)
    np.testing.assert_array_equal(a, b)
    assert sha256_hex(a) == sha256_hex(b)


def test_small_workload_shapes_and_determinism():
    w = WORKLOADS["cobs_decode_128k"].scaled(batch=1, n_ctx=4096, n_kv_heads=2, n_q_heads=4)
    x1, x2 = make_decode_inputs(w), make_decode_inputs(w)
    assert x1["K"].dtype == np.uint16 and x1["K"].shape == (1, 2, 4096, 128)
    assert sha256_hex(x1["K"]) == sha256_hex(x2["K"])
    assert len(x1["needles"]) == 1 and len(set(x1["needles"][0].tolist())) == 4
    assert all(1 <= b < (4096 - 1024) // 64 for b in x1["needles"][0])
    p = WORKLOADS["swa_prefill_8k"].scaled(seq_len=256, n_q_heads=4, n_kv_heads=2)
    y = make_prefill_inputs(p)
    assert y["Q"].shape == (1, 4, 256, 128) and y["K"].shape == (1, 2, 256, 128)
    assert np.abs(bf16_bits_to_f32(y["K"])).max() < 4  # N(0,1) * 0.5
