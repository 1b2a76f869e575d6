"""Seeded synthetic inputs shared by the oracle checks, the GPU tests and the benchmark.

This package draws random tensors and rounds them to the storage dtype.  It
holds none of the attention method's arithmetic: no scores, no summaries, no
softmax.  Both the CPU oracle and the GPU path consume exactly the bits it
produces.
"""

from .generators import (  # noqa: F401
    bf16_bits,
    bf16_bits_to_f32,
    normal_f32,
    orthonormal_rows,
    sha256_hex,
)
from .workloads import (  # noqa: F401
    DecodeWorkload,
    PrefillWorkload,
    WORKLOADS,
    make_decode_inputs,
    make_prefill_inputs,
)
