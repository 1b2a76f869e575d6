"""CPU oracle for block-sparse, sliding-window and local+global attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import this package.  The GPU library
never imports it, and it never imports the GPU library: the two share no
code.  Everything here is plain numpy in float64, written to be read against
the source pages, not to be fast.

Sources (cited by title and section throughout):

* "COBS: Cumulant Order Block Sparse Attention", AI-written Japanese explainer
  at gist.science/ja/paper/2607.09052 (the "COBS explainer"), technical
  summary sections 2.1 (selection oracle), 2.2 (cumulant expansion),
  2.3 (COBS method), 4.3 (ablations), 5 (limitations).
* "LLMアテンション機構" (LLM attention mechanism), jisaku.com glossary (the
  "attention glossary"): "Self-Attentionの計算原理" (the four steps of scaled
  dot-product attention), the variants table, FAQ Q2 (GQA).
* "スライディングウィンドウアテンション" (sliding window attention), jisaku.com
  glossary (the "SWA glossary"): "概要と動作原理" (band matrix), "SWAの拡張
  手法" (global, sink, ...), "FlashAttentionとの組み合わせ".
* "ローカル・グローバルアテンション" (local-global attention), jisaku.com glossary
  (the "local-global glossary"): local window, global tokens and their
  placement, the graph view (2-hop reach).

Every function here has a pin in tests/ (closed forms, library routines,
brute force on tiny inputs, invariants); none is "parity unpinned".
"""

from .attention import (  # noqa: F401
    prefill_allowed,
    masked_attention_rows,
    prefill,
)
from .selector import (  # noqa: F401
    round_to_bf16,
    quantize_e2m1_rows,
    dequantize_e2m1_rows,
    E2M1_MAGNITUDES,
    query_subspace_basis,
    block_summaries,
    head_scores,
    exact_mass_scores,
    group_scores,
    forced_token_mask,
    candidate_blocks,
    top_k_blocks,
)
from .decode import (  # noqa: F401
    decode_token_set,
    sparse_decode_group,
    decode_step,
)
from .sparse_prefill import (  # noqa: F401
    TILE as SPARSE_PREFILL_TILE,
    tile_candidates,
    sparse_prefill_selection,
    sparse_prefill_allowed,
    sparse_prefill,
)
