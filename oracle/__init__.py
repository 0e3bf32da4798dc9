"""CPU oracle for the decode-step query-aware sparse-attention path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute this package; only the tests, the package smoke check and the
benchmark's CPU-baseline leg use it.

It is a plain, slow, float64 NumPy implementation of what the method computes,
written from the pages:

* Vortex (CMU CSD PhD blog post, "Vortex"): block top-k attention,
  block-mean summaries, GQA-grouped block scoring, paged KV layout
  ("Why Long Generations Are Expensive", Fig. 1 and its equation;
  "Writing an algorithm: vFlow"; "Why New Ideas Are Hard to Deploy", Fig. 2).
* LeanSparse ("LeanSparse: Memory-Efficient Serving for Native
  Sparse-Attention LLMs"): the learned indexer's weighted-ReLU head
  aggregation (§5, Eq. 6) and coarse-to-fine candidate refinement (§5).
* LeanSparse §5, "Approximate scoring with PQ": PQ32 codes, k-means
  codebooks, coarse scores with centroids and exact refinement (pq.py).
* ByteCross ("Where Activation Sparsity and KV-Cache Sparsity Cross in LLM
  Decoding"): merging attention over disjoint token sets by log-sum-exp
  (App. A) and the byte account of a decode step (§3.1, Eq. 1-4).

It shares no code with the HIP library and imports nothing from it. Its own
bit-level decoders turn bf16 / fp8-e4m3fn storage into exact float64 values;
results are rounded once, round-to-nearest-even, to the output dtype.

Parity status per function is listed in each module's header; every function
here is pinned by tests under ``tests/`` against values that do not come from
the oracle itself (brute force, exact rationals, closed forms, the pages'
worked example), except where a header says "parity unpinned".
"""

from . import method, numerics, pq  # noqa: F401
from .numerics import (  # noqa: F401
    bf16_to_f64, fp8e4m3fn_to_f64, f64_to_bf16_bits, f64_to_f32, fraction_to_bf16_bits,
)
from .method import (  # noqa: F401
    BatchView, block_summaries, block_scores, select_blocks, select_blocks_batch,
    attention_over_tokens, sparse_attention, dense_attention, lse_merge,
    indexer_token_scores, select_tokens, mla_attention, decode_step,
    tokens_of_blocks, topk_from_keep_ratio, forced_blocks, indexer_block_scores,
    coarse_to_fine_select, block_bounds, bound_scores, approx_select_tokens, remap_bucket,
    window_tokens, window_attention, snapkv_scores, snapkv_select,
)
