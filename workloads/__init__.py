"""Seeded synthetic inputs for the decode-step sparse-attention path.

This package is shared by the CPU oracle (``oracle/``), the tests and the
benchmark. It only *draws* inputs: random queries, paged K/V pools, page
tables, hot blocks, indexer keys. It holds none of the method's arithmetic
(no summaries, scores, selection or attention), so neither side of a parity
check can borrow the other's computation through it.
"""

from .configs import (  # noqa: F401
    BlockTopKConfig,
    IndexerConfig,
    CoarseToFineConfig,
    PqConfig,
    PQ32_128K,
    TINY_4K,
    LLAMA8B_32K_B16,
    RAGGED_B64,
    INDEXER_128K,
    COARSE_TO_FINE_950K,
    reduced,
)
from .generate import (  # noqa: F401
    BlockTopKInputs,
    make_block_topk_inputs,
    IndexerInputs,
    make_indexer_inputs,
    indexer_queries,
    pq_init_tokens,
    bf16_bits,
    fp8_bits,
)
