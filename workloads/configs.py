"""The five synthetic decode-step workloads, as plain data.

Context lengths follow the ByteCross paper's convention ("Where Activation
Sparsity and KV-Cache Sparsity Cross in LLM Decoding", §3): K means 1,024
tokens, so 32K = 32,768 and 950K = 972,800.

Block size equals page size (16 tokens for the block top-k workloads, as in
the Vortex post's default of 16-token blocks, "Is it actually fast?").
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional, Tuple


@dataclass(frozen=True)
class BlockTopKConfig:
    """Block top-k over block-mean key summaries of a paged GQA KV cache."""

    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    # Every request holds `context` tokens, unless `ragged_range` is set, in
    # which case lengths are drawn log-uniformly in [lo, hi].
    context: int
    ragged_range: Optional[Tuple[int, int]] = None
    # k blocks chosen by score on top of the forced ones; -1 => from keep_ratio
    topk: int = 64
    keep_ratio: Optional[float] = None
    n_sink: int = 1
    n_recent: int = 2
    # "contiguous": request r owns pages [r*nb, (r+1)*nb) in order.
    # "permuted": one seeded permutation of exactly the used pages.
    # "pool": pages scattered in a larger shared pool (pool_occupancy used).
    page_table: str = "permuted"
    pool_occupancy: float = 1.0
    # Hot blocks per (request, kv-head): keys moved toward the group's query.
    n_hot: Optional[int] = None
    hot_fraction: Optional[float] = None
    hot_shift_sigma: float = 2.0
    group_agg: str = "max"
    out_dtype: str = "bf16"
    seed: int = 1000

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


@dataclass(frozen=True)
class IndexerConfig:
    """Learned-indexer token selection + sparse MLA attention."""

    name: str
    batch: int
    context: int
    index_heads: int = 64
    index_dim: int = 128
    page_size: int = 64
    topk_tokens: int = 2048
    mla_heads: int = 128
    kv_lora_dim: int = 512
    rope_dim: int = 64
    n_clusters: int = 16
    cluster_sigma: float = 0.5
    seed: int = 1003


@dataclass(frozen=True)
class CoarseToFineConfig(IndexerConfig):
    """Coarse block-mean indexer scores -> candidate blocks -> exact token top-k."""

    coarse_block: int = 64
    coarse_topk_blocks: int = 256
    seed: int = 1004


@dataclass(frozen=True)
class PqConfig(IndexerConfig):
    """PQ32 coarse scores -> top-C candidate tokens -> exact rerank -> top-k."""

    n_candidates: int = 2048
    kmeans_iters: int = 8
    seed: int = 1005


# Tiny single-request step: 1 layer, 8 q heads / 2 kv heads, d 64, 4K context,
# contiguous page table, 8 hot blocks, top-16 + block 0 + last block, fp32 out.
TINY_4K = BlockTopKConfig(
    name="tiny_4k_b1_h8kv2_d64",
    batch=1, num_q_heads=8, num_kv_heads=2, head_dim=64, page_size=16,
    context=4096, topk=16, n_sink=1, n_recent=1, page_table="contiguous",
    n_hot=8, out_dtype="fp32", seed=1001,
)

# Llama-3-8B-shaped decode attention: 16 requests x 32K, 32 q / 8 kv heads,
# d 128, permuted page table, 2% hot blocks, top-64 + 1 sink + 2 recent.
LLAMA8B_32K_B16 = BlockTopKConfig(
    name="llama8b_32k_b16_top64",
    batch=16, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
    context=32768, topk=64, n_sink=1, n_recent=2, page_table="permuted",
    hot_fraction=0.02, out_dtype="bf16", seed=1002,
)

# Ragged batch: 64 requests, lengths log-uniform in [2K, 128K], shared pool at
# 70% occupancy; the keep ratio is chosen per run (1/64, 1/16, 1/4, or 1.0).
RAGGED_B64 = BlockTopKConfig(
    name="ragged_b64_2k_128k",
    batch=64, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
    context=0, ragged_range=(2048, 131072), topk=-1, keep_ratio=1.0 / 16,
    n_sink=1, n_recent=2, page_table="pool", pool_occupancy=0.7,
    hot_fraction=0.02, out_dtype="bf16", seed=1003,
)

INDEXER_128K = IndexerConfig(name="indexer_fp8_128k_b8_top2048", batch=8,
                             context=131072)

COARSE_TO_FINE_950K = CoarseToFineConfig(
    name="coarse_to_fine_950k_b4", batch=4, context=972800)


# PQ32 coarse-to-fine indexing: 8 requests x 128K tokens in 64-token pages,
# 64 indexer heads x 128, codebooks trained on the cache, C = 2,048
# candidates, top-512 tokens after the exact rerank.
PQ32_128K = PqConfig(name="pq32_128k_b8_c2048_top512", batch=8, context=131072,
                     topk_tokens=512)


def reduced(cfg, **changes):
    """A copy of `cfg` with some fields replaced (smaller parity-test shapes)."""
    name = changes.pop("name", None) or (cfg.name + "_reduced")
    return dataclasses.replace(cfg, name=name, **changes)
