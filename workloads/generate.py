"""Seeded generators for the synthetic decode-step inputs.

Small index structures (sequence lengths, page tables, hot-block choices,
queries, head weights) are always drawn on the CPU from a CPU generator, so
they do not depend on the device. The large pools (paged K/V, latent KV,
indexer keys) are drawn on the requested device; the same seed therefore
gives the same tables everywhere but device-dependent pool values. Parity
checks always hand the *same* tensors to both sides, so this never matters
for correctness; it only keeps full-size generation on the GPU fast.

Nothing here computes any part of the method itself.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np
import torch

from .configs import BlockTopKConfig, IndexerConfig, CoarseToFineConfig

BF16_NAN_BITS = 0x7FC0


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bf16 bit patterns of a torch bfloat16 tensor as numpy uint16."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def fp8_bits(t: torch.Tensor) -> np.ndarray:
    """Raw OCP e4m3fn bit patterns of a torch float8 tensor as numpy uint8."""
    assert t.dtype == torch.float8_e4m3fn
    return t.detach().cpu().contiguous().view(torch.uint8).numpy()


def _cpu_gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _dev_gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn_bf16(shape, gen, device) -> torch.Tensor:
    """N(0,1) samples rounded to bf16, drawn in chunks to bound temporaries."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    chunk = 1 << 26
    for s in range(0, flat.numel(), chunk):
        e = min(flat.numel(), s + chunk)
        flat[s:e] = torch.randn(e - s, generator=gen, device=device,
                                dtype=torch.float32).to(torch.bfloat16)
    return out


# --------------------------------------------------------------------------
# Block top-k workloads (GQA, block-mean summaries)
# --------------------------------------------------------------------------

@dataclass
class BlockTopKInputs:
    cfg: BlockTopKConfig
    q: torch.Tensor              # [B][Hq][D] bf16 (on device)
    k_pool: torch.Tensor         # [num_pages][Hkv][P][D] bf16
    v_pool: torch.Tensor         # [num_pages][Hkv][P][D] bf16
    page_indptr: torch.Tensor    # [B+1] int32
    page_indices: torch.Tensor   # [nnz] int32, physical page ids in logical order
    seq_lens: torch.Tensor       # [B] int32, tokens cached (current one included)
    topk: int                    # k blocks chosen by score (forced excluded); -1: keep ratio
    hot_blocks: Dict = field(default_factory=dict)  # (r, g) -> list of logical blocks
    unused_pages: Optional[torch.Tensor] = None     # int64 page ids no request uses

    @property
    def num_pages(self) -> int:
        return int(self.k_pool.shape[0])

    def max_blocks(self) -> int:
        P = self.cfg.page_size
        return int(max((int(L) + P - 1) // P for L in self.seq_lens.tolist()))

    def to(self, device) -> "BlockTopKInputs":
        mv = lambda t: None if t is None else t.to(device)
        return BlockTopKInputs(self.cfg, mv(self.q), mv(self.k_pool), mv(self.v_pool),
                               mv(self.page_indptr), mv(self.page_indices),
                               mv(self.seq_lens), self.topk, dict(self.hot_blocks),
                               mv(self.unused_pages))


def _seq_lens(cfg: BlockTopKConfig, gen: torch.Generator) -> List[int]:
    if cfg.ragged_range is None:
        return [cfg.context] * cfg.batch
    lo, hi = cfg.ragged_range
    u = torch.rand(cfg.batch, generator=gen, dtype=torch.float64)
    lens = torch.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))
    return [int(min(hi, max(lo, round(float(x))))) for x in lens]


def make_block_topk_inputs(cfg: BlockTopKConfig, device="cpu", seed: Optional[int] = None,
                           poison_unused: bool = False,
                           seq_lens: Optional[List[int]] = None) -> BlockTopKInputs:
    """Draw one decode step's inputs for a block top-k workload.

    Random sub-streams, in order: sequence lengths, q (CPU), page table (CPU),
    hot blocks (CPU), K pool, V pool (device).
    """
    seed = cfg.seed if seed is None else seed
    cg = _cpu_gen(seed)
    B, Hq, Hkv, D, P = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.page_size
    G = Hq // Hkv
    lens = list(seq_lens) if seq_lens is not None else _seq_lens(cfg, cg)
    assert len(lens) == B
    nbs = [(L + P - 1) // P for L in lens]
    used = sum(nbs)

    q_cpu = torch.randn(B, Hq, D, generator=cg, dtype=torch.float32).to(torch.bfloat16)

    # page table
    if cfg.page_table == "contiguous":
        num_pages = used
        phys = torch.arange(used, dtype=torch.int64)
    elif cfg.page_table == "permuted":
        num_pages = used
        phys = torch.randperm(used, generator=cg)
    elif cfg.page_table == "pool":
        num_pages = max(used, math.ceil(used / cfg.pool_occupancy))
        phys = torch.randperm(num_pages, generator=cg)[:used]
    else:
        raise ValueError(cfg.page_table)
    indptr = [0]
    for nb in nbs:
        indptr.append(indptr[-1] + nb)
    page_indptr = torch.tensor(indptr, dtype=torch.int32)
    page_indices = phys.to(torch.int32)

    # hot blocks per (r, g), drawn among complete blocks outside the forced set
    hot: Dict = {}
    for r in range(B):
        nb, L = nbs[r], lens[r]
        n_complete = L // P
        lo = min(cfg.n_sink, nb)
        hi = min(n_complete, max(0, nb - cfg.n_recent))
        cands = list(range(lo, hi))
        if cfg.n_hot is not None:
            nh = cfg.n_hot
        elif cfg.hot_fraction:
            nh = int(round(cfg.hot_fraction * nb))
        else:
            nh = 0
        nh = min(nh, len(cands))
        for g in range(Hkv):
            if nh == 0:
                hot[(r, g)] = []
                continue
            pick = torch.randperm(len(cands), generator=cg)[:nh]
            hot[(r, g)] = sorted(cands[i] for i in pick.tolist())

    dg = _dev_gen(seed + 7919, device)
    k_pool = _randn_bf16((num_pages, Hkv, P, D), dg, device)
    v_pool = _randn_bf16((num_pages, Hkv, P, D), dg, device)

    # Move the keys of each hot block toward its group's query direction by
    # hot_shift_sigma standard deviations (the pool is N(0,1)).
    if any(len(v) for v in hot.values()):
        qf = q_cpu.float().view(B, Hkv, G, D).sum(dim=2)           # [B][Hkv][D]
        u = qf / qf.norm(dim=-1, keepdim=True).clamp_min(1e-30)
        pages, heads, shifts = [], [], []
        for (r, g), blocks in hot.items():
            for b in blocks:
                pages.append(int(page_indices[indptr[r] + b]))
                heads.append(g)
                shifts.append(u[r, g])
        pages_t = torch.tensor(pages, dtype=torch.int64, device=device)
        heads_t = torch.tensor(heads, dtype=torch.int64, device=device)
        shift = (cfg.hot_shift_sigma * torch.stack(shifts)).to(device)  # [n][D]
        blk = k_pool[pages_t, heads_t].float()                          # [n][P][D]
        k_pool[pages_t, heads_t] = (blk + shift[:, None, :]).to(torch.bfloat16)

    unused = None
    if num_pages > used:
        mask = torch.ones(num_pages, dtype=torch.bool)
        mask[phys] = False
        unused = torch.nonzero(mask).flatten()
        if poison_unused:
            ud = unused.to(device)
            nan = torch.tensor(BF16_NAN_BITS, dtype=torch.int16).view(torch.bfloat16).item()
            k_pool[ud] = nan
            v_pool[ud] = nan

    topk = cfg.topk   # -1: the keep ratio decides k per request (the oracle's rule)
    return BlockTopKInputs(cfg, q_cpu.to(device), k_pool, v_pool,
                           page_indptr.to(device), page_indices.to(device),
                           torch.tensor(lens, dtype=torch.int32).to(device),
                           topk, hot, unused)


# --------------------------------------------------------------------------
# Learned-indexer workloads (fp8 indexer keys, MLA latent KV)
# --------------------------------------------------------------------------

@dataclass
class IndexerInputs:
    cfg: IndexerConfig
    q_idx: torch.Tensor          # [B][Hi][Di] bf16
    head_w: torch.Tensor         # [B][Hi] fp32
    idx_keys: torch.Tensor       # [idx_pages][P][Di] float8_e4m3fn
    idx_scale: torch.Tensor      # [idx_pages][P] fp32 (per-token dequant scale)
    idx_indptr: torch.Tensor     # [B+1] int32
    idx_indices: torch.Tensor    # int32 physical indexer pages
    q_mla: torch.Tensor          # [B][Hm][576] bf16
    latent: torch.Tensor         # [kv_pages][P][576] bf16
    kv_indptr: torch.Tensor      # [B+1] int32
    kv_indices: torch.Tensor     # int32 physical latent pages
    seq_lens: torch.Tensor       # [B] int32


def _clustered(n_tok: int, dim: int, n_clusters: int, sigma: float, dg, device):
    """Keys around `n_clusters` N(0, I) centroids with N(0, sigma^2 I) spread."""
    cent = torch.randn(n_clusters, dim, generator=dg, device=device)
    out = torch.empty(n_tok, dim, device=device, dtype=torch.float32)
    chunk = 1 << 20
    for s in range(0, n_tok, chunk):
        e = min(n_tok, s + chunk)
        c = torch.randint(0, n_clusters, (e - s,), generator=dg, device=device)
        out[s:e] = cent[c] + sigma * torch.randn(e - s, dim, generator=dg, device=device)
    return out


def _indexer_queries(cfg: IndexerConfig, cg: torch.Generator):
    """Indexer queries (bf16), head weights (N(0,1)/sqrt(H), fp32) and MLA
    queries (bf16), drawn in that order from the CPU generator."""
    B = cfg.batch
    q_idx = torch.randn(B, cfg.index_heads, cfg.index_dim, generator=cg).to(torch.bfloat16)
    head_w = (torch.randn(B, cfg.index_heads, generator=cg) / math.sqrt(cfg.index_heads)).float()
    q_mla = torch.randn(B, cfg.mla_heads, cfg.kv_lora_dim + cfg.rope_dim,
                        generator=cg).to(torch.bfloat16)
    return q_idx, head_w, q_mla


def indexer_queries(cfg: IndexerConfig, seed: int, device="cpu"):
    """Another set of (q_idx, head_w, q_mla) for the same cache: the first
    draws of make_indexer_inputs(cfg, seed=seed)."""
    q_idx, head_w, q_mla = _indexer_queries(cfg, _cpu_gen(seed))
    return q_idx.to(device), head_w.to(device), q_mla.to(device)


def make_indexer_inputs(cfg: IndexerConfig, device="cpu", seed: Optional[int] = None) -> IndexerInputs:
    seed = cfg.seed if seed is None else seed
    cg = _cpu_gen(seed)
    B, P, L = cfg.batch, cfg.page_size, cfg.context
    nb = (L + P - 1) // P
    used = B * nb
    q_idx, head_w, q_mla = _indexer_queries(cfg, cg)
    idx_perm = torch.randperm(used, generator=cg).to(torch.int32)
    kv_perm = torch.randperm(used, generator=cg).to(torch.int32)
    indptr = torch.arange(0, used + 1, nb, dtype=torch.int32)

    dg = _dev_gen(seed + 104729, device)
    keys = _clustered(used * P, cfg.index_dim, cfg.n_clusters, cfg.cluster_sigma, dg, device)
    amax = keys.abs().amax(dim=-1).clamp_min(1e-12)
    scale = (amax / 448.0).float()
    k8 = (keys / scale[:, None]).to(torch.float8_e4m3fn)
    del keys
    lat = _clustered(used * P, cfg.kv_lora_dim + cfg.rope_dim, cfg.n_clusters,
                     cfg.cluster_sigma, dg, device).to(torch.bfloat16)
    return IndexerInputs(
        cfg, q_idx.to(device), head_w.to(device),
        k8.view(used, P, cfg.index_dim), scale.view(used, P),
        indptr.to(device), idx_perm.to(device),
        q_mla.to(device), lat.view(used, P, -1), indptr.clone().to(device),
        kv_perm.to(device), torch.full((B,), L, dtype=torch.int32).to(device))


def pq_init_tokens(n_tokens: int, seed: int, k: int = 256) -> torch.Tensor:
    """k distinct token indices in [0, n_tokens) (seeded): the k-means
    starting points, drawn here so both sides take the same ones."""
    g = _cpu_gen(seed)
    if n_tokens >= k:
        return torch.randperm(n_tokens, generator=g)[:k].to(torch.int32)
    return torch.randint(0, n_tokens, (k,), generator=g).to(torch.int32)
