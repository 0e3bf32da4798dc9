"""The method, step by step, in float64 (oracle; TEST INFRASTRUCTURE ONLY).

Notation follows the Vortex post ("Why Long Generations Are Expensive"):
blocks j of b consecutive tokens, mean key k̄_j, score s_j = q · k̄_j,
I = top-k_j(s_j), o = softmax(q K_I^T / sqrt(d)) V_I. Block = page here
(the paged layout of "Why New Ideas Are Hard to Deploy", Fig. 2): logical
block j of request r is physical page page_indices[page_indptr[r] + j], and
summaries are stored per physical page, as the post's vTensor section says
named cache entries live in pages of the KV allocator.

Readings where the pages leave a step open (each also listed in the design
notes of the repository):
* GQA: query head h belongs to kv head g = h // (Hq / Hkv). The group score
  is aggregated over the group's query heads (the vFlow listing reduces the
  score over the head axis); one selection per (request, kv head) is shared by
  its group. Aggregator: max (default) or mean.
* Block scores are unscaled dot products; the softmax uses sm_scale.
* Forced blocks: the first n_sink blocks and the last n_recent blocks, plus
  the last block whenever it is partial (only full blocks have summaries: they
  are built "when a block fills up"). Forced blocks are not ranked; k more are
  chosen from the other complete blocks.
* Ranking is by (score descending, block index ascending): ties go to the
  lowest index. The result is emitted in ascending block order.
* The cache holds L tokens including the current one; attention covers tokens
  t < L of the selected blocks.

Parity status: every function below is pinned by tests/test_oracle_method.py
against brute force, exact rationals, closed forms, softmax invariants or the
post's Fig. 1 example; none is "parity unpinned".
"""

from __future__ import annotations

from dataclasses import dataclass
from fractions import Fraction
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

from .numerics import (
    bf16_to_f64, fp8e4m3fn_to_f64, f64_to_bf16_bits, f64_to_f32,
    fraction_to_bf16_bits, fraction_to_f32, sum_is_exact_in_f64,
)


# --------------------------------------------------------------------------
# Paged batch view (vTensor-style: batch size, index pointer, page list)
# --------------------------------------------------------------------------

@dataclass
class BatchView:
    page_indptr: np.ndarray    # [B+1]
    page_indices: np.ndarray   # [nnz] physical page ids, logical order
    seq_lens: np.ndarray       # [B] tokens in cache (current one included)
    page_size: int

    def __post_init__(self):
        self.page_indptr = np.asarray(self.page_indptr, dtype=np.int64)
        self.page_indices = np.asarray(self.page_indices, dtype=np.int64)
        self.seq_lens = np.asarray(self.seq_lens, dtype=np.int64)

    @property
    def batch(self) -> int:
        return len(self.seq_lens)

    def pages(self, r: int) -> np.ndarray:
        return self.page_indices[self.page_indptr[r]:self.page_indptr[r + 1]]

    def num_blocks(self, r: int) -> int:
        return int(-(-int(self.seq_lens[r]) // self.page_size))

    def num_complete(self, r: int) -> int:
        return int(self.seq_lens[r]) // self.page_size

    def token_page_slot(self, r: int, t: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
        t = np.asarray(t, dtype=np.int64)
        return self.pages(r)[t // self.page_size], t % self.page_size


def _decode(bits: np.ndarray, fmt: str) -> np.ndarray:
    if fmt == "bf16":
        return bf16_to_f64(bits)
    if fmt == "fp8_e4m3fn":
        return fp8e4m3fn_to_f64(bits)
    if fmt == "fp32":
        return np.asarray(bits, dtype=np.float32).astype(np.float64)
    raise ValueError(fmt)


def _round_out(x: np.ndarray, out_dtype: str) -> np.ndarray:
    if out_dtype == "bf16":
        return f64_to_bf16_bits(x)
    if out_dtype == "fp32":
        return f64_to_f32(x)
    if out_dtype == "fp64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(out_dtype)


# --------------------------------------------------------------------------
# Block summaries: mean key of each full page, rounded once
# --------------------------------------------------------------------------

def block_summaries(key_bits: np.ndarray, page_ids: Sequence[int], *,
                    key_format: str = "bf16", key_scales: Optional[np.ndarray] = None,
                    out_dtype: str = "bf16") -> np.ndarray:
    """Mean key of each listed physical page, per head (Vortex, "Writing an
    algorithm: vFlow": the block-top-k cache step stores the mean of the keys
    over the in-block axis).

    key_bits: [num_pages][H][P][D] (or [num_pages][P][D] for single-head
    indexer pools). key_scales: optional per-token dequantisation scale
    [num_pages][P] (fp8 indexer keys): the summand is scale_t * key_t.
    Returns [n][H][D] (or [n][D]) bits / values in out_dtype.

    The sum over the P tokens is exact (checked; rows whose float64 sum could
    be inexact are summed as exact rationals), division by P = 2**m is exact,
    and the mean is rounded once to out_dtype.
    """
    page_ids = np.asarray(page_ids, dtype=np.int64)
    kb = np.asarray(key_bits)
    single = kb.ndim == 3
    k = _decode(kb[page_ids], key_format)
    if single:
        k = k[:, None]                                   # [n][1][P][D]
    if key_scales is not None:
        s = np.asarray(key_scales, dtype=np.float32)[page_ids].astype(np.float64)
        k = k * s[:, None, :, None]                      # exact: 24b x 4b
    P = k.shape[2]
    assert P & (P - 1) == 0, "page size must be a power of two"
    terms = np.moveaxis(k, 2, -1)                        # [n][H][D][P]
    total = terms.sum(axis=-1)
    mean = total / P
    exact = sum_is_exact_in_f64(terms, axis=-1)
    if out_dtype == "bf16":
        out = f64_to_bf16_bits(mean)
    else:
        out = _round_out(mean, out_dtype)
    for idx in zip(*np.nonzero(~exact)):               # rare: exact rationals
        fr = sum((Fraction(float(v)) for v in terms[idx]), Fraction(0)) / P
        out[idx] = fraction_to_bf16_bits(fr) if out_dtype == "bf16" else fraction_to_f32(fr)
    return out[:, 0] if single else out


# --------------------------------------------------------------------------
# Quest bounds: element-wise max and min key of each full page
# --------------------------------------------------------------------------

def block_bounds(key_bits: np.ndarray, page_ids: Sequence[int]) -> np.ndarray:
    """Element-wise maximum and minimum key of each listed physical page, per
    head (Vortex, "Writing an algorithm: vFlow": Quest's cache step keeps the
    block-wise Max and Min of the keys). key_bits: bf16 bits [num_pages][H][P][D].
    Returns bf16 bits [n][H][2][D]: row 0 the maximum, row 1 the minimum.
    Exact: the maximum and minimum of bf16 values are bf16 values."""
    page_ids = np.asarray(page_ids, dtype=np.int64)
    k = bf16_to_f64(np.asarray(key_bits)[page_ids])       # [n][H][P][D]
    hi = k.max(axis=2)
    lo = k.min(axis=2)
    return f64_to_bf16_bits(np.stack([hi, lo], axis=2))


def bound_scores(q_bits: np.ndarray, bounds: np.ndarray, batch: BatchView, r: int, g: int,
                 *, num_kv_heads: int, agg: str = "max") -> np.ndarray:
    """Quest score of request r's complete blocks for kv head g (Vortex,
    "Writing an algorithm: vFlow", the Quest listing): for each block j and
    query head h of the group, the element-wise Maximum of q_h * max_j and
    q_h * min_j, summed over the dims -- the largest value q_h . k can take
    for a key inside the block's box -- then agg over the group's heads
    (max, the listing's reduction over heads, or mean). bounds: bf16 bits
    [num_pages][Hkv][2][D] from block_bounds. Returns float64 [num_complete(r)]."""
    Hq = q_bits.shape[1]
    G = Hq // num_kv_heads
    q = bf16_to_f64(q_bits[r, g * G:(g + 1) * G])                  # [G][D]
    nc = batch.num_complete(r)
    pages = batch.pages(r)[:nc]
    b = bf16_to_f64(np.asarray(bounds)[pages, g])                   # [nc][2][D]
    hi, lo = b[:, 0], b[:, 1]
    s = np.maximum(q[None] * hi[:, None], q[None] * lo[:, None])     # [nc][G][D]
    per_head = s.sum(axis=2)                                         # [nc][G]
    if agg == "max":
        return per_head.max(axis=1) if nc else np.zeros(0)
    if agg == "mean":
        return per_head.mean(axis=1) if nc else np.zeros(0)
    raise ValueError(agg)


# --------------------------------------------------------------------------
# Scoring
# --------------------------------------------------------------------------

def block_scores(q_bits: np.ndarray, summaries: np.ndarray, batch: BatchView, r: int, g: int,
                 *, num_kv_heads: int, agg: str = "max",
                 summary_format: str = "bf16") -> np.ndarray:
    """Scores of request r's complete blocks for kv head g: for each block j,
    agg over the group's query heads h of q_h . k̄_j (Vortex, block top-k
    equation; GQA grouping from the vFlow listing). Returns float64
    [num_complete(r)]. summaries: [num_pages][Hkv][D] in summary_format."""
    Hq = q_bits.shape[1]
    G = Hq // num_kv_heads
    q = bf16_to_f64(q_bits[r, g * G:(g + 1) * G])                  # [G][D]
    nc = batch.num_complete(r)
    pages = batch.pages(r)[:nc]
    S = _decode(np.asarray(summaries)[pages, g], summary_format)    # [nc][D]
    per_head = S @ q.T                                               # [nc][G]
    if agg == "max":
        return per_head.max(axis=1) if nc else np.zeros(0)
    if agg == "mean":
        return per_head.mean(axis=1) if nc else np.zeros(0)
    raise ValueError(agg)


def indexer_token_scores(q_idx_bits: np.ndarray, head_w: np.ndarray, key_bits: np.ndarray,
                         key_scales: np.ndarray, batch: BatchView, r: int,
                         tokens: Optional[np.ndarray] = None) -> np.ndarray:
    """Learned-indexer score of tokens of request r (LeanSparse §5, Eq. 6,
    with the original key in place of the PQ centroids):
    s_t = sum_h w_h * ReLU(q_h . k_t), k_t = scale_t * fp8_t dequantised.
    key_bits: [pages][P][Di] fp8 bits; key_scales: [pages][P] fp32.
    Returns float64 scores for `tokens` (default: every cached token)."""
    L = int(batch.seq_lens[r])
    t = np.arange(L) if tokens is None else np.asarray(tokens, dtype=np.int64)
    page, slot = batch.token_page_slot(r, t)
    k = fp8e4m3fn_to_f64(np.asarray(key_bits)[page, slot])                 # [T][Di]
    k = k * np.asarray(key_scales, dtype=np.float32)[page, slot].astype(np.float64)[:, None]
    q = bf16_to_f64(q_idx_bits[r])                                          # [Hi][Di]
    w = np.asarray(head_w, dtype=np.float32)[r].astype(np.float64)          # [Hi]
    return np.maximum(k @ q.T, 0.0) @ w


def indexer_block_scores(q_idx_bits: np.ndarray, head_w: np.ndarray, summaries: np.ndarray,
                         batch: BatchView, r: int, *, summary_format: str = "bf16",
                         blocks: Optional[np.ndarray] = None) -> np.ndarray:
    """Coarse indexer score of request r's blocks from block-mean indexer keys:
    s_j = sum_h w_h * ReLU(q_h . k̄_j) (Eq. 6 of LeanSparse applied to the
    compact representation). summaries: [pages][Di]. Default blocks: every
    block whose summary exists (complete blocks)."""
    b = np.arange(batch.num_complete(r)) if blocks is None else np.asarray(blocks, dtype=np.int64)
    S = _decode(np.asarray(summaries)[batch.pages(r)[b]], summary_format)   # [nb][Di]
    q = bf16_to_f64(q_idx_bits[r])
    w = np.asarray(head_w, dtype=np.float32)[r].astype(np.float64)
    return np.maximum(S @ q.T, 0.0) @ w


# --------------------------------------------------------------------------
# Selection
# --------------------------------------------------------------------------

def forced_blocks(nb: int, n_complete: int, n_sink: int, n_recent: int) -> List[int]:
    f = set(range(min(n_sink, nb))) | set(range(max(0, nb - n_recent), nb))
    if n_complete < nb:            # partial last block: never scored, always kept
        f.add(nb - 1)
    return sorted(f)


def topk_from_keep_ratio(nb: int, n_complete: int, keep_ratio: float, n_sink: int,
                         n_recent: int) -> int:
    """k for a keep-ratio budget: the request keeps max(|F|, ceil(ratio * nb))
    blocks in all, forced blocks F included (the ByteCross paper counts its
    sink tokens inside the kept fraction r_KV, §3.2 and §4.1). The product
    ratio * nb is taken in fp32, the precision the kernels take it in, since
    it decides an integer."""
    nf = len(forced_blocks(nb, n_complete, n_sink, n_recent))
    total = int(np.ceil(np.float32(keep_ratio) * np.float32(nb)))
    return max(nf, total) - nf


def rank_top(scores: np.ndarray, candidates: Iterable[int], k: int) -> List[int]:
    """First k candidates under the order (score descending, index ascending)."""
    order = sorted(candidates, key=lambda j: (-float(scores[j]), j))
    return order[:max(0, k)]


def select_blocks(scores: np.ndarray, nb: int, n_complete: int, k: int,
                  n_sink: int, n_recent: int) -> List[int]:
    """Top-k blocks by score plus forced sink/recent blocks, ascending
    (Vortex, block top-k equation; static sink + recent window from the
    StreamingLLM mention in "Why Long Generations Are Expensive").
    scores: [n_complete] float64 for the complete blocks."""
    forced = forced_blocks(nb, n_complete, n_sink, n_recent)
    fs = set(forced)
    cands = [j for j in range(n_complete) if j not in fs]
    return sorted(fs | set(rank_top(scores, cands, k)))


def select_tokens(scores: np.ndarray, k: int, candidates: Optional[Iterable[int]] = None,
                  forced: Iterable[int] = ()) -> List[int]:
    """Top-k tokens by (score desc, token asc) among `candidates` (default all),
    plus `forced`, ascending (token-granular selection of the learned indexer,
    LeanSparse §2.1 / §5)."""
    fs = set(forced)
    cands = range(len(scores)) if candidates is None else candidates
    cands = [t for t in cands if t not in fs]
    return sorted(fs | set(rank_top(scores, cands, k)))


def remap_bucket(scores: np.ndarray, bins: int = 4096) -> np.ndarray:
    """Bucket of each score for the top-k's first digit (Vortex, "Making it
    fast": a monotonic remap of the scores spreads them over the buckets).
    The reading taken here: the plainest such remap, linear between the
    smallest and largest score of the ranked units, in fp32 (the precision
    the kernels rank in), each operation rounded once:
        span = mx - mn;  scale = bins / span;  t = (s - mn) * scale
        bucket = bins - 1 if t >= bins - 1, floor(t) if t >= 1, else 0.
    Every bucket is 0 when span is not a positive finite number (all scores
    equal). Non-decreasing in s, so a higher bucket never holds a lower
    score."""
    f = np.asarray(scores, dtype=np.float64).astype(np.float32)
    if f.size == 0:
        return np.zeros(0, dtype=np.int64)
    mn, mx = f.min(), f.max()
    with np.errstate(invalid="ignore", over="ignore"):
        span = np.float32(mx - mn)
        if not (np.isfinite(span) and span > 0):
            return np.zeros(f.size, dtype=np.int64)
        scale = np.float32(np.float32(bins) / span)
        t = (f - mn).astype(np.float32) * scale
        b = np.where(t >= bins - 1, bins - 1, np.where(t >= 1, np.floor(t), 0))
    return np.nan_to_num(b, nan=0).astype(np.int64)


def approx_select_tokens(scores: np.ndarray, k: int,
                         candidates: Optional[Iterable[int]] = None,
                         bins: int = 4096) -> List[int]:
    """Approximate top-k (Vortex, "Making it fast": a monotonic remap of the
    scores into buckets and an early exit that stops refining once enough
    winners are certain, filling the rest from the boundary bucket): with
    buckets from remap_bucket over the ranked units' scores, every unit whose
    bucket is above the bucket b* holding the k-th best, then units of b* in
    ascending index order until there are k (the page samples the boundary
    bucket; index order is the deterministic reading). Ascending ids."""
    cands = np.arange(len(scores)) if candidates is None else np.asarray(list(candidates))
    k = min(max(0, k), len(cands))
    if k == 0:
        return []
    b = remap_bucket(np.asarray(scores)[cands], bins)
    kth = np.sort(b)[::-1][k - 1]
    above = cands[b > kth]
    fill = np.sort(cands[b == kth])[:k - len(above)]
    return sorted(int(t) for t in np.concatenate([above, fill]))


def tokens_of_blocks(blocks: Iterable[int], page_size: int, seq_len: int) -> np.ndarray:
    t = [b * page_size + s for b in blocks for s in range(page_size)]
    t = np.asarray(t, dtype=np.int64)
    return t[t < seq_len]


# --------------------------------------------------------------------------
# Attention over a token set, split-K merge
# --------------------------------------------------------------------------

def attention_over_tokens(q: np.ndarray, K: np.ndarray, V: np.ndarray,
                          sm_scale: float) -> Tuple[np.ndarray, float]:
    """Exact softmax attention of one query over T tokens (float64):
    z_t = sm_scale * q . K_t; o = sum_t e^{z_t - M} V_t / sum_t e^{z_t - M};
    lse = M + ln sum_t e^{z_t - M}, M = max_t z_t. T = 0 gives o = 0,
    lse = -inf."""
    if K.shape[0] == 0:
        return np.zeros(V.shape[1]), -np.inf
    z = float(sm_scale) * (K @ q)
    M = z.max()
    w = np.exp(z - M)
    Z = w.sum()
    return (w @ V) / Z, float(M + np.log(Z))


def lse_merge(parts: Sequence[Tuple[np.ndarray, float]]) -> Tuple[np.ndarray, float]:
    """Merge attention results over disjoint token sets by log-sum-exp (the
    ByteCross paper merges its sink call with the window call this way, App. A):
    o = sum_s e^{lse_s - M} o_s / sum_s e^{lse_s - M}, lse = M + ln sum_s e^{lse_s - M}."""
    lses = np.array([p[1] for p in parts], dtype=np.float64)
    if np.all(np.isneginf(lses)):
        return np.zeros_like(parts[0][0]), -np.inf
    M = lses.max()
    w = np.exp(lses - M)
    o = sum(wi * p[0] for wi, p in zip(w, parts)) / w.sum()
    return o, float(M + np.log(w.sum()))


def sparse_attention(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray,
                     batch: BatchView, r: int, g: int, blocks: Sequence[int], *,
                     num_kv_heads: int, sm_scale: float,
                     out_dtype: str = "bf16") -> Tuple[np.ndarray, np.ndarray]:
    """Attention of every query head of kv group g of request r over the
    tokens of the selected blocks (Vortex block top-k equation). K/V pools:
    [pages][Hkv][P][D] bf16 bits. Returns (out [G][Dv] in out_dtype,
    lse float64 [G])."""
    Hq = q_bits.shape[1]
    G = Hq // num_kv_heads
    P = batch.page_size
    t = tokens_of_blocks(blocks, P, int(batch.seq_lens[r]))
    page, slot = batch.token_page_slot(r, t)
    K = bf16_to_f64(np.asarray(k_bits)[page, g, slot])                 # [T][D]
    V = bf16_to_f64(np.asarray(v_bits)[page, g, slot])                 # [T][Dv]
    outs, lses = [], []
    for h in range(g * G, (g + 1) * G):
        o, lse = attention_over_tokens(bf16_to_f64(q_bits[r, h]), K, V, sm_scale)
        outs.append(o)
        lses.append(lse)
    return _round_out(np.stack(outs), out_dtype), np.array(lses)


def window_tokens(seq_len: int, n_sink: int, window: int) -> np.ndarray:
    """Tokens of the sink + recent window (ByteCross, Appendix A, after
    attention sinks): the first min(n_sink, L) tokens and the last `window`
    tokens, without repeats, ascending."""
    L = int(seq_len)
    ns = min(int(n_sink), L)
    lo = max(ns, L - int(window))
    return np.concatenate([np.arange(ns), np.arange(lo, L)]).astype(np.int64)


def window_attention(q_bits, k_bits, v_bits, batch: BatchView, r: int, g: int, *,
                     n_sink: int, window: int, num_kv_heads: int, sm_scale: float,
                     out_dtype: str = "bf16") -> Tuple[np.ndarray, np.ndarray]:
    """Attention of every query head of kv group g of request r over the
    sink + recent window tokens, read in place (one exact softmax over the
    union; the paper's two calls merged by log-sum-exp give the same)."""
    Hq = q_bits.shape[1]
    G = Hq // num_kv_heads
    t = window_tokens(int(batch.seq_lens[r]), n_sink, window)
    page, slot = batch.token_page_slot(r, t)
    K = bf16_to_f64(np.asarray(k_bits)[page, g, slot])
    V = bf16_to_f64(np.asarray(v_bits)[page, g, slot])
    outs, lses = [], []
    for h in range(g * G, (g + 1) * G):
        o, lse = attention_over_tokens(bf16_to_f64(q_bits[r, h]), K, V, sm_scale)
        outs.append(o)
        lses.append(lse)
    return _round_out(np.stack(outs), out_dtype), np.array(lses)


def snapkv_scores(q_obs_bits: np.ndarray, k_bits: np.ndarray, batch: BatchView, r: int, g: int,
                  *, num_kv_heads: int, sm_scale: float) -> np.ndarray:
    """One-time SnapKV-style scores of request r's cache for kv head g
    (ByteCross §4.1 and Appendix A, "Scored selection"): the last W prompt
    tokens' queries q_obs [B][W][Hq][D] (bf16 bits; observation query w sits
    at position L - W + w and attends positions <= its own) each give a
    softmax over the cache; the score of position t is the sum of those
    probabilities over the W queries and the group's query heads (pooled).
    Returns float64 [L]."""
    W, Hq = q_obs_bits.shape[1], q_obs_bits.shape[2]
    G = Hq // num_kv_heads
    L = int(batch.seq_lens[r])
    t = np.arange(L)
    page, slot = batch.token_page_slot(r, t)
    K = bf16_to_f64(np.asarray(k_bits)[page, g, slot])                  # [L][D]
    score = np.zeros(L)
    for w in range(W):
        pos = L - W + w
        if pos < 0:            # a request shorter than the window: no such query
            continue
        for h in range(g * G, (g + 1) * G):
            z = float(sm_scale) * (K[:pos + 1] @ bf16_to_f64(q_obs_bits[r, w, h]))
            e = np.exp(z - z.max())
            score[:pos + 1] += e / e.sum()
    return score


def snapkv_select(q_obs_bits: np.ndarray, k_bits: np.ndarray, batch: BatchView, r: int, g: int,
                  *, num_kv_heads: int, sm_scale: float, n_sink: int, budget: int,
                  pool: int = 7) -> List[int]:
    """Positions kept for kv head g of request r: the first n_sink positions
    and the W observation positions are forced; the rest of the budget goes to
    the prefix positions [n_sink, L - W) with the largest pooled score, the
    scores averaged over a window of `pool` positions centred on each (zero
    outside the prefix [0, L - W), divisor `pool`); ties to the lowest
    position. Ascending."""
    W = q_obs_bits.shape[1]
    L = int(batch.seq_lens[r])
    s = snapkv_scores(q_obs_bits, k_bits, batch, r, g, num_kv_heads=num_kv_heads,
                      sm_scale=sm_scale)
    npre = max(0, L - W)
    pre = np.concatenate([np.zeros(pool // 2), s[:npre], np.zeros(pool // 2)])
    pooled = np.array([pre[i:i + pool].sum() for i in range(npre)]) / pool
    forced = set(range(min(n_sink, npre))) | set(range(npre, L))
    cands = [t for t in range(npre) if t not in forced]
    k = max(0, budget - len(forced))
    return sorted(forced | set(rank_top(pooled, cands, k)))


def dense_attention(q_bits, k_bits, v_bits, batch: BatchView, r: int, g: int, *,
                    num_kv_heads: int, sm_scale: float, out_dtype: str = "bf16"):
    """The k = all case: every block of the request selected."""
    return sparse_attention(q_bits, k_bits, v_bits, batch, r, g,
                            range(batch.num_blocks(r)), num_kv_heads=num_kv_heads,
                            sm_scale=sm_scale, out_dtype=out_dtype)


def mla_attention(q_bits: np.ndarray, latent_bits: np.ndarray, batch: BatchView, r: int,
                  tokens: Sequence[int], *, v_dim: int, sm_scale: float,
                  out_dtype: str = "bf16") -> Tuple[np.ndarray, np.ndarray]:
    """Multi-head latent attention over selected tokens: every query head
    attends the single shared latent head; keys are the full latent row
    (compressed content + rope part), values its first v_dim entries (Vortex,
    "Designing for a new architecture"). q: [B][H][Dk] bf16; latent pool:
    [pages][P][Dk] bf16. Returns (out [H][v_dim], lse [H])."""
    page, slot = batch.token_page_slot(r, np.asarray(tokens, dtype=np.int64))
    C = bf16_to_f64(np.asarray(latent_bits)[page, slot])                 # [T][Dk]
    K, V = C, C[:, :v_dim]
    outs, lses = [], []
    for h in range(q_bits.shape[1]):
        o, lse = attention_over_tokens(bf16_to_f64(q_bits[r, h]), K, V, sm_scale)
        outs.append(o)
        lses.append(lse)
    return _round_out(np.stack(outs), out_dtype), np.array(lses)


# --------------------------------------------------------------------------
# One decode step of block top-k over a paged GQA cache
# --------------------------------------------------------------------------

def select_blocks_batch(q_bits, summaries, batch: BatchView, pairs, *, num_kv_heads: int,
                        topk: int, n_sink: int, n_recent: int, agg: str = "max",
                        summary_format: str = "bf16", score_mode: str = "mean") -> Dict:
    """Scores and selections for the (r, g) pairs listed. score_mode "mean":
    summaries are block-mean keys (block_scores); "bounds": Quest bounds
    [num_pages][Hkv][2][D] (bound_scores)."""
    res = {}
    for r, g in pairs:
        if score_mode == "bounds":
            s = bound_scores(q_bits, summaries, batch, r, g, num_kv_heads=num_kv_heads, agg=agg)
        elif score_mode == "mean":
            s = block_scores(q_bits, summaries, batch, r, g, num_kv_heads=num_kv_heads,
                             agg=agg, summary_format=summary_format)
        else:
            raise ValueError(score_mode)
        sel = select_blocks(s, batch.num_blocks(r), batch.num_complete(r), topk,
                            n_sink, n_recent)
        res[(r, g)] = (s, sel)
    return res


def decode_step(q_bits, k_bits, v_bits, batch: BatchView, *, num_kv_heads: int, topk: int,
                n_sink: int, n_recent: int, sm_scale: float, agg: str = "max",
                out_dtype: str = "bf16", pairs=None, summaries=None,
                score_mode: str = "mean") -> Dict:
    """Summaries of the requests' complete pages (unless given: block means,
    or Quest bounds when score_mode is "bounds"), block scores, selection and
    attention for each (r, g) in `pairs` (default: all)."""
    if pairs is None:
        pairs = [(r, g) for r in range(batch.batch) for g in range(num_kv_heads)]
    if summaries is None:
        pages = sorted({int(p) for r in {r for r, _ in pairs}
                        for p in batch.pages(r)[:batch.num_complete(r)]})
        kb = np.asarray(k_bits)
        rows = (2,) if score_mode == "bounds" else ()
        summaries = np.zeros((kb.shape[0], kb.shape[1]) + rows + (kb.shape[3],), dtype=np.uint16)
        if pages:
            build = block_bounds if score_mode == "bounds" else block_summaries
            summaries[pages] = build(k_bits, pages)
    sel = select_blocks_batch(q_bits, summaries, batch, pairs, num_kv_heads=num_kv_heads,
                              topk=topk, n_sink=n_sink, n_recent=n_recent, agg=agg,
                              score_mode=score_mode)
    out = {}
    for (r, g), (s, blocks) in sel.items():
        o, lse = sparse_attention(q_bits, k_bits, v_bits, batch, r, g, blocks,
                                  num_kv_heads=num_kv_heads, sm_scale=sm_scale,
                                  out_dtype=out_dtype)
        out[(r, g)] = {"scores": s, "selected": blocks, "out": o, "lse": lse}
    return {"summaries": summaries, "pairs": out}


# --------------------------------------------------------------------------
# Coarse-to-fine token selection with a learned indexer
# --------------------------------------------------------------------------

def coarse_to_fine_select(q_idx_bits: np.ndarray, head_w: np.ndarray, key_bits: np.ndarray,
                          key_scales: np.ndarray, summaries: np.ndarray, batch: BatchView,
                          r: int, *, topk_blocks: int, n_recent_blocks: int, topk_tokens: int,
                          summary_format: str = "bf16") -> Dict:
    """Coarse-to-fine selection of request r (LeanSparse §5: a coarse pass
    over a compact representation picks candidate blocks, then exact indexer
    scores of the candidates' tokens pick the tokens; tokens outside the
    kept blocks cannot come back):
      1. coarse score of every complete block from its block-mean key,
      2. the top topk_blocks blocks plus the last n_recent_blocks (and a
         partial last block) -- select_blocks with no sink,
      3. exact Eq. 6 score of every cached token of those blocks,
      4. the top topk_tokens of them by (score desc, token asc).
    Returns {"blocks", "block_scores", "tokens" (ascending), "token_scores"}."""
    nb, nc = batch.num_blocks(r), batch.num_complete(r)
    L = int(batch.seq_lens[r])
    sb = indexer_block_scores(q_idx_bits, head_w, summaries, batch, r,
                              summary_format=summary_format)
    blocks = select_blocks(sb, nb, nc, topk_blocks, 0, n_recent_blocks)
    toks = tokens_of_blocks(blocks, batch.page_size, L)
    st = indexer_token_scores(q_idx_bits, head_w, key_bits, key_scales, batch, r, tokens=toks)
    full = np.full(L, -np.inf)
    full[toks] = st
    sel = select_tokens(full, topk_tokens, candidates=toks.tolist())
    return {"blocks": blocks, "block_scores": sb, "tokens": sel,
            "token_scores": dict(zip(toks.tolist(), st.tolist()))}
