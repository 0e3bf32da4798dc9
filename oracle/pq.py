"""PQ32 coarse scoring with exact refinement, in float64 (oracle; TEST
INFRASTRUCTURE ONLY).

LeanSparse ("LeanSparse: Memory-Efficient Serving for Native Sparse-Attention
LLMs"), §5, "Approximate scoring with PQ" and "Retrieving and refining
candidates": a 128-dim indexer key is cut into 32 subvectors of 4 dims, each
stored as a one-byte index into that subspace's codebook of 256 centroids
(trained offline by k-means). The coarse score of a key is the indexer score
(Eq. 6) with each subvector replaced by its centroid; the C best keys by that
score are candidates, their original keys (plus the recent keys not yet
encoded) are scored exactly, and the final top-k comes from those.

Readings where the page leaves a step open:
* Codebooks are per subspace (C_j in Eq. 6), bf16 [32][256][4]; the keys the
  codes stand for are the dequantised indexer keys x = scale * fp8.
* Encoding picks the centroid of least squared Euclidean distance. The
  distance decides an integer, so it is defined to the bit: in float64,
  d_t = x_t - c_t, then ((d_0 d_0 + d_1 d_1) + d_2 d_2) + d_3 d_3, each
  operation rounded once; ties go to the lowest centroid.
* k-means (Lloyd): centroid c of subspace j starts as subvector j of key
  init[c], rounded to bf16; each iteration encodes every training key, then
  sets each centroid with members to their mean and leaves the others. The
  mean is taken in fixed point so that its value does not depend on the order
  of the sum: each member value v becomes the integer rint(v * 2^24) (round
  half to even), the integers are summed exactly, the sum (below 2^53) and
  the count become float64, and mean = (sum / count) * 2^-24 (one float64
  division) is rounded once to bf16.
* Only keys of complete pages have codes (a page is encoded when it fills);
  the tokens of the partial last page are the "recent keys", scored exactly.
* Ranking keys of both passes are (score desc, token asc).
* Miss filter ("Retrieving and refining candidates"): the candidates whose
  original key is resident are kept; a miss is dropped when its approximate
  score is below theta = s_(k) - sd, read as: s_(k) the k-th largest
  approximate score among all of the request's candidates (hits and misses;
  the smallest when there are at most k), sd the sample standard deviation
  (denominator n - 1; 0 for fewer than two) of those same scores, both in
  float64 from the fp32 scores; "below" is strict, so a score equal to theta
  is kept.

Parity status: pinned by tests/test_oracle_pq.py (hand-worked k-means and
fixed-point means, brute-force nearest centroids with exact rationals, codes
of keys that are centroids, the reduction of the coarse score to the exact
indexer score when every subvector is a centroid, and the reduction of the
two-pass selection to the exact token top-k when C covers every token);
the miss filter by hand-worked thresholds (sample versus population
deviation, the k-th largest, equality kept, hits kept).
"""

from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from .method import BatchView, indexer_token_scores, select_tokens
from .numerics import bf16_to_f64, f64_to_bf16_bits, fp8e4m3fn_to_f64

PQ_SUBSPACES = 32
PQ_SUBDIM = 4
PQ_CENTROIDS = 256
PQ_FIXED_BITS = 24


def dequantize_index_keys(key_bits: np.ndarray, key_scales: np.ndarray) -> np.ndarray:
    """x = scale * fp8 value, exact in float64. key_bits [..][128] fp8 bits,
    key_scales [..] fp32."""
    k = fp8e4m3fn_to_f64(np.asarray(key_bits))
    s = np.asarray(key_scales, dtype=np.float32).astype(np.float64)
    return k * s[..., None]


def _sq_dist(x: np.ndarray, c: np.ndarray) -> np.ndarray:
    """Squared distance of subvectors x [n][4] to centroids c [K][4] in the
    defined order: ((d0*d0 + d1*d1) + d2*d2) + d3*d3 -> [n][K]."""
    d = x[:, None, :] - c[None, :, :]
    sq = d * d
    return ((sq[..., 0] + sq[..., 1]) + sq[..., 2]) + sq[..., 3]


def pq_encode(x: np.ndarray, codebooks_bits: np.ndarray) -> np.ndarray:
    """Codes [n][32] uint8 of keys x [n][128] (float64): per subspace, the
    index of the nearest centroid (lowest index on ties)."""
    x = np.asarray(x, dtype=np.float64)
    cb = bf16_to_f64(np.asarray(codebooks_bits))          # [32][K][4]
    n = x.shape[0]
    S = cb.shape[0]
    codes = np.zeros((n, S), dtype=np.int64)
    for j in range(S):
        sub = x[:, PQ_SUBDIM * j:PQ_SUBDIM * (j + 1)]
        for i0 in range(0, n, 4096):
            codes[i0:i0 + 4096, j] = np.argmin(_sq_dist(sub[i0:i0 + 4096], cb[j]), axis=1)
    return codes.astype(np.uint8 if cb.shape[1] <= 256 else np.int64)


def fixed_point_mean_bf16(values: np.ndarray) -> np.ndarray:
    """Mean over axis 0 of values [m][4] (m >= 1) by the fixed-point rule,
    rounded once to bf16 (bits)."""
    v = np.asarray(values, dtype=np.float64)
    ints = np.rint(v * float(2 ** PQ_FIXED_BITS)).astype(np.int64)
    tot = [int(t) for t in ints.sum(axis=0, dtype=object)]
    if any(abs(t) >= 2 ** 53 for t in tot):
        raise ValueError("fixed-point sum out of the exact range")
    mean = (np.array(tot, dtype=np.float64) / np.float64(v.shape[0])) * 2.0 ** -PQ_FIXED_BITS
    return f64_to_bf16_bits(mean)


def pq_kmeans(x: np.ndarray, init: Sequence[int], iters: int) -> np.ndarray:
    """Codebooks (bf16 bits [32][K][4], K = len(init)) trained by Lloyd's
    iterations on keys x [n][128] from centroid c = key init[c]."""
    x = np.asarray(x, dtype=np.float64)
    init = np.asarray(init, dtype=np.int64)
    K = len(init)
    cb = f64_to_bf16_bits(x[init].reshape(K, PQ_SUBSPACES, PQ_SUBDIM).transpose(1, 0, 2))
    for _ in range(iters):
        codes = pq_encode(x, cb).astype(np.int64)
        new = cb.copy()
        for j in range(PQ_SUBSPACES):
            sub = x[:, PQ_SUBDIM * j:PQ_SUBDIM * (j + 1)]
            for c in np.unique(codes[:, j]):
                new[j, c] = fixed_point_mean_bf16(sub[codes[:, j] == c])
        cb = new
    return cb


def pq_decode(codes: np.ndarray, codebooks_bits: np.ndarray) -> np.ndarray:
    """Keys [n][128] (float64) rebuilt from codes [n][32]: centroid
    C_j[code_j] in place of subvector j."""
    cb = bf16_to_f64(np.asarray(codebooks_bits))
    codes = np.asarray(codes, dtype=np.int64)
    parts = [cb[j][codes[:, j]] for j in range(codes.shape[1])]
    return np.concatenate(parts, axis=1)


def pq_token_scores(q_idx_bits: np.ndarray, head_w: np.ndarray, codes_pool: np.ndarray,
                    codebooks_bits: np.ndarray, batch: BatchView, r: int,
                    tokens: Optional[np.ndarray] = None) -> np.ndarray:
    """Coarse score of tokens of request r (LeanSparse §5, Eq. 6):
    s~_t = sum_h w_h ReLU(sum_j q_h,j . C_j[c_t,j]). codes_pool: [pages][P][32]
    uint8. Default tokens: every token of the complete pages."""
    nc = batch.num_complete(r)
    t = np.arange(nc * batch.page_size) if tokens is None else np.asarray(tokens, np.int64)
    page, slot = batch.token_page_slot(r, t)
    k = pq_decode(np.asarray(codes_pool)[page, slot], codebooks_bits)      # [T][128]
    q = bf16_to_f64(q_idx_bits[r])
    w = np.asarray(head_w, dtype=np.float32)[r].astype(np.float64)
    return np.maximum(k @ q.T, 0.0) @ w


def pq_refine_select(q_idx_bits: np.ndarray, head_w: np.ndarray, key_bits: np.ndarray,
                     key_scales: np.ndarray, codes_pool: np.ndarray,
                     codebooks_bits: np.ndarray, batch: BatchView, r: int, *,
                     n_candidates: int, topk: int) -> Dict:
    """Two-pass selection of request r: the top n_candidates tokens of the
    complete pages by coarse score, then the top topk of those candidates and
    the partial page's tokens by exact indexer score. Returns the coarse
    scores, the candidates (ascending), the exact scores of the refined set
    (candidates then tail, both ascending) and the selection (ascending)."""
    L = int(batch.seq_lens[r])
    nc = batch.num_complete(r)
    coarse = pq_token_scores(q_idx_bits, head_w, codes_pool, codebooks_bits, batch, r)
    cand = select_tokens(coarse, n_candidates)
    refined = np.array(cand + list(range(nc * batch.page_size, L)), dtype=np.int64)
    exact = indexer_token_scores(q_idx_bits, head_w, key_bits, key_scales, batch, r,
                                 tokens=refined)
    pick = select_tokens(exact, topk)
    return {"coarse": coarse, "candidates": cand, "refined": refined, "exact": exact,
            "selected": sorted(int(refined[i]) for i in pick)}


def pq_miss_filter(tokens: Sequence[int], scores: np.ndarray, resident: np.ndarray,
                   topk: int) -> Dict:
    """Miss filter before the exact rerank (LeanSparse §5, "Retrieving and
    refining candidates"): of the candidates `tokens` with approximate scores
    `scores` (fp32 values) and residency flags `resident` (the original key is
    on the GPU), keep every hit and every miss whose score is at least
    theta = s_(min(k, n)) - sd, with s_(j) the j-th largest score and sd the
    sample standard deviation of the n scores (0 when n < 2), in float64.
    Returns the kept tokens (ascending), theta, and the number of misses kept
    (the ones whose keys cross the host link)."""
    t = np.asarray(tokens, dtype=np.int64)
    s = np.asarray(scores, dtype=np.float64).astype(np.float32).astype(np.float64)
    res = np.asarray(resident, dtype=bool)
    n = len(t)
    if n == 0:
        return {"kept": [], "theta": float("nan"), "misses_kept": 0}
    kth = np.sort(s)[::-1][min(max(topk, 1), n) - 1]
    sd = float(np.std(s, ddof=1)) if n >= 2 else 0.0
    theta = float(kth) - sd
    keep = res | (s >= theta)
    return {"kept": sorted(int(x) for x in t[keep]), "theta": theta,
            "misses_kept": int((keep & ~res).sum())}
