"""Decode-step query-aware sparse attention for MI355X (gfx950).

Thin Python binding over libls.so (include/ls.h): argument marshalling only.
Every step of the path runs in the library's HIP kernels; PyTorch only
provides device memory and the current stream. Importing this package loads
the in-tree libls.so and raises ImportError if it has not been built.
"""

from __future__ import annotations

import ctypes as C
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

from . import _lib
from ._lib import (LS_AGG_MAX, LS_AGG_MEAN, LS_DTYPE_BF16, LS_DTYPE_FP32,  # noqa: F401
                   LS_BATCH_BAD_INDPTR, LS_BATCH_LENGTH_BEYOND_MAX_BLOCKS,
                   LS_BATCH_LENGTH_BEYOND_PAGES, LS_BATCH_NEGATIVE_LENGTH,
                   LS_BATCH_PAGE_OUT_OF_RANGE,
                   LS_CAND_BLOCKS, LS_CAND_TOKENS, LS_DTYPE_FP8_E4M3FN, LS_SCORE_BOUNDS,
                   LS_SCORE_MEAN, LS_SEL_BLOCKS,
                   LS_SEL_TOKENS, LsBatch, LsError,
                   LsIndexerParams, LsPool, LsSelectParams, check)

_L = _lib.load()

__all__ = ["PagedBatch", "build_block_summaries", "build_block_bounds", "score_select", "sparse_attn_decode",
           "score_select_workspace_size", "sparse_attn_decode_workspace_size",
           "attn_num_splits", "version", "LsError", "sparse_decode_step",
           "sparse_decode_step_workspace", "sparse_decode_step_noalloc", "stream_read",
           "check_batch", "debug_enable", "debug_enabled", "debug_report", "indexer_select", "indexer_select_workspace_size",
           "indexer_score_stride", "sparse_mla_decode", "sparse_mla_decode_workspace_size",
           "mla_num_splits", "pq_encode", "pq_train", "pq_select", "window_attn_decode",
           "snapkv_select", "snapkv_gather"]

_DT = {torch.bfloat16: LS_DTYPE_BF16, torch.float32: LS_DTYPE_FP32,
       torch.float8_e4m3fn: LS_DTYPE_FP8_E4M3FN}


def version() -> str:
    return _L.ls_version().decode()


@dataclass
class PagedBatch:
    """CSR page table of a ragged batch (device int32 tensors) plus the host
    bound max_blocks >= ceil(seq_len / page_size) for every request."""
    page_indptr: torch.Tensor
    page_indices: torch.Tensor
    seq_lens: torch.Tensor
    max_blocks: int

    @property
    def batch_size(self) -> int:
        return int(self.seq_lens.numel())

    def c(self) -> LsBatch:
        for t in (self.page_indptr, self.page_indices, self.seq_lens):
            _need(t, torch.int32)
        return LsBatch(self.batch_size, int(self.max_blocks), self.page_indptr.data_ptr(),
                       self.page_indices.data_ptr(), self.seq_lens.data_ptr())


def _need(t: torch.Tensor, dtype=None):
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"expected {dtype}, got {t.dtype}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream) -> C.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _pool(t: torch.Tensor, num_heads: int, page_size: int, head_dim: int) -> LsPool:
    return LsPool(int(t.shape[0]), num_heads, page_size, head_dim, _DT[t.dtype])


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> torch.Tensor:
    """The caller's workspace, or a new zero-filled one (the selection,
    attention and step calls need a workspace that is zero before its first
    use; every call leaves it zero)."""
    if ws is not None:
        return ws
    return torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ summaries

def build_block_summaries(keys: torch.Tensor, page_ids: torch.Tensor, summaries: torch.Tensor,
                          key_scales: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Mean key of every listed full page, per head, rounded once.

    keys: bf16 [pages][Hkv][P][D], or fp8-e4m3fn [pages][P][D] with
    key_scales fp32 [pages][P]. summaries: [pages][Hkv][D] (or [pages][D])
    bf16 or fp32; rows of the listed pages are overwritten."""
    _need(keys); _need(page_ids, torch.int32); _need(summaries)
    if keys.dim() == 4:
        pool = _pool(keys, keys.shape[1], keys.shape[2], keys.shape[3])
    else:
        pool = _pool(keys, 1, keys.shape[1], keys.shape[2])
    if key_scales is not None:
        _need(key_scales, torch.float32)
    check(_L.ls_build_block_summaries(keys.data_ptr(), _ptr(key_scales), pool,
                                      page_ids.data_ptr(), int(page_ids.numel()),
                                      summaries.data_ptr(), _DT[summaries.dtype],
                                      _stream(stream)))
    return summaries


def build_block_bounds(keys: torch.Tensor, page_ids: torch.Tensor, bounds: torch.Tensor,
                       stream=None) -> torch.Tensor:
    """Quest bounds of every listed page: the element-wise maximum and
    minimum key over the page's tokens, per head.

    keys: bf16 [pages][Hkv][P][D]; bounds: bf16 [pages][Hkv][2][D] (maximum
    row, then minimum row); rows of the listed pages are overwritten."""
    _need(keys, torch.bfloat16); _need(page_ids, torch.int32); _need(bounds, torch.bfloat16)
    n, H, P, D = keys.shape
    if tuple(bounds.shape) != (n, H, 2, D):
        raise ValueError(f"bounds must be [{n}][{H}][2][{D}], got {tuple(bounds.shape)}")
    check(_L.ls_build_block_bounds(keys.data_ptr(), _pool(keys, H, P, D), page_ids.data_ptr(),
                                   int(page_ids.numel()), bounds.data_ptr(), _stream(stream)))
    return bounds


def _score_mode(mode: str, summaries: torch.Tensor, head_dim: int) -> int:
    """LS_SCORE_MEAN for block-mean summaries [pages][Hkv][D], LS_SCORE_BOUNDS
    for Quest bounds [pages][Hkv][2][D]."""
    if mode == "mean":
        if summaries.dim() != 3 or summaries.shape[2] != head_dim:
            raise ValueError("block-mean summaries must be [pages][Hkv][D]")
        return LS_SCORE_MEAN
    if mode == "bounds":
        if summaries.dim() != 4 or summaries.shape[2] != 2 or summaries.shape[3] != head_dim:
            raise ValueError("Quest bounds must be [pages][Hkv][2][D]")
        return LS_SCORE_BOUNDS
    raise ValueError(f"score_mode {mode!r} (expected 'mean' or 'bounds')")


# ------------------------------------------------------------------ selection

def score_select_workspace_size(batch_size: int, num_kv_heads: int, max_blocks: int) -> int:
    return int(_L.ls_score_select_workspace_size(batch_size, num_kv_heads, max_blocks))


def score_select(q: torch.Tensor, summaries: torch.Tensor, page_size: int, batch: PagedBatch, *,
                 topk: int, n_sink: int, n_recent: int, max_selected: int,
                 group_agg: str = "max", keep_ratio: float = 0.0, score_mode: str = "mean",
                 selected: Optional[torch.Tensor] = None,
                 selected_count: Optional[torch.Tensor] = None,
                 scores_out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None,
                 stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Top-k blocks per (request, kv head) by GQA-aggregated summary score,
    plus forced sink/recent blocks, ascending. Returns (selected, counts)."""
    _need(q, torch.bfloat16); _need(summaries, torch.bfloat16)
    B, Hq, D = q.shape
    Hkv = summaries.shape[1]
    dev = q.device
    if selected is None:
        selected = torch.empty(B, Hkv, max_selected, dtype=torch.int32, device=dev)
    if selected_count is None:
        selected_count = torch.empty(B, Hkv, dtype=torch.int32, device=dev)
    _need(selected, torch.int32); _need(selected_count, torch.int32)
    if scores_out is not None:
        _need(scores_out, torch.float32)
    ws_bytes = score_select_workspace_size(B, Hkv, batch.max_blocks)
    ws = _workspace(ws_bytes, dev, workspace)
    params = LsSelectParams(C.sizeof(LsSelectParams),
                            LS_AGG_MAX if group_agg == "max" else LS_AGG_MEAN,
                            int(topk), float(keep_ratio), int(n_sink), int(n_recent),
                            int(max_selected), _score_mode(score_mode, summaries, D))
    pool = LsPool(int(summaries.shape[0]), int(Hkv), int(page_size), int(D), LS_DTYPE_BF16)
    check(_L.ls_score_select(q.data_ptr(), LS_DTYPE_BF16, int(Hq), summaries.data_ptr(), pool,
                             batch.c(), C.byref(params), selected.data_ptr(),
                             selected_count.data_ptr(), _ptr(scores_out), _ptr(ws),
                             0 if ws is None else ws.numel() * ws.element_size(),
                             _stream(stream)))
    return selected, selected_count


# ------------------------------------------------------------- batch checks

def check_batch(batch: PagedBatch, page_size: int, num_pages: int,
                report: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Check the batch's device data against a pool of num_pages pages of
    page_size tokens; returns the 4-word device report (kinds found,
    violating requests, first violating request or -1, requests checked)."""
    if report is None:
        report = torch.empty(4, dtype=torch.int32, device=batch.seq_lens.device)
    _need(report, torch.int32)
    check(_L.ls_check_batch(batch.c(), int(page_size), int(num_pages), report.data_ptr(),
                            _stream(stream)))
    return report


def debug_enable(on: bool = True) -> None:
    """Debug mode: every call that takes a batch checks it first and adds what
    it finds into the library's per-GPU debug words."""
    _L.ls_debug_enable(1 if on else 0)


def debug_enabled() -> bool:
    return bool(_L.ls_debug_enabled())


def debug_report() -> Tuple[int, int, int, int]:
    """The current GPU's debug words (kinds found, calls with a violation,
    violating requests, calls checked), then cleared; synchronises."""
    out = (C.c_int32 * 4)()
    check(_L.ls_debug_report(C.cast(out, C.c_void_p)))
    return tuple(int(x) for x in out)


# ------------------------------------------------------------------ attention

def stream_read(src: torch.Tensor, sink: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One streaming read of the whole of `src` (the bandwidth reference);
    returns the sink words."""
    _need(src)
    if sink is None:
        sink = torch.empty(int(_L.ls_stream_read_sink_words()), dtype=torch.int32,
                           device=src.device)
    check(_L.ls_stream_read(src.data_ptr(), src.numel() * src.element_size(), sink.data_ptr(),
                            _stream(stream)))
    return sink


def attn_num_splits(max_selected: int) -> int:
    return int(_L.ls_attn_num_splits(int(max_selected)))



def sparse_attn_decode_workspace_size(batch_size: int, num_q_heads: int, head_dim: int,
                                      max_selected: int, max_blocks: int) -> int:
    return int(_L.ls_sparse_attn_decode_workspace_size(batch_size, num_q_heads, head_dim,
                                                       max_selected, max_blocks))


def sparse_attn_decode(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                       batch: PagedBatch, selected: Optional[torch.Tensor],
                       selected_count: Optional[torch.Tensor], *, sm_scale: float,
                       out: Optional[torch.Tensor] = None, out_dtype=torch.bfloat16,
                       lse: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None,
                       stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Exact attention of every query head over the tokens of its group's
    selected blocks (selected=None: every block, the dense k = all path)."""
    _need(q, torch.bfloat16); _need(k_pool, torch.bfloat16); _need(v_pool, torch.bfloat16)
    B, Hq, D = q.shape
    _, Hkv, P, _ = k_pool.shape
    dev = q.device
    if out is None:
        out = torch.empty(B, Hq, D, dtype=out_dtype, device=dev)
    _need(out)
    if lse is not None:
        _need(lse, torch.float32)
    max_sel = int(selected.shape[-1]) if selected is not None else 0
    if selected is not None:
        _need(selected, torch.int32); _need(selected_count, torch.int32)
    ws_bytes = sparse_attn_decode_workspace_size(B, Hq, D, max_sel, batch.max_blocks)
    ws = _workspace(ws_bytes, dev, workspace)
    pool = _pool(k_pool, int(Hkv), int(P), int(D))
    check(_L.ls_sparse_attn_decode(q.data_ptr(), LS_DTYPE_BF16, int(Hq), k_pool.data_ptr(),
                                   v_pool.data_ptr(), pool, batch.c(), _ptr(selected),
                                   _ptr(selected_count), max_sel, float(sm_scale),
                                   out.data_ptr(), _DT[out.dtype], _ptr(lse), ws.data_ptr(),
                                   ws.numel() * ws.element_size(), _stream(stream)))
    return out, lse


# ------------------------------------------------------------------ fused step

def sparse_decode_step_workspace(batch_size: int, num_q_heads: int, num_kv_heads: int,
                                 head_dim: int, max_blocks: int, max_selected: int,
                                 device) -> torch.Tensor:
    """A zero-filled workspace for sparse_decode_step (it must be zero before
    the first call; every call leaves it zero, so it can be reused by calls
    that do not run concurrently)."""
    n = int(_L.ls_sparse_decode_step_workspace_size(batch_size, num_q_heads, num_kv_heads,
                                                   head_dim, max_blocks, max_selected))
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)


def sparse_decode_step(q: torch.Tensor, summaries: torch.Tensor, k_pool: torch.Tensor,
                       v_pool: torch.Tensor, batch: PagedBatch, *, topk: int, n_sink: int,
                       n_recent: int, max_selected: int, sm_scale: float,
                       group_agg: str = "max", keep_ratio: float = 0.0,
                       score_mode: str = "mean", selected: Optional[torch.Tensor] = None,
                       selected_count: Optional[torch.Tensor] = None,
                       out: Optional[torch.Tensor] = None, out_dtype=torch.bfloat16,
                       lse: Optional[torch.Tensor] = None,
                       new_pages: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None, stream=None):
    """score_select + sparse_attn_decode as one call (one launch for requests
    of at most 8192 blocks). new_pages (int32, optional):
    pages that filled at this step, whose summaries the call also rebuilds
    (they must be forced blocks of this call, e.g. last blocks with
    n_recent >= 1). Returns (out, lse, selected, selected_count)."""
    _need(q, torch.bfloat16); _need(summaries, torch.bfloat16)
    _need(k_pool, torch.bfloat16); _need(v_pool, torch.bfloat16)
    B, Hq, D = q.shape
    _, Hkv, P, _ = k_pool.shape
    dev = q.device
    if selected is None:
        selected = torch.empty(B, Hkv, max_selected, dtype=torch.int32, device=dev)
    if selected_count is None:
        selected_count = torch.empty(B, Hkv, dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty(B, Hq, D, dtype=out_dtype, device=dev)
    if workspace is None:
        workspace = sparse_decode_step_workspace(B, Hq, int(Hkv), D, batch.max_blocks,
                                                 max_selected, dev)
    _need(selected, torch.int32); _need(selected_count, torch.int32); _need(out)
    if lse is not None:
        _need(lse, torch.float32)
    params = LsSelectParams(C.sizeof(LsSelectParams),
                            LS_AGG_MAX if group_agg == "max" else LS_AGG_MEAN,
                            int(topk), float(keep_ratio), int(n_sink), int(n_recent),
                            int(max_selected), _score_mode(score_mode, summaries, D))
    n_new = 0
    if new_pages is not None:
        _need(new_pages, torch.int32)
        n_new = int(new_pages.numel())
    pool = _pool(k_pool, int(Hkv), int(P), int(D))
    check(_L.ls_sparse_decode_step(q.data_ptr(), LS_DTYPE_BF16, int(Hq), summaries.data_ptr(),
                                   k_pool.data_ptr(), v_pool.data_ptr(), pool, batch.c(),
                                   C.byref(params), selected.data_ptr(), selected_count.data_ptr(),
                                   float(sm_scale), out.data_ptr(), _DT[out.dtype], _ptr(lse),
                                   _ptr(new_pages), n_new, workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, lse, selected, selected_count


def sparse_decode_step_noalloc(q: torch.Tensor, summaries: torch.Tensor, k_pool: torch.Tensor,
                               v_pool: torch.Tensor, batch: PagedBatch, *, topk: int,
                               n_sink: int, n_recent: int, max_selected: int, sm_scale: float,
                               selected: torch.Tensor, selected_count: torch.Tensor,
                               out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                               group_agg: str = "max", keep_ratio: float = 0.0,
                               score_mode: str = "mean",
                               new_pages: Optional[torch.Tensor] = None, stream=None):
    """sparse_decode_step with the library's fixed scratch array instead of
    a workspace (no device allocation; outputs are the caller's)."""
    _need(q, torch.bfloat16); _need(summaries, torch.bfloat16)
    _need(k_pool, torch.bfloat16); _need(v_pool, torch.bfloat16)
    _need(selected, torch.int32); _need(selected_count, torch.int32); _need(out)
    if lse is not None:
        _need(lse, torch.float32)
    B, Hq, D = q.shape
    _, Hkv, P, _ = k_pool.shape
    params = LsSelectParams(C.sizeof(LsSelectParams),
                            LS_AGG_MAX if group_agg == "max" else LS_AGG_MEAN,
                            int(topk), float(keep_ratio), int(n_sink), int(n_recent),
                            int(max_selected), _score_mode(score_mode, summaries, D))
    n_new = 0
    if new_pages is not None:
        _need(new_pages, torch.int32)
        n_new = int(new_pages.numel())
    pool = _pool(k_pool, int(Hkv), int(P), int(D))
    check(_L.ls_sparse_decode_step_noalloc(q.data_ptr(), LS_DTYPE_BF16, int(Hq),
                                           summaries.data_ptr(), k_pool.data_ptr(),
                                           v_pool.data_ptr(), pool, batch.c(), C.byref(params),
                                           selected.data_ptr(), selected_count.data_ptr(),
                                           float(sm_scale), out.data_ptr(), _DT[out.dtype],
                                           _ptr(lse), _ptr(new_pages), n_new, _stream(stream)))
    return out, lse, selected, selected_count


# ------------------------------------------------------------ learned indexer

def indexer_score_stride(granularity: str, max_units: int) -> int:
    g = LS_SEL_TOKENS if granularity == "tokens" else LS_SEL_BLOCKS
    return int(_L.ls_indexer_score_stride(g, int(max_units)))


def indexer_select_workspace_size(batch_size: int, granularity: str, max_units: int) -> int:
    g = LS_SEL_TOKENS if granularity == "tokens" else LS_SEL_BLOCKS
    return int(_L.ls_indexer_select_workspace_size(int(batch_size), g, int(max_units)))


def indexer_select(q: torch.Tensor, head_weights: torch.Tensor, keys: torch.Tensor,
                   page_size: int, batch: PagedBatch, *, granularity: str, topk: int,
                   max_selected: int, key_scales: Optional[torch.Tensor] = None,
                   cand_blocks: Optional[torch.Tensor] = None,
                   cand_counts: Optional[torch.Tensor] = None,
                   n_sink: int = 0, n_recent: int = 0, token_candidates: bool = False,
                   approx: int = 0,
                   selected: Optional[torch.Tensor] = None,
                   selected_count: Optional[torch.Tensor] = None,
                   scores_out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None,
                   stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Top-k tokens (fp8 indexer keys [pages][P][128], granularity "tokens")
    or blocks (bf16 block-mean keys [pages][128], granularity "blocks") per
    request by the learned-indexer score sum_h w_h ReLU(sigma q_h . k).
    Returns (selected [B][max_selected], counts [B])."""
    _need(q, torch.bfloat16); _need(head_weights, torch.float32); _need(keys)
    B, H, D = q.shape
    dev = q.device
    tokens = granularity == "tokens"
    g = LS_SEL_TOKENS if tokens else LS_SEL_BLOCKS
    if selected is None:
        selected = torch.empty(B, max_selected, dtype=torch.int32, device=dev)
    if selected_count is None:
        selected_count = torch.empty(B, dtype=torch.int32, device=dev)
    _need(selected, torch.int32); _need(selected_count, torch.int32)
    cand_cap = 0
    if cand_blocks is not None:
        _need(cand_blocks, torch.int32); _need(cand_counts, torch.int32)
        cand_cap = int(cand_blocks.shape[-1])
    if key_scales is not None:
        _need(key_scales, torch.float32)
    if scores_out is not None:
        _need(scores_out, torch.float32)
    if tokens and token_candidates:
        max_units = cand_cap + page_size
    elif tokens:
        max_units = (cand_cap if cand_blocks is not None else batch.max_blocks) * page_size
    else:
        max_units = batch.max_blocks
    ws = _workspace(int(_L.ls_indexer_select_workspace_size(B, g, max_units)), dev, workspace)
    params = LsIndexerParams(C.sizeof(LsIndexerParams), g, int(topk), int(n_sink),
                             int(n_recent), int(max_selected),
                             LS_CAND_TOKENS if token_candidates else LS_CAND_BLOCKS,
                             int(approx))
    pool = LsPool(int(keys.shape[0]), 1, int(page_size), int(D), _DT[keys.dtype])
    check(_L.ls_indexer_select(q.data_ptr(), LS_DTYPE_BF16, int(H), head_weights.data_ptr(),
                               keys.data_ptr(), _ptr(key_scales), pool, batch.c(),
                               _ptr(cand_blocks), _ptr(cand_counts), cand_cap, C.byref(params),
                               selected.data_ptr(), selected_count.data_ptr(), _ptr(scores_out),
                               _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return selected, selected_count


# ----------------------------------------------------------------- sparse MLA

def mla_num_splits(max_tokens: int) -> int:
    return int(_L.ls_mla_num_splits(int(max_tokens)))


def sparse_mla_decode_workspace_size(batch_size: int, num_q_heads: int, max_tokens: int) -> int:
    return int(_L.ls_sparse_mla_decode_workspace_size(int(batch_size), int(num_q_heads),
                                                      int(max_tokens)))


def sparse_mla_decode(q: torch.Tensor, latent: torch.Tensor, batch: PagedBatch,
                      selected: Optional[torch.Tensor], selected_count: Optional[torch.Tensor], *,
                      sm_scale: float, out: Optional[torch.Tensor] = None,
                      out_dtype=torch.bfloat16, lse: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None,
                      stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Attention of every query head over the latent rows [pages][P][576] of
    the selected tokens (values: the first 512 entries). selected = None
    attends every cached token. Returns (out [B][H][512], lse or None)."""
    _need(q, torch.bfloat16); _need(latent, torch.bfloat16)
    B, H, Dk = q.shape
    P = int(latent.shape[1])
    dev = q.device
    if out is None:
        out = torch.empty(B, H, 512, dtype=out_dtype, device=dev)
    _need(out)
    if lse is not None:
        _need(lse, torch.float32)
    max_sel = 0
    if selected is not None:
        _need(selected, torch.int32); _need(selected_count, torch.int32)
        max_sel = int(selected.shape[-1])
    cap = max_sel if selected is not None else batch.max_blocks * P
    ws = _workspace(sparse_mla_decode_workspace_size(B, H, cap), dev, workspace)
    pool = LsPool(int(latent.shape[0]), 1, P, int(Dk), LS_DTYPE_BF16)
    check(_L.ls_sparse_mla_decode(q.data_ptr(), LS_DTYPE_BF16, int(H), latent.data_ptr(), pool,
                                  batch.c(), _ptr(selected), _ptr(selected_count), max_sel,
                                  float(sm_scale), out.data_ptr(), _DT[out.dtype], _ptr(lse),
                                  _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return out, lse


# ------------------------------------------------------------------ PQ32

def _fp8_pool(keys: torch.Tensor) -> LsPool:
    return LsPool(int(keys.shape[0]), 1, int(keys.shape[1]), int(keys.shape[2]),
                  LS_DTYPE_FP8_E4M3FN)


def pq_encode(keys: torch.Tensor, key_scales: Optional[torch.Tensor], page_ids: torch.Tensor,
              codebooks: torch.Tensor, codes: torch.Tensor, stream=None) -> torch.Tensor:
    """PQ32 codes [pages][P][32] uint8 of every token of the listed pages
    (nearest of 256 centroids per 4-dim subspace; codebooks bf16 [32][256][4])."""
    _need(keys, torch.float8_e4m3fn); _need(page_ids, torch.int32)
    _need(codebooks, torch.bfloat16); _need(codes, torch.uint8)
    if key_scales is not None:
        _need(key_scales, torch.float32)
    check(_L.ls_pq_encode(keys.data_ptr(), _ptr(key_scales), _fp8_pool(keys), page_ids.data_ptr(),
                          int(page_ids.numel()), codebooks.data_ptr(), codes.data_ptr(),
                          _stream(stream)))
    return codes


def pq_train(keys: torch.Tensor, key_scales: Optional[torch.Tensor], page_ids: torch.Tensor,
             init_tokens: torch.Tensor, iters: int, codebooks: Optional[torch.Tensor] = None,
             stream=None) -> torch.Tensor:
    """k-means codebooks bf16 [32][256][4] over the tokens of the listed pages,
    from centroids at the 256 tokens init_tokens (int32, indices into the
    listed pages' tokens)."""
    _need(keys, torch.float8_e4m3fn); _need(page_ids, torch.int32)
    _need(init_tokens, torch.int32)
    if init_tokens.numel() != 256:
        raise ValueError("init_tokens must hold 256 token indices")
    if key_scales is not None:
        _need(key_scales, torch.float32)
    dev = keys.device
    if codebooks is None:
        codebooks = torch.empty(32, 256, 4, dtype=torch.bfloat16, device=dev)
    _need(codebooks, torch.bfloat16)
    ws = torch.empty(int(_L.ls_pq_train_workspace_size()), dtype=torch.uint8, device=dev)
    check(_L.ls_pq_train(keys.data_ptr(), _ptr(key_scales), _fp8_pool(keys), page_ids.data_ptr(),
                         int(page_ids.numel()), init_tokens.data_ptr(), int(iters),
                         codebooks.data_ptr(), ws.data_ptr(), ws.numel(), _stream(stream)))
    return codebooks


def pq_select(q: torch.Tensor, head_weights: torch.Tensor, codes: torch.Tensor,
              codebooks: torch.Tensor, batch: PagedBatch, n_candidates: int, *,
              candidates: Optional[torch.Tensor] = None,
              counts: Optional[torch.Tensor] = None,
              scores_out: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None,
              stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """The n_candidates tokens of each request's complete pages with the best
    PQ coarse score sum_h w_h ReLU(q_h . decoded key), ascending token ids.
    codes: [pages][P][32] uint8. Returns (candidates [B][n], counts [B])."""
    _need(q, torch.bfloat16); _need(head_weights, torch.float32)
    _need(codes, torch.uint8); _need(codebooks, torch.bfloat16)
    B, H, D = q.shape
    dev = q.device
    if candidates is None:
        candidates = torch.empty(B, max(1, n_candidates), dtype=torch.int32, device=dev)
    if counts is None:
        counts = torch.empty(B, dtype=torch.int32, device=dev)
    _need(candidates, torch.int32); _need(counts, torch.int32)
    if scores_out is not None:
        _need(scores_out, torch.float32)
    P = int(codes.shape[1])
    max_units = batch.max_blocks * P
    ws = _workspace(int(_L.ls_indexer_select_workspace_size(B, LS_SEL_TOKENS, max_units)), dev,
                    workspace)
    pool = LsPool(int(codes.shape[0]), 1, P, 128, LS_DTYPE_FP8_E4M3FN)
    check(_L.ls_pq_select(q.data_ptr(), LS_DTYPE_BF16, int(H), head_weights.data_ptr(),
                          codes.data_ptr(), codebooks.data_ptr(), pool, batch.c(),
                          int(n_candidates), candidates.data_ptr(), counts.data_ptr(),
                          _ptr(scores_out), ws.data_ptr(), ws.numel() * ws.element_size(),
                          _stream(stream)))
    return candidates, counts


def pq_filter_misses(candidates: torch.Tensor, counts: torch.Tensor, scores: torch.Tensor,
                     resident: Optional[torch.Tensor], topk: int, *,
                     kept: Optional[torch.Tensor] = None,
                     kept_counts: Optional[torch.Tensor] = None,
                     misses_kept: Optional[torch.Tensor] = None,
                     stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Miss filter over candidates [B][cap] (counts [B]) with approximate
    scores [B][stride] at token t and a residency bitmap [B][words] int32
    (bit t % 32 of word t / 32; None: every key a miss). Returns (kept
    [B][cap], kept_counts [B], misses_kept [B])."""
    _need(candidates, torch.int32); _need(counts, torch.int32); _need(scores, torch.float32)
    B, cap = candidates.shape
    dev = candidates.device
    if resident is not None:
        _need(resident, torch.int32)
    words = 0 if resident is None else int(resident.shape[1])
    if kept is None:
        kept = torch.empty(B, cap, dtype=torch.int32, device=dev)
    if kept_counts is None:
        kept_counts = torch.empty(B, dtype=torch.int32, device=dev)
    if misses_kept is None:
        misses_kept = torch.empty(B, dtype=torch.int32, device=dev)
    _need(kept, torch.int32); _need(kept_counts, torch.int32); _need(misses_kept, torch.int32)
    check(_L.ls_pq_filter_misses(candidates.data_ptr(), counts.data_ptr(), int(cap),
                                 scores.data_ptr(), int(scores.shape[1]), _ptr(resident), words,
                                 int(B), int(topk), kept.data_ptr(), kept_counts.data_ptr(),
                                 misses_kept.data_ptr(), _stream(stream)))
    return kept, kept_counts, misses_kept


# ------------------------------------------------------------ sink + window

def window_attn_decode(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                       batch: PagedBatch, *, n_sink: int, window: int, sm_scale: float,
                       out: Optional[torch.Tensor] = None, out_dtype=torch.bfloat16,
                       lse: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None,
                       stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Exact attention of every query head over its request's first n_sink
    tokens and last `window` tokens, read in place."""
    _need(q, torch.bfloat16); _need(k_pool, torch.bfloat16); _need(v_pool, torch.bfloat16)
    B, Hq, D = q.shape
    _, Hkv, P, _ = k_pool.shape
    dev = q.device
    if out is None:
        out = torch.empty(B, Hq, D, dtype=out_dtype, device=dev)
    _need(out)
    if lse is not None:
        _need(lse, torch.float32)
    n = int(_L.ls_window_attn_decode_workspace_size(B, Hq, D, batch.max_blocks, int(n_sink),
                                                     int(window)))
    ws = _workspace(n, dev, workspace)
    check(_L.ls_window_attn_decode(q.data_ptr(), LS_DTYPE_BF16, int(Hq), k_pool.data_ptr(),
                                   v_pool.data_ptr(), _pool(k_pool, int(Hkv), int(P), int(D)),
                                   batch.c(), int(n_sink), int(window), float(sm_scale),
                                   out.data_ptr(), _DT[out.dtype], _ptr(lse), ws.data_ptr(),
                                   ws.numel() * ws.element_size(), _stream(stream)))
    return out, lse


# ------------------------------------------------------------ SnapKV-style

def snapkv_select(q_obs: torch.Tensor, k_pool: torch.Tensor, batch: PagedBatch, *,
                  max_len: int, sm_scale: float, n_sink: int, budget: int,
                  scores_out: Optional[torch.Tensor] = None, stream=None):
    """One-time selection of each (request, kv head)'s kept positions from
    the attention of the last prompt queries q_obs [B][W][Hq][D]. Returns
    (selected [B][Hkv][budget], counts [B][Hkv])."""
    _need(q_obs, torch.bfloat16); _need(k_pool, torch.bfloat16)
    B, W, Hq, D = q_obs.shape
    _, Hkv, P, _ = k_pool.shape
    dev = q_obs.device
    sel = torch.empty(B, Hkv, budget, dtype=torch.int32, device=dev)
    cnt = torch.empty(B, Hkv, dtype=torch.int32, device=dev)
    if scores_out is not None:
        _need(scores_out, torch.float32)
    n = int(_L.ls_snapkv_select_workspace_size(B, int(Hkv), int(max_len)))
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
    check(_L.ls_snapkv_select(q_obs.data_ptr(), LS_DTYPE_BF16, int(Hq), int(W), k_pool.data_ptr(),
                              _pool(k_pool, int(Hkv), int(P), int(D)), batch.c(), int(max_len),
                              float(sm_scale), int(n_sink), int(budget), sel.data_ptr(),
                              cnt.data_ptr(), _ptr(scores_out), ws.data_ptr(), ws.numel(),
                              _stream(stream)))
    return sel, cnt


def snapkv_gather(k_pool: torch.Tensor, v_pool: torch.Tensor, batch: PagedBatch,
                  selected: torch.Tensor, counts: torch.Tensor, stream=None):
    """Kept K and V rows, contiguous: [B][Hkv][ceil(budget/16)*16][D] each."""
    _need(k_pool, torch.bfloat16); _need(v_pool, torch.bfloat16)
    _need(selected, torch.int32); _need(counts, torch.int32)
    B, Hkv, budget = selected.shape
    _, _, P, D = k_pool.shape
    pad = -(-budget // 16) * 16
    k_out = torch.empty(B, Hkv, pad, D, dtype=torch.bfloat16, device=k_pool.device)
    v_out = torch.empty_like(k_out)
    check(_L.ls_snapkv_gather(k_pool.data_ptr(), v_pool.data_ptr(),
                              _pool(k_pool, int(Hkv), int(P), int(D)), batch.c(),
                              selected.data_ptr(), counts.data_ptr(), int(budget),
                              k_out.data_ptr(), v_out.data_ptr(), _stream(stream)))
    return k_out, v_out
