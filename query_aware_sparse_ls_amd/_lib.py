"""ctypes declarations of libls.so's C ABI (include/ls.h). Marshalling only."""

from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libls.so")

LS_OK, LS_ERR_INVALID, LS_ERR_UNSUPPORTED, LS_ERR_WORKSPACE, LS_ERR_HIP = range(5)
LS_DTYPE_BF16, LS_DTYPE_FP32, LS_DTYPE_FP8_E4M3FN = 1, 2, 3
LS_AGG_MAX, LS_AGG_MEAN = 0, 1
LS_SEL_TOKENS, LS_SEL_BLOCKS = 0, 1
LS_SCORE_MEAN, LS_SCORE_BOUNDS = 0, 1
LS_CAND_BLOCKS, LS_CAND_TOKENS = 0, 1
(LS_BATCH_BAD_INDPTR, LS_BATCH_NEGATIVE_LENGTH, LS_BATCH_LENGTH_BEYOND_PAGES,
 LS_BATCH_LENGTH_BEYOND_MAX_BLOCKS, LS_BATCH_PAGE_OUT_OF_RANGE) = 1, 2, 4, 8, 16

# every function the header declares, with its ctypes signature
EXPORTS = {}


class LsPool(C.Structure):
    _fields_ = [("num_pages", C.c_int32), ("num_heads", C.c_int32), ("page_size", C.c_int32),
                ("head_dim", C.c_int32), ("dtype", C.c_int32)]


class LsBatch(C.Structure):
    _fields_ = [("batch_size", C.c_int32), ("max_blocks", C.c_int32),
                ("page_indptr", C.c_void_p), ("page_indices", C.c_void_p),
                ("seq_lens", C.c_void_p)]


class LsSelectParams(C.Structure):
    _fields_ = [("struct_size", C.c_int32), ("group_agg", C.c_int32), ("topk", C.c_int32),
                ("keep_ratio", C.c_float), ("n_sink", C.c_int32), ("n_recent", C.c_int32),
                ("max_selected", C.c_int32), ("score_mode", C.c_int32)]


class LsIndexerParams(C.Structure):
    _fields_ = [("struct_size", C.c_int32), ("granularity", C.c_int32), ("topk", C.c_int32),
                ("n_sink", C.c_int32), ("n_recent", C.c_int32), ("max_selected", C.c_int32),
                ("candidates", C.c_int32), ("approx", C.c_int32)]


_P = C.c_void_p
_SIGS = {
    "ls_build_block_summaries": (C.c_int, [_P, _P, LsPool, _P, C.c_int32, _P, C.c_int32, _P]),
    "ls_build_block_bounds": (C.c_int, [_P, LsPool, _P, C.c_int32, _P, _P]),
    "ls_score_select_workspace_size": (C.c_size_t, [C.c_int32, C.c_int32, C.c_int32]),
    "ls_score_select": (C.c_int, [_P, C.c_int32, C.c_int32, _P, LsPool, LsBatch,
                                  C.POINTER(LsSelectParams), _P, _P, _P, _P, C.c_size_t, _P]),
    "ls_sparse_attn_decode_workspace_size": (C.c_size_t, [C.c_int32] * 5),
    "ls_sparse_attn_decode": (C.c_int, [_P, C.c_int32, C.c_int32, _P, _P, LsPool, LsBatch, _P,
                                        _P, C.c_int32, C.c_float, _P, C.c_int32, _P, _P,
                                        C.c_size_t, _P]),
    "ls_sparse_decode_step_workspace_size": (C.c_size_t, [C.c_int32] * 6),
    "ls_sparse_decode_step": (C.c_int, [_P, C.c_int32, C.c_int32, _P, _P, _P, LsPool, LsBatch,
                                        C.POINTER(LsSelectParams), _P, _P, C.c_float, _P,
                                        C.c_int32, _P, _P, C.c_int32, _P, C.c_size_t, _P]),
    "ls_noalloc_scratch_bytes": (C.c_size_t, []),
    "ls_sparse_decode_step_noalloc": (C.c_int, [_P, C.c_int32, C.c_int32, _P, _P, _P, LsPool,
                                                LsBatch, C.POINTER(LsSelectParams), _P, _P,
                                                C.c_float, _P, C.c_int32, _P, _P, C.c_int32, _P]),
    "ls_indexer_score_stride": (C.c_int32, [C.c_int32, C.c_int32]),
    "ls_indexer_select_workspace_size": (C.c_size_t, [C.c_int32, C.c_int32, C.c_int32]),
    "ls_indexer_select": (C.c_int, [_P, C.c_int32, C.c_int32, _P, _P, _P, LsPool, LsBatch, _P,
                                    _P, C.c_int32, C.POINTER(LsIndexerParams), _P, _P, _P, _P,
                                    C.c_size_t, _P]),
    "ls_mla_num_splits": (C.c_int32, [C.c_int32]),
    "ls_sparse_mla_decode_workspace_size": (C.c_size_t, [C.c_int32, C.c_int32, C.c_int32]),
    "ls_sparse_mla_decode": (C.c_int, [_P, C.c_int32, C.c_int32, _P, LsPool, LsBatch, _P, _P,
                                       C.c_int32, C.c_float, _P, C.c_int32, _P, _P, C.c_size_t,
                                       _P]),
    "ls_window_attn_decode_workspace_size": (C.c_size_t, [C.c_int32] * 6),
    "ls_window_attn_decode": (C.c_int, [_P, C.c_int32, C.c_int32, _P, _P, LsPool, LsBatch,
                                        C.c_int32, C.c_int32, C.c_float, _P, C.c_int32, _P, _P,
                                        C.c_size_t, _P]),
    "ls_snapkv_select_workspace_size": (C.c_size_t, [C.c_int32] * 3),
    "ls_snapkv_select": (C.c_int, [_P, C.c_int32, C.c_int32, C.c_int32, _P, LsPool, LsBatch,
                                   C.c_int32, C.c_float, C.c_int32, C.c_int32, _P, _P, _P, _P,
                                   C.c_size_t, _P]),
    "ls_snapkv_gather": (C.c_int, [_P, _P, LsPool, LsBatch, _P, _P, C.c_int32, _P, _P, _P]),
    "ls_pq_encode": (C.c_int, [_P, _P, LsPool, _P, C.c_int32, _P, _P, _P]),
    "ls_pq_train_workspace_size": (C.c_size_t, []),
    "ls_pq_train": (C.c_int, [_P, _P, LsPool, _P, C.c_int32, _P, C.c_int32, _P, _P, C.c_size_t,
                              _P]),
    "ls_pq_select": (C.c_int, [_P, C.c_int32, C.c_int32, _P, _P, _P, LsPool, LsBatch, C.c_int32,
                               _P, _P, _P, _P, C.c_size_t, _P]),
    "ls_pq_filter_misses": (C.c_int, [_P, _P, C.c_int32, _P, C.c_int32, _P, C.c_int32, C.c_int32,
                                      C.c_int32, _P, _P, _P, _P]),
    "ls_last_error": (C.c_char_p, []),
    "ls_version": (C.c_char_p, []),
    "ls_attn_num_splits": (C.c_int32, [C.c_int32]),
    "ls_stream_read_sink_words": (C.c_int32, []),
    "ls_stream_read": (C.c_int, [_P, C.c_size_t, _P, _P]),
    "ls_check_batch": (C.c_int, [LsBatch, C.c_int32, C.c_int32, _P, _P]),
    "ls_debug_enable": (None, [C.c_int32]),
    "ls_debug_enabled": (C.c_int32, []),
    "ls_debug_report": (C.c_int, [_P]),
}

_lib = None


class LsError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libls status {status}: {message}")
        self.status = status


def load() -> C.CDLL:
    """Load the in-tree libls.so; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} not found: build the HIP library first "
            "(python query_aware_sparse_ls_amd/build.py, or __graft_entry__.build())")
    lib = C.CDLL(LIB_PATH)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
        EXPORTS[name] = fn
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != LS_OK:
        raise LsError(status, load().ls_last_error().decode())
