"""The C ABI: the library loads, exports every function include/ls.h declares,
and rejects invalid arguments on the host before any HIP call (these tests
never launch a kernel, so they run without a GPU)."""

import ctypes as C
import os
import re
import subprocess

import pytest

from query_aware_sparse_ls_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ls.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ls_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    lib = _lib.load()
    names = _declared()
    assert {"ls_build_block_summaries", "ls_score_select", "ls_sparse_attn_decode"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    nm = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                        text=True).stdout
    exported = set(re.findall(r" T (ls_\w+)", nm))
    assert set(names) <= exported
    # and the binding declares a signature for each
    assert set(names) == set(_lib._SIGS)


def test_version_and_empty_error():
    lib = _lib.load()
    assert b"gfx950" in lib.ls_version()
    assert b"abi 6" in lib.ls_version()


def _pool(**kw):
    d = dict(num_pages=8, num_heads=8, page_size=16, head_dim=128, dtype=_lib.LS_DTYPE_BF16)
    d.update(kw)
    return _lib.LsPool(**d)


def _batch(**kw):
    d = dict(batch_size=2, max_blocks=4, page_indptr=16, page_indices=32, seq_lens=48)
    d.update(kw)
    return _lib.LsBatch(**d)


def _params(**kw):
    d = dict(struct_size=C.sizeof(_lib.LsSelectParams), group_agg=0, topk=2, keep_ratio=0.0,
             n_sink=1, n_recent=1, max_selected=4)
    d.update(kw)
    return _lib.LsSelectParams(**d)


FAKE = 4096  # never dereferenced: every call below fails validation first


def _score(lib, p=None, pool=None, batch=None, **kw):
    args = dict(q=FAKE, q_dtype=_lib.LS_DTYPE_BF16, num_q_heads=32, summaries=FAKE,
                pool=pool or _pool(), batch=batch or _batch(), sel=FAKE, cnt=FAKE,
                scores=None, ws=None, ws_bytes=0)
    args.update(kw)
    pp = C.byref(p) if p is not None else None
    return lib.ls_score_select(args["q"], args["q_dtype"], args["num_q_heads"], args["summaries"],
                               args["pool"], args["batch"], pp, args["sel"], args["cnt"],
                               args["scores"], args["ws"], args["ws_bytes"], None)


def test_score_select_validation():
    lib = _lib.load()
    assert _score(lib, p=None) == _lib.LS_ERR_INVALID
    assert b"params" in lib.ls_last_error()
    assert _score(lib, p=_params(struct_size=4)) == _lib.LS_ERR_INVALID
    assert _score(lib, p=_params(), pool=_pool(head_dim=96)) == _lib.LS_ERR_UNSUPPORTED
    assert _score(lib, p=_params(), pool=_pool(page_size=8)) == _lib.LS_ERR_UNSUPPORTED
    assert _score(lib, p=_params(), num_q_heads=30) == _lib.LS_ERR_INVALID
    assert _score(lib, p=_params(), num_q_heads=24) == _lib.LS_ERR_UNSUPPORTED  # group 3
    assert _score(lib, p=_params(), num_q_heads=128) == _lib.LS_ERR_UNSUPPORTED  # group 16
    assert b"1, 2, 4, 8" in lib.ls_last_error()
    for hq in (8, 16, 64):                                    # groups 1, 2, 8 pass validation
        assert _score(lib, p=_params(), num_q_heads=hq, ws=FAKE, ws_bytes=16) == \
            _lib.LS_ERR_WORKSPACE
    # Quest bounds only with group 4
    assert _score(lib, p=_params(score_mode=_lib.LS_SCORE_BOUNDS), num_q_heads=16) == \
        _lib.LS_ERR_UNSUPPORTED
    assert b"group 4" in lib.ls_last_error()
    assert _score(lib, p=_params(), q_dtype=_lib.LS_DTYPE_FP32) == _lib.LS_ERR_UNSUPPORTED
    assert _score(lib, p=_params(group_agg=7)) == _lib.LS_ERR_INVALID
    assert _score(lib, p=_params(score_mode=2)) == _lib.LS_ERR_INVALID
    assert b"score_mode" in lib.ls_last_error()
    assert _score(lib, p=_params(score_mode=_lib.LS_SCORE_BOUNDS, max_selected=10000),
                  batch=_batch(max_blocks=9000)) == _lib.LS_ERR_UNSUPPORTED   # bounds <= 8192
    assert _score(lib, p=_params(topk=-3)) == _lib.LS_ERR_INVALID
    assert _score(lib, p=_params(topk=-1, keep_ratio=1.5)) == _lib.LS_ERR_INVALID
    assert _score(lib, p=_params(max_selected=2)) == _lib.LS_ERR_INVALID
    assert b"max_selected" in lib.ls_last_error()
    assert _score(lib, p=_params(), batch=_batch(page_indptr=None)) == _lib.LS_ERR_INVALID
    assert _score(lib, p=_params(), batch=_batch(max_blocks=20000)) == _lib.LS_ERR_UNSUPPORTED
    assert _score(lib, p=_params(), sel=None) == _lib.LS_ERR_INVALID
    # workspace too small (no scores_out given)
    assert _score(lib, p=_params(), ws=FAKE, ws_bytes=16) == _lib.LS_ERR_WORKSPACE
    # empty batch: valid, nothing enqueued
    assert _score(lib, p=_params(), batch=_batch(batch_size=0)) == _lib.LS_OK
    assert lib.ls_last_error() == b""


def test_attention_validation():
    lib = _lib.load()

    def call(**kw):
        a = dict(q=FAKE, q_dtype=_lib.LS_DTYPE_BF16, hq=32, k=FAKE, v=FAKE, pool=_pool(),
                 batch=_batch(), sel=FAKE, cnt=FAKE, max_sel=8, scale=0.1, out=FAKE,
                 out_dtype=_lib.LS_DTYPE_BF16, lse=None, ws=FAKE, ws_bytes=0)
        a.update(kw)
        return lib.ls_sparse_attn_decode(a["q"], a["q_dtype"], a["hq"], a["k"], a["v"], a["pool"],
                                         a["batch"], a["sel"], a["cnt"], a["max_sel"], a["scale"],
                                         a["out"], a["out_dtype"], a["lse"], a["ws"],
                                         a["ws_bytes"], None)

    assert call() == _lib.LS_ERR_WORKSPACE
    assert call(sel=None) == _lib.LS_ERR_INVALID                 # one of the pair missing
    assert call(out_dtype=_lib.LS_DTYPE_FP8_E4M3FN) == _lib.LS_ERR_UNSUPPORTED
    assert call(scale=float("inf")) == _lib.LS_ERR_INVALID
    assert call(pool=_pool(dtype=_lib.LS_DTYPE_FP32)) == _lib.LS_ERR_UNSUPPORTED
    assert call(k=None) == _lib.LS_ERR_INVALID
    assert call(ws=FAKE + 1, ws_bytes=1 << 30) == _lib.LS_ERR_INVALID   # misaligned workspace
    assert call(q=FAKE + 2, ws=FAKE, ws_bytes=1 << 30) == _lib.LS_ERR_INVALID  # misaligned q
    assert call(batch=_batch(batch_size=0)) == _lib.LS_OK
    assert call(hq=24) == _lib.LS_ERR_UNSUPPORTED                 # group 3
    assert call(hq=64) == _lib.LS_ERR_WORKSPACE                   # group 8: valid
    assert call(hq=8, sel=None, cnt=None) == _lib.LS_ERR_WORKSPACE   # group 1, dense
    need = lib.ls_sparse_attn_decode_workspace_size(2, 32, 128, 8, 4)
    assert need >= 2 * 32 * lib.ls_attn_num_splits(8) * 130 * 4
    assert lib.ls_attn_num_splits(67) == 9 and lib.ls_attn_num_splits(2048) == 256


def test_summaries_validation():
    lib = _lib.load()
    f = lib.ls_build_block_summaries
    assert f(FAKE, None, _pool(), FAKE, -1, FAKE, _lib.LS_DTYPE_BF16, None) == _lib.LS_ERR_INVALID
    assert f(FAKE, None, _pool(), FAKE, 0, FAKE, _lib.LS_DTYPE_BF16, None) == _lib.LS_OK
    assert f(FAKE, None, _pool(page_size=12), FAKE, 1, FAKE, 1, None) == _lib.LS_ERR_UNSUPPORTED
    assert f(FAKE, None, _pool(dtype=_lib.LS_DTYPE_FP8_E4M3FN, num_heads=1), FAKE, 1, FAKE, 1,
             None) == _lib.LS_ERR_INVALID                      # fp8 needs scales
    assert f(FAKE, FAKE, _pool(), FAKE, 1, FAKE, 1, None) == _lib.LS_ERR_INVALID  # bf16 + scales
    assert f(FAKE, None, _pool(), FAKE, 1, FAKE, _lib.LS_DTYPE_FP8_E4M3FN,
             None) == _lib.LS_ERR_UNSUPPORTED
    assert f(None, None, _pool(), FAKE, 1, FAKE, 1, None) == _lib.LS_ERR_INVALID


def test_step_validation():
    lib = _lib.load()

    def call(p=None, **kw):
        a = dict(q=FAKE, summ=FAKE, k=FAKE, v=FAKE, pool=_pool(), batch=_batch(), sel=FAKE,
                 cnt=FAKE, scale=0.1, out=FAKE, out_dtype=_lib.LS_DTYPE_BF16, lse=None,
                 new=None, n_new=0, ws=FAKE, ws_bytes=0)
        a.update(kw)
        pp = C.byref(p if p is not None else _params())
        return lib.ls_sparse_decode_step(a["q"], _lib.LS_DTYPE_BF16, 32, a["summ"], a["k"], a["v"],
                                         a["pool"], a["batch"], pp, a["sel"], a["cnt"],
                                         a["scale"], a["out"], a["out_dtype"], a["lse"],
                                         a["new"], a["n_new"], a["ws"], a["ws_bytes"], None)

    assert call() == _lib.LS_ERR_WORKSPACE
    assert call(n_new=-1) == _lib.LS_ERR_INVALID
    assert call(n_new=2) == _lib.LS_ERR_INVALID                  # pages missing
    assert b"new_page_ids" in lib.ls_last_error()
    # a page that just filled must be a forced (recent) block of the call
    assert call(p=_params(n_recent=0), new=FAKE, n_new=2) == _lib.LS_ERR_INVALID
    assert b"n_recent" in lib.ls_last_error()
    assert call(batch=_batch(batch_size=0), new=FAKE, n_new=2) == _lib.LS_OK


def test_noalloc_step_validation():
    """The no-allocation step validates like the step, and rejects on the host
    any shape whose scratch need exceeds the library's fixed array."""
    lib = _lib.load()
    assert lib.ls_noalloc_scratch_bytes() == 32 << 20

    def call(p=None, **kw):
        a = dict(q=FAKE, summ=FAKE, k=FAKE, v=FAKE, pool=_pool(num_pages=1 << 20),
                 batch=_batch(), sel=FAKE, cnt=FAKE, scale=0.1, out=FAKE,
                 out_dtype=_lib.LS_DTYPE_BF16, lse=None, new=None, n_new=0)
        a.update(kw)
        pp = C.byref(p if p is not None else _params())
        return lib.ls_sparse_decode_step_noalloc(a["q"], _lib.LS_DTYPE_BF16, 32, a["summ"],
                                                 a["k"], a["v"], a["pool"], a["batch"], pp,
                                                 a["sel"], a["cnt"], a["scale"], a["out"],
                                                 a["out_dtype"], a["lse"], a["new"], a["n_new"],
                                                 None)

    assert call(n_new=2) == _lib.LS_ERR_INVALID                  # pages missing
    assert call(p=_params(struct_size=3)) == _lib.LS_ERR_INVALID
    assert call(batch=_batch(batch_size=0)) == _lib.LS_OK
    # 1024 (request, kv head) pairs x 8192 blocks: 32 MiB of scores alone
    big = _batch(batch_size=128, max_blocks=8192)
    assert call(batch=big, p=_params(max_selected=8192)) == _lib.LS_ERR_UNSUPPORTED
    assert b"scratch" in lib.ls_last_error()
    need = lib.ls_sparse_decode_step_workspace_size(128, 32, 8, 128, 8192, 8192)
    assert need > lib.ls_noalloc_scratch_bytes()


def test_bounds_validation():
    lib = _lib.load()
    f = lib.ls_build_block_bounds
    assert f(FAKE, _pool(), FAKE, -1, FAKE, None) == _lib.LS_ERR_INVALID
    assert f(FAKE, _pool(), FAKE, 0, FAKE, None) == _lib.LS_OK
    assert f(FAKE, _pool(page_size=12), FAKE, 1, FAKE, None) == _lib.LS_ERR_UNSUPPORTED
    assert f(FAKE, _pool(head_dim=96), FAKE, 1, FAKE, None) == _lib.LS_ERR_UNSUPPORTED
    assert f(FAKE, _pool(dtype=_lib.LS_DTYPE_FP8_E4M3FN), FAKE, 1, FAKE,
             None) == _lib.LS_ERR_UNSUPPORTED                  # bf16 keys only
    assert f(FAKE, _pool(num_heads=0), FAKE, 1, FAKE, None) == _lib.LS_ERR_INVALID
    assert f(None, _pool(), FAKE, 1, FAKE, None) == _lib.LS_ERR_INVALID
    assert f(FAKE, _pool(), FAKE, 1, None, None) == _lib.LS_ERR_INVALID


def _ipool(**kw):
    d = dict(num_pages=8, num_heads=1, page_size=64, head_dim=128,
             dtype=_lib.LS_DTYPE_FP8_E4M3FN)
    d.update(kw)
    return _lib.LsPool(**d)


def _iparams(**kw):
    d = dict(struct_size=C.sizeof(_lib.LsIndexerParams), granularity=_lib.LS_SEL_TOKENS, topk=8,
             n_sink=0, n_recent=0, max_selected=8, candidates=_lib.LS_CAND_BLOCKS, approx=0)
    d.update(kw)
    return _lib.LsIndexerParams(**d)


def test_indexer_token_candidates_and_approx_validation():
    lib = _lib.load()

    def call(p, cand=FAKE, cap=4, pool=None, batch=None):
        return lib.ls_indexer_select(FAKE, _lib.LS_DTYPE_BF16, 64, FAKE, FAKE, None,
                                     pool or _ipool(), batch or _batch(), cand, FAKE, cap,
                                     C.byref(p), FAKE, FAKE, None, None, 0, None)

    assert call(_iparams(candidates=3)) == _lib.LS_ERR_INVALID
    assert call(_iparams(candidates=_lib.LS_CAND_TOKENS), cand=None) == _lib.LS_ERR_INVALID
    assert call(_iparams(candidates=_lib.LS_CAND_TOKENS, granularity=_lib.LS_SEL_BLOCKS),
                pool=_ipool(dtype=_lib.LS_DTYPE_BF16)) == _lib.LS_ERR_INVALID
    assert call(_iparams(approx=3)) == _lib.LS_ERR_INVALID
    assert call(_iparams(approx=2)) == _lib.LS_ERR_INVALID
    assert call(_iparams(approx=1, granularity=_lib.LS_SEL_BLOCKS), cand=None,
                pool=_ipool(dtype=_lib.LS_DTYPE_BF16)) == _lib.LS_ERR_UNSUPPORTED
    assert call(_iparams(candidates=_lib.LS_CAND_TOKENS),
                pool=_ipool(num_pages=1 << 26)) == _lib.LS_ERR_UNSUPPORTED   # rows >= 2^31
    # valid arguments but no workspace: the workspace check is last
    assert call(_iparams(candidates=_lib.LS_CAND_TOKENS, approx=1)) == _lib.LS_ERR_WORKSPACE
    # empty batch: valid, nothing enqueued
    assert call(_iparams(candidates=_lib.LS_CAND_TOKENS),
                batch=_batch(batch_size=0)) == _lib.LS_OK


def test_pq_validation():
    lib = _lib.load()
    enc = lib.ls_pq_encode
    assert enc(FAKE, None, _ipool(), FAKE, -1, FAKE, FAKE, None) == _lib.LS_ERR_INVALID
    assert enc(FAKE, None, _ipool(), FAKE, 0, FAKE, FAKE, None) == _lib.LS_OK
    assert enc(FAKE, None, _ipool(dtype=_lib.LS_DTYPE_BF16), FAKE, 1, FAKE, FAKE,
               None) == _lib.LS_ERR_UNSUPPORTED
    assert enc(FAKE, None, _ipool(head_dim=64), FAKE, 1, FAKE, FAKE, None) == _lib.LS_ERR_UNSUPPORTED
    assert enc(FAKE, None, _ipool(page_size=8), FAKE, 1, FAKE, FAKE, None) == _lib.LS_ERR_UNSUPPORTED
    assert enc(FAKE, None, _ipool(), FAKE, 1, FAKE + 8, FAKE, None) == _lib.LS_ERR_INVALID  # align
    assert enc(FAKE, None, _ipool(), FAKE, 1, FAKE, None, None) == _lib.LS_ERR_INVALID
    tr = lib.ls_pq_train
    ws = lib.ls_pq_train_workspace_size()
    assert ws >= 32 * 256 * 4 * 8 + 32 * 256 * 4
    assert tr(FAKE, None, _ipool(), FAKE, 0, FAKE, 1, FAKE, FAKE, ws, None) == _lib.LS_ERR_INVALID
    assert tr(FAKE, None, _ipool(), FAKE, 4, FAKE, 1001, FAKE, FAKE, ws, None) == _lib.LS_ERR_INVALID
    assert tr(FAKE, None, _ipool(), FAKE, 4, None, 1, FAKE, FAKE, ws, None) == _lib.LS_ERR_INVALID
    assert tr(FAKE, None, _ipool(), FAKE, 4, FAKE, 1, FAKE, FAKE, ws - 1,
              None) == _lib.LS_ERR_WORKSPACE
    assert tr(FAKE, None, _ipool(), FAKE, 4, FAKE, 1, FAKE, FAKE + 16, ws,
              None) == _lib.LS_ERR_INVALID                                   # workspace align
    sel = lib.ls_pq_select

    def s(**kw):
        a = dict(q=FAKE, qd=_lib.LS_DTYPE_BF16, h=64, w=FAKE, codes=FAKE, cb=FAKE, pool=_ipool(),
                 batch=_batch(), n=16, cand=FAKE, cnt=FAKE, ws=None, wsb=0)
        a.update(kw)
        return sel(a["q"], a["qd"], a["h"], a["w"], a["codes"], a["cb"], a["pool"], a["batch"],
                   a["n"], a["cand"], a["cnt"], None, a["ws"], a["wsb"], None)

    assert s(h=48) == _lib.LS_ERR_UNSUPPORTED
    assert s(qd=_lib.LS_DTYPE_FP32) == _lib.LS_ERR_UNSUPPORTED
    assert s(n=-1) == _lib.LS_ERR_INVALID
    assert s(cand=None) == _lib.LS_ERR_INVALID
    assert s(codes=FAKE + 4) == _lib.LS_ERR_INVALID                          # codes 8-byte aligned
    assert s(batch=_batch(max_blocks=5000)) == _lib.LS_ERR_UNSUPPORTED       # > 262144 tokens
    assert s() == _lib.LS_ERR_WORKSPACE
    assert s(batch=_batch(batch_size=0)) == _lib.LS_OK


def test_window_and_snapkv_validation():
    lib = _lib.load()

    def win(**kw):
        a = dict(q=FAKE, hq=32, pool=_pool(), batch=_batch(), ns=4, w=100, scale=0.1,
                 out=FAKE, odt=_lib.LS_DTYPE_BF16, ws=None, wsb=0)
        a.update(kw)
        return lib.ls_window_attn_decode(a["q"], _lib.LS_DTYPE_BF16, a["hq"], FAKE, FAKE,
                                         a["pool"], a["batch"], a["ns"], a["w"], a["scale"],
                                         a["out"], a["odt"], None, a["ws"], a["wsb"], None)

    assert win(ns=-1) == _lib.LS_ERR_INVALID
    assert win(w=-5) == _lib.LS_ERR_INVALID
    assert win(hq=16) == _lib.LS_ERR_UNSUPPORTED                       # group 2
    assert win(pool=_pool(num_pages=1 << 22)) == _lib.LS_ERR_UNSUPPORTED
    assert win(scale=float("nan")) == _lib.LS_ERR_INVALID
    assert win(odt=_lib.LS_DTYPE_FP8_E4M3FN) == _lib.LS_ERR_UNSUPPORTED
    assert win() == _lib.LS_ERR_WORKSPACE
    assert win(batch=_batch(batch_size=0)) == _lib.LS_OK
    need = lib.ls_window_attn_decode_workspace_size(2, 32, 128, 4, 4, 100)
    assert need >= 2 * 32 * 130 * 4

    def snap(**kw):
        a = dict(hq=32, nobs=64, pool=_pool(), batch=_batch(), max_len=64, ns=4, bud=16,
                 sel=FAKE, ws=None, wsb=0)
        a.update(kw)
        return lib.ls_snapkv_select(FAKE, _lib.LS_DTYPE_BF16, a["hq"], a["nobs"], FAKE, a["pool"],
                                    a["batch"], a["max_len"], 0.1, a["ns"], a["bud"], a["sel"],
                                    FAKE, None, a["ws"], a["wsb"], None)

    assert snap(nobs=0) == _lib.LS_ERR_UNSUPPORTED
    assert snap(nobs=65) == _lib.LS_ERR_UNSUPPORTED
    assert snap(max_len=131073) == _lib.LS_ERR_UNSUPPORTED
    assert snap(hq=64) == _lib.LS_ERR_UNSUPPORTED                      # group 8
    assert snap(bud=0) == _lib.LS_ERR_INVALID
    assert snap(sel=None) == _lib.LS_ERR_INVALID
    assert snap() == _lib.LS_ERR_WORKSPACE
    assert snap(batch=_batch(batch_size=0)) == _lib.LS_OK
    assert lib.ls_snapkv_select_workspace_size(2, 8, 64) > 0
    assert lib.ls_snapkv_select_workspace_size(2, 8, 131073) == 0
    g = lib.ls_snapkv_gather
    assert g(FAKE, FAKE, _pool(), _batch(), FAKE, FAKE, 0, FAKE, FAKE, None) == _lib.LS_ERR_INVALID
    assert g(FAKE, FAKE, _pool(), _batch(), None, FAKE, 8, FAKE, FAKE, None) == _lib.LS_ERR_INVALID
    assert g(FAKE, FAKE, _pool(), _batch(batch_size=0), FAKE, FAKE, 8, FAKE, FAKE,
             None) == _lib.LS_OK


def test_stream_read_validation():
    """The stream-read reference rejects null and misaligned arguments on
    the host and launches nothing for zero bytes."""
    lib = _lib.load()
    assert lib.ls_stream_read_sink_words() > 0
    assert lib.ls_stream_read(FAKE, 0, FAKE, None) == _lib.LS_OK
    assert lib.ls_stream_read(None, 64, FAKE, None) == _lib.LS_ERR_INVALID
    assert lib.ls_stream_read(FAKE, 64, None, None) == _lib.LS_ERR_INVALID
    assert lib.ls_stream_read(FAKE + 8, 64, FAKE, None) == _lib.LS_ERR_INVALID
    assert lib.ls_stream_read(FAKE, 40, FAKE, None) == _lib.LS_ERR_INVALID
    assert b"aligned" in lib.ls_last_error()


def test_pq_filter_misses_validation():
    lib = _lib.load()
    F = FAKE

    def call(cap=8, stride=16, words=1, res=F, batch=2, topk=4, cand=F, kept=F):
        return lib.ls_pq_filter_misses(cand, F, cap, F, stride, res, words, batch, topk, kept, F,
                                       None, None)

    assert call(cap=0) == _lib.LS_ERR_UNSUPPORTED
    assert call(cap=4097) == _lib.LS_ERR_UNSUPPORTED
    assert call(stride=0) == _lib.LS_ERR_INVALID
    assert call(words=-1) == _lib.LS_ERR_INVALID
    assert call(topk=0) == _lib.LS_ERR_INVALID
    assert call(batch=-1) == _lib.LS_ERR_INVALID
    assert call(res=None) == _lib.LS_ERR_INVALID          # words > 0 needs a bitmap
    assert call(cand=None) == _lib.LS_ERR_INVALID
    assert call(kept=None) == _lib.LS_ERR_INVALID
    assert call(batch=0, cand=None) == _lib.LS_OK         # empty batch: nothing enqueued


def test_check_batch_and_debug_validation():
    """The batch check rejects a null or misaligned report, a bad pool
    geometry and a bad batch on the host; debug mode switches without a HIP
    call, and reading the debug words needs a host buffer."""
    lib = _lib.load()
    b = _batch()
    assert lib.ls_check_batch(b, 16, 8, None, None) == _lib.LS_ERR_INVALID
    assert lib.ls_check_batch(b, 16, 8, FAKE + 2, None) == _lib.LS_ERR_INVALID
    assert lib.ls_check_batch(b, 0, 8, FAKE, None) == _lib.LS_ERR_INVALID
    assert lib.ls_check_batch(b, 16, 0, FAKE, None) == _lib.LS_ERR_INVALID
    assert lib.ls_check_batch(_batch(batch_size=-1), 16, 8, FAKE, None) == _lib.LS_ERR_INVALID
    assert lib.ls_check_batch(_batch(seq_lens=None), 16, 8, FAKE, None) == _lib.LS_ERR_INVALID
    assert lib.ls_check_batch(_batch(max_blocks=0), 16, 8, FAKE, None) == _lib.LS_ERR_INVALID
    assert lib.ls_debug_report(None) == _lib.LS_ERR_INVALID
    was = lib.ls_debug_enabled()
    try:
        lib.ls_debug_enable(1)
        assert lib.ls_debug_enabled() == 1
        lib.ls_debug_enable(0)
        assert lib.ls_debug_enabled() == 0
    finally:
        lib.ls_debug_enable(was)


@pytest.mark.parametrize("value,want", [("1", 1), ("yes", 1), ("0", 0), ("", 0), (None, 0)])
def test_debug_mode_from_environment(value, want):
    """LS_DEBUG turns debug mode on when the library first looks (a fresh
    process per case; no HIP call is made)."""
    env = {k: v for k, v in os.environ.items() if k != "LS_DEBUG"}
    if value is not None:
        env["LS_DEBUG"] = value
    code = ("import ctypes, sys; lib = ctypes.CDLL(sys.argv[1]); "
            "print(lib.ls_debug_enabled())")
    out = subprocess.run(["python3", "-c", code, _lib.LIB_PATH], env=env, capture_output=True,
                         text=True, check=True).stdout.strip()
    assert out == str(want)
