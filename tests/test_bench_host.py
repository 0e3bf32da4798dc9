"""Host logic of bench.py (no GPU): the one-GPU contract, the repeat-block
summary (medians, ranges, % of the stream read, cost beyond byte time), the
byte account of a ragged step, and the oracle worker processes."""

import math
import subprocess
import sys
import os

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr


def _block(step_ms, stream_ms, dense_ms, order):
    def cell(ms, nbytes):
        return {"median_ms_per_step": ms, "min_ms_per_step": ms, "max_ms_per_step": ms,
                "steps_per_launch": 8, "launches": 20, "bytes_per_step": nbytes}
    return {"order": order, "cells": {"step": cell(step_ms, 100e6),
                                      "stream_read": cell(stream_ms, 100e6),
                                      "dense": cell(dense_ms, 1000e6)}}


def test_repeat_block_summary():
    blocks = [_block(0.040, 0.020, 0.200, ["step", "stream_read", "dense"]),
              _block(0.050, 0.025, 0.220, ["stream_read", "dense", "step"]),
              _block(0.044, 0.022, 0.250, ["dense", "step", "stream_read"])]
    s = bench.summarize_blocks(blocks, "step")
    assert s["blocks"] == 3 and s["launches_per_block"] == 20
    st = s["cells"]["step"]
    assert st["median_ms_per_step"] == pytest.approx(0.044)
    assert st["range_ms_per_step"] == [0.04, 0.05]
    assert st["GBps_at_median"] == pytest.approx(100e6 / 0.044e-3 / 1e9, abs=0.1)
    # the step moves the stream read's bytes in twice its time, in every block
    assert s["pct_of_stream_read"]["step"]["median"] == pytest.approx(50.0)
    assert s["pct_of_stream_read"]["step"]["range"] == [50.0, 50.0]
    # c_b = t_b - t_D * B_b / B_D, per block (paired), in microseconds
    cb = sorted((t - d * 0.1) * 1e3 for t, d in ((0.040, 0.200), (0.050, 0.220),
                                                 (0.044, 0.250)))
    assert s["beyond_byte_time"]["step"]["c_b_us_median"] == pytest.approx(cb[1], abs=1e-3)
    assert s["beyond_byte_time"]["step"]["c_b_us_range"] == pytest.approx([cb[0], cb[2]],
                                                                          abs=1e-3)
    assert "stream_read" not in s["beyond_byte_time"]


def test_ragged_step_byte_account():
    """Two requests of 40 and 32 tokens (page 16), 2 kv heads, D 8: request
    0 has blocks 0, 1 complete and a partial block 2 of 8 tokens; request 1
    has two complete blocks and its last page filled at this step."""
    from workloads.configs import BlockTopKConfig

    cfg = BlockTopKConfig(name="t", batch=2, num_q_heads=4, num_kv_heads=2, head_dim=8,
                          page_size=16, context=0, topk=1, n_sink=1, n_recent=1)

    class Inp:
        pass
    inp = Inp()
    inp.cfg = cfg
    inp.seq_lens = torch.tensor([40, 32], dtype=torch.int32)
    inp.q = torch.zeros(2, 4, 8)
    # selections: r0 g0 {0, 2} (16 + 8 tokens), r0 g1 {1, 2} (16 + 8),
    # r1 g0 {0, 1} (32), r1 g1 {1} (16); the slot past the count is ignored
    sel = torch.tensor([[[0, 2, 7], [1, 2, 7]], [[0, 1, 7], [1, 7, 7]]], dtype=torch.int32)
    cnt = torch.tensor([[2, 2], [2, 1]], dtype=torch.int32)
    b = bench.ragged_pair_bytes(inp, sel, cnt, n_sink=1, n_recent=1)
    assert b["selected_kv"] == (24 + 24 + 32 + 16) * 8 * 2 * 2
    # complete non-forced blocks: r0: block 1 (0 is the sink, 2 the recent
    # partial block); r1: none (0 sink, 1 recent); per kv head
    assert b["summaries"] == 2 * 1 * 8 * 2
    assert b["q_out_pagetable"] == 2 * 2 * 4 * 8 * 2 + (3 + 2) * 4
    assert b["summary_update"] == 1 * 2 * (16 * 8 * 2 + 8 * 2)


def test_oracle_pool_times_the_oracle_on_host_cores():
    from workloads import LLAMA8B_32K_B16, make_block_topk_inputs, reduced
    cfg = reduced(LLAMA8B_32K_B16, batch=2, context=1024)
    inp = make_block_topk_inputs(cfg, device="cpu")
    pool = bench.OraclePool(2)
    try:
        r = bench.cpu_baseline(pool, inp, cfg, requests=[0, 1], topk=inp.topk, keep_ratio=0.0,
                               score_mode="mean", sm_scale=1 / math.sqrt(cfg.head_dim),
                               step_bytes_total=1e6, budget_s=1.0)
    finally:
        pool.close()
    assert r["kind"] == "oracle" and r["cores"] == 2 and r["unit"] == "calls/s"
    assert r["value"] > 0 and r["cpu_model"]
    assert r["single_core_seconds_per_call"] >= r["seconds_per_call"]
    assert r["effective_GBps"] == pytest.approx(1e6 * r["value"] / 1e9)
