"""Benchmark of the decode-step sparse-attention hot path on one MI355X.

One step = the whole path for one batch of synthetic input:
  1. summaries of the pages that just filled (ls_build_block_summaries),
  2. GQA block scoring + top-k + forced sink/recent, and
  3. split-K attention over the selected blocks,
where 2 + 3 run as ONE persistent launch (ls_sparse_decode_step) by default
(--separate: ls_score_select then ls_sparse_attn_decode). Step 1 runs on a
side stream, forked and joined inside the step: the pages that just filled
are in the recent window, so this step's selection does not read their
summaries.

Workload: Llama-3-8B-shaped decode attention, 16 requests x 32K tokens,
32 query / 8 KV heads, head_dim 128, 16-token pages in a seeded random
permutation page table, bf16 K/V ~ N(0,1) with 2% hot blocks, top-64 blocks
+ 1 sink + 2 recent per KV head, bf16 output.

Timing: R input replicas (each its own pools, summaries, page table and
query), R x step bytes >> the 256 MB Infinity Cache, so consecutive steps
cannot be served from it. One HIP graph holds one step per replica; it is
replayed, and the timed region (hipEvents on the launch stream, bracketed by
device synchronisations) covers exactly `steps` steps. A second, eager pass
puts hipEvents around each library call (behind a GPU-side sleep so the host
enqueues ahead of the device) for the per-call durations the roofline uses.

Prints ONE JSON line.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X published HBM3E bandwidth


def step_bytes(B, Hq, Hkv, D, P, nb, n_sel, n_cand, n_new_pages, out_bytes=2):
    """Algorithmic bytes of one step: what the method itself must move.

    Per (request, kv head): the candidate summaries scanned (n_cand rows of
    D bf16) and the selected blocks' K and V (n_sel * P tokens * D * 2 B * 2).
    Per request: q (Hq * D bf16), output (Hq * D), page table (nb int32).
    Summary update: the new pages' keys read (Hkv * P * D bf16) and their
    summaries written (Hkv * D bf16)."""
    summ = B * Hkv * n_cand * D * 2
    kv = B * Hkv * n_sel * P * D * 2 * 2
    misc = B * Hq * D * 2 + B * Hq * D * out_bytes + B * nb * 4
    upd = n_new_pages * Hkv * (P * D * 2 + D * 2)
    return {"summaries": summ, "selected_kv": kv, "q_out_pagetable": misc, "summary_update": upd,
            "total": summ + kv + misc + upd}


def make_replica(cfg, seed, device):
    import torch
    import query_aware_sparse_ls_amd as ls
    from workloads import make_block_topk_inputs
    inp = make_block_topk_inputs(cfg, device=device, seed=seed)
    P, Hkv, D = cfg.page_size, cfg.num_kv_heads, cfg.head_dim
    B, Hq = cfg.batch, cfg.num_q_heads
    batch = ls.PagedBatch(inp.page_indptr, inp.page_indices, inp.seq_lens, inp.max_blocks())
    # full summary build once (setup, not timed): every complete page
    lens = inp.seq_lens.cpu().tolist()
    indptr = inp.page_indptr.cpu().tolist()
    idx = inp.page_indices.cpu()
    full = torch.cat([idx[indptr[r]:indptr[r] + lens[r] // P] for r in range(B)])
    # the pages that filled at this step: the last page of requests whose
    # length is a multiple of the page size
    new = [int(idx[indptr[r] + lens[r] // P - 1]) for r in range(B) if lens[r] % P == 0]
    summ = torch.zeros(inp.num_pages, Hkv, D, dtype=torch.bfloat16, device=device)
    ls.build_block_summaries(inp.k_pool, full.to(torch.int32).to(device), summ)
    maxsel = min(batch.max_blocks, inp.topk + cfg.n_sink + cfg.n_recent + 1)
    rep = dict(inp=inp, batch=batch, summ=summ,
               ws_step=ls.sparse_decode_step_workspace(B, Hq, Hkv, D, batch.max_blocks,
                                                       maxsel, device),
               new_pages=torch.tensor(new, dtype=torch.int32, device=device),
               sel=torch.empty(B, Hkv, maxsel, dtype=torch.int32, device=device),
               cnt=torch.empty(B, Hkv, dtype=torch.int32, device=device),
               out=torch.empty(B, Hq, D, dtype=torch.bfloat16, device=device),
               ws_sel=torch.empty(ls.score_select_workspace_size(B, Hkv, batch.max_blocks),
                                  dtype=torch.uint8, device=device),
               ws_attn=torch.empty(ls.sparse_attn_decode_workspace_size(
                   B, Hq, D, maxsel, batch.max_blocks), dtype=torch.uint8, device=device),
               maxsel=maxsel)
    return rep


def run_step(rep, cfg, sm_scale, fused=True, side=None, timers=None):
    """One step. With `side`, the summary update runs on that stream, forked
    from and joined back into the current stream. With `timers` (eager timing
    pass) events bracket each call: [update, select(+attend), attend]."""
    import torch
    import query_aware_sparse_ls_amd as ls
    inp = rep["inp"]
    ev = timers
    main = torch.cuda.current_stream()
    if side is not None:
        side.wait_stream(main)
        with torch.cuda.stream(side):
            ls.build_block_summaries(inp.k_pool, rep["new_pages"], rep["summ"])
    else:
        if ev: ev[0].record()
        ls.build_block_summaries(inp.k_pool, rep["new_pages"], rep["summ"])
    if ev: ev[1].record()
    if fused:
        ls.sparse_decode_step(inp.q, rep["summ"], inp.k_pool, inp.v_pool, rep["batch"],
                              topk=inp.topk, n_sink=cfg.n_sink, n_recent=cfg.n_recent,
                              max_selected=rep["maxsel"], sm_scale=sm_scale,
                              group_agg=cfg.group_agg, selected=rep["sel"],
                              selected_count=rep["cnt"], out=rep["out"],
                              workspace=rep["ws_step"])
        if ev: ev[2].record()
    else:
        ls.score_select(inp.q, rep["summ"], cfg.page_size, rep["batch"], topk=inp.topk,
                        n_sink=cfg.n_sink, n_recent=cfg.n_recent, max_selected=rep["maxsel"],
                        group_agg=cfg.group_agg, selected=rep["sel"], selected_count=rep["cnt"],
                        workspace=rep["ws_sel"])
        if ev: ev[2].record()
        ls.sparse_attn_decode(inp.q, inp.k_pool, inp.v_pool, rep["batch"], rep["sel"],
                              rep["cnt"], sm_scale=sm_scale, out=rep["out"],
                              workspace=rep["ws_attn"])
    if ev: ev[3].record()
    if side is not None:
        main.wait_stream(side)


def cpu_baseline(rep, cfg, sm_scale, budget_s: float):
    """Time the oracle (unchanged, one thread) on whole requests of replica 0:
    summary update of the request's new page, scores, selection and attention
    for all its kv heads. Scaled to one call (all requests)."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle
    from workloads import bf16_bits
    inp = rep["inp"]
    P, Hkv, D, G = cfg.page_size, cfg.num_kv_heads, cfg.head_dim, cfg.group
    times, done = [], 0
    with threadpool_limits(1):
        for r in range(cfg.batch):
            L = int(inp.seq_lens[r])
            nb = -(-L // P)
            p0 = int(inp.page_indptr[r])
            pages = inp.page_indices[p0:p0 + nb].long()
            k = bf16_bits(inp.k_pool[pages].contiguous())
            v = bf16_bits(inp.v_pool[pages].contiguous())
            q = bf16_bits(inp.q[r:r + 1].contiguous())
            bv = oracle.BatchView(np.array([0, nb]), np.arange(nb), np.array([L]), P)
            nc = L // P
            summ = np.zeros((nb, Hkv, D), dtype=np.uint16)
            summ[:nc] = oracle.block_summaries(k, np.arange(nc))      # setup: not timed
            t0 = time.perf_counter()
            new = [nc - 1] if L % P == 0 and nc > 0 else []
            if new:
                summ[new] = oracle.block_summaries(k, new)
            oracle.decode_step(q, k, v, bv, num_kv_heads=Hkv, topk=inp.topk, n_sink=cfg.n_sink,
                               n_recent=cfg.n_recent, sm_scale=np.float32(sm_scale),
                               agg=cfg.group_agg, out_dtype="bf16", summaries=summ)
            times.append(time.perf_counter() - t0)
            done += 1
            if sum(times) >= budget_s:
                break
    per_request = sum(times) / done
    per_call = per_request * cfg.batch
    return {"value": 1.0 / per_call, "unit": "calls/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} of {cfg.batch} requests of one call (all {Hkv} kv heads each: "
                      f"new-page summary, scores, top-k selection, attention), float64 NumPy, "
                      f"one thread; scaled x{cfg.batch / done:.1f} to a full call",
            "seconds_per_call": per_call}


def copy_calibration(nbytes: int) -> int:
    """A plain device-to-device copy of nbytes (for scaling PMC byte counters:
    FETCH_SIZE and WRITE_SIZE of this kernel should read nbytes each)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "launches": 3}), flush=True)
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--replicas", type=int, default=8)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--separate", action="store_true",
                    help="time ls_score_select + ls_sparse_attn_decode instead of the fused step")
    ap.add_argument("--copy-calibrate", type=int, default=0, metavar="BYTES")
    args = ap.parse_args(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the sparse-attention path has no multi-GPU mode "
              "(run with --gpus 1).", file=sys.stderr)
        return 2
    if args.copy_calibrate:
        return copy_calibration(args.copy_calibrate)

    import torch
    import query_aware_sparse_ls_amd as ls
    from workloads import LLAMA8B_32K_B16

    cfg = LLAMA8B_32K_B16
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sm_scale = 1.0 / math.sqrt(cfg.head_dim)
    fused = not args.separate
    R = max(1, args.replicas)
    reps = [make_replica(cfg, cfg.seed + i, dev) for i in range(R)]
    torch.cuda.synchronize()
    print(f"# {R} replicas ready, {torch.cuda.memory_allocated() / 2**30:.1f} GiB",
          file=sys.stderr, flush=True)

    inp0 = reps[0]["inp"]
    P, Hkv, D, Hq, B = cfg.page_size, cfg.num_kv_heads, cfg.head_dim, cfg.num_q_heads, cfg.batch
    nb = cfg.context // P
    n_forced = cfg.n_sink + cfg.n_recent
    n_sel = inp0.topk + n_forced
    n_cand = nb - n_forced
    nbytes = step_bytes(B, Hq, Hkv, D, P, nb, n_sel, n_cand, int(reps[0]["new_pages"].numel()))
    main_stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()

    for i in range(max(1, args.warmup)):
        run_step(reps[i % R], cfg, sm_scale, fused, side)
    torch.cuda.synchronize()

    graph = None
    if not args.no_graph:
        cap = torch.cuda.Stream()
        cap.wait_stream(main_stream)
        with torch.cuda.stream(cap):
            for i in range(R):
                run_step(reps[i], cfg, sm_scale, fused, side)
        main_stream.wait_stream(cap)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(R):
                run_step(reps[i], cfg, sm_scale, fused, side)
        torch.cuda.synchronize()
        for _ in range(max(1, args.warmup // R)):
            graph.replay()
        torch.cuda.synchronize()
    print("# timing", file=sys.stderr, flush=True)

    replays = max(1, args.steps // R)
    steps = replays * R
    t0e, t1e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0e.record()
    if graph is not None:
        for _ in range(replays):
            graph.replay()
    else:
        for i in range(steps):
            run_step(reps[i % R], cfg, sm_scale, fused, side)
    t1e.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0e.elapsed_time(t1e) / steps

    # per-call durations: eager, events around each call, GPU given a head start
    n_eager = min(steps, 8 * R)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_eager)]
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2e8))
    for i in range(n_eager):
        run_step(reps[i % R], cfg, sm_scale, fused, None, timers=evs[i])
    torch.cuda.synchronize()
    avg = lambda a, b: sum(e[a].elapsed_time(e[b]) for e in evs) / n_eager
    upd, first, second = avg(0, 1), avg(1, 2), avg(2, 3)

    calls_per_s = 1e3 / ms_step
    gbps = nbytes["total"] / (ms_step * 1e-3) / 1e9
    sel_bytes = B * Hkv * n_sel * 4 + B * Hkv * 4      # selection written (+ counts)
    fused_bytes = nbytes["total"] - nbytes["summary_update"] + sel_bytes
    if fused:
        dom_ms, dom_bytes = first, fused_bytes
        dom_name = "decode_step_kernel (scoring + top-k + split-K attention + merge, one launch)"
    else:
        dom_ms = second
        dom_bytes = nbytes["selected_kv"] + B * Hq * D * 4 + sel_bytes + B * nb * 4
        dom_name = "ls_sparse_attn_decode (split-K attention + combine kernels)"
    dom_gbps = dom_bytes / (dom_ms * 1e-3) / 1e9

    res = {
        "metric": "sparse decode attention calls/sec + achieved HBM GB/s (% of peak) at 8B/32K/B16",
        "value": round(calls_per_s, 1), "unit": "calls/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "batch": B, "context": cfg.context, "q_heads": Hq,
                   "kv_heads": Hkv, "head_dim": D, "page_size": P, "topk": inp0.topk,
                   "n_sink": cfg.n_sink, "n_recent": cfg.n_recent, "replicas": R,
                   "path": "fused" if fused else "separate",
                   "timing": "hip graph" if graph is not None else "eager"},
        "step_bytes": nbytes["total"], "step_bytes_breakdown": nbytes,
        "achieved_GBps_step": round(gbps, 1),
        "pct_of_hbm_peak_step": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "call_ms": ({"summary_update": round(upd, 5), "decode_step": round(first, 5)} if fused
                    else {"summary_update": round(upd, 5), "score_select": round(first, 5),
                          "sparse_attn_decode": round(second, 5)}),
        "roofline": {"kernel": dom_name, "bound": "hbm", "achieved": round(dom_gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(dom_gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "bytes_per_launch": dom_bytes, "avg_launch_ms": round(dom_ms, 5)},
        "wall_s_timed": round(wall, 4),
        "device": torch.cuda.get_device_name(0),
    }
    if not args.no_cpu_baseline:
        print("# cpu baseline", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(reps[0], cfg, sm_scale, args.cpu_seconds)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
