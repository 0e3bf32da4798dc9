"""Benchmark of the decode-step sparse-attention hot path on one MI355X.

One step = the whole path for one batch of synthetic input:
  1. summaries of the pages that just filled,
  2. GQA block scoring + top-k + forced sink/recent, and
  3. attention over the selected blocks,
all in ONE library call (ls_sparse_decode_step with the filled pages; one
launch: the pairs' workgroups plus a few that rebuild those summaries --
the pages that just filled are recent blocks, so this step's selection does
not read them). --separate: ls_build_block_summaries on a side stream, then
ls_score_select, then ls_sparse_attn_decode.

Workload: Llama-3-8B-shaped decode attention, 16 requests x 32K tokens,
32 query / 8 KV heads, head_dim 128, 16-token pages in a seeded random
permutation page table, bf16 K/V ~ N(0,1) with 2% hot blocks, top-64 blocks
+ 1 sink + 2 recent per KV head, bf16 output.

Timing (ByteCross App. A and App. E adapted):
  * R input replicas (each its own pools, summaries, page table and query),
    R x step bytes >> the 256 MB Infinity Cache, so consecutive steps
    cannot be served from it.
  * The JSON line's value: exactly --steps steps cycling over the replicas
    in one HIP graph, after --warmup eager steps and one untimed launch of
    the graph; one HIP-event pair on the launch stream, device-synchronised
    on both sides.
  * Repeat blocks: --blocks fresh processes (this script again), started
    one after the other before this process makes its first GPU call. Each
    builds its own replicas and times every cell of the session -- the step,
    a plain streaming read of the step's byte count (ls_stream_read), and
    k = all attention -- in an order rotated by the block index: 10 untimed
    then 20 timed launches of a graph of the cell's steps, median per step.
    Reported: the median over the blocks and their range; % of the stream
    read's bandwidth and the cost beyond byte time at the dense rate
    (c_b = t_b - t_D * B_b / B_D, ByteCross §4.3 and App. D), each paired
    within a block.
  * Per-call durations (roofline): back-to-back eager launches of one call
    between two HIP events, behind a GPU-side sleep. Also one call alone
    (latency), and the same graph on one replica (warm, labelled so).
  * Oracle baseline: the oracle as it stands, in one process per host core
    (os.sched_getaffinity, at most 16; one BLAS thread each; spawned before
    the first GPU call), parallel over (request, kv head) units of one
    replica, for about --cpu-seconds CPU seconds; the CPU model and the
    process count are recorded.

--path ragged: the batch-64 sweep (lengths log-uniform in [2K, 128K], a
shared pool at 70% occupancy): the fused step at keep 1/64, 1/16 and 1/4,
each one cell, k = all, and the stream read; --keep names the cell the
value is for. Bytes per step come from the selections the steps make.

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


def step_bytes(B, Hq, Hkv, D, P, nb, n_sel, n_cand, n_new_pages, out_bytes=2, rows=1):
    """Algorithmic bytes of one step: what the method itself must move.

    Per (request, kv head): the candidate summaries scanned (n_cand * rows
    rows of D bf16: rows = 1 for block means, 2 for Quest bounds) and the
    selected blocks' K and V (n_sel * P tokens * D * 2 B * 2).
    Per request: q (Hq * D bf16), output (Hq * D), page table (nb int32).
    Summary update: the new pages' keys read (Hkv * P * D bf16) and their
    summaries written (Hkv * rows * D bf16)."""
    summ = B * Hkv * n_cand * rows * D * 2
    kv = B * Hkv * n_sel * P * D * 2 * 2
    misc = B * Hq * D * 2 + B * Hq * D * out_bytes + B * nb * 4
    upd = n_new_pages * Hkv * (P * D * 2 + rows * D * 2)
    return {"summaries": summ, "selected_kv": kv, "q_out_pagetable": misc, "summary_update": upd,
            "total": summ + kv + misc + upd}


def make_replica(cfg, seed, device, score_mode="mean"):
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
    if score_mode == "bounds":
        summ = torch.zeros(inp.num_pages, Hkv, 2, D, dtype=torch.bfloat16, device=device)
        ls.build_block_bounds(inp.k_pool, full.to(torch.int32).to(device), summ)
    else:
        summ = torch.zeros(inp.num_pages, Hkv, D, dtype=torch.bfloat16, device=device)
        ls.build_block_summaries(inp.k_pool, full.to(torch.int32).to(device), summ)
    maxsel = min(batch.max_blocks, inp.topk + cfg.n_sink + cfg.n_recent + 1)
    rep = dict(inp=inp, batch=batch, summ=summ, mode=score_mode,
               ws_step=ls.sparse_decode_step_workspace(B, Hq, Hkv, D, batch.max_blocks,
                                                       maxsel, device),
               new_pages=torch.tensor(new, dtype=torch.int32, device=device),
               sel=torch.empty(B, Hkv, maxsel, dtype=torch.int32, device=device),
               cnt=torch.empty(B, Hkv, dtype=torch.int32, device=device),
               out=torch.empty(B, Hq, D, dtype=torch.bfloat16, device=device),
               ws_sel=torch.zeros(ls.score_select_workspace_size(B, Hkv, batch.max_blocks),
                                  dtype=torch.uint8, device=device),
               ws_attn=torch.zeros(ls.sparse_attn_decode_workspace_size(
                   B, Hq, D, maxsel, batch.max_blocks), dtype=torch.uint8, device=device),
               maxsel=maxsel)
    return rep


def call_update(rep):
    """Summaries (or bounds) of the pages that filled at this step."""
    import query_aware_sparse_ls_amd as ls
    if rep["mode"] == "bounds":
        ls.build_block_bounds(rep["inp"].k_pool, rep["new_pages"], rep["summ"])
    else:
        ls.build_block_summaries(rep["inp"].k_pool, rep["new_pages"], rep["summ"])


def call_first(rep, cfg, sm_scale, fused):
    """The whole step (fused), or scoring + selection (separate)."""
    import query_aware_sparse_ls_amd as ls
    inp = rep["inp"]
    if fused:
        ls.sparse_decode_step(inp.q, rep["summ"], inp.k_pool, inp.v_pool, rep["batch"],
                              topk=inp.topk, n_sink=cfg.n_sink, n_recent=cfg.n_recent,
                              max_selected=rep["maxsel"], sm_scale=sm_scale,
                              group_agg=cfg.group_agg, selected=rep["sel"],
                              selected_count=rep["cnt"], out=rep["out"],
                              new_pages=rep["new_pages"], workspace=rep["ws_step"],
                              score_mode=rep["mode"])
    else:
        ls.score_select(inp.q, rep["summ"], cfg.page_size, rep["batch"], topk=inp.topk,
                        n_sink=cfg.n_sink, n_recent=cfg.n_recent, max_selected=rep["maxsel"],
                        group_agg=cfg.group_agg, selected=rep["sel"], selected_count=rep["cnt"],
                        workspace=rep["ws_sel"], score_mode=rep["mode"])


def call_second(rep, sm_scale):
    """Attention over the selection (separate path only)."""
    import query_aware_sparse_ls_amd as ls
    inp = rep["inp"]
    ls.sparse_attn_decode(inp.q, inp.k_pool, inp.v_pool, rep["batch"], rep["sel"], rep["cnt"],
                          sm_scale=sm_scale, out=rep["out"], workspace=rep["ws_attn"])


def run_step(rep, cfg, sm_scale, fused=True, side=None):
    """One step. Fused: ONE library call, which also rebuilds the summaries
    of the pages that filled at this step (they are recent blocks, so this
    step does not score them). Separate: the summary update on `side`
    (forked from and joined back into the current stream), then selection,
    then attention."""
    import torch
    if fused:
        call_first(rep, cfg, sm_scale, fused)
        return
    main = torch.cuda.current_stream()
    if side is not None:
        side.wait_stream(main)
        with torch.cuda.stream(side):
            call_update(rep)
    else:
        call_update(rep)
    call_first(rep, cfg, sm_scale, fused)
    call_second(rep, sm_scale)
    if side is not None:
        main.wait_stream(side)


def per_call_ms(reps, cfg, sm_scale, fused, n):
    """Mean duration of each library call of the step: n launches of one call
    back to back (cycling over the replicas) between two HIP events on the
    launch stream, queued behind a GPU-side sleep so that the host is ahead
    of the device and the launches run back to back."""
    import torch
    R = len(reps)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2e8))
    ev[0].record()
    if not fused:   # the fused call rebuilds them itself
        for i in range(n):
            call_update(reps[i % R])
    ev[1].record()
    for i in range(n):
        call_first(reps[i % R], cfg, sm_scale, fused)
    ev[2].record()
    if not fused:
        for i in range(n):
            call_second(reps[i % R], sm_scale)
    ev[3].record()
    torch.cuda.synchronize()
    return [ev[a].elapsed_time(ev[a + 1]) / n for a in range(3)]


# ------------------------------------------------------- oracle baseline ----
#
# The oracle, as it stands, on the host's cores: one process per core (one
# BLAS thread each), parallel over (request, kv head) units. The processes are
# spawned before this process touches the GPU; later they read a sample of
# one replica's inputs from memory-mapped files, prepare their units (the
# summaries of the complete pages: setup, not timed), meet at a barrier, and
# run passes over their units until their share of the time budget is spent.

def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _oracle_units(job, barrier):
    """Prepare the job's units, wait for the others, then time passes over
    them. A unit (r, g) is kv head g of sampled request r alone: its G query
    heads, its K/V pages and its summaries (GQA groups do not interact)."""
    import numpy as np
    import oracle
    d, m = job["dir"], job["meta"]
    kmm = np.load(os.path.join(d, "k.npy"), mmap_mode="r")     # [pages][Hkv][P][D] bf16 bits
    vmm = np.load(os.path.join(d, "v.npy"), mmap_mode="r")
    q = np.load(os.path.join(d, "q.npy"))                       # [requests][Hq][D] bf16 bits
    off, lens, P, G = m["page_offsets"], m["seq_lens"], m["page_size"], m["group"]
    bounds = m["score_mode"] == "bounds"
    build = oracle.block_bounds if bounds else oracle.block_summaries
    units = []
    for r, g in job["units"]:
        L = int(lens[r])
        nb, nc = -(-L // P), L // P
        k = kmm[off[r]:off[r] + nb, g:g + 1]
        v = vmm[off[r]:off[r] + nb, g:g + 1]
        qu = np.ascontiguousarray(q[r:r + 1, g * G:(g + 1) * G])
        bv = oracle.BatchView(np.array([0, nb]), np.arange(nb), np.array([L]), P)
        summ = np.zeros((nb, 1) + ((2,) if bounds else ()) + (k.shape[-1],), dtype=np.uint16)
        if nc:
            summ[:nc] = build(k, np.arange(nc))
        topk = m["topk"]
        if topk < 0:
            topk = oracle.topk_from_keep_ratio(nb, nc, m["keep_ratio"], m["n_sink"], m["n_recent"])
        units.append((L, nc, k, v, qu, bv, summ, topk))
    barrier.wait()
    t0 = time.perf_counter()
    passes, el = 0, 0.0
    while units:
        for L, nc, k, v, qu, bv, summ, topk in units:
            if L % P == 0 and nc:               # the page that filled at this step
                summ[[nc - 1]] = build(k, [nc - 1])
            oracle.decode_step(qu, k, v, bv, num_kv_heads=1, topk=topk, n_sink=m["n_sink"],
                               n_recent=m["n_recent"], sm_scale=np.float32(m["sm_scale"]),
                               agg=m["agg"], out_dtype=m["out_dtype"], summaries=summ,
                               score_mode=m["score_mode"])
        passes += 1
        el = time.perf_counter() - t0
        if el >= job["budget_s"]:
            break
    return {"passes": passes, "seconds": el, "units": len(units)}


_ONE_THREAD_VARS = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")


def _oracle_worker(w, jobs, results, barrier):
    # one thread per process (also set in the environment the process was
    # started with); limit whatever pools NumPy and the oracle loaded
    for var in _ONE_THREAD_VARS:
        os.environ[var] = "1"
    import numpy  # noqa: F401
    import oracle  # noqa: F401
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        while True:
            job = jobs.get()
            if job is None:
                return
            try:
                res = _oracle_units(job, barrier)
            except BaseException as e:      # report it; never leave the others waiting
                res = {"error": repr(e)}
                barrier.abort()
            res["worker"] = w
            results.put(res)


class OraclePool:
    """Oracle worker processes (spawned: fresh interpreters that never touch
    the GPU). Start it before the first GPU call of this process."""

    def __init__(self, n: int):
        import multiprocessing as mp
        ctx = mp.get_context("spawn")
        self.n = n
        self.barrier = ctx.Barrier(n + 1)
        self.jobs = [ctx.Queue() for _ in range(n)]
        self.results = ctx.Queue()
        self.procs = [ctx.Process(target=_oracle_worker,
                                  args=(w, self.jobs[w], self.results, self.barrier), daemon=True)
                      for w in range(n)]
        # the children inherit this environment: one BLAS / OpenMP thread each
        saved = {v: os.environ.get(v) for v in _ONE_THREAD_VARS}
        os.environ.update({v: "1" for v in _ONE_THREAD_VARS})
        try:
            for p in self.procs:
                p.start()
        finally:
            for v, x in saved.items():
                if x is None:
                    os.environ.pop(v, None)
                else:
                    os.environ[v] = x

    def run(self, job_dir: str, meta: dict, units, cost, budget_s: float,
            timeout_s: float = 600.0):
        """Deal `units` to the workers, the costliest first, each to the
        worker with the least cost so far (cost: e.g. the unit's tokens);
        returns the workers' {passes, seconds, units} records and the wall
        time from the barrier."""
        per, load = [[] for _ in range(self.n)], [0.0] * self.n
        for u, c in sorted(zip(units, cost), key=lambda uc: -uc[1]):
            w = load.index(min(load))
            per[w].append(u)
            load[w] += c
        for w in range(self.n):
            self.jobs[w].put({"dir": job_dir, "meta": meta, "units": per[w],
                              "budget_s": budget_s})
        self.barrier.wait(timeout=timeout_s)
        t0 = time.perf_counter()
        recs = [self.results.get(timeout=timeout_s) for _ in range(self.n)]
        wall = time.perf_counter() - t0
        errs = [r["error"] for r in recs if "error" in r]
        if errs:
            raise RuntimeError(f"oracle worker failed: {errs[0]}")
        return recs, wall

    def close(self):
        for q in self.jobs:
            q.put(None)
        for p in self.procs:
            p.join(timeout=30)


def oracle_workers() -> int:
    """Worker processes for the oracle: the cores this process may run on
    (sched_getaffinity), at most 16 (one GPU's share of a host's cores)."""
    return max(1, min(len(os.sched_getaffinity(0)), 16))


def write_oracle_sample(dirpath: str, inp, requests):
    """The listed requests' pages (logical order) of one replica as .npy
    files: k, v [pages][Hkv][P][D] and q [requests][Hq][D], bf16 bits."""
    import numpy as np
    import torch
    P = inp.cfg.page_size
    indptr = inp.page_indptr.cpu().tolist()
    lens = inp.seq_lens.cpu().tolist()
    ids, offs = [], [0]
    for r in requests:
        nb = -(-int(lens[r]) // P)
        ids.append(inp.page_indices[indptr[r]:indptr[r] + nb].long())
        offs.append(offs[-1] + nb)
    ids = torch.cat(ids)
    for name, pool in (("k", inp.k_pool), ("v", inp.v_pool)):
        arr = np.lib.format.open_memmap(os.path.join(dirpath, name + ".npy"), mode="w+",
                                        dtype=np.uint16, shape=(len(ids),) + tuple(pool.shape[1:]))
        for s in range(0, len(ids), 4096):
            part = pool[ids[s:s + 4096]].view(torch.int16).cpu().numpy().view(np.uint16)
            arr[s:s + len(part)] = part
        arr.flush()
        del arr
    q = inp.q[torch.tensor(list(requests), device=inp.q.device)]
    np.save(os.path.join(dirpath, "q.npy"), q.view(torch.int16).cpu().numpy().view(np.uint16))
    return offs[:-1], [int(lens[r]) for r in requests]


def cpu_baseline(pool: OraclePool, inp, cfg, *, requests, topk, keep_ratio, score_mode,
                 sm_scale, step_bytes_total, budget_s):
    """Oracle calls/s on the host cores over a sample of one replica's
    requests (every kv head of each): wall seconds per pass over the sample,
    scaled by batch / sampled requests to one call. A single-core time per
    call is the sum of the workers' per-pass times, scaled the same way."""
    import tempfile
    requests = list(requests)
    G = cfg.num_q_heads // cfg.num_kv_heads
    with tempfile.TemporaryDirectory(prefix="ls_oracle_") as d:
        offs, lens = write_oracle_sample(d, inp, requests)
        meta = {"page_offsets": offs, "seq_lens": lens, "page_size": cfg.page_size, "group": G,
                "topk": int(topk), "keep_ratio": float(keep_ratio), "n_sink": cfg.n_sink,
                "n_recent": cfg.n_recent, "sm_scale": float(sm_scale), "agg": cfg.group_agg,
                "out_dtype": "fp32" if cfg.out_dtype == "fp32" else "bf16",
                "score_mode": score_mode}
        units = [(i, g) for i in range(len(requests)) for g in range(cfg.num_kv_heads)]
        recs, wall = pool.run(d, meta, units, [lens[i] for i, _ in units], budget_s / pool.n)
    busy = [r for r in recs if r["units"]]
    per_pass = [r["seconds"] / r["passes"] for r in busy]
    scale = cfg.batch / len(requests)
    par = max(per_pass) * scale
    single = sum(per_pass) * scale
    cpu_s = sum(r["seconds"] for r in busy)
    return {"value": 1.0 / par, "unit": "calls/s", "cores": pool.n, "kind": "oracle",
            "cpu_model": cpu_model(), "affinity_cores": len(os.sched_getaffinity(0)),
            "seconds_per_call": par, "single_core_seconds_per_call": single,
            "effective_GBps": step_bytes_total / par / 1e9,
            "sample": (f"{len(requests)} of {cfg.batch} requests of one replica x "
                       f"{cfg.num_kv_heads} kv heads = {len(units)} (request, kv head) units "
                       f"over {pool.n} processes (one BLAS thread each, units dealt by "
                       f"length), "
                       f"{min(r['passes'] for r in busy)}-{max(r['passes'] for r in busy)} passes "
                       f"each, {cpu_s:.1f} CPU-s in {wall:.1f} s wall; per unit: the page that "
                       f"filled, {'Quest bound' if score_mode == 'bounds' else 'block'} scores, "
                       f"selection and attention, float64 NumPy; one call = the slowest "
                       f"process's time per pass x {scale:g}")}


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


PROFILE_DIR = os.path.join(ROOT, "profiles")
CSRC_DIR = os.path.join(ROOT, "query_aware_sparse_ls_amd", "csrc")


def library_source_digest() -> str:
    """sha256 over every HIP/C++ source of the library (names and bytes, in
    name order). A traffic figure taken from PMC counters is reported only
    while this digest equals the one stored next to it."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC_DIR)):
        if name.endswith((".hip", ".h", ".cpp")):
            h.update(name.encode())
            with open(os.path.join(CSRC_DIR, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def stored_traffic(kernel_key: str):
    """HBM bytes per launch of `kernel_key` from the committed PMC summary
    (profiles/<kernel_key>.md, a JSON object on its `traffic-json:` line),
    or None when there is none or the library sources changed since."""
    path = os.path.join(PROFILE_DIR, kernel_key + ".md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("traffic-json:"):
            rec = json.loads(line.split(":", 1)[1])
            if rec.get("source_sha256") != library_source_digest():
                return None
            return rec
    return None


def _kernel_stats(csv_path: str):
    import csv
    rows = {}
    for row in csv.DictReader(open(csv_path)):
        rows[row["Name"]] = {"calls": int(row["Calls"]), "avg_us": float(row["AverageNs"]) / 1e3,
                             "min_us": float(row["MinNs"]) / 1e3,
                             "max_us": float(row["MaxNs"]) / 1e3}
    return rows


def _counter_per_dispatch(csv_path: str, counter: str, match: str):
    """Mean value of `counter` over the dispatches whose kernel name contains
    `match`, with the dispatch count and the grid size seen."""
    import csv
    vals, grids = [], set()
    for row in csv.DictReader(open(csv_path)):
        if row["Counter_Name"] == counter and match in row["Kernel_Name"]:
            vals.append(float(row["Counter_Value"]))
            grids.add(int(row["Grid_Size"]))
    if not vals:
        raise SystemExit(f"no {counter} samples for kernels matching {match!r} in {csv_path}")
    return sum(vals) / len(vals), len(vals), sorted(grids)


def summarize_profiles(args) -> int:
    """Write profiles/<kernel_key>.md from rocprofv3 CSV output: the
    kernel-trace statistics, FETCH_SIZE / WRITE_SIZE per dispatch of the
    kernel, and the same counters for a plain copy of a known byte count,
    which scale the kernel's counters to bytes. `--kernel-match` may list
    several kernels separated by '|' (the launches of one library call): the
    traffic is then the sum of their per-dispatch means."""
    key = args.kernel_key
    matches = args.kernel_match.split("|")
    stats = _kernel_stats(os.path.join(args.kt_dir, "run_kernel_stats.csv"))
    per = []
    for m in matches:
        f, nf, grid = _counter_per_dispatch(os.path.join(args.fetch_dir, "run_counter_collection.csv"),
                                            "FETCH_SIZE", m)
        w, nw, _ = _counter_per_dispatch(os.path.join(args.write_dir, "run_counter_collection.csv"),
                                         "WRITE_SIZE", m)
        per.append((m, f, nf, grid, w, nw))
    fetch = sum(p[1] for p in per)
    write = sum(p[4] for p in per)
    cb = args.copy_bytes
    cfetch, _, _ = _counter_per_dispatch(os.path.join(args.copy_fetch_dir, "run_counter_collection.csv"),
                                         "FETCH_SIZE", "copyBuffer")
    cwrite, _, _ = _counter_per_dispatch(os.path.join(args.copy_write_dir, "run_counter_collection.csv"),
                                         "WRITE_SIZE", "copyBuffer")
    f_scale = cb / (cfetch * 1024.0)      # bytes per counted KiB
    w_scale = cb / (cwrite * 1024.0)
    traffic = fetch * 1024.0 * f_scale + write * 1024.0 * w_scale
    ours = {n: v for n, v in stats.items() if "ls::" in n}
    lines = [f"# {key}: kernel time and HBM traffic", "",
             f"Workload: {args.workload}", "",
             "## Kernel trace (rocprofv3 --kernel-trace --stats)", "",
             "```", args.kt_cmd, "```", "",
             "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for n, v in sorted(ours.items(), key=lambda kv: -kv[1]["avg_us"] * kv[1]["calls"]):
        lines.append(f"| `{n[:110]}` | {v['calls']} | {v['avg_us']:.2f} | {v['min_us']:.2f} | "
                     f"{v['max_us']:.2f} |")
    lines += ["", "## HBM counters per dispatch (rocprofv3 --pmc, one counter per run)", "",
              "```", args.fetch_cmd, args.write_cmd, args.copy_fetch_cmd, args.copy_write_cmd, "```", ""]
    for m, f, nf, grid, w, nw in per:
        lines.append(f"* kernel `{m}` (grid {grid}): FETCH_SIZE {f:.1f} KiB over {nf} dispatches, "
                     f"WRITE_SIZE {w:.1f} KiB over {nw} dispatches")
    lines += [f"* plain copy (`__amd_rocclr_copyBuffer`, {cb} bytes read and written): "
              f"FETCH_SIZE {cfetch:.1f} KiB, WRITE_SIZE {cwrite:.1f} KiB",
              f"* scale (copy bytes / counter bytes): FETCH_SIZE x {f_scale:.4f}, "
              f"WRITE_SIZE x {w_scale:.4f}",
              f"* traffic per launch{' (sum over the kernels)' if len(per) > 1 else ''}: "
              f"{fetch * 1024 * f_scale:.0f} B read + "
              f"{write * 1024 * w_scale:.0f} B written = {traffic:.0f} B", ""]
    rec = {"kernel": args.kernel_match, "traffic_bytes": round(traffic),
           "read_bytes": round(fetch * 1024 * f_scale),
           "write_bytes": round(write * 1024 * w_scale), "fetch_kib": fetch, "write_kib": write,
           "copy_bytes": cb, "copy_fetch_kib": cfetch, "copy_write_kib": cwrite,
           "source_sha256": library_source_digest()}
    lines.append("traffic-json: " + json.dumps(rec))
    os.makedirs(PROFILE_DIR, exist_ok=True)
    with open(os.path.join(PROFILE_DIR, key + ".md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps(rec))
    return 0



# ------------------------------------------------- learned-indexer paths ----

def indexer_step_bytes(cfg, coarse: bool, pq: bool = False, kept_mean=None):
    """Algorithmic bytes of one learned-indexer step (per call, all requests).
    Token keys are fp8 (1 B per dim) with one fp32 scale per token; latent
    rows are 576 bf16 (the whole row is read: key = all 576 dims). PQ32: 32 B
    of codes per complete-page token, then the candidates' keys, and the
    codes of the pages that filled this step (keys read, codes written).
    With the miss filter (kept_mean: kept candidates per request, measured),
    the coarse scores are written and read back, the filter reads the
    residency bits, and only the kept candidates' keys are read."""
    B, L, H, D, P = cfg.batch, cfg.context, cfg.index_heads, cfg.index_dim, cfg.page_size
    k = cfg.topk_tokens
    dk = cfg.kv_lora_dim + cfg.rope_dim
    d = {"q_idx_w": B * H * (D * 2 + 4), "selection": B * k * 4,
         "mla_kv": B * k * dk * 2, "q_mla": B * cfg.mla_heads * dk * 2,
         "out": B * cfg.mla_heads * cfg.kv_lora_dim * 2}
    if pq:
        C = cfg.n_candidates
        d["pq_codes"] = B * (L // P) * P * 32
        d["candidates"] = B * C * 4 * 2                   # written, then read
        d["candidate_keys"] = B * (C + L % P) * (D + 4)
        d["encode_new_pages"] = B * P * (D + 4 + 32)
        if kept_mean is not None:
            d["candidate_keys"] = int(round(B * (kept_mean + L % P) * (D + 4)))
            d["coarse_scores"] = B * (L // P) * P * 4 + B * C * 4   # written; candidates' read
            d["residency_bits"] = B * C * 4
            d["kept"] = B * C * 4 * 2
    elif coarse:
        nb = L // P
        kb = cfg.coarse_topk_blocks + 1                  # + the forced last block
        d["coarse_summaries"] = B * (nb - 1) * D * 2     # every complete, non-forced block
        d["block_selection"] = B * kb * 4
        d["candidate_keys"] = B * kb * P * (D + 4)
    else:
        d["indexer_keys"] = B * L * (D + 4)
    d["total"] = sum(d.values())
    return d


def bench_indexer(args, coarse: bool, pq: bool = False) -> int:
    """Time the learned-indexer path: token top-k over every cached token
    (128K workload), coarse block top-k -> exact token top-k among the kept
    blocks (950K workload), or PQ32 coarse top-C -> exact rerank of the
    candidates (128K workload); then sparse MLA over the selected tokens."""
    import numpy as np
    import torch
    import query_aware_sparse_ls_amd as ls
    from workloads import (COARSE_TO_FINE_950K, INDEXER_128K, PQ32_128K, indexer_queries,
                           make_indexer_inputs, pq_init_tokens)
    cfg = PQ32_128K if pq else (COARSE_TO_FINE_950K if coarse else INDEXER_128K)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, P, k = cfg.batch, cfg.page_size, cfg.topk_tokens
    nb = cfg.context // P
    sm = 1.0 / math.sqrt(cfg.kv_lora_dim + cfg.rope_dim)
    R = max(1, args.replicas or 8)
    reps = []
    base = make_indexer_inputs(cfg, device=dev)
    summ = None
    codes = codebooks = None
    if pq:
        # one cache with its codebooks (trained on it) and codes, built once
        # (setup, not timed); replicas differ in their queries
        npg = base.idx_keys.shape[0]
        ids = torch.arange(npg, dtype=torch.int32, device=dev)
        init = pq_init_tokens(npg * P, cfg.seed).to(dev)
        codebooks = ls.pq_train(base.idx_keys, base.idx_scale, ids, init, cfg.kmeans_iters)
        codes = torch.zeros(npg, P, 32, dtype=torch.uint8, device=dev)
        ls.pq_encode(base.idx_keys, base.idx_scale, ids, codebooks, codes)
        lens = base.seq_lens.cpu().tolist()
        indptr = base.idx_indptr.cpu().tolist()
        idx = base.idx_indices.cpu()
        new_pages = torch.tensor([int(idx[indptr[r] + lens[r] // P - 1]) for r in range(B)
                                  if lens[r] % P == 0], dtype=torch.int32, device=dev)
    if coarse:
        # one cache; replicas differ in their queries and own a copy of the
        # block means (read in full every step)
        npg = base.idx_keys.shape[0]
        summ = torch.zeros(npg, cfg.index_dim, dtype=torch.bfloat16, device=dev)
        ls.build_block_summaries(base.idx_keys, torch.arange(npg, dtype=torch.int32, device=dev),
                                 summ, key_scales=base.idx_scale)
    for i in range(R):
        if coarse or pq:
            q_idx, w, q_mla = indexer_queries(cfg, cfg.seed + 7 * i, dev)
            inp = base
            rep = dict(q_idx=q_idx, w=w, q_mla=q_mla)
            if coarse:
                rep["summ"] = summ.clone()
        else:
            inp = base if i == 0 else make_indexer_inputs(cfg, device=dev, seed=cfg.seed + 7 * i)
            rep = dict(q_idx=inp.q_idx, w=inp.head_w, q_mla=inp.q_mla)
        rep.update(inp=inp,
                   ib=ls.PagedBatch(inp.idx_indptr, inp.idx_indices, inp.seq_lens, nb),
                   kb=ls.PagedBatch(inp.kv_indptr, inp.kv_indices, inp.seq_lens, nb),
                   sel=torch.empty(B, k, dtype=torch.int32, device=dev),
                   cnt=torch.empty(B, dtype=torch.int32, device=dev),
                   out=torch.empty(B, cfg.mla_heads, cfg.kv_lora_dim, dtype=torch.bfloat16,
                                   device=dev),
                   ws_mla=torch.zeros(ls.sparse_mla_decode_workspace_size(B, cfg.mla_heads, k),
                                      dtype=torch.uint8, device=dev))
        if pq and args.miss_filter:
            # the keys a previous step left resident: a seeded Bernoulli mask
            # with the given hit rate (no cache is simulated)
            hits = np.random.default_rng(cfg.seed + 101 * i).random((B, nb * P)) < args.miss_filter
            words = (nb * P + 31) // 32
            padded = np.zeros((B, words * 32), dtype=np.uint64)
            padded[:, :nb * P] = hits
            w32 = (padded.reshape(B, words, 32) << np.arange(32, dtype=np.uint64)).sum(-1)
            rep.update(res=torch.from_numpy(w32.astype(np.uint32).view(np.int32)).to(dev),
                       csc=torch.empty(B, ls.indexer_score_stride("tokens", nb * P),
                                       device=dev),
                       kept=torch.empty(B, cfg.n_candidates, dtype=torch.int32, device=dev),
                       kcnt=torch.empty(B, dtype=torch.int32, device=dev),
                       mk=torch.empty(B, dtype=torch.int32, device=dev))
        if pq:
            C = cfg.n_candidates
            rep.update(cand=torch.empty(B, C, dtype=torch.int32, device=dev),
                       ccnt=torch.empty(B, dtype=torch.int32, device=dev),
                       ws_c=torch.empty(ls.indexer_select_workspace_size(B, "tokens", nb * P),
                                        dtype=torch.uint8, device=dev),
                       ws_t=torch.empty(ls.indexer_select_workspace_size(B, "tokens", C + P),
                                        dtype=torch.uint8, device=dev))
        elif coarse:
            kb = cfg.coarse_topk_blocks + 2
            rep.update(bsel=torch.empty(B, kb, dtype=torch.int32, device=dev),
                       bcnt=torch.empty(B, dtype=torch.int32, device=dev),
                       ws_b=torch.empty(ls.indexer_select_workspace_size(B, "blocks", nb),
                                        dtype=torch.uint8, device=dev),
                       ws_t=torch.empty(ls.indexer_select_workspace_size(B, "tokens", kb * P),
                                        dtype=torch.uint8, device=dev))
        else:
            rep["ws_t"] = torch.empty(ls.indexer_select_workspace_size(B, "tokens", nb * P),
                                      dtype=torch.uint8, device=dev)
        reps.append(rep)
    torch.cuda.synchronize()
    print(f"# {R} replicas ready, {torch.cuda.memory_allocated() / 2**30:.1f} GiB",
          file=sys.stderr, flush=True)

    def c_blocks(rp):
        ls.indexer_select(rp["q_idx"], rp["w"], rp["summ"], P, rp["ib"], granularity="blocks",
                          topk=cfg.coarse_topk_blocks, n_recent=1,
                          max_selected=cfg.coarse_topk_blocks + 2, selected=rp["bsel"],
                          selected_count=rp["bcnt"], workspace=rp["ws_b"])

    def c_tokens(rp):
        inp = rp["inp"]
        ls.indexer_select(rp["q_idx"], rp["w"], inp.idx_keys, P, rp["ib"], granularity="tokens",
                          topk=k, max_selected=k, key_scales=inp.idx_scale,
                          cand_blocks=rp.get("kept", rp.get("cand", rp.get("bsel"))),
                          cand_counts=rp.get("kcnt", rp.get("ccnt", rp.get("bcnt"))),
                          token_candidates=pq, approx=args.approx_topk,
                          selected=rp["sel"], selected_count=rp["cnt"], workspace=rp["ws_t"])

    def c_encode(rp):
        ls.pq_encode(rp["inp"].idx_keys, rp["inp"].idx_scale, new_pages, codebooks, codes)

    def c_pq(rp):
        ls.pq_select(rp["q_idx"], rp["w"], codes, codebooks, rp["ib"], cfg.n_candidates,
                     candidates=rp["cand"], counts=rp["ccnt"], scores_out=rp.get("csc"),
                     workspace=rp["ws_c"])

    def c_filter(rp):
        ls.pq_filter_misses(rp["cand"], rp["ccnt"], rp["csc"], rp["res"], k, kept=rp["kept"],
                            kept_counts=rp["kcnt"], misses_kept=rp["mk"])

    def c_mla(rp):
        ls.sparse_mla_decode(rp["q_mla"], rp["inp"].latent, rp["kb"], rp["sel"], rp["cnt"],
                             sm_scale=sm, out=rp["out"], workspace=rp["ws_mla"])

    calls = ([("coarse_block_select", c_blocks)] if coarse else []) + \
        ([("pq_encode_new_pages", c_encode), ("pq_coarse_select", c_pq)] if pq else []) + \
        ([("pq_miss_filter", c_filter)] if pq and args.miss_filter else []) + \
        [("token_select", c_tokens), ("sparse_mla", c_mla)]

    def step(rp):
        for _, f in calls:
            f(rp)

    for i in range(max(1, args.warmup)):
        step(reps[i % R])
    torch.cuda.synchronize()
    main_stream = torch.cuda.current_stream()
    cap = torch.cuda.Stream()
    cap.wait_stream(main_stream)
    with torch.cuda.stream(cap):
        for rp in reps:
            step(rp)
    main_stream.wait_stream(cap)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for rp in reps:
            step(rp)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    replays = max(1, args.steps // R)
    steps = replays * R
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(replays):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # per-call durations: n launches of one call back to back between events
    n = min(steps, 4 * R)
    per = {}
    for name, f in calls:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(int(1e8))
        a.record()
        for i in range(n):
            f(reps[i % R])
        b.record()
        torch.cuda.synchronize()
        per[name] = a.elapsed_time(b) / n
    filt = None
    if pq and args.miss_filter:
        # what the filter did in the last step of every replica
        kc = torch.stack([rp["kcnt"] for rp in reps]).float()
        mk = torch.stack([rp["mk"] for rp in reps]).float()
        cc = torch.stack([rp["ccnt"] for rp in reps]).float()
        filt = {"hit_rate": args.miss_filter, "candidates_mean": round(cc.mean().item(), 1),
                "kept_mean": round(kc.mean().item(), 1),
                "misses_kept_mean": round(mk.mean().item(), 1),
                "misses_dropped_mean": round((cc - kc).mean().item(), 1)}
    nbytes = indexer_step_bytes(cfg, coarse, pq, kept_mean=filt["kept_mean"] if filt else None)
    gbps = nbytes["total"] / (ms * 1e-3) / 1e9
    dom = max(per, key=per.get)
    if dom == "token_select":
        dbytes = (nbytes["candidate_keys"] if coarse or pq else nbytes["indexer_keys"]) + \
            nbytes["q_idx_w"] + nbytes["selection"]
    elif dom == "pq_coarse_select":
        dbytes = nbytes["pq_codes"] + nbytes["q_idx_w"] + B * cfg.n_candidates * 4
    elif dom == "pq_encode_new_pages":
        dbytes = nbytes["encode_new_pages"]
    elif dom == "sparse_mla":
        dbytes = nbytes["mla_kv"] + nbytes["q_mla"] + nbytes["out"] + nbytes["selection"]
    else:
        dbytes = nbytes["coarse_summaries"] + nbytes["q_idx_w"] + nbytes["block_selection"]
    dgbps = dbytes / (per[dom] * 1e-3) / 1e9
    recall = None
    if args.approx_topk:
        # recall of the approximate top-k against the exact one (replica 0)
        rp = reps[0]
        step(rp)
        ex_sel = torch.empty_like(rp["sel"])
        ex_cnt = torch.empty_like(rp["cnt"])
        ls.indexer_select(rp["q_idx"], rp["w"], rp["inp"].idx_keys, P, rp["ib"],
                          granularity="tokens", topk=k, max_selected=k,
                          key_scales=rp["inp"].idx_scale,
                          cand_blocks=rp.get("cand", rp.get("bsel")),
                          cand_counts=rp.get("ccnt", rp.get("bcnt")), token_candidates=pq,
                          selected=ex_sel, selected_count=ex_cnt)
        torch.cuda.synchronize()
        hits = 0
        for r in range(B):
            hits += len(set(rp["sel"][r, :int(rp["cnt"][r])].tolist()) &
                        set(ex_sel[r, :int(ex_cnt[r])].tolist()))
        recall = {"approx_topk_vs_exact": round(hits / float(ex_cnt.sum().item()), 4)}
    if pq and not args.approx_topk:
        # recall against the exact top-k over every token (GPU, replica 0):
        # the coarse top-k alone, and the top-C + exact rerank of the step
        rp = reps[0]
        step(rp)
        ex, exn = ls.indexer_select(rp["q_idx"], rp["w"], base.idx_keys, P, rp["ib"],
                                    granularity="tokens", topk=k, max_selected=k,
                                    key_scales=base.idx_scale)
        direct, dn = ls.pq_select(rp["q_idx"], rp["w"], codes, codebooks, rp["ib"], k)
        torch.cuda.synchronize()

        def rec(a, an):
            hits = 0
            for r in range(B):
                sa = set(a[r, :int(an[r])].tolist())
                hits += len(sa & set(ex[r, :int(exn[r])].tolist()))
            return round(hits / float(exn.sum().item()), 4)
        recall = {f"pq_direct_top{k}": rec(direct, dn),
                  f"c{cfg.n_candidates}_rerank_top{k}": rec(rp["sel"], rp["cnt"])}
    if pq:
        metric = "PQ32 coarse-to-fine token selection + sparse MLA decode calls/sec"
    elif coarse:
        metric = "coarse-to-fine indexer selection + sparse MLA decode calls/sec"
    else:
        metric = "learned-indexer token selection + sparse MLA decode calls/sec"
    res = {"metric": metric,
           "value": round(1e3 / ms, 1), "unit": "calls/s", "n_gpus": 1, "steps": steps,
           "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": cfg.name, "batch": B, "context": cfg.context,
                      "index_heads": cfg.index_heads, "topk_tokens": k,
                      "mla_heads": cfg.mla_heads, "page_size": P, "replicas": R,
                      **({"coarse_topk_blocks": cfg.coarse_topk_blocks} if coarse else {}),
                      **({"n_candidates": cfg.n_candidates, "kmeans_iters": cfg.kmeans_iters}
                         if pq else {}),
                      **({"miss_filter": filt} if filt else {}),
                      "token_topk": ("approximate (remapped first digit, boundary bucket "
                                     "in index order)" if args.approx_topk else "exact")},
           "step_bytes": nbytes["total"], "step_bytes_breakdown": nbytes,
           "achieved_GBps_step": round(gbps, 1),
           "pct_of_hbm_peak_step": round(100 * gbps / HBM_PEAK_GBPS, 2),
           "call_ms": {kk: round(v, 5) for kk, v in per.items()},
           "roofline": {"kernel": dom + " (library call)", "bound": "hbm",
                        "achieved": round(dgbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                        "frac": round(dgbps / HBM_PEAK_GBPS, 4), "traffic": None,
                        "algorithmic_bytes_per_launch": dbytes,
                        "avg_launch_ms": round(per[dom], 5)},
           "device": torch.cuda.get_device_name(0)}
    if not (coarse or pq or args.approx_topk):
        # the exact token top-k over every cached token: the committed
        # counters cover this call's three launches
        tkey = f"{dom}.{cfg.name}"
        tr = stored_traffic(tkey)
        if tr is not None:
            res["roofline"]["traffic"] = tr["traffic_bytes"]
            res["roofline"]["traffic_source"] = f"profiles/{tkey}.md"
    if recall is not None:
        res["recall_vs_exact"] = recall
    print(json.dumps(res), flush=True)
    return 0


def bench_dense(args, window: bool = False) -> int:
    """Time the k = all path: split-K attention over every block of the
    8B/32K/B16 workload (ls_sparse_attn_decode with no selection), the dense
    baseline the sparse step's speedup is judged against; or (window) the
    sink + recent window of the same batch: 4 sinks and the last 30% of the
    tokens, read in place (ls_window_attn_decode)."""
    import torch
    import query_aware_sparse_ls_amd as ls
    from workloads import LLAMA8B_32K_B16, make_block_topk_inputs
    cfg = LLAMA8B_32K_B16
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, Hq, Hkv, D, P = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.page_size
    sm = 1.0 / math.sqrt(D)
    R = max(1, min(args.replicas or 2, 2))    # one step reads 2 GiB: no cache reuse either way
    N_SINK, WIN = 4, int(0.3 * cfg.context)   # the window: 4 sinks + 30% of the tokens
    reps = []
    for i in range(R):
        inp = make_block_topk_inputs(cfg, device=dev, seed=cfg.seed + i)
        b = ls.PagedBatch(inp.page_indptr, inp.page_indices, inp.seq_lens, inp.max_blocks())
        reps.append(dict(inp=inp, batch=b,
                         out=torch.empty(B, Hq, D, dtype=torch.bfloat16, device=dev),
                         ws=torch.empty(max(ls.sparse_attn_decode_workspace_size(
                             B, Hq, D, 0, b.max_blocks), int(ls._lib.EXPORTS[
                                 "ls_window_attn_decode_workspace_size"](
                                 B, Hq, D, b.max_blocks, N_SINK, WIN))),
                             dtype=torch.uint8, device=dev)))
    torch.cuda.synchronize()
    print(f"# {R} replicas ready, {torch.cuda.memory_allocated() / 2**30:.1f} GiB",
          file=sys.stderr, flush=True)

    def call(rp):
        inp = rp["inp"]
        if window:
            ls.window_attn_decode(inp.q, inp.k_pool, inp.v_pool, rp["batch"], n_sink=N_SINK,
                                  window=WIN, sm_scale=sm, out=rp["out"], workspace=rp["ws"])
        else:
            ls.sparse_attn_decode(inp.q, inp.k_pool, inp.v_pool, rp["batch"], None, None,
                                  sm_scale=sm, out=rp["out"], workspace=rp["ws"])

    for i in range(max(1, args.warmup)):
        call(reps[i % R])
    torch.cuda.synchronize()
    steps = max(R, args.steps // R * R)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(1e8))     # the host enqueues ahead of the device
    e0.record()
    for i in range(steps):
        call(reps[i % R])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    L = cfg.context
    ntok = min(L, N_SINK + WIN) if window else L
    kv = B * ntok * Hkv * D * 2 * 2
    nbytes = {"kv": kv, "q_out_pagetable": B * Hq * D * 2 * 2 + B * (-(-ntok // P) + 1) * 4}
    nbytes["total"] = sum(nbytes.values())
    gbps = nbytes["total"] / (ms * 1e-3) / 1e9
    key = "attn_window_kernel.llama8b_32k_b16_window" if window else \
        "plan_attn_kernel.llama8b_32k_b16_dense"
    tr = stored_traffic(key)
    res = {"metric": ("sink + recent window decode attention calls/sec at 8B/32K/B16" if window
                      else "dense (k = all) split-K decode attention calls/sec at 8B/32K/B16"),
           "value": round(1e3 / ms, 2), "unit": "calls/s", "n_gpus": 1, "steps": steps,
           "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": cfg.name + (" window" if window else " dense"), "batch": B,
                      "context": L, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D,
                      "page_size": P, "replicas": R, "timing": "eager, back-to-back calls",
                      **({"n_sink": N_SINK, "window": WIN} if window else {})},
           "step_bytes": nbytes["total"], "step_bytes_breakdown": nbytes,
           "roofline": {"kernel": ("ls::attn_window_kernel<128> + ls::attn_combine_kernel<128> "
                                   "(one library call)" if window else
                                   "ls::plan_attn_kernel<128, true> (one launch)"),
                        "bound": "hbm",
                        "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                        "frac": round(gbps / HBM_PEAK_GBPS, 4),
                        "traffic": tr["traffic_bytes"] if tr else None,
                        "algorithmic_bytes_per_launch": nbytes["total"],
                        "avg_launch_ms": round(ms, 5),
                        "traffic_source": (f"profiles/{key}.md" if tr else None)},
           "device": torch.cuda.get_device_name(0)}
    print(json.dumps(res), flush=True)
    return 0


def bench_summaries(args) -> int:
    """Full summary builds: the block means of every complete page of the
    16 x 32K bf16 key cache (8 KV heads, D 128: 1.07 GB read, 67 MB written),
    and of the fp8 indexer key cache of 4 x 950K tokens in 64-token pages
    (128 B per token plus its fp32 scale), each timed over back-to-back
    builds alternating two replicas between HIP events."""
    import torch
    import query_aware_sparse_ls_amd as ls
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = torch.Generator(device="cuda").manual_seed(11)
    res = {"metric": "block summary build GB/s (% of HBM peak)", "unit": "GB/s", "n_gpus": 1,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic", "config": {"workload": "summaries: 16 x 32K bf16 keys (8 kv "
                                                        "heads, D 128, 16-token pages); 4 x 950K "
                                                        "fp8 indexer keys (64-token pages)"}}

    def timed(fn, n):
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(n):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    # bf16: 16 x 2048 pages x 8 heads x 16 tokens x 128 dims
    num_pages, H, P, D = 16 * 2048, 8, 16, 128
    keys = [torch.randn(num_pages, H, P, D, generator=g, device=dev).to(torch.bfloat16)
            for _ in range(2)]
    ids = torch.randperm(num_pages, device=dev).to(torch.int32)
    outs = [torch.empty(num_pages, H, D, dtype=torch.bfloat16, device=dev) for _ in range(2)]
    ms = timed(lambda i: ls.build_block_summaries(keys[i % 2], ids, outs[i % 2]), max(4, args.steps // 20))
    nbytes = num_pages * H * P * D * 2 + num_pages * H * D * 2 + num_pages * 4
    gbps = nbytes / (ms * 1e-3) / 1e9
    res["value"] = round(gbps, 1)
    res["bf16_build"] = {"ms": round(ms, 5), "bytes": nbytes, "GBps": round(gbps, 1),
                         "pct_of_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2)}
    # the chip's streaming rate over a buffer of the same size (what a read
    # of these bytes can take at best on this part)
    sink = torch.empty(int(ls._lib.EXPORTS["ls_stream_read_sink_words"]()), dtype=torch.int32,
                       device=dev)
    flat = [k.view(-1)[: nbytes // 2] if k.numel() * 2 >= nbytes else k.view(-1) for k in keys]
    ms_sr = timed(lambda i: ls.stream_read(flat[i % 2], sink), max(4, args.steps // 20))
    sr = flat[0].numel() * 2 / (ms_sr * 1e-3) / 1e9
    res["bf16_build"]["stream_read_GBps"] = round(sr, 1)
    res["bf16_build"]["pct_of_stream_read"] = round(100 * gbps / sr, 2)
    res["roofline"] = {"kernel": "ls::summaries_bf16_kernel<128, false, 16>", "bound": "hbm",
                       "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                       "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                       "algorithmic_bytes_per_launch": nbytes, "avg_launch_ms": round(ms, 5)}
    tr = stored_traffic("summaries_bf16_kernel.summaries_b16_32k_bf16")
    if tr is not None:
        res["roofline"]["traffic"] = tr["traffic_bytes"]
        res["roofline"]["traffic_source"] = "profiles/summaries_bf16_kernel.summaries_b16_32k_bf16.md"
    del keys, outs, flat
    torch.cuda.empty_cache()
    # fp8 indexer keys: 4 x 15,200 pages of 64 tokens x 128 bytes, fp32 scales
    npg, P8 = 4 * 15200, 64
    k8 = [torch.randint(0, 0x7e, (npg, P8, 128), generator=g, device=dev, dtype=torch.int32)
          .to(torch.uint8) for _ in range(2)]
    sc = [torch.rand(npg, P8, generator=g, device=dev) for _ in range(2)]
    ids8 = torch.arange(npg, dtype=torch.int32, device=dev)
    o8 = [torch.empty(npg, 128, dtype=torch.bfloat16, device=dev) for _ in range(2)]
    ms8 = timed(lambda i: ls.build_block_summaries(k8[i % 2].view(torch.float8_e4m3fn), ids8,
                                                   o8[i % 2], key_scales=sc[i % 2]),
                max(4, args.steps // 20))
    nb8 = npg * P8 * (128 + 4) + npg * 128 * 2 + npg * 4
    g8 = nb8 / (ms8 * 1e-3) / 1e9
    res["fp8_indexer_build"] = {"ms": round(ms8, 5), "bytes": nb8, "GBps": round(g8, 1),
                                "pct_of_hbm_peak": round(100 * g8 / HBM_PEAK_GBPS, 2),
                                "pct_of_stream_read": round(100 * g8 / sr, 2)}
    res["device"] = torch.cuda.get_device_name(0)
    print(json.dumps(res), flush=True)
    return 0


def bench_snapkv(args) -> int:
    """SnapKV-style selection on the 8B/32K/B16 batch: the one-time selection
    (64 observation queries, 4 sinks, budget 30% of the context) and gather,
    timed once per replica, then the decode step: dense split-K attention over
    each (request, KV head)'s gathered buffer."""
    import torch
    import query_aware_sparse_ls_amd as ls
    from workloads import LLAMA8B_32K_B16, make_block_topk_inputs
    cfg = LLAMA8B_32K_B16
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, Hq, Hkv, D, L = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.context
    W, NS, BUD = 64, 4, int(0.3 * cfg.context)
    sm = 1.0 / math.sqrt(D)
    R = max(1, min(args.replicas or 2, 2))
    reps, sel_ms = [], []
    for i in range(R):
        inp = make_block_topk_inputs(cfg, device=dev, seed=cfg.seed + i)
        g = torch.Generator().manual_seed(cfg.seed + 17 * i)
        qo = torch.randn(B, W, Hq, D, generator=g).to(torch.bfloat16).to(dev)
        b = ls.PagedBatch(inp.page_indptr, inp.page_indices, inp.seq_lens, inp.max_blocks())
        ls.snapkv_select(qo, inp.k_pool, b, max_len=L, sm_scale=sm, n_sink=NS, budget=BUD)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        sel, cnt = ls.snapkv_select(qo, inp.k_pool, b, max_len=L, sm_scale=sm, n_sink=NS,
                                    budget=BUD)
        k_out, v_out = ls.snapkv_gather(inp.k_pool, inp.v_pool, b, sel, cnt)
        e1.record()
        torch.cuda.synchronize()
        sel_ms.append(e0.elapsed_time(e1))
        pairs, nblk = B * Hkv, k_out.shape[2] // 16
        vb = ls.PagedBatch(torch.arange(0, pairs * nblk + 1, nblk, dtype=torch.int32, device=dev),
                           torch.arange(pairs * nblk, dtype=torch.int32, device=dev),
                           cnt.reshape(-1).contiguous(), nblk)
        reps.append(dict(q=inp.q.reshape(pairs, 4, D).contiguous(),
                         k=k_out.reshape(pairs * nblk, 1, 16, D),
                         v=v_out.reshape(pairs * nblk, 1, 16, D), batch=vb,
                         out=torch.empty(pairs, 4, D, dtype=torch.bfloat16, device=dev),
                         ws=torch.empty(ls.sparse_attn_decode_workspace_size(
                             pairs, 4, D, 0, nblk), dtype=torch.uint8, device=dev),
                         ntok=int(cnt.sum().item())))
        del inp
    torch.cuda.synchronize()

    def call(rp):
        ls.sparse_attn_decode(rp["q"], rp["k"], rp["v"], rp["batch"], None, None, sm_scale=sm,
                              out=rp["out"], workspace=rp["ws"])

    for i in range(max(1, args.warmup)):
        call(reps[i % R])
    torch.cuda.synchronize()
    steps = max(R, args.steps // R * R)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(1e8))
    e0.record()
    for i in range(steps):
        call(reps[i % R])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    ntok = reps[0]["ntok"]
    nbytes = ntok * D * 2 * 2 + B * Hq * D * 2 * 2
    gbps = nbytes / (ms * 1e-3) / 1e9
    res = {"metric": "SnapKV-style decode attention calls/sec over the gathered buffer at "
                     "8B/32K/B16",
           "value": round(1e3 / ms, 2), "unit": "calls/s", "n_gpus": 1, "steps": steps,
           "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": cfg.name + " snapkv", "batch": B, "context": L, "q_heads": Hq,
                      "kv_heads": Hkv, "head_dim": D, "observation_queries": W, "n_sink": NS,
                      "budget": BUD, "replicas": R, "timing": "eager, back-to-back calls"},
           "one_time_select_and_gather_ms": [round(x, 3) for x in sel_ms],
           "step_bytes": nbytes,
           "roofline": {"kernel": "ls::plan_attn_kernel<128, true> "
                                  "(one launch over the gathered buffer)", "bound": "hbm",
                        "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                        "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                        "algorithmic_bytes_per_launch": nbytes, "avg_launch_ms": round(ms, 5)},
           "device": torch.cuda.get_device_name(0)}
    print(json.dumps(res), flush=True)
    return 0


# -------------------------------------------------- the timing protocol ----
#
# A Cell is one measured operation of a session: fn(i) enqueues one step of
# it on replica i on the current stream; nbytes is its algorithmic bytes per
# step (mean over the replicas); steps is the number of steps one graph
# launch holds when the cell is timed as a repeat block.

class Cell:
    def __init__(self, name, fn, nbytes, steps, kernel=""):
        self.name, self.fn, self.nbytes, self.steps, self.kernel = name, fn, nbytes, steps, kernel


def capture(fns):
    """One HIP graph of fns in order (each enqueues work on the current
    stream), captured after one eager pass of the same work."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for f in fns:
            f()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    torch.cuda.synchronize()
    return g


def cell_graph(cell, R, n, replica=None):
    """A graph of n steps of `cell`, cycling over the R replicas (or all on
    one replica)."""
    return capture([(lambda i=i: cell.fn(i % R if replica is None else replica))
                    for i in range(n)])


def launch_ms(g, launches, warm):
    """Durations (ms) of `launches` replays of g, each between two HIP events
    on the launch stream, after `warm` untimed replays."""
    import torch
    for _ in range(warm):
        g.replay()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(launches)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def measure_cells(sess, order, launches, warm):
    """Median, min and max ms per step of every cell, one cell after the
    other in `order`: `launches` timed replays of a graph of cell.steps
    steps, after `warm` untimed ones."""
    import statistics
    out = {}
    for name in order:
        c = sess["cells"][name]
        print(f"#   {name}: graph of {c.steps} steps", file=sys.stderr, flush=True)
        g = cell_graph(c, sess["R"], c.steps)
        per = [m / c.steps for m in launch_ms(g, launches, warm)]
        del g
        out[name] = {"median_ms_per_step": statistics.median(per), "min_ms_per_step": min(per),
                     "max_ms_per_step": max(per), "steps_per_launch": c.steps,
                     "launches": launches, "bytes_per_step": c.nbytes}
    return out


def child_block(args) -> int:
    """One repeat block in a fresh process: the session's cells in an order
    rotated by the block index; one JSON line on stdout."""
    import torch
    b = args.child_block
    torch.cuda.set_device(0)
    sess = make_session(args, torch.device("cuda:0"), block=b)
    names = list(sess["cells"])
    order = names[b % len(names):] + names[:b % len(names)]
    cells = measure_cells(sess, order, args.launches, args.warm_launches)
    print(json.dumps({"block": b, "pid": os.getpid(), "order": order, "cells": cells}), flush=True)
    return 0


def run_blocks(args, argv):
    """The repeat blocks: this script again with --child-block i, one fresh
    process after the other, all before this process makes a GPU call."""
    import subprocess
    out = []
    for b in range(args.blocks):
        print(f"# repeat block {b + 1}/{args.blocks} (fresh process)", file=sys.stderr, flush=True)
        p = subprocess.run([sys.executable, "-u", os.path.abspath(__file__)] + list(argv)
                           + ["--child-block", str(b)], stdout=subprocess.PIPE, text=True,
                           timeout=args.block_timeout)
        if p.returncode != 0:
            raise SystemExit(f"repeat block {b} ended with status {p.returncode}")
        out.append(json.loads(p.stdout.strip().splitlines()[-1]))
    return out


def summarize_blocks(blocks, primary):
    """Per cell: the median over the blocks of their medians, and the range;
    per block, paired with the primary cell in the same process: % of the
    stream-read bandwidth and the cost beyond byte time at the dense rate
    (t_b - t_D * B_b / B_D, ByteCross §4.3 and App. D)."""
    import statistics
    names = list(blocks[0]["cells"])
    cells = {}
    for n in names:
        meds = [b["cells"][n]["median_ms_per_step"] for b in blocks]
        nbytes = blocks[0]["cells"][n]["bytes_per_step"]
        m = statistics.median(meds)
        cells[n] = {"median_ms_per_step": round(m, 6),
                    "range_ms_per_step": [round(min(meds), 6), round(max(meds), 6)],
                    "per_block_ms_per_step": [round(x, 6) for x in meds],
                    "bytes_per_step": nbytes, "GBps_at_median": round(nbytes / (m * 1e-3) / 1e9, 1),
                    "pct_of_hbm_peak_at_median": round(100 * nbytes / (m * 1e-3) / 1e9
                                                       / HBM_PEAK_GBPS, 2)}
    res = {"blocks": len(blocks), "orders": [b["order"] for b in blocks],
           "launches_per_block": blocks[0]["cells"][primary]["launches"], "cells": cells}

    def gbps(b, n):
        c = b["cells"][n]
        return c["bytes_per_step"] / (c["median_ms_per_step"] * 1e-3) / 1e9

    if "stream_read" in names:
        ratios = {n: [100 * gbps(b, n) / gbps(b, "stream_read") for b in blocks]
                  for n in names if n != "stream_read"}
        res["pct_of_stream_read"] = {n: {"median": round(statistics.median(v), 2),
                                         "range": [round(min(v), 2), round(max(v), 2)]}
                                     for n, v in ratios.items()}
    if "dense" in names:
        beyond = {}
        for n in names:
            if n in ("dense", "stream_read"):
                continue
            cb = []
            for b in blocks:
                tb, td = b["cells"][n]["median_ms_per_step"], b["cells"]["dense"]["median_ms_per_step"]
                cb.append((tb - td * b["cells"][n]["bytes_per_step"]
                           / b["cells"]["dense"]["bytes_per_step"]) * 1e3)
            beyond[n] = {"c_b_us_median": round(statistics.median(cb), 3),
                         "c_b_us_range": [round(min(cb), 3), round(max(cb), 3)]}
        res["beyond_byte_time"] = beyond
    return res


def eager_mean_ms(fn, R, n):
    """Mean duration of n eager launches of fn (cycling over the replicas)
    between two HIP events, queued behind a GPU-side sleep so that the
    launches run back to back."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2e8))
    a.record()
    for i in range(n):
        fn(i % R)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def single_call_us(fn, R, n=21):
    """Median latency of one call alone (synchronised before and after)."""
    import statistics
    import torch
    ts = []
    for j in range(n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        fn(j % R)
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b) * 1e3)
    return statistics.median(ts)


def contract_timing(sess, args):
    """Exactly args.steps steps of the primary cell, cycling over the
    replicas, after args.warmup eager steps and one untimed launch of the
    same graph; one HIP-event pair on the launch stream, synchronised on
    both sides. Returns (ms per step, wall seconds, timing label)."""
    import torch
    c, R, K = sess["cells"][sess["primary"]], sess["R"], args.steps
    for i in range(max(1, args.warmup)):
        c.fn(i % R)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if args.no_graph:
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        a.record()
        for i in range(K):
            c.fn(i % R)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / K, time.perf_counter() - w0, "eager"
    g = cell_graph(c, R, K)
    g.replay()
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    return a.elapsed_time(b) / K, wall, "hip graph"


# ------------------------------------------------------------- sessions ----

def stream_cell(reps, nbytes, steps):
    """The stream-read reference over nbytes of each replica's K pool."""
    import torch
    import query_aware_sparse_ls_amd as ls
    n16 = int(nbytes) // 16 * 16
    srcs = [r["inp"].k_pool.view(-1).view(torch.uint8)[:n16] for r in reps]
    sink = torch.empty(int(ls._lib.EXPORTS["ls_stream_read_sink_words"]()), dtype=torch.int32,
                       device=reps[0]["inp"].q.device)
    return Cell("stream_read", lambda i: ls.stream_read(srcs[i], sink), n16, steps,
                "ls::stream_read_kernel")


def dense_cell(reps, sm_scale, nbytes, steps):
    """k = all: split-K attention over every cached token (no selection)."""
    import torch
    import query_aware_sparse_ls_amd as ls
    inp0 = reps[0]["inp"]
    B, Hq, D = inp0.q.shape
    ws = [torch.zeros(ls.sparse_attn_decode_workspace_size(B, Hq, D, 0, r["batch"].max_blocks),
                      dtype=torch.uint8, device=inp0.q.device) for r in reps]
    out = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=inp0.q.device)

    def fn(i):
        inp = reps[i]["inp"]
        ls.sparse_attn_decode(inp.q, inp.k_pool, inp.v_pool, reps[i]["batch"], None, None,
                              sm_scale=sm_scale, out=out, workspace=ws[i])
    return Cell("dense", fn, nbytes, steps, "ls::plan_attn_kernel<128, true>")


def make_session(args, dev, block=None):
    sess = ragged_session(args, dev, block) if args.path == "ragged" else \
        block_topk_session(args, dev, block)
    if getattr(args, "only_primary", False):
        sess["cells"] = {sess["primary"]: sess["cells"][sess["primary"]]}
    return sess


def block_topk_session(args, dev, block=None):
    """Llama-3-8B-shaped decode at 16 x 32K: the step (fused, or the
    separate calls), the stream read of the step's byte count, and k = all."""
    import torch
    from workloads import LLAMA8B_32K_B16
    cfg = LLAMA8B_32K_B16
    sm = 1.0 / math.sqrt(cfg.head_dim)
    fused = not args.separate
    R = args.replicas or 8
    reps = [make_replica(cfg, cfg.seed + i, dev, args.score) for i in range(R)]
    torch.cuda.synchronize()
    print(f"# {R} replicas ready, {torch.cuda.memory_allocated() / 2**30:.1f} GiB"
          + ("" if block is None else f" (block {block})"), file=sys.stderr, flush=True)
    inp0 = reps[0]["inp"]
    P, Hkv, D, Hq, B = cfg.page_size, cfg.num_kv_heads, cfg.head_dim, cfg.num_q_heads, cfg.batch
    nb = cfg.context // P
    n_forced = cfg.n_sink + cfg.n_recent
    quest = args.score == "bounds"
    nbytes = step_bytes(B, Hq, Hkv, D, P, nb, inp0.topk + n_forced, nb - n_forced,
                        int(reps[0]["new_pages"].numel()), rows=2 if quest else 1)
    side = torch.cuda.Stream()
    dense_bytes = B * Hkv * cfg.context * D * 2 * 2 + 2 * B * Hq * D * 2 + B * nb * 4
    cells = {"step": Cell("step", lambda i: run_step(reps[i], cfg, sm, fused, side),
                          nbytes["total"], args.steps),
             "stream_read": stream_cell(reps, nbytes["total"], args.steps),
             "dense": dense_cell(reps, sm, dense_bytes, min(args.steps, 2 * R))}
    return {"cfg": cfg, "reps": reps, "R": R, "cells": cells, "primary": "step",
            "sm_scale": sm, "fused": fused, "quest": quest, "nbytes": nbytes, "side": side}


KEEPS = {"1/64": 1.0 / 64, "1/16": 1.0 / 16, "1/4": 1.0 / 4}


def ragged_pair_bytes(inp, sel, cnt, n_sink, n_recent):
    """Algorithmic bytes of one keep-ratio step on a ragged batch, from the
    selection the step made: the selected blocks' tokens (a partial last
    block counts its cached tokens), the complete non-forced blocks'
    summaries, q, output, the page table, and the pages that filled."""
    import torch
    cfg = inp.cfg
    P, D, Hq, Hkv = cfg.page_size, cfg.head_dim, cfg.num_q_heads, cfg.num_kv_heads
    lens = inp.seq_lens.long()
    pos = torch.arange(sel.shape[2], device=sel.device)
    valid = pos[None, None, :] < cnt.long()[:, :, None]
    tok = (lens[:, None, None] - sel.long() * P).clamp(0, P)
    tokens = int((tok * valid).sum())
    cand = 0
    n_new = 0
    for L in lens.cpu().tolist():
        nb, nc = -(-L // P), L // P
        forced = set(range(min(n_sink, nb))) | set(range(max(0, nb - n_recent), nb))
        cand += nc - sum(1 for b in forced if b < nc)
        n_new += 1 if (L % P == 0 and nc) else 0
    nb_all = sum(-(-L // P) for L in lens.cpu().tolist())
    return {"summaries": Hkv * cand * D * 2, "selected_kv": tokens * D * 2 * 2,
            "q_out_pagetable": 2 * inp.q.shape[0] * Hq * D * 2 + nb_all * 4,
            "summary_update": n_new * Hkv * (P * D * 2 + D * 2)}


def ragged_session(args, dev, block=None):
    """The batch-64 ragged sweep (lengths log-uniform in [2K, 128K], shared
    page pool at 70% occupancy): the fused step at keep 1/64, 1/16 and 1/4,
    k = all, and the stream read of the primary keep ratio's bytes."""
    import torch
    import query_aware_sparse_ls_amd as ls
    from workloads import RAGGED_B64, make_block_topk_inputs
    cfg = RAGGED_B64
    P, Hkv, D, Hq, B = cfg.page_size, cfg.num_kv_heads, cfg.head_dim, cfg.num_q_heads, cfg.batch
    sm = 1.0 / math.sqrt(D)
    R = args.replicas or 3
    reps = []
    for i in range(R):
        inp = make_block_topk_inputs(cfg, device=dev, seed=cfg.seed + i)
        batch = ls.PagedBatch(inp.page_indptr, inp.page_indices, inp.seq_lens, inp.max_blocks())
        lens = inp.seq_lens.cpu().tolist()
        indptr = inp.page_indptr.cpu().tolist()
        idx = inp.page_indices.cpu()
        full = torch.cat([idx[indptr[r]:indptr[r] + lens[r] // P] for r in range(B)])
        new = [int(idx[indptr[r] + lens[r] // P - 1]) for r in range(B)
               if lens[r] % P == 0 and lens[r] >= P]
        summ = torch.zeros(inp.num_pages, Hkv, D, dtype=torch.bfloat16, device=dev)
        ls.build_block_summaries(inp.k_pool, full.to(torch.int32).to(dev), summ)
        rep = dict(inp=inp, batch=batch, summ=summ,
                   new_pages=torch.tensor(new, dtype=torch.int32, device=dev), keeps={})
        mb = batch.max_blocks
        for name, kr in KEEPS.items():
            maxsel = min(mb, max(cfg.n_sink + cfg.n_recent + 1,
                                 math.ceil(float(torch.tensor(kr, dtype=torch.float32)) * mb) + 1))
            rep["keeps"][name] = dict(
                ratio=kr, maxsel=maxsel,
                ws=ls.sparse_decode_step_workspace(B, Hq, Hkv, D, mb, maxsel, dev),
                sel=torch.empty(B, Hkv, maxsel, dtype=torch.int32, device=dev),
                cnt=torch.empty(B, Hkv, dtype=torch.int32, device=dev),
                out=torch.empty(B, Hq, D, dtype=torch.bfloat16, device=dev))
        reps.append(rep)
    torch.cuda.synchronize()
    print(f"# {R} ragged replicas ready, {torch.cuda.memory_allocated() / 2**30:.1f} GiB"
          + ("" if block is None else f" (block {block})"), file=sys.stderr, flush=True)

    def step(i, name):
        rp = reps[i]
        k = rp["keeps"][name]
        inp = rp["inp"]
        ls.sparse_decode_step(inp.q, rp["summ"], inp.k_pool, inp.v_pool, rp["batch"], topk=-1,
                              keep_ratio=k["ratio"], n_sink=cfg.n_sink, n_recent=cfg.n_recent,
                              max_selected=k["maxsel"], sm_scale=sm, group_agg=cfg.group_agg,
                              selected=k["sel"], selected_count=k["cnt"], out=k["out"],
                              new_pages=rp["new_pages"], workspace=k["ws"])

    def select(i, name):
        rp = reps[i]
        k = rp["keeps"][name]
        ls.score_select(rp["inp"].q, rp["summ"], P, rp["batch"], topk=-1, keep_ratio=k["ratio"],
                        n_sink=cfg.n_sink, n_recent=cfg.n_recent, max_selected=k["maxsel"],
                        group_agg=cfg.group_agg, selected=k["sel"], selected_count=k["cnt"],
                        workspace=k["ws_sel"])

    def attend(i, name):
        rp = reps[i]
        k = rp["keeps"][name]
        inp = rp["inp"]
        ls.sparse_attn_decode(inp.q, inp.k_pool, inp.v_pool, rp["batch"], k["sel"], k["cnt"],
                              sm_scale=sm, out=k["out"], workspace=k["ws_attn"])

    for rp in reps:
        mb = rp["batch"].max_blocks
        for k in rp["keeps"].values():
            k["ws_sel"] = torch.zeros(ls.score_select_workspace_size(B, Hkv, mb),
                                      dtype=torch.uint8, device=dev)
            k["ws_attn"] = torch.zeros(ls.sparse_attn_decode_workspace_size(
                B, Hq, D, k["maxsel"], mb), dtype=torch.uint8, device=dev)

    # bytes per step from the selections themselves (one untimed step each)
    cells, breakdown, positions = {}, {}, {}
    for name in KEEPS:
        parts = []
        for i in range(R):
            step(i, name)
            k = reps[i]["keeps"][name]
            parts.append(ragged_pair_bytes(reps[i]["inp"], k["sel"], k["cnt"], cfg.n_sink,
                                           cfg.n_recent))
        mean = {key: sum(p[key] for p in parts) / R for key in parts[0]}
        mean["total"] = sum(mean.values())
        breakdown[name] = mean
        positions[name] = sum(int(reps[i]["keeps"][name]["cnt"].sum()) for i in range(R)) / R
        cells["keep_" + name] = Cell("keep_" + name, lambda i, n=name: step(i, n), mean["total"],
                                     args.steps)
    dense_bytes = sum(float(r["inp"].seq_lens.long().sum()) * Hkv * D * 2 * 2
                      + 2 * B * Hq * D * 2 + 4 * sum(-(-int(L) // P)
                                                     for L in r["inp"].seq_lens.tolist())
                      for r in reps) / R
    cells["dense"] = dense_cell(reps, sm, dense_bytes, min(args.steps, 2 * R))
    primary = "keep_" + args.keep
    cells["stream_read"] = stream_cell(reps, cells[primary].nbytes, args.steps)
    return {"cfg": cfg, "reps": reps, "R": R, "cells": cells, "primary": primary,
            "sm_scale": sm, "breakdown": breakdown, "positions": positions, "step": step,
            "select": select, "attend": attend}


# ----------------------------------------------------------------- main ----

METRIC = "sparse decode attention calls/sec + achieved HBM GB/s (% of peak) at 8B/32K/B16"


def bench_block_topk(args, argv) -> int:
    """The block top-k decode step (default path) or the ragged sweep."""
    if args.child_block is not None:
        return child_block(args)
    if args.only_primary:
        args.blocks, args.no_cpu_baseline = 0, True
    pool = None
    if not args.no_cpu_baseline:
        pool = OraclePool(oracle_workers())        # spawned before any GPU call here
    try:
        blocks = run_blocks(args, argv) if args.blocks > 0 else []
        return _bench_block_topk_parent(args, blocks, pool)
    finally:
        if pool is not None:
            pool.close()


def _bench_block_topk_parent(args, blocks, pool) -> int:
    import statistics
    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sess = make_session(args, dev)
    cfg, R, cells = sess["cfg"], sess["R"], sess["cells"]
    prim = cells[sess["primary"]]
    ragged = args.path == "ragged"
    print("# timing", file=sys.stderr, flush=True)
    ms_step, wall, timing = contract_timing(sess, args)
    steps = args.steps
    if blocks:
        rb = summarize_blocks(blocks, sess["primary"])
    else:   # no fresh-process blocks asked for: one block in this process
        print("# cells in this process", file=sys.stderr, flush=True)
        rb = summarize_blocks([{"order": list(cells), "cells": measure_cells(
            sess, list(cells), args.launches, args.warm_launches)}], sess["primary"])
        rb["in_parent_process"] = True
    lat_us = single_call_us(prim.fn, R)
    warm_g = cell_graph(prim, R, steps, replica=0)
    warm_ms = launch_ms(warm_g, 1, 1)[0] / steps
    del warm_g

    calls_per_s = 1e3 / ms_step
    gbps = prim.nbytes / (ms_step * 1e-3) / 1e9
    B = cfg.batch
    if ragged:
        # the step is three launches (scoring, ranking, attention); the
        # attention call alone is one kernel, the one moving the most bytes
        step_ms = eager_mean_ms(prim.fn, R, 4 * R)
        sel_ms = eager_mean_ms(lambda i: sess["select"](i, args.keep), R, 4 * R)
        att_ms = eager_mean_ms(lambda i: sess["attend"](i, args.keep), R, 4 * R)
        bd = sess["breakdown"][args.keep]
        Hq, D = cfg.num_q_heads, cfg.head_dim
        n_pos = sess["positions"][args.keep]
        dom_ms = att_ms
        dom_bytes = bd["selected_kv"] + 2 * B * Hq * D * 2 + n_pos * 4 * 2 + B * cfg.num_kv_heads * 4
        dom_key = f"plan_attn_kernel.ragged_b64_keep{args.keep.replace('/', 'of')}"
        dom_match = "plan_attn_kernel<128, false>"
        call_ms = {"decode_step_with_summary_refresh": round(step_ms, 5),
                   "score_select": round(sel_ms, 5), "sparse_attn_decode": round(att_ms, 5)}
    else:
        cfg8 = cfg
        upd, first, second = per_call_ms(sess["reps"], cfg8, sess["sm_scale"], sess["fused"],
                                         min(steps, 8 * R))
        quest = sess["quest"]
        n_sel = sess["reps"][0]["inp"].topk + cfg.n_sink + cfg.n_recent
        nb = cfg.context // cfg.page_size
        sel_bytes = B * cfg.num_kv_heads * n_sel * 4 + B * cfg.num_kv_heads * 4
        if sess["fused"]:
            dom_ms, dom_bytes = first, prim.nbytes + sel_bytes
            dom_key = "step_item_kernel.llama8b_32k_b16" + ("_quest" if quest else "")
            dom_match = f"ls::step_item_kernel<128, 2048, {'true' if quest else 'false'}>"
            call_ms = {"decode_step_with_summary_refresh": round(first, 5)}
        else:
            nbd = sess["nbytes"]
            dom_ms = second
            dom_bytes = (nbd["selected_kv"] + B * cfg.num_q_heads * cfg.head_dim * 2 + sel_bytes
                         + B * nb * 4)
            dom_key = "attn_item_kernel.llama8b_32k_b16" + ("_quest" if quest else "")
            dom_match = "ls::attn_item_kernel<128, 2048>"
            call_ms = {"summary_update": round(upd, 5), "score_select": round(first, 5),
                       "sparse_attn_decode": round(second, 5)}
    dom_gbps = dom_bytes / (dom_ms * 1e-3) / 1e9
    tr = stored_traffic(dom_key)
    sr = rb["cells"].get("stream_read")
    workload = (f"ragged_b64_2k_128k keep {args.keep}" if ragged
                else cfg.name + (" quest bounds" if sess["quest"] else ""))
    config = {"workload": workload, "batch": B, "q_heads": cfg.num_q_heads,
              "kv_heads": cfg.num_kv_heads, "head_dim": cfg.head_dim,
              "page_size": cfg.page_size, "n_sink": cfg.n_sink, "n_recent": cfg.n_recent,
              "replicas": R, "timing": timing}
    if ragged:
        config.update({"context": "log-uniform [2048, 131072] per request, pool 70% occupied",
                       "keep_ratio": args.keep, "path": "fused"})
    else:
        config.update({"context": cfg.context, "topk": sess["reps"][0]["inp"].topk,
                       "path": "fused" if sess["fused"] else "separate",
                       "block_scores": "quest bounds" if sess["quest"] else "block-mean keys"})
    res = {
        "metric": METRIC if not ragged else
        "sparse decode attention calls/sec + achieved HBM GB/s (% of peak) at ragged B64 2K-128K",
        "value": round(calls_per_s, 1), "unit": "calls/s", "n_gpus": 1,
        "steps": steps, "steps_requested": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "config": config,
        "step_bytes": round(prim.nbytes),
        "step_bytes_breakdown": sess["breakdown"][args.keep] if ragged else sess["nbytes"],
        "achieved_GBps_step": round(gbps, 1),
        "pct_of_hbm_peak_step": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "pct_of_stream_read_step": rb.get("pct_of_stream_read", {}).get(sess["primary"]),
        "stream_read": None if sr is None else {
            "bytes": sr["bytes_per_step"], "ms_median": sr["median_ms_per_step"],
            "GBps_median": sr["GBps_at_median"], "pct_of_hbm_peak": sr["pct_of_hbm_peak_at_median"],
            "kernel": "ls::stream_read_kernel (4 KB chunks per wave round, 16-byte non-temporal loads)"},
        "beyond_byte_time": rb.get("beyond_byte_time"),
        "repeat_blocks": rb,
        "single_call_latency_us": round(lat_us, 2),
        "warm_same_replica_ms_per_step": round(warm_ms, 5),
        "call_ms": call_ms,
        "roofline": {"kernel": dom_match, "bound": "hbm", "achieved": round(dom_gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(dom_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": tr["traffic_bytes"] if tr else None,
                     "algorithmic_bytes_per_launch": round(dom_bytes),
                     "avg_launch_ms": round(dom_ms, 5),
                     "traffic_source": f"profiles/{dom_key}.md" if tr else None},
        "wall_s_timed": round(wall, 4),
        "device": torch.cuda.get_device_name(0),
    }
    if ragged:
        res["cells"] = {n: {"ms_per_step_median": c["median_ms_per_step"],
                            "calls_per_s_median": round(1e3 / c["median_ms_per_step"], 1),
                            "GBps": c["GBps_at_median"],
                            "pct_of_hbm_peak": c["pct_of_hbm_peak_at_median"],
                            "bytes_per_step": round(c["bytes_per_step"])}
                        for n, c in rb["cells"].items()}
        res["ragged_bytes_breakdown"] = sess["breakdown"]
    if pool is not None:
        print(f"# cpu baseline ({pool.n} processes)", file=sys.stderr, flush=True)
        inp0 = sess["reps"][0]["inp"]
        if ragged:
            order = sorted(range(B), key=lambda r: int(inp0.seq_lens[r]))
            sample = [order[s * B // 8 + B // 16] for s in range(8)]   # one per length octile
            topk, kr = -1, KEEPS[args.keep]
        else:
            sample, topk, kr = list(range(B)), inp0.topk, 0.0
        res["cpu_baseline"] = cpu_baseline(
            pool, inp0, cfg, requests=sample, topk=topk, keep_ratio=kr,
            score_mode="bounds" if (not ragged and sess["quest"]) else "mean",
            sm_scale=sess["sm_scale"], step_bytes_total=prim.nbytes, budget_s=args.cpu_seconds)
    print(json.dumps(res), flush=True)
    return 0


def main(argv=None) -> int:
    argv = list(sys.argv[1:] if argv is None else argv)
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400,
                    help="steps in the timed region (exactly; one graph of that many steps)")
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--replicas", type=int, default=0,
                    help="input replicas cycled by the steps (default: 8 at 16 x 32K, 3 ragged)")
    ap.add_argument("--blocks", type=int, default=3,
                    help="repeat blocks, each in a fresh process started before this one "
                         "touches the GPU (0: one block in this process)")
    ap.add_argument("--launches", type=int, default=20, help="timed graph launches per block")
    ap.add_argument("--warm-launches", type=int, default=10)
    ap.add_argument("--block-timeout", type=float, default=400.0)
    ap.add_argument("--child-block", type=int, default=None, help=argparse.SUPPRESS)
    ap.add_argument("--only-primary", action="store_true",
                    help="time only the cell the value is for (no repeat blocks, no oracle): "
                         "for profiling one kernel's launches")
    ap.add_argument("--keep", choices=tuple(KEEPS), default="1/16",
                    help="ragged path: the keep ratio the JSON line's value is for")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU seconds (all processes together) for the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--separate", action="store_true",
                    help="time ls_score_select + ls_sparse_attn_decode instead of the fused step")
    ap.add_argument("--copy-calibrate", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (PMC byte-counter scale)")
    ap.add_argument("--summarize-profiles", action="store_true",
                    help="write profiles/<kernel-key>.md from rocprofv3 CSV directories")
    for a in ("kernel-key", "kernel-match", "workload", "kt-dir", "fetch-dir", "write-dir",
              "copy-fetch-dir", "copy-write-dir", "kt-cmd", "fetch-cmd", "write-cmd",
              "copy-fetch-cmd", "copy-write-cmd"):
        ap.add_argument("--" + a, default="")
    ap.add_argument("--copy-bytes", type=int, default=0)
    ap.add_argument("--approx-topk", type=int, nargs="?", const=1, default=0, choices=(0, 1),
                    help="indexer paths: the approximate token top-k (early exit after the "
                         "remapped first digit, the boundary bucket filled in index order) "
                         "instead of the exact one; reports its recall")
    ap.add_argument("--miss-filter", type=float, default=0.0, metavar="HIT_RATE",
                    help="pq path: the miss filter before the exact rerank, with a seeded "
                         "residency mask of this hit rate (0: no filter)")
    ap.add_argument("--score", choices=("mean", "bounds"), default="mean",
                    help="block-topk path: block-mean summaries (default) or Quest bounds")
    ap.add_argument("--path", choices=("block-topk", "ragged", "indexer", "coarse-to-fine",
                                       "dense", "pq", "window", "snapkv", "summaries"),
                    default="block-topk",
                    help="block-topk: the 8B/32K/B16 block top-k step (default); ragged: the "
                         "batch-64 sweep, lengths 2K-128K, keep 1/64, 1/16, 1/4 and k = all; "
                         "indexer: token top-2048 of 8 x 128K + sparse MLA; coarse-to-fine: "
                         "4 x 950K; dense: k = all split-K attention on the 8B/32K/B16 "
                         "workload; pq: PQ32 top-2048 candidates + exact rerank to top-512 of "
                         "8 x 128K + sparse MLA")
    args = ap.parse_args(argv)
    if args.summarize_profiles:
        return summarize_profiles(args)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the sparse-attention path has no multi-GPU mode "
              "(run with --gpus 1).", file=sys.stderr)
        return 2
    if args.steps < 1:
        print("--steps must be at least 1", file=sys.stderr)
        return 2
    if args.copy_calibrate:
        return copy_calibration(args.copy_calibrate)
    if args.path == "snapkv":
        return bench_snapkv(args)
    if args.path == "summaries":
        return bench_summaries(args)
    if args.path in ("dense", "window"):
        return bench_dense(args, window=args.path == "window")
    if args.path in ("block-topk", "ragged"):
        return bench_block_topk(args, argv)
    return bench_indexer(args, coarse=args.path == "coarse-to-fine", pq=args.path == "pq")


if __name__ == "__main__":
    sys.exit(main())
