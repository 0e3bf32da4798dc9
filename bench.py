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

Timing: R input replicas (each its own pools, summaries, page table and
query), R x step bytes >> the 256 MB Infinity Cache, so consecutive steps
cannot be served from it. One HIP graph holds one step per replica; it is
replayed, and the timed region (hipEvents on the launch stream, bracketed by
device synchronisations) covers exactly `steps` steps. A second, eager pass
times each library call alone: 8R launches of it back to back between two
hipEvents (behind a GPU-side sleep so the host enqueues ahead of the device);
that mean launch duration prices the roofline line.

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


def cpu_baseline(rep, cfg, sm_scale, budget_s: float):
    """Time the oracle (unchanged, one thread) on whole requests of replica 0:
    summary update of the request's new page, scores, selection and attention
    for all its kv heads. Requests are taken in turn (wrapping around) until
    `budget_s` seconds of oracle time are spent; the mean time per request,
    times the batch size, is the time of one call."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle
    from workloads import bf16_bits
    inp = rep["inp"]
    P, Hkv = cfg.page_size, cfg.num_kv_heads
    bounds = rep["mode"] == "bounds"
    build = oracle.block_bounds if bounds else oracle.block_summaries
    prepared = {}

    def prepare(r):
        L = int(inp.seq_lens[r])
        nb = -(-L // P)
        p0 = int(inp.page_indptr[r])
        pages = inp.page_indices[p0:p0 + nb].long()
        k = bf16_bits(inp.k_pool[pages].contiguous())
        v = bf16_bits(inp.v_pool[pages].contiguous())
        q = bf16_bits(inp.q[r:r + 1].contiguous())
        bv = oracle.BatchView(np.array([0, nb]), np.arange(nb), np.array([L]), P)
        nc = L // P
        summ = np.zeros((nb, Hkv) + ((2,) if bounds else ()) + (cfg.head_dim,), dtype=np.uint16)
        summ[:nc] = build(k, np.arange(nc))                        # setup: not timed
        return L, nc, k, v, q, bv, summ

    times = []
    with threadpool_limits(1):
        while sum(times) < budget_s:
            r = len(times) % cfg.batch
            if r not in prepared:
                prepared[r] = prepare(r)
            L, nc, k, v, q, bv, summ = prepared[r]
            t0 = time.perf_counter()
            new = [nc - 1] if L % P == 0 and nc > 0 else []
            if new:
                summ[new] = build(k, new)
            oracle.decode_step(q, k, v, bv, num_kv_heads=Hkv, topk=inp.topk, n_sink=cfg.n_sink,
                               n_recent=cfg.n_recent, sm_scale=np.float32(sm_scale),
                               agg=cfg.group_agg, out_dtype="bf16", summaries=summ,
                               score_mode=rep["mode"])
            times.append(time.perf_counter() - t0)
    per_call = sum(times) / len(times) * cfg.batch
    return {"value": 1.0 / per_call, "unit": "calls/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(times)} request-steps ({len(times) / cfg.batch:.1f} calls' worth; "
                      f"each: new-page {'bounds' if bounds else 'summary'}, "
                      f"{'Quest bound ' if bounds else ''}scores, top-k selection and attention for all "
                      f"{Hkv} kv heads of one request), float64 NumPy on one thread, "
                      f"{sum(times):.1f} s; mean per request x {cfg.batch} requests = one call",
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
    which scale the kernel's counters to bytes."""
    key, match = args.kernel_key, args.kernel_match
    stats = _kernel_stats(os.path.join(args.kt_dir, "run_kernel_stats.csv"))
    fetch, nf, grid = _counter_per_dispatch(os.path.join(args.fetch_dir, "run_counter_collection.csv"),
                                            "FETCH_SIZE", match)
    write, nw, _ = _counter_per_dispatch(os.path.join(args.write_dir, "run_counter_collection.csv"),
                                         "WRITE_SIZE", match)
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
              "```", args.fetch_cmd, args.write_cmd, args.copy_fetch_cmd, args.copy_write_cmd, "```", "",
              f"* kernel `{match}` (grid {grid}): FETCH_SIZE {fetch:.1f} KiB over {nf} dispatches, "
              f"WRITE_SIZE {write:.1f} KiB over {nw} dispatches",
              f"* plain copy (`__amd_rocclr_copyBuffer`, {cb} bytes read and written): "
              f"FETCH_SIZE {cfetch:.1f} KiB, WRITE_SIZE {cwrite:.1f} KiB",
              f"* scale (copy bytes / counter bytes): FETCH_SIZE x {f_scale:.4f}, "
              f"WRITE_SIZE x {w_scale:.4f}",
              f"* traffic per launch: {fetch * 1024 * f_scale:.0f} B read + "
              f"{write * 1024 * w_scale:.0f} B written = {traffic:.0f} B", ""]
    rec = {"kernel": match, "traffic_bytes": round(traffic), "read_bytes": round(fetch * 1024 * f_scale),
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

def indexer_step_bytes(cfg, coarse: bool, pq: bool = False):
    """Algorithmic bytes of one learned-indexer step (per call, all requests).
    Token keys are fp8 (1 B per dim) with one fp32 scale per token; latent
    rows are 576 bf16 (the whole row is read: key = all 576 dims). PQ32: 32 B
    of codes per complete-page token, then the candidates' keys, and the
    codes of the pages that filled this step (keys read, codes written)."""
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
    R = max(1, args.replicas)
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
                   ws_mla=torch.empty(ls.sparse_mla_decode_workspace_size(B, cfg.mla_heads, k),
                                      dtype=torch.uint8, device=dev))
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
                          cand_blocks=rp.get("cand", rp.get("bsel")),
                          cand_counts=rp.get("ccnt", rp.get("bcnt")), token_candidates=pq,
                          approx=args.approx_topk,
                          selected=rp["sel"], selected_count=rp["cnt"], workspace=rp["ws_t"])

    def c_encode(rp):
        ls.pq_encode(rp["inp"].idx_keys, rp["inp"].idx_scale, new_pages, codebooks, codes)

    def c_pq(rp):
        ls.pq_select(rp["q_idx"], rp["w"], codes, codebooks, rp["ib"], cfg.n_candidates,
                     candidates=rp["cand"], counts=rp["ccnt"], workspace=rp["ws_c"])

    def c_mla(rp):
        ls.sparse_mla_decode(rp["q_mla"], rp["inp"].latent, rp["kb"], rp["sel"], rp["cnt"],
                             sm_scale=sm, out=rp["out"], workspace=rp["ws_mla"])

    calls = ([("coarse_block_select", c_blocks)] if coarse else []) + \
        ([("pq_encode_new_pages", c_encode), ("pq_coarse_select", c_pq)] if pq else []) + \
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
    nbytes = indexer_step_bytes(cfg, coarse, pq)
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
                      "token_topk": (f"approximate ({args.approx_topk} digit"
                                     f"{'s' if args.approx_topk > 1 else ''})"
                                     if args.approx_topk else "exact")},
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
    R = max(1, min(args.replicas, 2))    # one step reads 2 GiB: no cache reuse either way
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
        "attn_chunk_kernel.llama8b_32k_b16_dense"
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
           "roofline": {"kernel": ("ls::attn_window_kernel<128>" if window else
                                   "ls::attn_chunk_kernel<128>") +
                                  " + ls::attn_combine_kernel<128> (one library call)",
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
    R = max(1, min(args.replicas, 2))
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
           "roofline": {"kernel": "ls::attn_chunk_kernel<128> + ls::attn_combine_kernel<128> "
                                  "(one library call over the gathered buffer)", "bound": "hbm",
                        "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                        "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                        "algorithmic_bytes_per_launch": nbytes, "avg_launch_ms": round(ms, 5)},
           "device": torch.cuda.get_device_name(0)}
    print(json.dumps(res), flush=True)
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
    ap.add_argument("--copy-calibrate", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (PMC byte-counter scale)")
    ap.add_argument("--summarize-profiles", action="store_true",
                    help="write profiles/<kernel-key>.md from rocprofv3 CSV directories")
    for a in ("kernel-key", "kernel-match", "workload", "kt-dir", "fetch-dir", "write-dir",
              "copy-fetch-dir", "copy-write-dir", "kt-cmd", "fetch-cmd", "write-cmd",
              "copy-fetch-cmd", "copy-write-cmd"):
        ap.add_argument("--" + a, default="")
    ap.add_argument("--copy-bytes", type=int, default=0)
    ap.add_argument("--approx-topk", type=int, nargs="?", const=1, default=0, choices=(0, 1, 2),
                    help="indexer paths: the approximate token top-k (early exit after 1 or 2 "
                         "radix digits, the boundary bucket filled in index order) instead of "
                         "the exact one; reports its recall")
    ap.add_argument("--score", choices=("mean", "bounds"), default="mean",
                    help="block-topk path: block-mean summaries (default) or Quest bounds")
    ap.add_argument("--path", choices=("block-topk", "indexer", "coarse-to-fine", "dense", "pq",
                                       "window", "snapkv"),
                    default="block-topk",
                    help="block-topk: the 8B/32K/B16 block top-k step (default); indexer: "
                         "token top-2048 of 8 x 128K + sparse MLA; coarse-to-fine: 4 x 950K; "
                         "dense: k = all split-K attention on the 8B/32K/B16 workload; pq: PQ32 "
                         "top-2048 candidates + exact rerank to top-512 of 8 x 128K + sparse MLA")
    args = ap.parse_args(argv)
    if args.summarize_profiles:
        return summarize_profiles(args)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the sparse-attention path has no multi-GPU mode "
              "(run with --gpus 1).", file=sys.stderr)
        return 2
    if args.copy_calibrate:
        return copy_calibration(args.copy_calibrate)
    if args.path == "snapkv":
        return bench_snapkv(args)
    if args.path in ("dense", "window"):
        return bench_dense(args, window=args.path == "window")
    if args.path != "block-topk":
        return bench_indexer(args, coarse=args.path == "coarse-to-fine", pq=args.path == "pq")

    import torch
    import query_aware_sparse_ls_amd as ls
    from workloads import LLAMA8B_32K_B16

    cfg = LLAMA8B_32K_B16
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sm_scale = 1.0 / math.sqrt(cfg.head_dim)
    fused = not args.separate
    R = max(1, args.replicas)
    reps = [make_replica(cfg, cfg.seed + i, dev, args.score) for i in range(R)]
    torch.cuda.synchronize()
    print(f"# {R} replicas ready, {torch.cuda.memory_allocated() / 2**30:.1f} GiB",
          file=sys.stderr, flush=True)

    inp0 = reps[0]["inp"]
    P, Hkv, D, Hq, B = cfg.page_size, cfg.num_kv_heads, cfg.head_dim, cfg.num_q_heads, cfg.batch
    nb = cfg.context // P
    n_forced = cfg.n_sink + cfg.n_recent
    n_sel = inp0.topk + n_forced
    n_cand = nb - n_forced
    quest = args.score == "bounds"
    nbytes = step_bytes(B, Hq, Hkv, D, P, nb, n_sel, n_cand, int(reps[0]["new_pages"].numel()),
                        rows=2 if quest else 1)
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

    # per-call durations (eager, back-to-back launches of one call)
    upd, first, second = per_call_ms(reps, cfg, sm_scale, fused, min(steps, 8 * R))

    calls_per_s = 1e3 / ms_step
    gbps = nbytes["total"] / (ms_step * 1e-3) / 1e9
    sel_bytes = B * Hkv * n_sel * 4 + B * Hkv * 4      # selection written (+ counts)
    fused_bytes = nbytes["total"] + sel_bytes           # summary refresh included
    if fused:
        # one (request, kv head) pair per workgroup plus the summary-refresh
        # workgroups: the whole call is one launch
        dom_ms, dom_bytes = first, fused_bytes
        dom_key = "step_item_kernel.llama8b_32k_b16" + ("_quest" if quest else "")
        dom_match = f"ls::step_item_kernel<128, 2048, {'true' if quest else 'false'}>"
    else:
        dom_ms = second
        dom_bytes = nbytes["selected_kv"] + B * Hq * D * 2 + sel_bytes + B * nb * 4
        dom_key = "attn_item_kernel.llama8b_32k_b16" + ("_quest" if quest else "")
        dom_match = "ls::attn_item_kernel<128, 2048>"
    dom_gbps = dom_bytes / (dom_ms * 1e-3) / 1e9
    tr = stored_traffic(dom_key)

    res = {
        "metric": "sparse decode attention calls/sec + achieved HBM GB/s (% of peak) at 8B/32K/B16",
        "value": round(calls_per_s, 1), "unit": "calls/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name + (" quest bounds" if quest else ""), "batch": B,
                   "context": cfg.context, "q_heads": Hq,
                   "kv_heads": Hkv, "head_dim": D, "page_size": P, "topk": inp0.topk,
                   "n_sink": cfg.n_sink, "n_recent": cfg.n_recent, "replicas": R,
                   "path": "fused" if fused else "separate",
                   "block_scores": "quest bounds" if quest else "block-mean keys",
                   "timing": "hip graph" if graph is not None else "eager"},
        "step_bytes": nbytes["total"], "step_bytes_breakdown": nbytes,
        "achieved_GBps_step": round(gbps, 1),
        "pct_of_hbm_peak_step": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "call_ms": ({"decode_step_with_summary_refresh": round(first, 5)} if fused
                    else {"summary_update": round(upd, 5), "score_select": round(first, 5),
                          "sparse_attn_decode": round(second, 5)}),
        "roofline": {"kernel": dom_match, "bound": "hbm", "achieved": round(dom_gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(dom_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": tr["traffic_bytes"] if tr else None,
                     "algorithmic_bytes_per_launch": dom_bytes,
                     "avg_launch_ms": round(dom_ms, 5),
                     "traffic_source": f"profiles/{dom_key}.md" if tr else None},
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
