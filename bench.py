"""Benchmark of the lightning-indexer hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input resident in
HBM: indexer_score_topk, the NVFP4 paged scorer followed by the per-row top-k, with
the scores kept in the workspace.  Prints ONE JSON line.  The default workload is the
long-context decode (T=32 queries, H=64, D=128, 64 keys per page, S=262144,
top_k=2048).  Steps are launched eagerly (--graph replays a captured HIP graph
instead).  The scorer and the select are also timed on their own (the split entry
points, each launched back to back) for the stage times and the scorer's roofline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--precision mfma|fp32]
                    [--graph] [--no-cpu-baseline] [--no-cold]

The decode workloads are also timed cold (key pool rotated through copies, reported
under "cold"; "value" stays the warm figure).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "query·key scores/s + ms per top-k=2048 call; % of HBM BW (decode) / MFMA peak"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
VALU_F32_PEAK_TFLOPS = 157.3
MFMA_F32_PEAK_TFLOPS = 157.3

WORKLOADS = {
    "tiny_decode": 1,
    "decode_T8_S65536": 2,
    "long_decode_T32_S262144": 3,
    "prefill_T4096": 4,
    "qsa_prefill": 5,
    # diagnostic, not a configuration: the long-decode shape with every row on its own
    # pages of a 604 MB pool, so that every key byte read comes from DRAM
    "hbm_true_T32_S262144": "diag",
    # one decode query of the QSA workload (its last prefill position) over all its blocks
    "qsa_decode": "qsa_decode",
    # attention of the QSA prefill rows over their selected blocks (workloads/attention.py)
    "qsa_prefill_attn": "attention",
    # the selected-entry gathers that consume the top-k (workloads/gather.py)
    "gather_T32_k2048": "gather",
    "qsa_gather_4096": "gather",
}
# Decode workloads also timed cold: the key pool rotates through enough copies that the
# copies read between two uses of one copy exceed twice the 256 MB last-level cache.
COLD_WORKLOADS = ("decode_T8_S65536", "long_decode_T32_S262144")
# the configuration the metric's HBM target is set on
DEFAULT_WORKLOAD = "long_decode_T32_S262144"
COLD_SPAN_BYTES = 2 * 256 * 2**20


# HBM traffic of one scorer launch, from two rocprofv3 --pmc passes (FETCH_SIZE, then
# WRITE_SIZE, KiB per dispatch of the split entry's scorer, the launch the roofline
# times) scaled by what the same counters read for a plain
# 256 MiB copy (FETCH_SIZE x 1.9998, WRITE_SIZE x 1.0); the summaries are under
# profiles/.  Valid only for the scorer sources they were taken with: a different
# source hash reports null.
TRAFFIC_COPY_FACTOR = {"FETCH_SIZE": 1.9998, "WRITE_SIZE": 1.0}
SCORER_SOURCES = {"csa": ['score.hip', 'nvfp4.hpp', 'common.hpp', 'internal.hpp'], "qsa": ['qsa.hip', 'common.hpp', 'internal.hpp']}
SCORER_TRAFFIC = {   # workload: (sources, sha, FETCH_SIZE KiB, WRITE_SIZE KiB per dispatch)
    "tiny_decode": ("csa", "1a53394b857b3ffd", 81.7, 16.0),
    "decode_T8_S65536": ("csa", "1a53394b857b3ffd", 3552.0, 2048.0),
    "long_decode_T32_S262144": ("csa", "1a53394b857b3ffd", 33796.7, 32776.0),
    "prefill_T4096": ("csa", "1a53394b857b3ffd", 35444.1, 65690.8),
    "qsa_prefill": ("qsa", "ec667992117eed46", 81970.8, 278861.5),
    "qsa_decode": ("qsa", "ec667992117eed46", 8279.1, 141.5),
    "hbm_true_T32_S262144": ("csa", "1a53394b857b3ffd", 229530.6, 32776.1),
}


def source_sha(kind):
    h = hashlib.sha256()
    for f in SCORER_SOURCES[kind]:
        with open(os.path.join(ROOT, "sparse_attention_lightning_block_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def scorer_traffic(workload):
    t = SCORER_TRAFFIC.get(workload)
    if t is None or source_sha(t[0]) != t[1]:
        return None
    return int((t[2] * TRAFFIC_COPY_FACTOR["FETCH_SIZE"] + t[3] * TRAFFIC_COPY_FACTOR["WRITE_SIZE"]) * 1024)


def key_bytes_per_entry(D, epb):
    # codes + scales + the page's global scale and block-table entry shared by epb keys
    return D / 2 + D / 16 + 8.0 / epb


def cpu_baseline(w, budget_s=20.0):
    """Time the CPU oracle (as it stands) on whole query rows until the budget is used."""
    from threadpoolctl import threadpool_info

    from oracle import indexer, nvfp4

    q = indexer.upcast(w.q, w.q_dtype)
    wt = w.w.astype(np.float64)
    pairs = 0
    rows = 0
    t0 = time.perf_counter()
    for t in range(w.T):
        c, g = nvfp4.dequant_row(w.keys_fp4, w.key_scale, w.key_gscale, w.block_table[t], w.valid_lens[t], w.epb)
        r = indexer.score_row(q[t], wt[t], c, g)
        indexer.topk(r, w.top_k)
        pairs += int(w.valid_lens[t])
        rows += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {
        "value": pairs / dt,
        "unit": "scores/s",
        "cores": int(min(threads, len(os.sched_getaffinity(0)))),
        "kind": "oracle",
        "sample": f"{rows} of {w.T} query rows ({pairs} pairs): NVFP4 decode, float64 scores, full sort top-k; "
                  f"{dt:.2f} s",
    }


def make_step(torch, stages, graph):
    """step(ev): run the stages in order, with ev[i] recorded before stage i and ev[-1]
    after the last (ev=None: no events).  With graph=True every stage is captured once
    into a HIP graph and replayed (the library allocates nothing and issues no memset,
    so its launches capture as plain kernel nodes); the events stay outside the graphs,
    on the same stream."""
    if graph:
        graphs = []
        for f in stages:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                f()
            graphs.append(g)
        torch.cuda.synchronize()
        runs = [g.replay for g in graphs]
    else:
        runs = list(stages)

    def step(ev):
        if ev is None:
            for r in runs:
                r()
            return
        for i, r in enumerate(runs):
            ev[i].record()
            r()
        ev[len(runs)].record()

    return step


def timed_steps(torch, step, n_stages, steps):
    """ms per step over `steps` back-to-back steps, and each stage's per-step times (ms).

    The steps are timed with one event before the first and one after the last, so no
    marker sits between the kernels of the timed region; the per-stage times come from a
    second pass over the same number of steps with an event around every stage."""
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_stages + 1)] for _ in range(steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    step(evs[0])  # one untimed pass through the replay path
    torch.cuda.synchronize()
    t_start.record()
    for i in range(steps):
        step(None)
    t_end.record()
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / steps
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    stage = [np.array([e[j].elapsed_time(e[j + 1]) for e in evs]) for j in range(n_stages)]
    return ms_per_step, stage


def cpu_baseline_qsa(w, budget_s=20.0):
    """Time the CPU oracle (as it stands) on the QSA chain for a bounded sample of rows."""
    from threadpoolctl import threadpool_info

    from oracle import indexer, qsa

    t0 = time.perf_counter()
    keys = qsa.block_pool(indexer.upcast(w.raw_keys, "bf16"), w.k_norm_w, 0, w.n_blocks, w.ratio, w.rot, w.theta,
                          w.eps)
    t_pool = time.perf_counter() - t0
    pairs = 0
    rows = 0
    t1 = time.perf_counter()
    for r0 in range(0, w.rows, 8):
        n = min(8, w.rows - r0)
        q = qsa.qprep_rows(indexer.upcast(w.qk[r0:r0 + n], "bf16"), w.q_norm_w, n, w.first_pos + r0,
                           w.n_heads * w.hd, w.n_heads, w.hd, w.rot, w.theta, w.eps)
        sc, valid = qsa.score_rows(q, keys, w.first_pos + r0, w.ratio)
        for i in range(n):
            indexer.topk(sc[i, : int(valid[i])], w.top_k)
        pairs += int(valid.sum())
        rows += n
        if time.perf_counter() - t1 > budget_s:
            break
    dt = time.perf_counter() - t1
    # the pooling is shared by all rows: charge it pro rata to the sampled rows
    dt_all = dt + t_pool * rows / w.rows
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {
        "value": pairs / dt_all,
        "unit": "scores/s",
        "cores": int(min(threads, len(os.sched_getaffinity(0)))),
        "kind": "oracle",
        "sample": f"{rows} of {w.rows} rows ({pairs} row-block pairs): query prep, float64 scores, full sort top-k "
                  f"({dt:.2f} s), plus {rows}/{w.rows} of the float64 block pooling ({t_pool:.2f} s in all)",
    }


def run_qsa(args, w):
    import torch

    import sparse_attention_lightning_block_amd as salb

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    raw = torch.from_numpy(w.raw_keys.view(np.int16).copy()).view(torch.bfloat16).to(dev)
    kw = torch.from_numpy(w.k_norm_w).to(dev)
    qk = torch.from_numpy(w.qk.view(np.int16).copy()).view(torch.bfloat16).to(dev)
    qw = torch.from_numpy(w.q_norm_w).to(dev)
    # the matrix-core path stores the pooled keys and prepared queries in fp16, the values
    # its MFMAs multiply (the same scores, bit for bit, as from fp32 storage)
    mfma = args.precision == "mfma" and w.hd in (64, 128) and w.n_heads in (16, 32, 64)
    sdt = torch.float16 if mfma else torch.float32
    keys = torch.empty((w.n_blocks, w.hd), dtype=sdt, device=dev)
    q = torch.empty((w.rows, w.n_heads, w.hd), dtype=sdt, device=dev)
    idx = torch.empty((w.rows, w.top_k), dtype=torch.int32, device=dev)
    # the matrix-core path scores with the 16-block sub-tile maxima and selects from the
    # sub-tiles that can hold a winner (qsa_score_select_f16 as its two halves); the FP32
    # path scores whole rows and runs the general select
    tiles = mfma and w.n_blocks <= 32768 and w.top_k <= 512
    s16 = (w.n_blocks + 15) // 16 * 16
    scores = torch.empty((w.rows, s16 if tiles else w.n_blocks), dtype=torch.float32, device=dev)
    tmax = torch.empty((w.rows, s16 // 16), dtype=torch.int32, device=dev) if tiles else None
    ws = torch.zeros(max(1, salb.indexer_topk_workspace_size(w.rows, w.n_blocks, w.top_k)), dtype=torch.uint8,
                     device=dev)

    def prep():
        salb.qsa_block_pool(raw, kw, keys, first_block=0, n_new=w.n_blocks, ratio=w.ratio, rot=w.rot, theta=w.theta,
                            eps=w.eps)
        salb.qsa_qprep_rows(qk, qw, n_heads=w.n_heads, hd=w.hd, first_pos=w.first_pos, rot=w.rot, theta=w.theta,
                            eps=w.eps, out=q)

    def score():
        if tiles:
            salb.qsa_score_rows_f16_tmax(q, keys, first_pos=w.first_pos, ratio=w.ratio, out=scores, tile_max=tmax)
        else:
            salb.qsa_score_rows(q, keys, first_pos=w.first_pos, ratio=w.ratio, precision=args.precision, out=scores)

    def select():
        if tiles:
            salb.qsa_select_tiles(scores, tmax, w.top_k, n_cols=w.n_blocks, first_pos=w.first_pos, ratio=w.ratio,
                                  out_idx=idx)
        else:
            salb.indexer_topk_select(scores, w.top_k, first_pos=w.first_pos, ratio=w.ratio, workspace=ws,
                                     out_idx=idx)

    stages = [prep, score, select]
    for _ in range(args.warmup):
        for f in stages:
            f()
    torch.cuda.synchronize()
    step = make_step(torch, stages, args.graph)
    ms_per_step, stage = timed_steps(torch, step, len(stages), args.steps)
    prep_ms, score_ms, select_ms = stage
    # stage averages with the stage launched back to back (no event between launches)
    prep_avg, score_avg, select_avg = (back_to_back_ms(torch, f, args.steps) for f in stages)
    pos = w.first_pos + np.arange(w.rows, dtype=np.int64)
    pairs = int(np.minimum((pos + 1) // w.ratio, w.n_blocks).sum())
    flops = 2.0 * pairs * w.n_heads * w.hd
    score_s = score_avg / 1e3
    tf = flops / score_s / 1e12
    peak = MFMA_F16_PEAK_TFLOPS if mfma else VALU_F32_PEAK_TFLOPS
    pool_bytes = w.n_blocks * w.ratio * w.hd * 2 + w.n_blocks * w.hd * keys.element_size()
    out = {
        "metric": METRIC,
        "value": pairs / (ms_per_step / 1e3),
        "unit": "scores/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if mfma else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "rows": w.rows, "heads": w.n_heads, "hd": w.hd, "raw_keys": w.n_blocks * w.ratio,
                   "ratio": w.ratio, "blocks": w.n_blocks, "top_k": w.top_k, "pairs": pairs,
                   "precision": args.precision, "storage": "f16" if mfma else "f32",
                   "select": "sub-tile" if tiles else "rows",
                   "launch": "hip_graph" if args.graph else "eager"},
        "step_ms": {"p50": float(np.median(prep_ms + score_ms + select_ms))},
        "stage_ms": {"pool_and_qprep": prep_avg, "score": score_avg, "select": select_avg},
        "roofline": {
            "bound": "mfma" if mfma else "alu",
            "achieved": round(tf, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(tf / peak, 4),
            "traffic": scorer_traffic(w.name) if mfma else None,
            "kernel": "qsa_score_mfma_kernel" if mfma else "qsa_score_f32_kernel",
            "kernel_avg_us": round(score_s * 1e6, 2),
            "flops_per_launch": int(flops),
            "pool": {"bytes_per_launch": pool_bytes, "stage_ms_with_qprep": float(np.median(prep_ms))},
        },
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_qsa(w),
    }
    print(json.dumps(out), flush=True)


def run_qsa_decode(args):
    """One QSA decode step on the QSA workload's cache: the new block pooled (n_new = 1) and
    the query prepared at its position (one launch), then its scores over every complete
    block and their top-k (qsa_score_topk)."""
    import torch

    import sparse_attention_lightning_block_amd as salb
    from workloads import make
    from workloads.device import bf16_tensor

    w = make(5)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    raw = bf16_tensor(w.raw_keys).to(dev)
    kw = torch.from_numpy(w.k_norm_w).to(dev)
    qw = torch.from_numpy(w.q_norm_w).to(dev)
    keys = torch.empty((w.n_blocks, w.hd), dtype=torch.float32, device=dev)
    salb.qsa_block_pool(raw, kw, keys, first_block=0, n_new=w.n_blocks, ratio=w.ratio, rot=w.rot, theta=w.theta,
                        eps=w.eps)
    r = w.rows - 1
    pos = w.first_pos + r
    nb = min(w.n_blocks, (pos + 1) // w.ratio)
    q_in = bf16_tensor(w.qk[r]).to(dev)
    q = torch.empty((w.n_heads, w.hd), dtype=torch.float32, device=dev)
    sc = torch.empty((1, nb), dtype=torch.float32, device=dev)
    idx = torch.empty((1, w.top_k), dtype=torch.int32, device=dev)
    ws = torch.empty(max(256, salb.indexer_topk_workspace_size(1, nb, w.top_k)), dtype=torch.uint8, device=dev)
    ws2 = torch.empty(max(256, salb.qsa_score_topk_workspace_size(nb, w.top_k)), dtype=torch.uint8, device=dev)

    def pool():
        salb.qsa_block_pool(raw, kw, keys, first_block=nb - 1, n_new=1, ratio=w.ratio, rot=w.rot, theta=w.theta,
                            eps=w.eps)

    def prep():
        salb.qsa_qprep(q_in, qw, n_heads=w.n_heads, hd=w.hd, pos=pos, rot=w.rot, theta=w.theta, eps=w.eps, out=q)

    q_rows, q_out = q_in.view(1, -1), q.view(1, w.n_heads, w.hd)

    def prep_one_launch():  # both of the above in one launch
        salb.qsa_decode_prep(raw, kw, keys, q_rows, qw, first_block=nb - 1, n_new=1, ratio=w.ratio,
                             n_heads=w.n_heads, hd=w.hd, first_pos=pos, rot=w.rot, theta=w.theta, eps=w.eps,
                             out=q_out)

    def score():
        salb.qsa_score(q, keys, n_blocks=nb, out=sc[0])

    def select():
        salb.indexer_topk_select(sc, w.top_k, workspace=ws, out_idx=idx)

    def score_topk():  # both of the above, the scores in the workspace (one launch fewer)
        salb.qsa_score_topk(q, keys, w.top_k, n_blocks=nb, workspace=ws2, out_idx=idx)

    def step():
        prep_one_launch()
        score_topk()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # A decode step is a short chain of small kernels: it runs both captured into one HIP
    # graph and replayed, and launched eagerly; the faster of the two is the step (two
    # calls per step launch fast enough from Python that the eager stream has no gaps,
    # while each graph node adds its own overhead), and both are reported.
    ms_graph, stage_g = timed_steps(torch, make_step(torch, [step], True), 1, args.steps)
    ms_eager, stage_e = timed_steps(torch, make_step(torch, [step], False), 1, args.steps)
    launch = "eager" if ms_eager <= ms_graph else "hip_graph"
    ms_per_step, stage = (ms_eager, stage_e) if launch == "eager" else (ms_graph, stage_g)
    pool_ms, prep_ms, fused_ms, score_ms, select_ms, st_ms = (
        back_to_back_ms(torch, f, args.steps) for f in (pool, prep, prep_one_launch, score, select, score_topk))
    key_bytes = nb * w.hd * 4 + w.n_heads * w.hd * 4 + nb * 4
    gbs = key_bytes / (score_ms / 1e3) / 1e9
    out = {
        "metric": METRIC,
        "value": nb / (ms_per_step / 1e3),
        "unit": "scores/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "qsa_decode", "pos": int(pos), "blocks": int(nb), "heads": w.n_heads, "hd": w.hd,
                   "top_k": w.top_k, "launch": launch},
        "ms_per_step_eager": ms_eager,
        "ms_per_step_graph": ms_graph,
        "step_ms": {"p10": float(np.percentile(stage[0], 10)), "p50": float(np.median(stage[0])),
                    "p90": float(np.percentile(stage[0], 90))},
        "stage_ms": {"prep_one_launch": fused_ms, "score_topk": st_ms, "score_alone": score_ms,
                     "select_alone": select_ms, "pool_one_block_alone": pool_ms, "qprep_alone": prep_ms},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": scorer_traffic("qsa_decode"),
                     "kernel": "qsa_decode_score_mfma_kernel",
                     "kernel_avg_us": round(score_ms * 1e3, 2), "bytes_per_launch": int(key_bytes),
                     "flops_per_launch": int(2 * nb * w.n_heads * w.hd)},
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_qsa_decode(w, r, pos, nb),
    }
    print(json.dumps(out), flush=True)


def cpu_baseline_qsa_decode(w, r, pos, nb):
    """The oracle decode step (query prep, scores over the pooled keys, full-sort top-k);
    the pooled keys come from the oracle too, outside the timed part."""
    from oracle import indexer, qsa

    keys = qsa.block_pool(indexer.upcast(w.raw_keys, "bf16"), w.k_norm_w, 0, nb, w.ratio, w.rot, w.theta, w.eps)
    t0 = time.perf_counter()
    q = qsa.qprep(indexer.upcast(w.qk[r], "bf16"), w.q_norm_w, w.n_heads, w.hd, w.rot, pos, w.theta, w.eps)
    indexer.topk(qsa.score_blocks(q, keys, nb), w.top_k)
    dt = time.perf_counter() - t0
    return {"value": nb / dt, "unit": "scores/s", "cores": int(len(os.sched_getaffinity(0))), "kind": "oracle",
            "sample": f"one decode query over {nb} blocks (prep, float64 scores, full-sort top-k): {dt:.3f} s"}


def run_attention(args):
    """Block-sparse prefill attention of the QSA prefill rows: one step is one call."""
    import torch

    import sparse_attention_lightning_block_amd as salb
    from oracle import attention
    from workloads.attention import qsa_prefill_attention
    from workloads.device import bf16_tensor

    w = qsa_prefill_attention()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q = bf16_tensor(w.q).to(dev)
    k = bf16_tensor(w.k_cache).to(dev)
    v = bf16_tensor(w.v_cache).to(dev)
    bt = torch.from_numpy(w.block_table).to(dev)
    lists = torch.from_numpy(w.lists).to(dev)
    out = torch.empty((w.rows, w.nq, w.hd), dtype=torch.float32, device=dev)

    def step():
        salb.qsa_prefill_attn(q, k, v, bt, lists, first_pos=w.first_pos, ratio=w.ratio, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ms_per_step, stage = timed_steps(torch, make_step(torch, [step], args.graph), 1, args.steps)
    kern_ms = back_to_back_ms(torch, step, args.steps)
    n_pos = [attention.attended_positions(w.lists[r], w.first_pos, r, w.ratio).size for r in range(w.rows)]
    pairs = int(np.sum(n_pos)) * w.nq                    # (row, head, position) triples
    flops = 4.0 * pairs * w.hd                           # q.k and p.v, 2 flops per multiply-add
    per_stream = int(np.sum(n_pos)) * w.nkv * w.hd * 2 * 2 + w.rows * w.nq * w.hd * (2 + 4)
    blocks = set()
    for r in range(w.rows):
        blocks.update((attention.attended_positions(w.lists[r], w.first_pos, r, w.ratio) // w.block_size).tolist())
    unique = len(blocks) * w.block_size * w.nkv * w.hd * 2 * 2 + w.rows * w.nq * w.hd * (2 + 4)
    kern_s = kern_ms / 1e3
    ridge = MFMA_F16_PEAK_TFLOPS / (HBM_PEAK_GBS / 1e3)
    mfma_bound = flops / unique > ridge
    tf = flops / kern_s / 1e12
    # below the ridge the binding traffic is what each row must gather: its own listed
    # blocks (lists are per row, and the cache is larger than the last-level cache)
    gbs = per_stream / kern_s / 1e9
    out_line = {
        "metric": METRIC,
        "value": pairs / (ms_per_step / 1e3),
        "unit": "query-head x position pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "qsa_prefill_attn", "rows": w.rows, "first_pos": w.first_pos, "ratio": w.ratio,
                   "topk": w.topk, "nq": w.nq, "nkv": w.nkv, "hd": w.hd, "block_size": w.block_size,
                   "launch": "hip_graph" if args.graph else "eager"},
        "step_ms": {"p10": float(np.percentile(stage[0], 10)), "p50": float(np.median(stage[0])),
                    "p90": float(np.percentile(stage[0], 90))},
        "roofline": {
            "bound": "mfma" if mfma_bound else "hbm",
            "achieved": round(tf, 2) if mfma_bound else round(gbs, 1),
            "peak": MFMA_F16_PEAK_TFLOPS if mfma_bound else HBM_PEAK_GBS,
            "unit": "TFLOP/s" if mfma_bound else "GB/s",
            "frac": round((tf / MFMA_F16_PEAK_TFLOPS) if mfma_bound else (gbs / HBM_PEAK_GBS), 4),
            "traffic": None, "kernel": "prefill_attn_kernel", "kernel_avg_us": round(kern_ms * 1e3, 2),
            "flops_per_launch": int(flops), "bytes_per_launch": int(per_stream), "unique_bytes_per_launch": int(unique),
            "ai_unique": round(flops / unique, 1), "ridge": round(ridge, 1),
            "fractions": {"mfma": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
                          "hbm_unique": round(unique / kern_s / 1e9 / HBM_PEAK_GBS, 4),
                          "hbm_per_stream": round(per_stream / kern_s / 1e9 / HBM_PEAK_GBS, 4)},
        },
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_attention(w, pairs),
    }
    print(json.dumps(out_line), flush=True)


def cpu_baseline_attention(w, pairs_all, budget_s=15.0):
    """The oracle attention on whole rows until the budget is used."""
    from oracle import attention, indexer

    done_pairs, rows = 0, 0
    t0 = time.perf_counter()
    for r in range(w.rows):
        pos = attention.attended_positions(w.lists[r], w.first_pos, r, w.ratio)
        logical = np.unique(pos // w.block_size)
        pages = w.block_table[logical]
        bt = np.zeros(w.block_table.shape, dtype=np.int64)
        bt[logical] = np.arange(logical.size)
        attention.prefill_attn(indexer.upcast(w.q[r:r + 1], "bf16"), indexer.upcast(w.k_cache[pages], "bf16"),
                               indexer.upcast(w.v_cache[pages], "bf16"), bt, w.lists[r:r + 1], w.first_pos + r, w.ratio,
                               w.block_size, w.nkv, w.hd ** -0.5)
        done_pairs += pos.size * w.nq
        rows += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": done_pairs / dt, "unit": "query-head x position pairs/s",
            "cores": int(len(os.sched_getaffinity(0))), "kind": "oracle",
            "sample": f"{rows} of {w.rows} rows ({done_pairs} pairs), float64 numpy: {dt:.2f} s"}


def run_gather(args, name):
    """The selected-entry gathers: one step is one gather call, timed back to back."""
    import torch

    import sparse_attention_lightning_block_amd as salb
    from workloads.device import bf16_tensor
    from workloads.gather import GATHER_WORKLOADS

    w = GATHER_WORKLOADS[name]()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if name.startswith("qsa"):
        k = bf16_tensor(w.k_cache).to(dev)
        v = bf16_tensor(w.v_cache).to(dev)
        bt = torch.from_numpy(w.block_table).to(dev)
        sel = torch.from_numpy(w.sel).to(dev)
        ko = torch.empty((w.n_sel, w.nkv, w.hd), dtype=torch.bfloat16, device=dev)
        vo = torch.empty_like(ko)

        def step():
            salb.qsa_gather(k, v, bt, sel, k_out=ko, v_out=vo)

        row = w.nkv * w.hd * 2
        bytes_moved = w.n_sel * (2 * row * 2 + 4 + 4)      # K and V rows read and written, position, table entry
        units, unit = w.n_sel, "positions"
        kernel = "qsa_gather_kernel"
        cfg = {"workload": name, "n_sel": w.n_sel, "block_size": w.block_size, "nkv": w.nkv, "hd": w.hd,
               "cache_tokens": w.n_blocks * w.block_size}
    else:
        fp8 = torch.from_numpy(w.fp8).to(dev)
        sc = torch.from_numpy(w.scale).to(dev)
        rope = bf16_tensor(w.rope_bits).to(dev)
        bt = torch.from_numpy(w.block_table).to(dev)
        idx = torch.from_numpy(w.topk_idx).to(dev)
        out = torch.empty((w.T, w.top_k, w.d_nope + w.d_rope), dtype=torch.bfloat16, device=dev)

        def step():
            salb.indexer_gather_kv(fp8, sc, rope, bt, idx, group=w.group, out=out)

        n = w.entries
        per_entry = w.d_nope + 4 * (w.d_nope // w.group) + 2 * w.d_rope      # FP8 codes, scales, rope
        bytes_moved = n * (per_entry + 4) + w.T * w.top_k * (4 + 2 * (w.d_nope + w.d_rope))
        units, unit = n, "entries"
        kernel = "gather_kv_kernel"
        cfg = {"workload": name, "T": w.T, "top_k": w.top_k, "entries": n, "entries_per_block": w.epb,
               "d_nope": w.d_nope, "d_rope": w.d_rope, "group": w.group}
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ms_per_step, stage = timed_steps(torch, make_step(torch, [step], args.graph), 1, args.steps)
    kern_ms = back_to_back_ms(torch, step, args.steps)
    gbs = bytes_moved / (kern_ms / 1e3) / 1e9
    out = {
        "metric": METRIC,
        "value": units / (ms_per_step / 1e3),
        "unit": f"{unit}/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": dict(cfg, launch="hip_graph" if args.graph else "eager"),
        "step_ms": {"p10": float(np.percentile(stage[0], 10)), "p50": float(np.median(stage[0])),
                    "p90": float(np.percentile(stage[0], 90))},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "kernel": kernel,
                     "kernel_avg_us": round(kern_ms * 1e3, 2), "bytes_per_launch": int(bytes_moved)},
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_gather(w, name, units, unit),
    }
    print(json.dumps(out), flush=True)


def cpu_baseline_gather(w, name, units, unit):
    """The oracle gather on the whole workload (a few seconds), as it stands."""
    from oracle import gather

    t0 = time.perf_counter()
    if name.startswith("qsa"):
        gather.qsa_gather(w.k_cache, w.v_cache, w.block_table, w.sel, w.block_size)
    else:
        gather.gather_kv(w.fp8, w.scale, w.rope_bits, w.block_table, w.topk_idx, w.epb, w.group)
    dt = time.perf_counter() - t0
    return {"value": units / dt, "unit": f"{unit}/s", "cores": 1, "kind": "oracle",
            "sample": f"the whole workload ({units} {unit}), numpy on one thread: {dt:.2f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(WORKLOADS))
    ap.add_argument("--precision", default="mfma", choices=["mfma", "fp32"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold (rotated key pool) timing")
    ap.add_argument("--graph", action="store_true",
                    help="replay each stage from a captured HIP graph (slower than eager launches on this "
                         "ROCm stack: a graph launch costs more than the kernel launches it replaces)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the indexer path here is a "
              "single-GPU kernel library; see the design notes for how it would shard.", file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_attention_lightning_block_amd as salb
    from workloads.device import to_dev
    from workloads import make, make_diag

    if WORKLOADS[args.workload] == "qsa_decode":
        run_qsa_decode(args)
        return
    if WORKLOADS[args.workload] == "attention":
        run_attention(args)
        return
    if WORKLOADS[args.workload] == "gather":
        run_gather(args, args.workload)
        return
    w = make_diag(args.workload) if WORKLOADS[args.workload] == "diag" else make(WORKLOADS[args.workload])
    if w.kind == "qsa":
        run_qsa(args, w)
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = to_dev(w, dev)
    n_cols = w.max_lb * w.epb
    idx = torch.empty((w.T, w.top_k), dtype=torch.int32, device=dev)
    val = torch.empty((w.T, w.top_k), dtype=torch.float32, device=dev)
    ws = torch.empty(max(256, salb.indexer_score_topk_workspace_size(w.T, w.max_lb, w.epb, w.top_k)),
                     dtype=torch.uint8, device=dev)

    def fused():   # one step: indexer_score_topk, scorer + select, scores kept in the workspace
        salb.indexer_score_topk(**d, top_k=w.top_k, precision=args.precision, workspace=ws, out_idx=idx,
                                out_scores=val)

    for _ in range(args.warmup):
        fused()
    torch.cuda.synchronize()
    step = make_step(torch, [fused], args.graph)
    ms_per_step, stage = timed_steps(torch, step, 1, args.steps)
    step_ms = stage[0]
    pairs = w.pairs
    value = pairs / (ms_per_step / 1e3)

    # The stages on their own, each launched back to back with one event pair around
    # the run (no marker between launches): the scorer as indexer_score_rows (the same
    # kernel as in the step, plus the -inf tails of the split entry), the select as
    # indexer_topk_select on those scores.
    scores = torch.empty((w.T, n_cols), dtype=torch.float32, device=dev)
    sel_ws = torch.empty(max(256, salb.indexer_topk_workspace_size(w.T, n_cols, w.top_k)), dtype=torch.uint8,
                         device=dev)
    score_ms = back_to_back_ms(torch, lambda: salb.indexer_score_rows(**d, n_cols=n_cols, precision=args.precision,
                                                                      out=scores), args.steps)
    select_ms = back_to_back_ms(torch, lambda: salb.indexer_topk_select(scores, w.top_k, valid_lens=d["valid_lens"],
                                                                        workspace=sel_ws, out_idx=idx, out_scores=val),
                                args.steps)
    cold = None
    if args.workload in COLD_WORKLOADS and not args.no_cold and not args.graph:
        cold = cold_timing(torch, salb, d, w, args, ws, idx, val)
    mfma = args.precision == "mfma"
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "scores/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if mfma else "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "T": w.T, "H": w.H, "D": w.D, "entries_per_block": w.epb, "S": n_cols, "top_k": w.top_k,
            "pairs": pairs, "precision": args.precision, "entry": "indexer_score_topk",
            "launch": "hip_graph" if args.graph else "eager",
        },
        "step_ms": {"p10": float(np.percentile(step_ms, 10)), "p50": float(np.median(step_ms)),
                    "p90": float(np.percentile(step_ms, 90))},
        "stage_ms": {"score": score_ms, "select": select_ms},
        "roofline": csa_roofline(w, score_ms / 1e3, args.precision),
        "cold": cold,
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline(w),
    }
    print(json.dumps(out), flush=True)


def back_to_back_ms(torch, fn, n):
    """Average ms of n back-to-back calls of fn.  The n calls are captured into one HIP
    graph (the library allocates nothing and issues no memset, so they capture as plain
    kernel nodes) and the graph is replayed between two events on the current stream,
    the stream the library launches on: the host's per-call cost, which exceeds the
    shortest kernels' run time, leaves no gap between the launches."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            fn()
    g.replay()  # the first replay uploads the graph
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    del g
    return a.elapsed_time(b) / n


def csa_bytes(w):
    """Algorithmic bytes of one scorer launch: per stream (each row reads its own block-table
    row of pages, as the API defines it) and unique (each page read once, whoever reads
    it), plus q, w and the valid scores written."""
    per_key = w.D / 2 + w.D / 16
    used = [-(-int(v) // w.epb) for v in w.valid_lens]
    q_bytes = w.T * w.H * w.D * (2 if w.q_dtype == "bf16" else 4) + w.T * w.H * 4
    out_bytes = w.pairs * 4
    per_stream = w.pairs * key_bytes_per_entry(w.D, w.epb) + q_bytes + out_bytes
    pages = set()
    for t in range(w.T):
        pages.update(w.block_table[t, : used[t]].tolist())
    unique = len(pages) * (w.epb * per_key + 4) + 4 * sum(used) + q_bytes + out_bytes
    return per_stream, unique


def csa_roofline(w, score_s, precision):
    """Roofline of the scorer, the dominant kernel.  The binding roof follows from the
    unique-byte intensity: above the fp16 ridge (2500 TFLOP/s over 8 TB/s) the matrix
    cores bind, below it HBM (rows on pages of their own).  All three fractions are
    reported beside each other."""
    flops = 2.0 * w.pairs * w.H * w.D
    per_stream, unique = csa_bytes(w)
    traffic = scorer_traffic(w.name) if precision == "mfma" else None
    tflops = flops / score_s / 1e12
    # the matrix peak of the path's own operand type: fp16 for the MFMA path, fp32 for FP32
    mpeak = MFMA_F16_PEAK_TFLOPS if precision == "mfma" else MFMA_F32_PEAK_TFLOPS
    ridge = mpeak / (HBM_PEAK_GBS / 1e3)
    ai_unique = flops / unique
    frac = {
        "mfma": round(tflops / mpeak, 4),
        "hbm_per_stream": round(per_stream / score_s / 1e9 / HBM_PEAK_GBS, 4),
        "hbm_unique": round(unique / score_s / 1e9 / HBM_PEAK_GBS, 4),
        "hbm_counter": None if traffic is None else round(traffic / score_s / 1e9 / HBM_PEAK_GBS, 4),
    }
    # the FP32 path runs on the fp32 matrix cores at D 64/128 (the vector ALUs otherwise)
    f32_mfma = precision != "mfma" and w.D in (64, 128)
    if f32_mfma:
        bound, achieved, peak, unit = "mfma", tflops, MFMA_F32_PEAK_TFLOPS, "TFLOP/s"
    elif precision != "mfma":
        bound, achieved, peak, unit = "alu", tflops, VALU_F32_PEAK_TFLOPS, "TFLOP/s"
    elif ai_unique > ridge:
        bound, achieved, peak, unit = "mfma", tflops, MFMA_F16_PEAK_TFLOPS, "TFLOP/s"
    else:
        bound, achieved, peak, unit = "hbm", per_stream / score_s / 1e9, HBM_PEAK_GBS, "GB/s"
    return {
        "bound": bound,
        "achieved": round(achieved, 2),
        "peak": peak,
        "unit": unit,
        "frac": round(achieved / peak, 4),
        "traffic": traffic,
        "kernel": ("score_mfma_group_kernel" if w.T >= 4 else "score_mfma_split_kernel") if precision == "mfma"
        else "score_f32mfma_kernel" if f32_mfma else "score_f32_kernel",
        "kernel_avg_us": round(score_s * 1e6, 2),
        "flops_per_launch": int(flops),
        "bytes_per_launch": int(per_stream),
        "unique_bytes_per_launch": int(unique),
        "ai_unique": round(ai_unique, 1),
        "ai_counter": None if traffic is None else round(flops / traffic, 1),
        "ridge": round(ridge, 1),
        "fractions": frac,
    }


def cold_timing(torch, salb, d, w, args, ws, idx, val):
    """The same step with the key pool (codes, scales, global scales) rotated through
    copies, so that a copy's keys have left the caches before it is used again."""
    pool = [d["keys_fp4"], d["key_scale"], d["key_gscale"]]
    pool_bytes = sum(t.numel() * t.element_size() for t in pool)
    copies = max(2, -(-COLD_SPAN_BYTES // pool_bytes))
    sets = [d] + [dict(d, keys_fp4=pool[0].clone(), key_scale=pool[1].clone(), key_gscale=pool[2].clone())
                  for _ in range(copies - 1)]
    turn = [0]

    def fused():
        salb.indexer_score_topk(**sets[turn[0] % copies], top_k=w.top_k, precision=args.precision, workspace=ws,
                                out_idx=idx, out_scores=val)
        turn[0] += 1

    for _ in range(min(args.warmup, copies)):
        fused()
    torch.cuda.synchronize()
    ms_per_step, _ = timed_steps(torch, make_step(torch, [fused], False), 1, args.steps)
    del sets
    return {
        "copies": copies,
        "pool_mb": round(pool_bytes / 2**20, 2),
        "ms_per_step": ms_per_step,
        "value": w.pairs / (ms_per_step / 1e3),
    }


if __name__ == "__main__":
    main()
