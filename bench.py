"""Benchmark of the lightning-indexer hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input resident in
HBM: the NVFP4 paged scorer (indexer_score_rows) and the per-row top-k
(indexer_topk_select) -- the same two stages indexer_score_topk runs.  Prints ONE
JSON line.  The default workload is the decode configuration
(T=8 queries, H=64, D=128, 64 keys per page, S=65536, top_k=2048).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--precision mfma|fp32]
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
MFMA_F16_PEAK_TFLOPS = 2516.0
VALU_F32_PEAK_TFLOPS = 157.3

WORKLOADS = {
    "tiny_decode": 1,
    "decode_T8_S65536": 2,
    "long_decode_T32_S262144": 3,
    "prefill_T4096": 4,
}


# HBM traffic of one scorer launch, from two rocprofv3 --pmc passes (FETCH_SIZE, then
# WRITE_SIZE, KiB per dispatch) scaled by what the same counters read for a plain
# 256 MiB copy (FETCH_SIZE x 1.9998, WRITE_SIZE x 1.0); the summaries are under
# profiles/.  Valid only for the scorer sources they were taken with: a different
# source hash reports null.
SCORER_SOURCES = ["score.hip", "nvfp4.hpp", "common.hpp", "internal.hpp"]
TRAFFIC_COPY_FACTOR = {"FETCH_SIZE": 1.9998, "WRITE_SIZE": 1.0}
SCORER_TRAFFIC_KIB = {   # workload: (FETCH_SIZE, WRITE_SIZE) KiB per dispatch
    "decode_T8_S65536": (3552.2, 2048.0),
    "long_decode_T32_S262144": (13693.5, 32768.8),
    "prefill_T4096": (35574.6, 65657.1),
}
SCORER_TRAFFIC_SHA = "bc82987ca976d653"


def scorer_source_sha():
    h = hashlib.sha256()
    for f in SCORER_SOURCES:
        with open(os.path.join(ROOT, "sparse_attention_lightning_block_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def scorer_traffic(workload):
    kib = SCORER_TRAFFIC_KIB.get(workload)
    if kib is None or scorer_source_sha() != SCORER_TRAFFIC_SHA:
        return None
    return int((kib[0] * TRAFFIC_COPY_FACTOR["FETCH_SIZE"] + kib[1] * TRAFFIC_COPY_FACTOR["WRITE_SIZE"]) * 1024)


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_T8_S65536", choices=sorted(WORKLOADS))
    ap.add_argument("--precision", default="mfma", choices=["mfma", "fp32"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the indexer path here is a "
              "single-GPU kernel library; see the design notes for how it would shard.", file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_attention_lightning_block_amd as salb
    from tests.parity import to_dev
    from workloads import make

    w = make(WORKLOADS[args.workload])
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = to_dev(w, dev)
    n_cols = w.max_lb * w.epb
    scores = torch.empty((w.T, n_cols), dtype=torch.float32, device=dev)
    idx = torch.empty((w.T, w.top_k), dtype=torch.int32, device=dev)
    val = torch.empty((w.T, w.top_k), dtype=torch.float32, device=dev)
    ws = torch.zeros(max(1, salb.indexer_topk_workspace_size(w.T, n_cols, w.top_k)), dtype=torch.uint8, device=dev)
    sc_view = scores

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        salb.indexer_score_rows(**d, n_cols=n_cols, precision=args.precision, out=sc_view)
        if ev is not None:
            ev[1].record()
        salb.indexer_topk_select(sc_view, w.top_k, valid_lens=d["valid_lens"], workspace=ws, out_idx=idx,
                                 out_scores=val)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        step(evs[i])
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    score_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    select_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    step_ms = score_ms + select_ms

    pairs = w.pairs
    value = pairs / (ms_per_step / 1e3)
    # dominant kernel: the scorer (one launch per step)
    bytes_alg = pairs * key_bytes_per_entry(w.D, w.epb) + w.T * w.H * w.D * (2 if w.q_dtype == "bf16" else 4) \
        + w.T * w.H * 4 + pairs * 4
    flops_alg = 2.0 * pairs * w.H * w.D
    score_avg_s = float(score_ms.mean()) / 1e3
    hbm_gbs = bytes_alg / score_avg_s / 1e9
    tflops = flops_alg / score_avg_s / 1e12
    mfma = args.precision == "mfma"
    roofline = {
        "bound": "hbm",
        "achieved": round(hbm_gbs, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(hbm_gbs / HBM_PEAK_GBS, 4),
        "traffic": scorer_traffic(w.name) if mfma else None,
        "kernel": ("score_mfma_group_kernel" if w.T >= 4 else "score_mfma_split_kernel") if mfma else "score_f32_kernel",
        "kernel_avg_us": round(score_avg_s * 1e6, 2),
        "bytes_per_launch": int(bytes_alg),
        "compute": {
            "achieved": round(tflops, 2),
            "peak": MFMA_F16_PEAK_TFLOPS if mfma else VALU_F32_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / (MFMA_F16_PEAK_TFLOPS if mfma else VALU_F32_PEAK_TFLOPS), 4),
            "flops_per_launch": int(flops_alg),
        },
    }
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
            "pairs": pairs, "precision": args.precision,
        },
        "step_ms": {"p10": float(np.percentile(step_ms, 10)), "p50": float(np.median(step_ms)),
                    "p90": float(np.percentile(step_ms, 90))},
        "stage_ms": {"score": float(np.median(score_ms)), "select": float(np.median(select_ms))},
        "roofline": roofline,
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline(w),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
