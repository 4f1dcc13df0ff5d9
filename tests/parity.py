"""Helpers shared by the GPU parity tests: moving workloads to the device, the
tolerances, and the top-k set rules.  Expected values come only from ``oracle``."""

from __future__ import annotations

import numpy as np
import torch

from oracle import indexer, nvfp4

FP32_REL = 1e-5      # FP32 path: |dI| <= 1e-5 |I| + 1e-6 * A
FP32_ABS_A = 1e-6
MFMA_ROWMAX = 2e-3   # matrix-core path: |dI| <= 2e-3 * max_s |I[t, s]|


def to_dev(w, device="cuda"):
    """Device tensors of a CSA workload."""
    if w.q_dtype == "bf16":
        q = torch.from_numpy(w.q.view(np.int16).copy()).view(torch.bfloat16)
    else:
        q = torch.from_numpy(w.q.copy())
    return dict(
        q=q.to(device),
        w=torch.from_numpy(w.w.copy()).to(device),
        keys_fp4=torch.from_numpy(w.keys_fp4.copy()).to(device),
        key_scale=torch.from_numpy(w.key_scale.copy()).to(device),
        key_gscale=torch.from_numpy(w.key_gscale.copy()).to(device),
        block_table=torch.from_numpy(w.block_table.copy()).to(device),
        valid_lens=torch.from_numpy(w.valid_lens.astype(np.int32)).to(device),
    )


def oracle_rows(w, rows=None):
    """Oracle score vectors (float64) and abs-product sums A for the given rows."""
    rows = range(w.T) if rows is None else rows
    q = indexer.upcast(w.q, w.q_dtype)
    wt = w.w.astype(np.float64)
    out, amag = {}, {}
    for t in rows:
        c, g = nvfp4.dequant_row(w.keys_fp4, w.key_scale, w.key_gscale, w.block_table[t], w.valid_lens[t], w.epb)
        out[t] = indexer.score_row(q[t], wt[t], c, g)
        k = np.abs(c * g[:, None])
        amag[t] = np.abs(wt[t]) @ (np.abs(q[t]) @ k.T)
    return out, amag


def score_tol(ref, amag, precision):
    if precision == "fp32":
        return FP32_REL * np.abs(ref) + FP32_ABS_A * amag
    m = np.max(np.abs(ref)) if ref.size else 0.0
    return np.full(ref.shape, MFMA_ROWMAX * m)


def check_scores(got_row, ref, amag, precision, what=""):
    got = np.asarray(got_row, dtype=np.float64)
    n = ref.shape[0]
    tol = score_tol(ref, amag, precision)
    err = np.abs(got[:n] - ref)
    bad = np.nonzero(err > tol)[0]
    assert bad.size == 0, (f"{what}: {bad.size} scores out of tolerance, first {bad[:5]}: "
                           f"got {got[bad[:5]]} ref {ref[bad[:5]]} tol {tol[bad[:5]]}")
    return float(err.max()) if n else 0.0


def check_topk(gpu_idx, gpu_val, ref, amag, k, precision, what="", tol=None):
    """Set rules: K_t winners in [0, valid), distinct, -1 padded; any disagreement with the
    oracle's set lies within the score tolerance (both sides may err: 2 tau) of the
    oracle's K-th score; the GPU order is its own scores descending, ties by index.
    ``tol`` (per entry) replaces the precision's score tolerance when given."""
    gpu_idx = np.asarray(gpu_idx)
    n = ref.shape[0]
    K = min(k, n)
    assert np.all(gpu_idx[K:] == -1), f"{what}: padding"
    g = gpu_idx[:K]
    assert len(set(g.tolist())) == K, f"{what}: duplicates"
    assert np.all((g >= 0) & (g < n)), f"{what}: index out of [0, valid)"
    if K == 0:
        return 0
    o_idx, o_val = indexer.topk(ref, k)
    vk = o_val[K - 1]
    if tol is None:
        tol = score_tol(ref, amag, precision)
    diff = set(g.tolist()) ^ set(o_idx[:K].tolist())
    tol_k = tol[o_idx[K - 1]]
    for s in diff:
        assert abs(ref[s] - vk) <= 2 * max(tol[s], tol_k), (
            f"{what}: entry {s} (score {ref[s]}) differs from the oracle set, k-th {vk}, tol {tol[s]}")
    if gpu_val is not None:
        v = np.asarray(gpu_val[:K], dtype=np.float64)
        assert np.all(np.isneginf(np.asarray(gpu_val[K:]))), f"{what}: score padding"
        for i in range(K - 1):
            assert v[i] > v[i + 1] or (v[i] == v[i + 1] and g[i] < g[i + 1]), f"{what}: order at {i}"
    return len(diff)
