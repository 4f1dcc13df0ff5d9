"""Helpers shared by the GPU parity tests: moving workloads to the device, the
tolerances, and the top-k set rules.  Expected values come only from ``oracle``."""

from __future__ import annotations

import numpy as np
from oracle import indexer, nvfp4
from workloads.device import to_dev  # noqa: F401  (re-exported for the tests)

FP32_REL = 1e-5      # FP32 path: |dI| <= 1e-5 |I| + 1e-6 * A
FP32_ABS_A = 1e-6
MFMA_ROWMAX = 2e-3   # matrix-core path: |dI| <= 2e-3 * max_s |I[t, s]|


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


def oracle_rows_all(w, rows=None):
    """oracle_rows for many rows of one workload: when every requested row reads the same
    block table (one sequence), the keys are dequantised once by the oracle for the longest
    row and each row takes its prefix; otherwise row by row.  Same results as oracle_rows."""
    rows = list(range(w.T)) if rows is None else list(rows)
    bt = w.block_table
    if not all(np.array_equal(bt[rows[0]], bt[t]) for t in rows):
        return oracle_rows(w, rows)
    n_max = max(int(w.valid_lens[t]) for t in rows)
    c, g = nvfp4.dequant_row(w.keys_fp4, w.key_scale, w.key_gscale, bt[rows[0]], n_max, w.epb)
    q = indexer.upcast(w.q, w.q_dtype)
    wt = w.w.astype(np.float64)
    kabs = np.abs(c * g[:, None])
    out, amag = {}, {}
    for t in rows:
        v = int(w.valid_lens[t])
        out[t] = indexer.score_row(q[t], wt[t], c[:v], g[:v])
        amag[t] = np.abs(wt[t]) @ (np.abs(q[t]) @ kabs[:v].T)
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


# Set differences the tests have seen beyond tau (but within 2 tau) of the oracle's K-th
# score, per check label; printed by tests that run with -s and summarised in the
# design notes.
BEYOND_TAU = {}
# Every top-k row check of the session: rows checked, rows whose set differs from the
# oracle's, and the differing entries (a differing pair counts twice: one in, one out).
TOPK_CHECKS = {"rows": 0, "rows_differing": 0, "entries_differing": 0}


def check_topk(gpu_idx, gpu_val, ref, amag, k, precision, what="", tol=None):
    """Set rules: K_t winners in [0, valid), distinct, -1 padded; the GPU order is its own
    scores descending, ties by index; any disagreement with the oracle's set lies near the
    oracle's K-th score.

    "Near" is checked at 2 tau: an entry whose GPU score errs up by tau can displace one
    whose GPU score errs down by tau, so two correct scorers can swap entries up to 2 tau
    apart.  The number of differing entries farther than tau (the literal reading) is
    recorded in BEYOND_TAU[what] and returned with the total: (n_diff, n_beyond_tau).
    ``tol`` (per entry) replaces the precision's score tolerance when given."""
    gpu_idx = np.asarray(gpu_idx)
    n = ref.shape[0]
    K = min(k, n)
    assert np.all(gpu_idx[K:] == -1), f"{what}: padding"
    g = gpu_idx[:K]
    assert len(set(g.tolist())) == K, f"{what}: duplicates"
    assert np.all((g >= 0) & (g < n)), f"{what}: index out of [0, valid)"
    if K == 0:
        TOPK_CHECKS["rows"] += 1
        return 0, 0
    o_idx, o_val = indexer.topk(ref, k)
    vk = o_val[K - 1]
    if tol is None:
        tol = score_tol(ref, amag, precision)
    diff = set(g.tolist()) ^ set(o_idx[:K].tolist())
    tol_k = tol[o_idx[K - 1]]
    beyond = 0
    for s in diff:
        t = max(tol[s], tol_k)
        assert abs(ref[s] - vk) <= 2 * t, (
            f"{what}: entry {s} (score {ref[s]}) differs from the oracle set, k-th {vk}, tol {tol[s]}")
        beyond += abs(ref[s] - vk) > t
    if beyond:
        BEYOND_TAU[what] = beyond
    TOPK_CHECKS["rows"] += 1
    TOPK_CHECKS["rows_differing"] += bool(diff)
    TOPK_CHECKS["entries_differing"] += len(diff)
    if gpu_val is not None:
        v = np.asarray(gpu_val[:K], dtype=np.float64)
        assert np.all(np.isneginf(np.asarray(gpu_val[K:]))), f"{what}: score padding"
        for i in range(K - 1):
            assert v[i] > v[i + 1] or (v[i] == v[i + 1] and g[i] < g[i + 1]), f"{what}: order at {i}"
    return len(diff), beyond
