"""Lightning-indexer scores and top-k (float64 oracle).

Test infrastructure only; see the package docstring.

Definition ([listing], header comment quoting eq. 16, and the scoring loop of the
main kernel):

    I[t, s] = sum_h w[t, h] * ReLU( q[t, h, :] . k[s, :] ),   s in [0, valid_len[t])
    Selected[t] = TopK(I[t, :], k)

One key vector k[s] per logical entry, shared by all heads (the kernel indexes the
key without a head index).  k[s] = c[s] * g[phys(s)] from ``oracle.nvfp4``; the
product is exact in float64, and so are the upcasts of fp32/bf16 q and fp32 w, so
the only roundings are those of the float64 dot products and sums.

Top-k order ([listing], the comparator of ``heap_insert`` and the final selection
sort): score descending, equal scores by increasing index.  The ``min(k, valid)``
winners come first; the remaining output slots are -1, as the kernel's heap is
initialised to (-inf, -1) and those entries sort last.  NaN scores rank below every
number (they never occur in the configured workloads).
"""

from __future__ import annotations

import numpy as np

from . import nvfp4


def upcast(x, dtype: str = "f32") -> np.ndarray:
    """float32 array, or bfloat16 given as uint16 bit patterns -> exact float64."""
    a = np.asarray(x)
    if dtype == "bf16":
        if a.dtype != np.uint16:
            raise TypeError("bf16 inputs are passed as uint16 bit patterns")
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return a.astype(np.float32).astype(np.float64)
    raise ValueError(dtype)


def score_row(q_t, w_t, c, g, chunk: int = 65536) -> np.ndarray:
    """I[s] for one query: q_t [H, D] f64, w_t [H] f64, c [n, D] f64, g [n] f64."""
    n = c.shape[0]
    out = np.empty(n, dtype=np.float64)
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        keys = c[a:b] * g[a:b, None]           # exact
        dots = q_t @ keys.T                    # [H, b-a]
        out[a:b] = w_t @ np.maximum(dots, 0.0)
    return out


def scores(q, w, keys_fp4, key_scale, key_gscale, block_table, valid_lens, epb, q_dtype="f32"):
    """List of per-query score vectors I[t, 0:valid_len[t]] in float64."""
    qf = upcast(q, q_dtype)
    wf = upcast(w, "f32")
    T = qf.shape[0]
    res = []
    for t in range(T):
        c, g = nvfp4.dequant_row(keys_fp4, key_scale, key_gscale, block_table[t], valid_lens[t], epb)
        res.append(score_row(qf[t], wf[t], c, g))
    return res


def topk(row_scores, k: int):
    """Indices [k] (int32, -1 padded) and scores [k] (float64, -inf padded) of the top k."""
    v = np.asarray(row_scores, dtype=np.float64)
    n = v.shape[0]
    order = np.lexsort((np.arange(n), -v))     # primary: score desc; secondary: index asc
    kk = min(k, n)
    idx = np.full(k, -1, dtype=np.int32)
    val = np.full(k, -np.inf, dtype=np.float64)
    idx[:kk] = order[:kk]
    val[:kk] = v[order[:kk]]
    return idx, val


def score_topk(q, w, keys_fp4, key_scale, key_gscale, block_table, valid_lens, epb, top_k, q_dtype="f32"):
    """(idx [T, k] int32, vals [T, k] float64, per-row scores list)."""
    rows = scores(q, w, keys_fp4, key_scale, key_gscale, block_table, valid_lens, epb, q_dtype)
    T = len(rows)
    idx = np.empty((T, top_k), dtype=np.int32)
    val = np.empty((T, top_k), dtype=np.float64)
    for t, r in enumerate(rows):
        idx[t], val[t] = topk(r, top_k)
    return idx, val, rows
