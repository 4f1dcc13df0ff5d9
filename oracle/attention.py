"""Block-sparse prefill attention over the selected blocks (float64 oracle).

Test infrastructure only; see the package docstring.

Source: [qsa.rs] "metrale_model_layers/layers/ops/qsa.rs", qsa_prefill_attn: for each
prefill row and query head, attention over exactly the blocks in the row's selection
list plus the incomplete tail, read from the paged K/V cache; the result overwrites
the row's context in the output.  Its arguments name the pieces: q, the paged k/v
caches with their block table and page size, the lists, rows, first_pos, topk, ratio,
nq and nkv heads, hd and the softmax scale inv_sqrt_d.

Readings where the page is silent (listed with the design notes):
* Row r sits at position pos = first_pos + r and has nb = floor((pos + 1) / ratio)
  complete blocks.  Block b covers positions [ratio * b, ratio * b + ratio).  The
  incomplete tail is positions [ratio * nb, pos]: the tokens after the last complete
  block, the row's own token included (empty when pos + 1 is a multiple of ratio).
* A list entry b attends its block when 0 <= b < nb; -1 (the padding of a top-k) and
  anything outside [0, nb) are skipped.  Entries are taken as given: a block listed
  twice would be attended twice (a top-k never lists one twice).
* Query head h reads KV head h // (nq / nkv) (grouped-query attention).
* Position s lives in cache page block_table[s // block_size], slot s % block_size;
  the caches are [pages, block_size, nkv, hd].
* out[r, h] = sum_j softmax_j(inv_sqrt_d * q[r, h] . k_j) * v_j over the attended
  positions j; a row with no attended position gets zeros.
"""

from __future__ import annotations

import numpy as np


def attended_positions(lists_row, first_pos, r, ratio):
    """Positions row r attends: its listed complete blocks, then the incomplete tail."""
    pos = first_pos + r
    nb = (pos + 1) // ratio
    out = []
    for b in np.asarray(lists_row, dtype=np.int64):
        if 0 <= b < nb:
            out.extend(range(int(b) * ratio, int(b) * ratio + ratio))
    out.extend(range(nb * ratio, pos + 1))
    return np.asarray(out, dtype=np.int64)


def prefill_attn(q, k_cache, v_cache, block_table, lists, first_pos, ratio, block_size, nkv, inv_sqrt_d):
    """out [rows, nq, hd] float64.  q [rows, nq, hd] and the caches as float64 (bf16
    inputs upcast exactly by the caller); lists [rows, topk] int."""
    q = np.asarray(q, dtype=np.float64)
    rows, nq, hd = q.shape
    group = nq // nkv
    kc = np.asarray(k_cache, dtype=np.float64)
    vc = np.asarray(v_cache, dtype=np.float64)
    bt = np.asarray(block_table, dtype=np.int64)
    out = np.zeros((rows, nq, hd))
    for r in range(rows):
        pos = attended_positions(lists[r], first_pos, r, ratio)
        if pos.size == 0:
            continue
        page, slot = bt[pos // block_size], pos % block_size
        for kvh in range(nkv):
            k = kc[page, slot, kvh]                   # [n, hd]
            v = vc[page, slot, kvh]
            for h in range(kvh * group, (kvh + 1) * group):
                s = (k @ q[r, h]) * inv_sqrt_d
                p = np.exp(s - s.max())
                out[r, h] = (p / p.sum()) @ v
    return out
