"""Seeded synthetic inputs for the block-sparse prefill attention.

Only random draws and bf16 packing: a paged bf16 K/V cache of one sequence, the
prefill rows' queries, and per row a list of distinct complete blocks (-1 padded, plus
a few entries outside the row's complete blocks that the attention must skip).
Streams: seed + [j] with j = 0 block table, 1 lists, 2 q, 3 keys, 4 values.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .configs import _rng, to_bf16_bits


@dataclass
class AttnWorkload:
    name: str
    rows: int
    first_pos: int
    ratio: int
    block_size: int
    nq: int
    nkv: int
    hd: int
    topk: int
    q: np.ndarray            # uint16 bf16 bits [rows, nq, hd]
    k_cache: np.ndarray      # uint16 bf16 bits [pages, block_size, nkv, hd]
    v_cache: np.ndarray
    block_table: np.ndarray  # int32 [pages]
    lists: np.ndarray        # int32 [rows, topk]


def make_attention(name, seed, rows, first_pos, ratio, block_size, nq, nkv, hd, topk, pad_frac=0.0,
                   junk=False) -> AttnWorkload:
    """Row r lists min(topk, complete blocks) distinct complete blocks in random order,
    then -1; ``pad_frac`` of the rows keep only half their entries; ``junk`` plants an
    entry at or past the row's complete blocks in some rows (skipped by the attention)."""
    r_bt, r_l, r_q, r_k, r_v = (_rng(seed, j) for j in range(5))
    n_pos = first_pos + rows
    pages = -(-n_pos // block_size)
    bt = r_bt.permutation(pages).astype(np.int32)
    q = to_bf16_bits(r_q.standard_normal((rows, nq, hd), dtype=np.float32))
    k = to_bf16_bits(r_k.standard_normal((pages, block_size, nkv, hd), dtype=np.float32))
    v = to_bf16_bits(r_v.standard_normal((pages, block_size, nkv, hd), dtype=np.float32))
    lists = np.full((rows, topk), -1, dtype=np.int32)
    for r in range(rows):
        nb = (first_pos + r + 1) // ratio
        n = min(topk, nb)
        if pad_frac and r_l.random() < pad_frac:
            n //= 2
        if n:
            lists[r, :n] = r_l.choice(nb, size=n, replace=False)
        if junk and topk > n and r % 3 == 0:
            lists[r, n] = nb + r % 2                 # not complete yet (or past the end)
    return AttnWorkload(name=name, rows=rows, first_pos=first_pos, ratio=ratio, block_size=block_size, nq=nq, nkv=nkv,
                        hd=hd, topk=topk, q=q, k_cache=k, v_cache=v, block_table=bt, lists=lists)


def qsa_prefill_attention():
    """The QSA prefill shape: 2048 rows at positions 522240 .. 524287, 16 positions per
    block, the top 256 blocks per row; a 524288-position cache in pages of 64, 32 query
    heads over 4 KV heads of 128 dims."""
    return make_attention("qsa_prefill_attn", [9], rows=2048, first_pos=522240, ratio=16, block_size=64, nq=32,
                          nkv=4, hd=128, topk=256)
