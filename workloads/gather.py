"""Seeded synthetic inputs for the selected-entry gathers.

Only random draws and storage encoding: FP8 E4M3 codes with an fp32 scale per
``group`` dims (absmax / 448, the largest E4M3 magnitude), bf16 bit patterns, block
tables and top-k index lists.  Nothing here decodes or gathers.

Streams: seed + [j] with j = 0 block table, 1 valid lengths, 2 nope values, 3 rope
values, 4 selected indices (the seed conventions of ``workloads.configs``).
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .configs import _rng, e4m3_encode_rne, to_bf16_bits


@dataclass
class GatherWorkload:
    name: str
    T: int
    P: int
    epb: int
    max_lb: int
    top_k: int
    d_nope: int
    d_rope: int
    group: int
    fp8: np.ndarray          # uint8 [P, epb, d_nope]
    scale: np.ndarray        # float32 [P, epb, d_nope / group]
    rope_bits: np.ndarray    # uint16 [P, epb, d_rope]
    block_table: np.ndarray  # int32 [T, max_lb]
    valid_lens: np.ndarray   # int32 [T]
    topk_idx: np.ndarray     # int32 [T, top_k], -1 padded
    source: Optional[np.ndarray] = None   # float32 [P, epb, d_nope] before quantisation

    @property
    def entries(self) -> int:
        return int((self.topk_idx >= 0).sum())


def make_gather(name, seed, T, P, epb, max_lb, top_k, d_nope=512, d_rope=64, group=128, amp=None,
                valid_lens=None, table="shared") -> GatherWorkload:
    """A paged FP8 + BF16 KV pool and, per row, top_k distinct entries of [0, valid_len)
    in random order (rows shorter than top_k select every entry, then -1)."""
    r_bt, r_v, r_x, r_r, r_s = (_rng(seed, j) for j in range(5))
    if table == "shared":
        bt = np.tile(r_bt.permutation(P)[:max_lb].astype(np.int32), (T, 1))
    else:
        bt = np.stack([r_bt.permutation(P)[:max_lb] for _ in range(T)]).astype(np.int32)
    if valid_lens is None:
        valid_lens = r_v.integers(max_lb * epb // 2, max_lb * epb + 1, size=T)
    vl = np.asarray(valid_lens, dtype=np.int32)
    if amp is None:
        x = r_x.standard_normal((P, epb, d_nope), dtype=np.float32)
    else:
        x = r_x.uniform(-amp, amp, size=(P, epb, d_nope)).astype(np.float32)
    g = x.reshape(P, epb, d_nope // group, group)
    amax = np.abs(g).max(axis=-1)
    scale = np.where(amax > 0, amax / 448.0, 1.0).astype(np.float32)
    codes = e4m3_encode_rne(g / scale[..., None]).reshape(P, epb, d_nope)
    rope = to_bf16_bits(r_r.standard_normal((P, epb, d_rope), dtype=np.float32))
    idx = np.full((T, top_k), -1, dtype=np.int32)
    for t in range(T):
        n = int(vl[t])
        k = min(top_k, n)
        idx[t, :k] = r_s.choice(n, size=k, replace=False) if k else []
    return GatherWorkload(name=name, T=T, P=P, epb=epb, max_lb=max_lb, top_k=top_k, d_nope=d_nope, d_rope=d_rope,
                          group=group, fp8=codes, scale=scale, rope_bits=rope, block_table=bt, valid_lens=vl,
                          topk_idx=idx, source=x)


@dataclass
class QsaGatherWorkload:
    name: str
    n_blocks: int
    block_size: int
    nkv: int
    hd: int
    k_cache: np.ndarray      # uint16 bf16 bits [n_blocks, block_size, nkv, hd]
    v_cache: np.ndarray
    block_table: np.ndarray  # int32 [n_blocks] (one sequence)
    sel: np.ndarray          # int32 [n_sel] token positions

    @property
    def n_sel(self) -> int:
        return int(self.sel.shape[0])


def make_qsa_gather(name, seed, n_blocks, block_size, nkv, hd, n_sel) -> QsaGatherWorkload:
    """A paged bf16 K/V cache of one sequence and n_sel distinct selected positions."""
    r_bt, _, r_k, r_v, r_s = (_rng(seed, j) for j in range(5))
    bt = r_bt.permutation(n_blocks).astype(np.int32)
    k = to_bf16_bits(r_k.standard_normal((n_blocks, block_size, nkv, hd), dtype=np.float32))
    v = to_bf16_bits(r_v.standard_normal((n_blocks, block_size, nkv, hd), dtype=np.float32))
    sel = np.sort(r_s.choice(n_blocks * block_size, size=n_sel, replace=False)).astype(np.int32)
    return QsaGatherWorkload(name=name, n_blocks=n_blocks, block_size=block_size, nkv=nkv, hd=hd, k_cache=k,
                             v_cache=v, block_table=bt, sel=sel)


def _gather_long_decode():
    """The long-context decode shape (32 queries, 4096 pages of 64 entries, valid lengths
    U{131072..262144}, top_k 2048) over a KV pool of 512 FP8 dims (fp32 scale per 128)
    and 64 bf16 rope dims per entry."""
    return make_gather("gather_T32_k2048", [6], T=32, P=8192, epb=64, max_lb=4096, top_k=2048, d_nope=512,
                       d_rope=64, group=128, valid_lens=_rng([6], 1).integers(131072, 262145, size=32))


def _qsa_gather_decode():
    """One query's selection in the QSA prefill shape: 256 blocks of 16 tokens (4096
    positions) gathered from a paged bf16 K/V cache of 262144 tokens (4096 pages of 64),
    4 KV heads of 128 dims."""
    return make_qsa_gather("qsa_gather_4096", [7], n_blocks=4096, block_size=64, nkv=4, hd=128, n_sel=4096)


GATHER_WORKLOADS = {
    "gather_T32_k2048": _gather_long_decode,
    "qsa_gather_4096": _qsa_gather_decode,
}
