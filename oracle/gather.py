"""Selected-entry gather (float64 oracle): the top-k indices turned into dense tiles.

Test infrastructure only; see the package docstring.

Sources:
* [commits] "nvfp4-megamoe-kernel -- commit graph of dsv4/kernels/indexer", commit
  c2f705a21a (gather_kv.cu): for each (query, selected entry), the entry is located in
  the paged pool through the block table, its FP8 part is dequantised to BF16, its
  BF16 RoPE part is copied exactly, and the result is a dense [T, top_k, head_dim]
  BF16 tile; the FP8 round trip is stated to stay under 0.01 absolute.
* [qsa.rs] "metrale_model_layers/layers/ops/qsa.rs", qsa_gather: the selected tokens'
  K and V rows are copied into contiguous [n_sel, nkv, hd] scratch, slot i holding
  the token at position sel[i] of the paged cache.

Readings where the pages are silent (listed with the design notes):
* CSA pool layout: per physical page p and slot e, ``fp8[p, e, :d_nope]`` (OCP E4M3
  codes), ``scale[p, e, :d_nope/group]`` (fp32, one per ``group`` consecutive dims)
  and ``rope[p, e, :d_rope]`` (bf16).  Output dims [0, d_nope) are the dequantised
  part, [d_nope, d_nope + d_rope) the RoPE part.
* Dequantised value: one round-to-nearest-even of the exact product e4m3 * scale to
  bfloat16 (the product is exact in float64), as for the NVFP4 keys.
* Index -1 (a padded top-k slot) gives an all-zero row.
* QSA cache layout: ``cache[phys_block, slot, kv_head, dim]``, position s at logical
  block s // block_size, slot s % block_size, physical block block_table[s // block_size].
"""

from __future__ import annotations

import numpy as np

from . import nvfp4


def bf16_rne(x) -> np.ndarray:
    """float64 values -> bfloat16 bit patterns (uint16), one round-to-nearest-even.

    Each value is split into its sign and |x| = m * 2^e with m in [1, 2) (frexp); the
    8-bit significand is m * 2^7 rounded half to even (numpy's rint), exactly, since
    both m * 2^7 and its rounding are exact in float64.  Magnitudes below the smallest
    normal bfloat16 are rounded on the subnormal grid 2^-133; overflow gives infinity.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.uint16)
    sign = np.signbit(x).astype(np.uint32) << 15
    a = np.abs(x)
    nan = np.isnan(a)
    m, e = np.frexp(a)                   # a = m * 2^e, m in [0.5, 1)
    m, e = m * 2.0, e - 1                # m in [1, 2)
    normal = (a != 0) & np.isfinite(a) & (e >= -126)
    sig = np.rint(np.where(normal, m, 0.0) * 128.0)          # 128 .. 256, ties to even
    carry = sig == 256.0
    sig = np.where(carry, 128.0, sig)
    e = np.where(carry, e + 1, e)
    bits = ((e + 127).astype(np.int64) << 7) | (sig.astype(np.int64) - 128)
    bits = np.where(e > 127, 0x7F80, bits)                     # overflow: infinity
    sub = (a != 0) & ~nan & (e < -126)
    sub_bits = np.rint(np.where(sub, a, 0.0) * 2.0 ** 133).astype(np.int64)   # may round up to 0x80
    res = np.where(normal, bits, np.where(sub, sub_bits, 0))
    res = np.where(np.isinf(a), 0x7F80, res)
    res = np.where(nan, 0x7FC0, res)
    out[...] = (res.astype(np.uint32) | sign).astype(np.uint16)
    return out


def gather_kv(fp8, scale, rope_bits, block_table, topk_idx, epb, group):
    """Dense BF16 tiles [T, k, d_nope + d_rope] (uint16 bit patterns) of the selected entries.

    fp8 [P, epb, d_nope] uint8, scale [P, epb, d_nope / group] float32, rope_bits
    [P, epb, d_rope] uint16, block_table [T, max_lb] int32, topk_idx [T, k] int32
    (logical entries, -1 padded).
    """
    fp8 = np.asarray(fp8, dtype=np.uint8)
    P, e, d_nope = fp8.shape
    if e != epb:
        raise ValueError("fp8 must be [P, epb, d_nope]")
    d_rope = rope_bits.shape[-1]
    idx = np.asarray(topk_idx, dtype=np.int64)
    T, k = idx.shape
    out = np.zeros((T, k, d_nope + d_rope), dtype=np.uint16)
    for t in range(T):
        sel = idx[t] >= 0
        s = idx[t][sel]
        phys, entry = nvfp4.resolve(block_table[t], s, epb)
        if s.size and (phys.min() < 0 or phys.max() >= P):
            raise ValueError("block_table entry outside the pool")
        codes = fp8.reshape(P * epb, d_nope)[entry]
        sc = np.asarray(scale, dtype=np.float32).reshape(P * epb, -1)[entry].astype(np.float64)
        vals = nvfp4.e4m3_decode(codes) * np.repeat(sc, group, axis=-1)   # exact in float64
        out[t, sel, :d_nope] = bf16_rne(vals)
        out[t, sel, d_nope:] = np.asarray(rope_bits).reshape(P * epb, d_rope)[entry]
    return out


def qsa_gather(k_cache, v_cache, block_table, sel, block_size):
    """(k_out, v_out) [n_sel, nkv, hd]: slot i holds the cache rows of position sel[i]."""
    s = np.asarray(sel, dtype=np.int64)
    lb = s // block_size
    phys = np.asarray(block_table, dtype=np.int64)[lb]
    slot = s % block_size
    return np.asarray(k_cache)[phys, slot], np.asarray(v_cache)[phys, slot]
