"""Thin PyTorch binding of the C ABI: each function marshals tensors into the C call
of the same name (pointers, sizes, the current HIP stream) and allocates outputs
and workspaces with torch.  All computation happens in the HIP library."""

from __future__ import annotations

from typing import Optional

import torch

from . import _lib
from ._lib import IDX_DTYPE_BF16, IDX_DTYPE_F32, IDX_F_VALIDATE, IDX_PREC_FP32, IDX_PREC_MFMA, check

PRECISION = {"fp32": IDX_PREC_FP32, "mfma": IDX_PREC_MFMA}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev(t: torch.Tensor, name: str, dtype=None, dims=None) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}")
    if dims is not None and t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dims")
    return t


def _row_stride(t: torch.Tensor) -> int:
    """Elements between rows of a 2-D tensor (a single row's stride is its width)."""
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def _q_dtype(q: torch.Tensor) -> int:
    return IDX_DTYPE_BF16 if q.dtype == torch.bfloat16 else IDX_DTYPE_F32


def indexer_score_rows(q, w, keys_fp4, key_scale, key_gscale, block_table, valid_lens, *, n_cols: int,
                       precision: str = "mfma", validate: bool = False,
                       out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """scores [T, n_cols] fp32: I[t, s] for s < valid_lens[t], -inf beyond.

    validate=True checks valid_lens and the block-table entries first (IDX_F_VALIDATE:
    the call then waits for the check) and raises IndexerError (code IDX_ERR_DATA) on
    out-of-range metadata."""
    _dev(q, "q", (torch.float32, torch.bfloat16), 3)
    _dev(w, "w", torch.float32, 2)
    _dev(keys_fp4, "keys_fp4", torch.uint8, 3)
    _dev(key_scale, "key_scale", torch.uint8, 3)
    _dev(key_gscale, "key_gscale", torch.float32, 1)
    _dev(block_table, "block_table", torch.int32, 2)
    _dev(valid_lens, "valid_lens", torch.int32, 1)
    T, H, D = q.shape
    P, epb, _ = keys_fp4.shape
    if out is None:
        out = torch.empty((T, n_cols), dtype=torch.float32, device=q.device)
    _dev(out, "out", torch.float32, 2)
    check(_lib.load().indexer_score_rows(
        _ptr(q), _q_dtype(q), _ptr(w), _ptr(keys_fp4), _ptr(key_scale), _ptr(key_gscale), _ptr(block_table),
        _row_stride(block_table), _ptr(valid_lens), T, H, D, epb, block_table.shape[1], P, PRECISION[precision],
        IDX_F_VALIDATE if validate else 0, _ptr(out), _row_stride(out), n_cols, _stream()))
    return out


def indexer_topk_workspace_size(rows: int, n_cols: int, top_k: int) -> int:
    return int(_lib.load().indexer_topk_workspace_size(rows, n_cols, top_k))


def indexer_topk_select(scores, top_k: int, *, valid_lens: Optional[torch.Tensor] = None, first_pos: int = 0,
                        ratio: int = 0, with_scores: bool = False, workspace: Optional[torch.Tensor] = None,
                        out_idx: Optional[torch.Tensor] = None, out_scores: Optional[torch.Tensor] = None):
    """(idx [rows, top_k] int32, scores [rows, top_k] fp32 or None).

    A caller-provided workspace is scratch of at least indexer_topk_workspace_size bytes
    (no initialisation needed)."""
    _dev(scores, "scores", torch.float32, 2)
    rows, n_cols = scores.shape
    dev = scores.device
    if valid_lens is not None:
        _dev(valid_lens, "valid_lens", torch.int32, 1)
    if out_idx is None:
        out_idx = torch.empty((rows, top_k), dtype=torch.int32, device=dev)
    if with_scores and out_scores is None:
        out_scores = torch.empty((rows, top_k), dtype=torch.float32, device=dev)
    if workspace is None:
        nbytes = indexer_topk_workspace_size(rows, n_cols, top_k)
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    check(_lib.load().indexer_topk_select(
        _ptr(scores), _row_stride(scores), _ptr(valid_lens), first_pos, ratio, rows, n_cols, top_k, _ptr(out_idx),
        _ptr(out_scores), _ptr(workspace), workspace.numel(), _stream()))
    return out_idx, out_scores


def indexer_score_topk_workspace_size(T: int, max_lb: int, epb: int, top_k: int) -> int:
    return int(_lib.load().indexer_score_topk_workspace_size(T, max_lb, epb, top_k))


def indexer_score_topk(q, w, keys_fp4, key_scale, key_gscale, block_table, valid_lens, *, top_k: int,
                       precision: str = "mfma", with_scores: bool = False, validate: bool = False,
                       workspace: Optional[torch.Tensor] = None, out_idx: Optional[torch.Tensor] = None,
                       out_scores: Optional[torch.Tensor] = None):
    """(idx [T, top_k] int32, scores [T, top_k] fp32 or None) = TopK of the indexer scores.

    A caller-provided workspace is scratch of at least indexer_score_topk_workspace_size
    bytes (no initialisation needed).  validate=True as for indexer_score_rows."""
    _dev(q, "q", (torch.float32, torch.bfloat16), 3)
    _dev(w, "w", torch.float32, 2)
    _dev(keys_fp4, "keys_fp4", torch.uint8, 3)
    _dev(key_scale, "key_scale", torch.uint8, 3)
    _dev(key_gscale, "key_gscale", torch.float32, 1)
    _dev(block_table, "block_table", torch.int32, 2)
    _dev(valid_lens, "valid_lens", torch.int32, 1)
    T, H, D = q.shape
    P, epb, _ = keys_fp4.shape
    max_lb = block_table.shape[1]
    dev = q.device
    if out_idx is None:
        out_idx = torch.empty((T, top_k), dtype=torch.int32, device=dev)
    if with_scores and out_scores is None:
        out_scores = torch.empty((T, top_k), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(indexer_score_topk_workspace_size(T, max_lb, epb, top_k), 256), dtype=torch.uint8,
                                device=dev)
    check(_lib.load().indexer_score_topk(
        _ptr(q), _q_dtype(q), _ptr(w), _ptr(keys_fp4), _ptr(key_scale), _ptr(key_gscale), _ptr(block_table),
        _row_stride(block_table), _ptr(valid_lens), T, H, D, epb, max_lb, P, top_k, PRECISION[precision],
        IDX_F_VALIDATE if validate else 0, _ptr(out_idx), _ptr(out_scores), _ptr(workspace), workspace.numel(),
        _stream()))
    return out_idx, out_scores


def indexer_score_topk_noalloc(q, w, keys_fp4, key_scale, key_gscale, block_table, valid_lens, *, top_k: int,
                               precision: str = "mfma", validate: bool = False, out_idx: Optional[torch.Tensor] = None,
                               out_scores: Optional[torch.Tensor] = None, with_scores: bool = False):
    """indexer_score_topk with the library's own per-GPU scratch instead of a workspace
    (for callers that cannot allocate device memory; the outputs are still the caller's)."""
    _dev(q, "q", (torch.float32, torch.bfloat16), 3)
    for t, name, dt, nd in ((w, "w", torch.float32, 2), (keys_fp4, "keys_fp4", torch.uint8, 3),
                            (key_scale, "key_scale", torch.uint8, 3), (key_gscale, "key_gscale", torch.float32, 1),
                            (block_table, "block_table", torch.int32, 2), (valid_lens, "valid_lens", torch.int32, 1)):
        _dev(t, name, dt, nd)
    T, H, D = q.shape
    P, epb, _ = keys_fp4.shape
    if out_idx is None:
        out_idx = torch.empty((T, top_k), dtype=torch.int32, device=q.device)
    if with_scores and out_scores is None:
        out_scores = torch.empty((T, top_k), dtype=torch.float32, device=q.device)
    check(_lib.load().indexer_score_topk_noalloc(
        _ptr(q), _q_dtype(q), _ptr(w), _ptr(keys_fp4), _ptr(key_scale), _ptr(key_gscale), _ptr(block_table),
        _row_stride(block_table), _ptr(valid_lens), T, H, D, epb, block_table.shape[1], P, top_k, PRECISION[precision],
        IDX_F_VALIDATE if validate else 0, _ptr(out_idx), _ptr(out_scores), _stream()))
    return out_idx, out_scores


def indexer_gather_kv(kv_fp8, kv_scale, kv_rope, block_table, topk_idx, *, group: int = 128,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Dense bf16 tiles [T, top_k, d_nope + d_rope] of the selected entries (-1: zeros)."""
    _dev(kv_fp8, "kv_fp8", torch.uint8, 3)
    _dev(kv_scale, "kv_scale", torch.float32, 3)
    _dev(kv_rope, "kv_rope", torch.bfloat16, 3)
    _dev(block_table, "block_table", torch.int32, 2)
    _dev(topk_idx, "topk_idx", torch.int32, 2)
    P, epb, d_nope = kv_fp8.shape
    d_rope = kv_rope.shape[2]
    T, top_k = topk_idx.shape
    if out is None:
        out = torch.empty((T, top_k, d_nope + d_rope), dtype=torch.bfloat16, device=kv_fp8.device)
    _dev(out, "out", torch.bfloat16, 3)
    check(_lib.load().indexer_gather_kv(
        _ptr(kv_fp8), _ptr(kv_scale), _ptr(kv_rope), _ptr(block_table), _row_stride(block_table), _ptr(topk_idx), T,
        top_k, epb, block_table.shape[1], P, d_nope, d_rope, group, _ptr(out), _stream()))
    return out


def qsa_gather(k_cache, v_cache, block_table, sel, *, k_out: Optional[torch.Tensor] = None,
               v_out: Optional[torch.Tensor] = None):
    """(k_out, v_out) [n_sel, nkv, hd]: the cache rows of the selected token positions."""
    _dev(k_cache, "k_cache", (torch.bfloat16, torch.float16), 4)
    _dev(v_cache, "v_cache", k_cache.dtype, 4)
    _dev(block_table, "block_table", torch.int32, 1)
    _dev(sel, "sel", torch.int32, 1)
    _, block_size, nkv, hd = k_cache.shape
    n_sel = sel.shape[0]
    if k_out is None:
        k_out = torch.empty((n_sel, nkv, hd), dtype=k_cache.dtype, device=k_cache.device)
    if v_out is None:
        v_out = torch.empty((n_sel, nkv, hd), dtype=k_cache.dtype, device=k_cache.device)
    check(_lib.load().qsa_gather(_ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(sel), _ptr(k_out),
                                 _ptr(v_out), n_sel, block_size, nkv, hd, _stream()))
    return k_out, v_out


def qsa_prefill_attn(q, k_cache, v_cache, block_table, lists, *, first_pos: int, ratio: int,
                     inv_sqrt_d: Optional[float] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Attention of each prefill row over its listed blocks plus its incomplete tail:
    [rows, nq, hd] fp32 from bf16 q [rows, nq, hd] and paged bf16 caches [pages, bs, nkv, hd]."""
    _dev(q, "q", torch.bfloat16, 3)
    _dev(k_cache, "k_cache", torch.bfloat16, 4)
    _dev(v_cache, "v_cache", torch.bfloat16, 4)
    _dev(block_table, "block_table", torch.int32, 1)
    rows, nq, hd = q.shape
    _, block_size, nkv, hd_k = k_cache.shape
    if hd_k != hd or v_cache.shape != k_cache.shape:
        raise ValueError("q, k_cache and v_cache must agree on hd and the caches on their shape")
    if lists is not None:
        _dev(lists, "lists", torch.int32, 2)
        if lists.shape[0] != rows:
            raise ValueError("lists must have one row per query row")
    topk = 0 if lists is None else lists.shape[1]
    if inv_sqrt_d is None:
        inv_sqrt_d = hd ** -0.5
    if out is None:
        out = torch.empty((rows, nq, hd), dtype=torch.float32, device=q.device)
    _dev(out, "out", torch.float32, 3)
    check(_lib.load().qsa_prefill_attn(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(lists),
                                       _ptr(out), rows, first_pos, topk, ratio, block_size, nq, nkv, hd, inv_sqrt_d,
                                       _stream()))
    return out


def qsa_block_pool(raw_keys, k_norm_w, block_keys, *, first_block: int, n_new: int, ratio: int, rot: int,
                   theta: float, eps: float) -> torch.Tensor:
    """Writes block_keys[first_block : first_block + n_new] from bf16 raw keys: fp32, or fp16
    (each fp32 result rounded to nearest even) when block_keys is a float16 tensor."""
    _dev(raw_keys, "raw_keys", torch.bfloat16, 2)
    _dev(k_norm_w, "k_norm_w", torch.float32, 1)
    f16 = block_keys.dtype == torch.float16
    _dev(block_keys, "block_keys", torch.float16 if f16 else torch.float32, 2)
    hd = raw_keys.shape[1]
    if (first_block + n_new) * ratio > raw_keys.shape[0] or first_block + n_new > block_keys.shape[0]:
        raise ValueError("block range exceeds the raw keys or the block-key table")
    fn = _lib.load().qsa_block_pool_f16 if f16 else _lib.load().qsa_block_pool
    check(fn(_ptr(raw_keys), _ptr(k_norm_w), _ptr(block_keys), first_block, n_new, ratio, hd, rot, theta, eps,
             _stream()))
    return block_keys


def qsa_qprep_rows(qk, q_norm_w, *, n_heads: int, hd: int, first_pos: int, rot: int, theta: float, eps: float,
                   out: Optional[torch.Tensor] = None, dtype=torch.float32) -> torch.Tensor:
    """Prepared queries [rows, n_heads, hd] from bf16 projection rows qk [rows, qkw]: fp32, or
    fp16 (rounded to nearest even) for dtype (or out) float16."""
    _dev(qk, "qk", torch.bfloat16, 2)
    _dev(q_norm_w, "q_norm_w", torch.float32, 1)
    rows, qkw = qk.shape
    if out is None:
        out = torch.empty((rows, n_heads, hd), dtype=dtype, device=qk.device)
    f16 = out.dtype == torch.float16
    _dev(out, "out", torch.float16 if f16 else torch.float32, 3)
    fn = _lib.load().qsa_qprep_rows_f16 if f16 else _lib.load().qsa_qprep_rows
    check(fn(_ptr(qk), _ptr(q_norm_w), _ptr(out), rows, first_pos, qkw, n_heads, hd, rot, theta, eps, _stream()))
    return out


def qsa_decode_prep(raw_keys, k_norm_w, block_keys, qk, q_norm_w, *, first_block: int, n_new: int, ratio: int,
                    n_heads: int, hd: int, first_pos: int, rot: int, theta: float, eps: float,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """qsa_block_pool (fp32 block keys) and qsa_qprep_rows (fp32 queries) in one launch: writes
    block_keys[first_block : first_block + n_new] and returns the prepared rows of qk."""
    _dev(raw_keys, "raw_keys", torch.bfloat16, 2)
    _dev(k_norm_w, "k_norm_w", torch.float32, 1)
    _dev(block_keys, "block_keys", torch.float32, 2)
    _dev(qk, "qk", torch.bfloat16, 2)
    _dev(q_norm_w, "q_norm_w", torch.float32, 1)
    if raw_keys.shape[1] != hd or block_keys.shape[1] != hd:
        raise ValueError("raw_keys and block_keys must have hd columns")
    if (first_block + n_new) * ratio > raw_keys.shape[0] or first_block + n_new > block_keys.shape[0]:
        raise ValueError("block range exceeds the raw keys or the block-key table")
    rows, qkw = qk.shape
    if out is None:
        out = torch.empty((rows, n_heads, hd), dtype=torch.float32, device=qk.device)
    _dev(out, "out", torch.float32, 3)
    check(_lib.load().qsa_decode_prep(_ptr(raw_keys), _ptr(k_norm_w), _ptr(block_keys), first_block, n_new, ratio,
                                      _ptr(qk), _ptr(q_norm_w), _ptr(out), rows, first_pos, qkw, n_heads, hd, rot,
                                      theta, eps, _stream()))
    return out


def qsa_qprep(q_in, q_norm_w, *, n_heads: int, hd: int, pos: int, rot: int, theta: float, eps: float,
              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One prepared decode query [n_heads, hd] fp32 from its bf16 projection [n_heads * hd]."""
    _dev(q_in, "q_in", torch.bfloat16, 1)
    _dev(q_norm_w, "q_norm_w", torch.float32, 1)
    if q_in.shape[0] < n_heads * hd:
        raise ValueError("q_in holds fewer than n_heads * hd values")
    if out is None:
        out = torch.empty((n_heads, hd), dtype=torch.float32, device=q_in.device)
    _dev(out, "out", torch.float32, 2)
    check(_lib.load().qsa_qprep(_ptr(q_in), _ptr(q_norm_w), _ptr(out), n_heads, hd, rot, pos, theta, eps,
                                _stream()))
    return out


def qsa_score(q, block_keys, *, n_blocks: Optional[int] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decode scores [n_blocks] fp32 of one prepared query [n_heads, hd] over the block keys."""
    _dev(q, "q", torch.float32, 2)
    _dev(block_keys, "block_keys", torch.float32, 2)
    n_heads, hd = q.shape
    nb = block_keys.shape[0] if n_blocks is None else n_blocks
    if nb > block_keys.shape[0]:
        raise ValueError("n_blocks exceeds the block-key table")
    if out is None:
        out = torch.empty((nb,), dtype=torch.float32, device=q.device)
    _dev(out, "out", torch.float32, 1)
    check(_lib.load().qsa_score(_ptr(q), _ptr(block_keys), _ptr(out), nb, n_heads, hd, _stream()))
    return out


def qsa_score_topk_workspace_size(n_blocks: int, top_k: int) -> int:
    return int(_lib.load().qsa_score_topk_workspace_size(n_blocks, top_k))


def qsa_score_topk(q, block_keys, top_k: int, *, n_blocks: Optional[int] = None, with_scores: bool = False,
                   workspace: Optional[torch.Tensor] = None, out_idx: Optional[torch.Tensor] = None,
                   out_scores: Optional[torch.Tensor] = None):
    """(idx [top_k] int32, scores [top_k] fp32 or None): the top_k blocks of one prepared
    decode query [n_heads, hd] over the first n_blocks block keys (qsa_score, then the
    select, with the scores kept in the workspace)."""
    _dev(q, "q", torch.float32, 2)
    _dev(block_keys, "block_keys", torch.float32, 2)
    n_heads, hd = q.shape
    nb = block_keys.shape[0] if n_blocks is None else n_blocks
    if nb > block_keys.shape[0]:
        raise ValueError("n_blocks exceeds the block-key table")
    dev = q.device
    if out_idx is None:
        out_idx = torch.empty((top_k,), dtype=torch.int32, device=dev)
    if with_scores and out_scores is None:
        out_scores = torch.empty((top_k,), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(qsa_score_topk_workspace_size(nb, top_k), 256), dtype=torch.uint8, device=dev)
    check(_lib.load().qsa_score_topk(_ptr(q), _ptr(block_keys), nb, n_heads, hd, top_k, _ptr(out_idx),
                                     _ptr(out_scores), _ptr(workspace), workspace.numel(), _stream()))
    return out_idx, out_scores


def qsa_score_rows_f16_tmax(q, block_keys, *, first_pos: int, ratio: int, n_blocks_max: Optional[int] = None,
                            out: Optional[torch.Tensor] = None, tile_max: Optional[torch.Tensor] = None):
    """(scores [rows, S] fp32, tile_max [rows, S / 16] int32 holding uint32 order keys), S =
    n_blocks_max rounded up to 16: qsa_score_rows of fp16 q and block keys, and the largest
    order key of every 16-block sub-tile (columns past n_blocks_max are not written)."""
    _dev(q, "q", torch.float16, 3)
    _dev(block_keys, "block_keys", torch.float16, 2)
    rows, n_heads, hd = q.shape
    nb = block_keys.shape[0] if n_blocks_max is None else n_blocks_max
    s16 = (nb + 15) // 16 * 16
    if out is None:
        out = torch.empty((rows, s16), dtype=torch.float32, device=q.device)
    if tile_max is None:
        tile_max = torch.empty((rows, s16 // 16), dtype=torch.int32, device=q.device)
    _dev(out, "out", torch.float32, 2)
    _dev(tile_max, "tile_max", torch.int32, 2)
    check(_lib.load().qsa_score_rows_f16_tmax(_ptr(q), _ptr(block_keys), _ptr(out), _ptr(tile_max), rows, nb,
                                              first_pos, _row_stride(out), _row_stride(tile_max), ratio, n_heads, hd,
                                              _stream()))
    return out, tile_max


def qsa_select_tiles(scores, tile_max, top_k: int, *, n_cols: int, first_pos: int, ratio: int,
                     with_scores: bool = False, out_idx: Optional[torch.Tensor] = None,
                     out_scores: Optional[torch.Tensor] = None):
    """(idx [rows, top_k] int32, scores [rows, top_k] fp32 or None): indexer_topk_select with the
    causal count over scores and tile maxima from qsa_score_rows_f16_tmax, reading only the
    sub-tiles that can hold a winner."""
    _dev(scores, "scores", torch.float32, 2)
    _dev(tile_max, "tile_max", torch.int32, 2)
    rows = scores.shape[0]
    dev = scores.device
    if out_idx is None:
        out_idx = torch.empty((rows, top_k), dtype=torch.int32, device=dev)
    if with_scores and out_scores is None:
        out_scores = torch.empty((rows, top_k), dtype=torch.float32, device=dev)
    check(_lib.load().qsa_select_tiles(_ptr(scores), _row_stride(scores), _ptr(tile_max), _row_stride(tile_max),
                                       first_pos, ratio, rows, n_cols, top_k, _ptr(out_idx), _ptr(out_scores),
                                       _stream()))
    return out_idx, out_scores


def qsa_score_select_f16_workspace_size(rows: int, n_blocks: int, top_k: int) -> int:
    return int(_lib.load().qsa_score_select_f16_workspace_size(rows, n_blocks, top_k))


def qsa_score_select_f16(q, block_keys, top_k: int, *, first_pos: int, ratio: int, n_blocks: Optional[int] = None,
                         with_scores: bool = False, workspace: Optional[torch.Tensor] = None,
                         out_idx: Optional[torch.Tensor] = None, out_scores: Optional[torch.Tensor] = None):
    """(idx [rows, top_k] int32, scores [rows, top_k] fp32 or None): the causal top_k blocks of
    every fp16 prepared query row over the first n_blocks fp16 block keys (qsa_score_rows on
    the matrix cores, then the select, with the scores kept in the workspace)."""
    _dev(q, "q", torch.float16, 3)
    _dev(block_keys, "block_keys", torch.float16, 2)
    rows, n_heads, hd = q.shape
    nb = block_keys.shape[0] if n_blocks is None else n_blocks
    if nb > block_keys.shape[0]:
        raise ValueError("n_blocks exceeds the block-key table")
    dev = q.device
    if out_idx is None:
        out_idx = torch.empty((rows, top_k), dtype=torch.int32, device=dev)
    if with_scores and out_scores is None:
        out_scores = torch.empty((rows, top_k), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(qsa_score_select_f16_workspace_size(rows, nb, top_k), 256), dtype=torch.uint8,
                                device=dev)
    check(_lib.load().qsa_score_select_f16(_ptr(q), _ptr(block_keys), rows, nb, first_pos, ratio, n_heads, hd, top_k,
                                           _ptr(out_idx), _ptr(out_scores), _ptr(workspace), workspace.numel(),
                                           _stream()))
    return out_idx, out_scores


def qsa_score_rows(q, block_keys, *, first_pos: int, ratio: int, n_blocks_max: Optional[int] = None,
                   precision: str = "mfma", out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """scores [rows, n_blocks_max] fp32 with -inf past each row's complete blocks.  fp16 q and
    block keys (the storage of the *_f16 pool and prep) take the matrix-core scorer."""
    f16 = q.dtype == torch.float16
    _dev(q, "q", torch.float16 if f16 else torch.float32, 3)
    _dev(block_keys, "block_keys", torch.float16 if f16 else torch.float32, 2)
    rows, n_heads, hd = q.shape
    nb = block_keys.shape[0] if n_blocks_max is None else n_blocks_max
    if out is None:
        out = torch.empty((rows, nb), dtype=torch.float32, device=q.device)
    _dev(out, "out", torch.float32, 2)
    if f16:
        if precision != "mfma":
            raise ValueError("fp16 q and block keys are scored on the matrix cores (precision='mfma')")
        check(_lib.load().qsa_score_rows_f16(_ptr(q), _ptr(block_keys), _ptr(out), rows, nb, first_pos,
                                             _row_stride(out), ratio, n_heads, hd, _stream()))
    else:
        check(_lib.load().qsa_score_rows(_ptr(q), _ptr(block_keys), _ptr(out), rows, nb, first_pos, _row_stride(out),
                                         ratio, n_heads, hd, PRECISION[precision], _stream()))
    return out


def indexer_debug_dequant(keys_fp4, key_scale, key_gscale, block_table_row, n: int, mode: int) -> torch.Tensor:
    """[n, D] fp32 decoder output for one block-table row (mode 0 code, 1 code*gscale, 2 fp16 operand)."""
    P, epb, half = keys_fp4.shape
    out = torch.empty((n, 2 * half), dtype=torch.float32, device=keys_fp4.device)
    check(_lib.load().indexer_debug_dequant(_ptr(keys_fp4), _ptr(key_scale), _ptr(key_gscale),
                                            _ptr(block_table_row), n, 2 * half, epb, P, mode, _ptr(out), _stream()))
    return out
