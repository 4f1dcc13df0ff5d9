"""QSA block-pooled indexer variant (float64 oracle).

Test infrastructure only; see the package docstring.

Sources ([qsa.rs] doc comments of the launchers):
* qsa_block_pool: a block key is the mean of ``ratio`` raw keys, then RMSNorm
  scaled by ``1 + w``, then RoPE at the block's first token position; nothing is
  launched when ``n_new == 0``.
* qsa_qprep / qsa_qprep_rows: per head, RMSNorm scaled by ``1 + w``, then partial
  RoPE at the row position ``first_pos + row``; q is read from rows of width
  ``qkw`` of the projection.
* qsa_score: ``scores[b] = sum_h relu(q_h . k_b) / sqrt(hd)`` for the ``n_blocks``
  blocks a decode query scores (every block it is given: no causal cut).
* qsa_qprep: one decode query, per head RMSNorm scaled by ``1 + w`` then partial RoPE
  at the query's position ``pos``.
* qsa_score_rows: per-row block scores; blocks at or past the row's count of
  complete blocks score -inf.

Readings where the page is silent (each is listed with the design notes):
* RMSNorm is x / sqrt(mean(x^2) + eps), the standard definition.
* RoPE pairs dimension i with i + rot/2 for i < rot/2 ("NeoX" half split), with
  inverse frequency theta^(-2i/rot); dimensions >= rot pass through.  The page
  names ``rot`` and ``theta`` but not the pairing: this convention is a choice,
  and parity against the original system is unpinned for it.
* The complete-block count of a row at position p is floor((p + 1) / ratio).
* Pooled block b is written to row b of the block-key table (rows
  first_block .. first_block + n_new - 1).
"""

from __future__ import annotations

import numpy as np


def rms_norm(x, weight, eps):
    """x / sqrt(mean(x^2, last axis) + eps) * (1 + weight), float64."""
    x = np.asarray(x, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x * r * (1.0 + np.asarray(weight, dtype=np.float64))


def rope(x, pos, rot, theta):
    """Partial rotary embedding of the first ``rot`` dims of x[..., D] at positions ``pos``.

    ``pos`` broadcasts against x's leading axes.  Angles are formed in float64.
    """
    x = np.asarray(x, dtype=np.float64).copy()
    if rot == 0:
        return x
    half = rot // 2
    i = np.arange(half, dtype=np.float64)
    inv_freq = np.power(float(theta), -2.0 * i / rot)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq
    cos, sin = np.cos(ang), np.sin(ang)
    a = x[..., :half].copy()
    b = x[..., half:rot].copy()
    x[..., :half] = a * cos - b * sin
    x[..., half:rot] = a * sin + b * cos
    return x


def block_pool(raw_keys, k_norm_w, first_block, n_new, ratio, rot, theta, eps):
    """Pooled keys of blocks first_block .. first_block+n_new-1 -> [n_new, hd] float64.

    raw_keys: [n_tokens, hd] float64 (bf16 inputs upcast exactly by the caller).
    """
    raw = np.asarray(raw_keys, dtype=np.float64)
    hd = raw.shape[1]
    if n_new == 0:
        return np.zeros((0, hd))
    b = np.arange(first_block, first_block + n_new, dtype=np.int64)
    grp = raw[first_block * ratio:(first_block + n_new) * ratio].reshape(n_new, ratio, hd)
    m = grp.mean(axis=1)
    n = rms_norm(m, k_norm_w, eps)
    return rope(n, b * ratio, rot, theta)


def qprep_rows(qk, q_norm_w, rows, first_pos, qkw, n_heads, hd, rot, theta, eps):
    """Prepared queries [rows, n_heads, hd] float64 from the projection rows qk[rows, qkw]."""
    qk = np.asarray(qk, dtype=np.float64)
    q = qk[:rows, : n_heads * hd].reshape(rows, n_heads, hd)
    n = rms_norm(q, q_norm_w, eps)
    pos = (first_pos + np.arange(rows, dtype=np.int64))[:, None]
    return rope(n, np.broadcast_to(pos, (rows, n_heads)), rot, theta)


def complete_blocks(first_pos, rows, ratio, n_blocks_max):
    """Per-row count of complete blocks, capped at the table width."""
    pos = first_pos + np.arange(rows, dtype=np.int64)
    return np.minimum((pos + 1) // ratio, n_blocks_max)


def score_rows(q, block_keys, first_pos, ratio, chunk: int = 8192):
    """S[r, b] = sum_h relu(q[r,h] . k_b) / sqrt(hd), -inf for b >= complete blocks."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(block_keys, dtype=np.float64)
    rows, H, hd = q.shape
    nb = k.shape[0]
    valid = complete_blocks(first_pos, rows, ratio, nb)
    out = np.full((rows, nb), -np.inf)
    inv = 1.0 / np.sqrt(float(hd))
    for r in range(rows):
        v = int(valid[r])
        for a in range(0, v, chunk):
            b = min(v, a + chunk)
            dots = q[r] @ k[a:b].T
            out[r, a:b] = np.maximum(dots, 0.0).sum(axis=0) * inv
    return out, valid


def qprep(q_in, q_norm_w, n_heads, hd, rot, pos, theta, eps):
    """One decode query [n_heads, hd] float64 from its projection q_in [n_heads * hd]:
    per head RMSNorm * (1 + w), then RoPE at position ``pos``."""
    q = np.asarray(q_in, dtype=np.float64)[: n_heads * hd].reshape(n_heads, hd)
    return rope(rms_norm(q, q_norm_w, eps), np.full(n_heads, pos), rot, theta)


def score_blocks(q, block_keys, n_blocks):
    """Decode scores [n_blocks]: sum_h relu(q[h] . k_b) / sqrt(hd) for b < n_blocks."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(block_keys, dtype=np.float64)[:n_blocks]
    return np.maximum(q @ k.T, 0.0).sum(axis=0) / np.sqrt(float(q.shape[-1]))
