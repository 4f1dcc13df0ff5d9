"""Copies of a workload's host arrays into device tensors (argument marshalling only).

Used by the GPU tests and the benchmark; it holds none of the indexer's arithmetic."""

from __future__ import annotations

import numpy as np
import torch


def bf16_tensor(bits) -> torch.Tensor:
    """A bfloat16 tensor with the given uint16 bit patterns (on the host)."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).view(torch.bfloat16)


def to_dev(w, device="cuda"):
    """Device tensors of a paged NVFP4 workload, keyed by the binding's argument names."""
    q = bf16_tensor(w.q) if w.q_dtype == "bf16" else torch.from_numpy(w.q.copy())
    return dict(
        q=q.to(device),
        w=torch.from_numpy(w.w.copy()).to(device),
        keys_fp4=torch.from_numpy(w.keys_fp4.copy()).to(device),
        key_scale=torch.from_numpy(w.key_scale.copy()).to(device),
        key_gscale=torch.from_numpy(w.key_gscale.copy()).to(device),
        block_table=torch.from_numpy(w.block_table.copy()).to(device),
        valid_lens=torch.from_numpy(w.valid_lens.astype(np.int32)).to(device),
    )
