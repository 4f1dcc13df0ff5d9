"""Seeded synthetic inputs for the indexer workloads.

This package only draws random numbers and packs them into the storage formats
the indexer consumes (NVFP4 key pools, block tables, q/w tensors, bf16 raw keys).
It contains none of the indexer's own arithmetic: no decoding, scoring, top-k,
pooling, normalisation or rotary embedding.  Both the CPU oracle's tests and the
GPU path's tests and benchmark draw their inputs from here.
"""

from .configs import CONFIGS, make, make_diag, Workload  # noqa: F401
