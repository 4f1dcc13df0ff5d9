"""CPU oracle for the lightning-indexer score + top-k path and its QSA block-pooled variant.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or link
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, tables, constants or helpers) and imports nothing
from ``sparse_attention_lightning_block_amd``.

Everything is plain numpy in float64, written from the pages the method is
described on:

* [listing]  "nvfp4-megamoe-kernel -- dsv4/kernels/indexer/indexer_score_topk.cu"
  (the source listing page: its header comment quoting eq. 16, the NVFP4 notes,
  ``dequant_fp4_scalar``, ``heap_insert``, the main kernel and its final sort);
* [commits]  "nvfp4-megamoe-kernel -- commit graph of dsv4/kernels/indexer"
  (commit messages c2f705a21a, 79ef87f9a9 with the E2M1 encoding table, and
  e74c84458c with the E2M1 magnitude LUT);
* [qsa.rs]   "metrale_model_layers/layers/ops/qsa.rs" (doc comments of the QSA
  launchers: qsa_block_pool, qsa_qprep / qsa_qprep_rows, qsa_score,
  qsa_score_rows, qsa_score_rows_tc).

Modules:
  nvfp4     -- E2M1 / E4M3 decode, block-table resolution, key dequantisation.
  indexer   -- I[t,s] = sum_h w[t,h] * ReLU(q[t,h] . k[s]) and the total-order top-k.
  qsa       -- block pooling, RMSNorm, partial RoPE, query prep, row and decode scores.
  gather    -- the selected entries as dense tiles (FP8 + BF16 pool, QSA K/V rows).
  attention -- prefill attention over the selected blocks plus the incomplete tail.
"""

from . import attention, gather, indexer, nvfp4, qsa  # noqa: F401
