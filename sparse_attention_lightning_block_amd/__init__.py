"""MI355X (gfx950) lightning-indexer score + top-k: a C-ABI HIP library with a thin
PyTorch binding.  The binding only marshals arguments; every step runs in the
hand-written HIP kernels of libsalb_indexer.so."""

from .ops import (  # noqa: F401
    indexer_debug_dequant,
    indexer_gather_kv,
    indexer_score_rows,
    indexer_score_topk,
    indexer_score_topk_noalloc,
    indexer_score_topk_workspace_size,
    indexer_topk_select,
    indexer_topk_workspace_size,
    qsa_block_pool,
    qsa_decode_prep,
    qsa_gather,
    qsa_prefill_attn,
    qsa_qprep,
    qsa_qprep_rows,
    qsa_score,
    qsa_score_rows,
    qsa_score_topk,
    qsa_score_topk_workspace_size,
    qsa_score_select_f16,
    qsa_score_select_f16_workspace_size,
    qsa_score_rows_f16_tmax,
    qsa_select_tiles,
)
from ._lib import IDX_ERR_DATA, IDX_F_VALIDATE, IndexerError, load  # noqa: F401
