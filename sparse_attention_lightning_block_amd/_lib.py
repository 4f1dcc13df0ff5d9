"""ctypes declarations of the C ABI in include/indexer.h.

Loading fails loudly when the HIP library has not been built: there is no other
implementation behind these names.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsalb_indexer.so")

IDX_OK = 0
IDX_ERR_NULL = 1
IDX_ERR_SHAPE = 2
IDX_ERR_WORKSPACE = 3
IDX_ERR_UNSUPPORTED = 4
IDX_ERR_HIP = 5
IDX_ERR_DATA = 6

IDX_F_VALIDATE = 1
IDX_NOALLOC_SCRATCH_BYTES = 128 << 20

IDX_DTYPE_F32 = 0
IDX_DTYPE_BF16 = 1
IDX_PREC_FP32 = 0
IDX_PREC_MFMA = 1

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_U32 = ctypes.c_uint32
_F = ctypes.c_float
_SZ = ctypes.c_size_t

# name -> (restype, argtypes), in header order
SIGNATURES = {
    "indexer_last_error": (ctypes.c_char_p, []),
    "indexer_score_rows": (_I, [_P, _I, _P, _P, _P, _P, _P, _I64, _P, _I, _I, _I, _I, _I, _I, _I, _U32, _P, _I64, _I,
                                _P]),
    "indexer_topk_workspace_size": (_SZ, [_I, _I, _I]),
    "indexer_topk_select": (_I, [_P, _I64, _P, _I64, _I, _I, _I, _I, _P, _P, _P, _SZ, _P]),
    "indexer_score_topk_workspace_size": (_SZ, [_I, _I, _I, _I]),
    "qsa_score_topk_workspace_size": (_SZ, [_U32, _I]),
    "qsa_score_topk": (_I, [_P, _P, _U32, _U32, _U32, _I, _P, _P, _P, _SZ, _P]),
    "qsa_score_select_f16_workspace_size": (_SZ, [_U32, _U32, _I]),
    "qsa_score_rows_f16_tmax": (_I, [_P, _P, _P, _P, _U32, _U32, _U32, _U32, _U32, _U32, _U32, _U32, _P]),
    "qsa_select_tiles": (_I, [_P, _I64, _P, _I64, _I64, _I, _I, _I, _I, _P, _P, _P]),
    "qsa_score_select_f16": (_I, [_P, _P, _U32, _U32, _U32, _U32, _U32, _U32, _I, _P, _P, _P, _SZ, _P]),
    "indexer_score_topk": (_I, [_P, _I, _P, _P, _P, _P, _P, _I64, _P, _I, _I, _I, _I, _I, _I, _I, _I, _U32, _P, _P,
                                _P, _SZ, _P]),
    "indexer_score_topk_noalloc": (_I, [_P, _I, _P, _P, _P, _P, _P, _I64, _P, _I, _I, _I, _I, _I, _I, _I, _I, _U32,
                                        _P, _P, _P]),
    "indexer_gather_kv": (_I, [_P, _P, _P, _P, _I64, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P]),
    "qsa_gather": (_I, [_P, _P, _P, _P, _P, _P, _U32, _U32, _U32, _U32, _P]),
    "qsa_prefill_attn": (_I, [_P, _P, _P, _P, _P, _P, _U32, _U32, _U32, _U32, _U32, _U32, _U32, _U32, _F, _P]),
    "qsa_block_pool": (_I, [_P, _P, _P, _U32, _U32, _U32, _U32, _U32, _F, _F, _P]),
    "qsa_block_pool_f16": (_I, [_P, _P, _P, _U32, _U32, _U32, _U32, _U32, _F, _F, _P]),
    "qsa_qprep_rows": (_I, [_P, _P, _P, _U32, _U32, _U32, _U32, _U32, _U32, _F, _F, _P]),
    "qsa_qprep_rows_f16": (_I, [_P, _P, _P, _U32, _U32, _U32, _U32, _U32, _U32, _F, _F, _P]),
    "qsa_qprep": (_I, [_P, _P, _P, _U32, _U32, _U32, _U32, _F, _F, _P]),
    "qsa_decode_prep": (_I, [_P, _P, _P, _U32, _U32, _U32, _P, _P, _P, _U32, _U32, _U32, _U32, _U32, _U32, _F, _F,
                             _P]),
    "qsa_score": (_I, [_P, _P, _P, _U32, _U32, _U32, _P]),
    "qsa_score_rows": (_I, [_P, _P, _P, _U32, _U32, _U32, _U32, _U32, _U32, _U32, _I, _P]),
    "qsa_score_rows_f16": (_I, [_P, _P, _P, _U32, _U32, _U32, _U32, _U32, _U32, _U32, _P]),
    "indexer_debug_dequant": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P]),
}

_lib = None


class IndexerError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """The library, loaded once.  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build the HIP library first "
            "(python -m sparse_attention_lightning_block_amd.build)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(rc: int) -> None:
    if rc != IDX_OK:
        msg = load().indexer_last_error()
        raise IndexerError(rc, msg.decode() if msg else "")
