"""The C-ABI library loads, exports every symbol include/indexer.h declares, and its host
argument checks reject bad calls before any HIP call (no GPU needed)."""

import ctypes
import os
import re

import pytest

from sparse_attention_lightning_block_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "indexer.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="HIP library not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_header_matches_binding():
    names = declared_functions()
    assert names == sorted(_lib.SIGNATURES), names


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def _score_rows(lib, **over):
    args = dict(q=8, q_dtype=0, w=16, keys=256, scale=512, gscale=1024, bt=2048, bt_stride=4, valid=4096, T=1, H=4,
                D=64, epb=16, max_lb=4, P=4, prec=1, flags=0, scores=8192, stride=64, n_cols=64)
    args.update(over)
    return lib.indexer_score_rows(args["q"], args["q_dtype"], args["w"], args["keys"], args["scale"], args["gscale"],
                                  args["bt"], args["bt_stride"], args["valid"], args["T"], args["H"], args["D"],
                                  args["epb"], args["max_lb"], args["P"], args["prec"], args["flags"], args["scores"],
                                  args["stride"], args["n_cols"], None)


def test_argument_checks_without_gpu():
    lib = _lib.load()
    assert _score_rows(lib, q=None) == _lib.IDX_ERR_NULL
    assert b"required" in lib.indexer_last_error()
    assert _score_rows(lib, D=96) == _lib.IDX_ERR_UNSUPPORTED
    assert _score_rows(lib, H=65) == _lib.IDX_ERR_UNSUPPORTED
    assert _score_rows(lib, epb=0) == _lib.IDX_ERR_SHAPE
    assert _score_rows(lib, bt_stride=3) == _lib.IDX_ERR_SHAPE
    assert _score_rows(lib, prec=7) == _lib.IDX_ERR_UNSUPPORTED
    assert _score_rows(lib, keys=264) == _lib.IDX_ERR_SHAPE       # misaligned key pool
    assert _score_rows(lib, stride=10) == _lib.IDX_ERR_SHAPE
    assert _score_rows(lib, flags=2) == _lib.IDX_ERR_UNSUPPORTED  # unknown flag bits
    assert b"flags" in lib.indexer_last_error()
    assert _score_rows(lib, T=0, flags=_lib.IDX_F_VALIDATE) == _lib.IDX_OK   # no work: no check, no launch
    assert _score_rows(lib, T=0) == _lib.IDX_OK                   # no work: no launch
    assert lib.indexer_last_error() == b""
    # select
    assert lib.indexer_topk_select(16, 64, None, 0, 0, 2, 64, 0, 32, None, None, 0, None) == _lib.IDX_ERR_UNSUPPORTED
    assert lib.indexer_topk_select(16, 64, None, 0, 0, 2, 64, 8, None, None, None, 0, None) == _lib.IDX_ERR_NULL
    assert lib.indexer_topk_select(16, 60, None, 0, 0, 2, 64, 8, 32, None, None, 0, None) == _lib.IDX_ERR_SHAPE
    assert lib.indexer_topk_select(16, 64, None, 0, 0, 0, 64, 8, 32, None, None, 0, None) == _lib.IDX_OK
    # fused: workspace too small is reported before any launch
    rc = lib.indexer_score_topk(8, 0, 16, 256, 512, 1024, 2048, 4, 4096, 1, 4, 64, 16, 4, 4, 8, 1, 0, 8192, None, 256,
                                16, None)
    assert rc == _lib.IDX_ERR_WORKSPACE
    rc = lib.indexer_score_topk(8, 0, 16, 256, 512, 1024, 2048, 4, 4096, 1, 4, 64, 16, 4, 4, 8, 1, 4, 8192, None, 256,
                                1 << 20, None)
    assert rc == _lib.IDX_ERR_UNSUPPORTED
    # QSA
    assert lib.qsa_block_pool(None, 16, 32, 0, 1, 16, 128, 64, 1e4, 1e-6, None) == _lib.IDX_ERR_NULL
    assert lib.qsa_block_pool(16, 16, 32, 0, 1, 16, 100, 64, 1e4, 1e-6, None) == _lib.IDX_ERR_UNSUPPORTED
    assert lib.qsa_block_pool(16, 16, 32, 0, 0, 16, 128, 64, 1e4, 1e-6, None) == _lib.IDX_OK
    assert lib.qsa_qprep_rows(16, 16, 32, 4, 0, 100, 1, 128, 64, 1e4, 1e-6, None) == _lib.IDX_ERR_SHAPE
    assert lib.qsa_score_rows(16, 32, 48, 4, 64, 0, 32, 16, 8, 128, 1, None) == _lib.IDX_ERR_SHAPE
    assert lib.indexer_debug_dequant(16, 16, 16, 16, 4, 64, 16, 4, 3, 64, None) == _lib.IDX_ERR_UNSUPPORTED


def test_workspace_sizes_are_device_independent():
    lib = _lib.load()
    small = lib.indexer_topk_workspace_size(4, 4096, 512)
    assert small == 0 or small == 256        # one segment: no candidate buffers
    big = lib.indexer_topk_workspace_size(32, 262144, 2048)
    assert big >= 2 * 32 * (262144 // 32768) * 2048 * 8
    fused = lib.indexer_score_topk_workspace_size(32, 4096, 64, 2048)
    assert fused >= 32 * 262144 * 4 + big
    assert lib.indexer_topk_workspace_size(0, 10, 10) == 0


def test_gather_argument_checks_without_gpu():
    lib = _lib.load()
    g = lambda **o: lib.indexer_gather_kv(*[dict(fp8=256, sc=512, rope=1024, bt=2048, bts=8, idx=4096, T=2, k=4,
                                                  epb=16, max_lb=8, P=8, dn=512, dr=64, grp=128, out=8192)
                                             .__or__(o)[n] for n in ("fp8", "sc", "rope", "bt", "bts", "idx", "T",
                                                                     "k", "epb", "max_lb", "P", "dn", "dr", "grp",
                                                                     "out")], None)
    assert g(T=0) == _lib.IDX_OK                         # no work: no launch
    assert g(out=None) == _lib.IDX_ERR_NULL
    assert g(dn=500) == _lib.IDX_ERR_UNSUPPORTED          # d_nope not a multiple of 16
    assert g(grp=96) == _lib.IDX_ERR_UNSUPPORTED          # group not dividing d_nope
    assert g(dr=4) == _lib.IDX_ERR_UNSUPPORTED
    assert g(bts=4) == _lib.IDX_ERR_SHAPE
    assert g(rope=None, dr=0, T=0) == _lib.IDX_OK          # no rope part: no rope pointer needed
    assert g(out=8200) == _lib.IDX_ERR_SHAPE              # misaligned output
    q = lambda **o: lib.qsa_gather(*[dict(k=256, v=512, bt=1024, sel=2048, ko=4096, vo=8192, n=3, bs=16, nkv=2,
                                          hd=128).__or__(o)[n] for n in ("k", "v", "bt", "sel", "ko", "vo", "n", "bs",
                                                                         "nkv", "hd")], None)
    assert q(n=0) == _lib.IDX_OK
    assert q(sel=None) == _lib.IDX_ERR_NULL
    assert q(hd=3, nkv=1) == _lib.IDX_ERR_UNSUPPORTED
    assert q(bs=0) == _lib.IDX_ERR_SHAPE


def test_qsa_decode_argument_checks_without_gpu():
    lib = _lib.load()
    assert lib.qsa_qprep(None, 16, 32, 32, 128, 64, 7, 1e4, 1e-6, None) == _lib.IDX_ERR_NULL
    assert lib.qsa_qprep(16, 16, 32, 32, 100, 64, 7, 1e4, 1e-6, None) == _lib.IDX_ERR_UNSUPPORTED
    assert lib.qsa_qprep(16, 16, 32, 32, 128, 65, 7, 1e4, 1e-6, None) == _lib.IDX_ERR_SHAPE     # odd rot
    assert lib.qsa_score(16, 32, 48, 10, 65, 128, None) == _lib.IDX_ERR_UNSUPPORTED             # 65 heads
    assert lib.qsa_score(16, 32, 48, 0, 32, 128, None) == _lib.IDX_OK                           # no blocks
    assert lib.qsa_score(16, 40, 48, 10, 32, 128, None) == _lib.IDX_ERR_SHAPE                   # misaligned keys


def test_qsa_decode_prep_argument_checks_without_gpu():
    """The one-launch decode prep applies both calls' checks before any HIP call."""
    lib = _lib.load()
    good = (16, 16, 32, 0, 1, 16, 48, 16, 64, 1, 0, 4096, 32, 128, 64, 1e4, 1e-6, None)
    bad = list(good); bad[0] = None                      # raw_keys
    assert lib.qsa_decode_prep(*bad) == _lib.IDX_ERR_NULL
    bad = list(good); bad[7] = None                      # q_norm_w
    assert lib.qsa_decode_prep(*bad) == _lib.IDX_ERR_NULL
    bad = list(good); bad[13] = 100                      # hd
    assert lib.qsa_decode_prep(*bad) == _lib.IDX_ERR_UNSUPPORTED
    bad = list(good); bad[11] = 100                      # qkw < n_heads * hd
    assert lib.qsa_decode_prep(*bad) == _lib.IDX_ERR_SHAPE
    bad = list(good); bad[2] = 40                        # block_keys misaligned
    assert lib.qsa_decode_prep(*bad) == _lib.IDX_ERR_SHAPE
    empty = list(good); empty[4] = 0; empty[9] = 0       # nothing to do: no launch
    assert lib.qsa_decode_prep(*empty) == _lib.IDX_OK


def test_qsa_score_topk_argument_checks_without_gpu():
    lib = _lib.load()
    n = lib.qsa_score_topk_workspace_size(32768, 256)
    assert n >= 32768 * 4 and n % 256 == 0
    assert lib.qsa_score_topk_workspace_size(0, 256) == 0
    assert lib.qsa_score_topk_workspace_size(100, 0) == 0
    assert lib.qsa_score_topk(None, 16, 100, 32, 128, 8, 16, None, 256, 1 << 20, None) == _lib.IDX_ERR_NULL
    assert lib.qsa_score_topk(16, 16, 100, 32, 100, 8, 16, None, 256, 1 << 20, None) == _lib.IDX_ERR_UNSUPPORTED
    assert lib.qsa_score_topk(16, 16, 100, 65, 128, 8, 16, None, 256, 1 << 20, None) == _lib.IDX_ERR_UNSUPPORTED
    assert lib.qsa_score_topk(16, 16, 100, 32, 128, 0, 16, None, 256, 1 << 20, None) == _lib.IDX_ERR_UNSUPPORTED
    # a workspace too small for the scores: rejected before any HIP call
    assert lib.qsa_score_topk(16, 16, 32768, 32, 128, 256, 16, None, 256, 1024, None) == _lib.IDX_ERR_WORKSPACE


def test_qsa_score_select_argument_checks_without_gpu():
    lib = _lib.load()
    # scores with rows padded to 16 blocks, then the sub-tile maxima (n_blocks <= 32768, top_k <= 512)
    n = lib.qsa_score_select_f16_workspace_size(2048, 32768, 256)
    assert n >= 2048 * 32768 * 4 + 2048 * 2048 * 4 and n % 256 == 0
    assert lib.qsa_score_select_f16_workspace_size(40, 700, 64) >= 40 * 704 * 4 + 40 * 44 * 4
    assert lib.qsa_score_select_f16_workspace_size(0, 700, 64) == 0
    assert lib.qsa_score_select_f16_workspace_size(40, 0, 64) == 0
    assert lib.qsa_score_select_f16_workspace_size(40, 700, 0) == 0
    # beyond the sub-tile select (top_k > 512): the general select's buffers instead
    assert lib.qsa_score_select_f16_workspace_size(4, 100000, 2048) > 4 * 100000 * 4
    def call(q=16, keys=16, rows=40, nb=700, ratio=16, nh=32, hd=128, k=64, idx=16, ws=256, wsb=1 << 30):
        return lib.qsa_score_select_f16(q, keys, rows, nb, 0, ratio, nh, hd, k, idx, None, ws, wsb, None)
    assert call(q=None) == _lib.IDX_ERR_NULL
    assert call(idx=None) == _lib.IDX_ERR_NULL
    assert call(hd=256) == _lib.IDX_ERR_UNSUPPORTED
    assert call(nh=48) == _lib.IDX_ERR_UNSUPPORTED
    assert call(ratio=0) == _lib.IDX_ERR_SHAPE
    assert call(k=0) == _lib.IDX_ERR_UNSUPPORTED
    assert call(q=17) == _lib.IDX_ERR_SHAPE
    # a workspace too small: rejected before any HIP call
    assert call(wsb=1024) == _lib.IDX_ERR_WORKSPACE
    assert call(ws=None) == _lib.IDX_ERR_WORKSPACE
    assert call(ws=264) == _lib.IDX_ERR_SHAPE
    assert call(rows=0) == _lib.IDX_OK


def test_qsa_score_tmax_and_tile_select_argument_checks_without_gpu():
    lib = _lib.load()
    def score(q=16, keys=16, sc=16, tm=16, rows=4, nb=700, stride=704, tstride=44, ratio=16, nh=32, hd=128):
        return lib.qsa_score_rows_f16_tmax(q, keys, sc, tm, rows, nb, 0, stride, tstride, ratio, nh, hd, None)
    assert score(tm=None) == _lib.IDX_ERR_NULL
    assert score(tstride=43) == _lib.IDX_ERR_SHAPE          # fewer than ceil(700 / 16) sub-tiles
    assert score(stride=699) == _lib.IDX_ERR_SHAPE
    assert score(hd=256) == _lib.IDX_ERR_UNSUPPORTED
    assert score(ratio=0) == _lib.IDX_ERR_SHAPE
    assert score(rows=0) == _lib.IDX_OK
    def sel(sc=16, stride=704, tm=16, tstride=44, ratio=16, rows=4, n=700, k=64, idx=16):
        return lib.qsa_select_tiles(sc, stride, tm, tstride, 0, ratio, rows, n, k, idx, None, None)
    assert sel(idx=None) == _lib.IDX_ERR_NULL
    assert sel(tm=None) == _lib.IDX_ERR_NULL
    assert sel(ratio=0) == _lib.IDX_ERR_SHAPE              # the causal count only
    assert sel(k=513) == _lib.IDX_ERR_UNSUPPORTED          # past the sub-tile select
    assert sel(n=40000, stride=40000, tstride=2500) == _lib.IDX_ERR_UNSUPPORTED
    assert sel(stride=700) == _lib.IDX_ERR_SHAPE           # rows must hold whole sub-tiles
    assert sel(sc=20) == _lib.IDX_ERR_SHAPE                # 16-byte aligned rows
    assert sel(tstride=40) == _lib.IDX_ERR_SHAPE
    assert sel(rows=0) == _lib.IDX_OK


def test_qsa_fp16_storage_argument_checks_without_gpu():
    lib = _lib.load()
    assert lib.qsa_block_pool_f16(None, 16, 32, 0, 1, 16, 128, 64, 1e4, 1e-6, None) == _lib.IDX_ERR_NULL
    assert lib.qsa_block_pool_f16(16, 16, 32, 0, 1, 16, 100, 64, 1e4, 1e-6, None) == _lib.IDX_ERR_UNSUPPORTED
    assert lib.qsa_block_pool_f16(16, 16, 40, 0, 1, 16, 128, 64, 1e4, 1e-6, None) == _lib.IDX_ERR_SHAPE
    assert lib.qsa_block_pool_f16(16, 16, 32, 0, 0, 16, 128, 64, 1e4, 1e-6, None) == _lib.IDX_OK
    assert lib.qsa_qprep_rows_f16(16, 16, 32, 4, 0, 100, 1, 128, 64, 1e4, 1e-6, None) == _lib.IDX_ERR_SHAPE
    assert lib.qsa_qprep_rows_f16(16, 16, 32, 0, 0, 128, 1, 128, 64, 1e4, 1e-6, None) == _lib.IDX_OK
    # fp16 inputs take the matrix-core scorer only: hd 64/128, 16/32/64 heads
    assert lib.qsa_score_rows_f16(16, 32, 48, 4, 64, 0, 64, 16, 32, 256, None) == _lib.IDX_ERR_UNSUPPORTED
    assert lib.qsa_score_rows_f16(16, 32, 48, 4, 64, 0, 64, 16, 8, 128, None) == _lib.IDX_ERR_UNSUPPORTED
    assert lib.qsa_score_rows_f16(16, 32, 48, 4, 64, 0, 32, 16, 32, 128, None) == _lib.IDX_ERR_SHAPE
    assert lib.qsa_score_rows_f16(None, 32, 48, 4, 64, 0, 64, 16, 32, 128, None) == _lib.IDX_ERR_NULL
    assert lib.qsa_score_rows_f16(16, 32, 48, 0, 64, 0, 64, 16, 32, 128, None) == _lib.IDX_OK
