"""GPU parity of the selected-entry gathers (indexer_gather_kv, qsa_gather) through the C
ABI against the oracle: bit-exact, since both are data movement with one defined
rounding.  Needs an MI355X."""

import numpy as np
import pytest
import torch

import sparse_attention_lightning_block_amd as salb
from oracle import gather
from workloads import make
from workloads.device import bf16_tensor, to_dev
from workloads.gather import GATHER_WORKLOADS, make_gather, make_qsa_gather

pytestmark = pytest.mark.gpu


def _dev_gather(w):
    return dict(kv_fp8=torch.from_numpy(w.fp8).cuda(), kv_scale=torch.from_numpy(w.scale).cuda(),
                kv_rope=bf16_tensor(w.rope_bits).cuda(), block_table=torch.from_numpy(w.block_table).cuda())


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("d_nope,d_rope,group,table", [(512, 64, 128, "shared"), (448, 64, 64, "per_row"),
                                                       (256, 0, 16, "shared"), (0, 64, 128, "per_row")])
def test_gather_kv_reduced(d_nope, d_rope, group, table):
    """Rows longer and shorter than top_k (-1 padding), shared and per-row tables, widths
    with and without a rope part: bit-exact against the oracle."""
    w = make_gather(f"g_{d_nope}_{d_rope}", [40, d_nope, d_rope], T=5, P=40, epb=16, max_lb=32, top_k=100,
                    d_nope=d_nope or 128, d_rope=d_rope, group=group, valid_lens=[512, 300, 100, 37, 0],
                    table=table)
    if d_nope == 0:       # a pool with no FP8 part
        w.fp8 = w.fp8[:, :, :0].copy()
        w.scale = w.scale[:, :, :0].copy()
        w.d_nope = 0
    d = _dev_gather(w)
    got = salb.indexer_gather_kv(**d, topk_idx=torch.from_numpy(w.topk_idx).cuda(), group=group)
    torch.cuda.synchronize()
    ref = gather.gather_kv(w.fp8, w.scale, w.rope_bits, w.block_table, w.topk_idx, w.epb, group)
    assert np.array_equal(_bits(got), ref)
    assert np.all(_bits(got)[4] == 0)           # an empty row: every slot padded


def test_gather_kv_rounds_each_product_once():
    """Random fp32 scales times every E4M3 code: about 2^-16 of the products fall within
    half an fp32 spacing of a bfloat16 tie, where rounding the fp32 product would go the
    wrong way; every element must equal the single rounding.  Plus the hand-worked value
    1.125 * 0x3f69c71c -> 0x3F83."""
    P, epb, d = 256, 64, 256
    rng = np.random.default_rng(41)
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    fp8 = rng.choice(codes, size=(P, epb, d)).astype(np.uint8)
    fp8[0, 0, :] = 0x39
    mant = rng.integers(0, 1 << 23, size=(P, epb, d // 16), dtype=np.uint32)
    expo = rng.integers(120, 130, size=(P, epb, d // 16), dtype=np.uint32)
    scale = ((expo << 23) | mant).view(np.float32)
    scale[0, 0, :] = np.array([0x3F69C71C], dtype=np.uint32).view(np.float32)[0]
    rope = np.zeros((P, epb, 0), np.uint16)
    bt = np.arange(P, dtype=np.int32)[None, :]
    idx = np.arange(P * epb, dtype=np.int32)[None, :]
    got = salb.indexer_gather_kv(torch.from_numpy(fp8).cuda(), torch.from_numpy(scale).cuda(),
                                 bf16_tensor(rope).cuda(), torch.from_numpy(bt).cuda(), torch.from_numpy(idx).cuda(),
                                 group=16)
    g = _bits(got)
    ref = gather.gather_kv(fp8, scale, rope, bt, idx, epb, 16)
    assert np.all(g[0, 0] == 0x3F83)
    assert np.array_equal(g, ref)


@pytest.mark.parametrize("cfg,reduced", [(2, 1), (3, 1)])
def test_gather_of_the_selected_entries(cfg, reduced):
    """The path's own output as the gather's input: indexer_score_topk on a paged pool,
    then indexer_gather_kv of a KV pool with the same pages and block table, against the
    oracle gather of the same indices."""
    w = make(cfg, reduced)
    d = to_dev(w)
    idx, _ = salb.indexer_score_topk(**d, top_k=w.top_k, precision="mfma")
    g = make_gather("kv_of_" + w.name, [42, cfg], T=w.T, P=w.P, epb=w.epb, max_lb=w.max_lb, top_k=w.top_k,
                    valid_lens=w.valid_lens)
    g.block_table = w.block_table
    dg = _dev_gather(g)
    dg["block_table"] = d["block_table"]
    got = salb.indexer_gather_kv(**dg, topk_idx=idx, group=g.group)
    torch.cuda.synchronize()
    ref = gather.gather_kv(g.fp8, g.scale, g.rope_bits, w.block_table, idx.cpu().numpy(), g.epb, g.group)
    assert np.array_equal(_bits(got), ref)


def test_gather_kv_full_size():
    """The benchmark's gather workload (32 rows x 2048 entries of a 8192-page pool):
    every row bit-exact."""
    w = GATHER_WORKLOADS["gather_T32_k2048"]()
    d = _dev_gather(w)
    got = salb.indexer_gather_kv(**d, topk_idx=torch.from_numpy(w.topk_idx).cuda(), group=w.group)
    g = _bits(got)
    ref = gather.gather_kv(w.fp8, w.scale, w.rope_bits, w.block_table, w.topk_idx, w.epb, w.group)
    assert np.array_equal(g, ref)


@pytest.mark.parametrize("n_blocks,block_size,nkv,hd,n_sel", [(64, 16, 2, 64, 300), (40, 7, 1, 8, 280),
                                                              (128, 64, 4, 128, 1)])
def test_qsa_gather(n_blocks, block_size, nkv, hd, n_sel):
    w = make_qsa_gather("qg", [43, block_size], n_blocks=n_blocks, block_size=block_size, nkv=nkv, hd=hd,
                        n_sel=n_sel)
    ko, vo = salb.qsa_gather(bf16_tensor(w.k_cache).cuda(), bf16_tensor(w.v_cache).cuda(),
                             torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.sel).cuda())
    rk, rv = gather.qsa_gather(w.k_cache, w.v_cache, w.block_table, w.sel, w.block_size)
    assert np.array_equal(_bits(ko), rk) and np.array_equal(_bits(vo), rv)


def test_qsa_gather_full_size():
    w = GATHER_WORKLOADS["qsa_gather_4096"]()
    ko, vo = salb.qsa_gather(bf16_tensor(w.k_cache).cuda(), bf16_tensor(w.v_cache).cuda(),
                             torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.sel).cuda())
    rk, rv = gather.qsa_gather(w.k_cache, w.v_cache, w.block_table, w.sel, w.block_size)
    assert np.array_equal(_bits(ko), rk) and np.array_equal(_bits(vo), rv)
