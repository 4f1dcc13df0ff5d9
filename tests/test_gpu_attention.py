"""GPU parity of the block-sparse prefill attention (qsa_prefill_attn) through the C
ABI against the oracle.  Needs an MI355X.

Tolerance: the scores and the softmax are fp32 from bf16 inputs (products exact, fp32
sums); each probability is rounded to fp16 (2^-12 relative) for the value product and
the values are exact in fp16, so an output errs by at most about 2^-12 of
sum_j w_j |v_j| (w the softmax weights).  That sum is the oracle's own attention with
|v| as the values; the test allows four times the bound plus 1e-6."""

import numpy as np
import pytest
import torch

import sparse_attention_lightning_block_amd as salb
from oracle import attention, indexer
from workloads import make
from workloads.attention import make_attention, qsa_prefill_attention
from workloads.device import bf16_tensor

pytestmark = pytest.mark.gpu


def _run(w, lists=None):
    lists = w.lists if lists is None else lists
    out = salb.qsa_prefill_attn(bf16_tensor(w.q).cuda(), bf16_tensor(w.k_cache).cuda(), bf16_tensor(w.v_cache).cuda(),
                                torch.from_numpy(w.block_table).cuda(),
                                None if lists.shape[1] == 0 else torch.from_numpy(lists).cuda(),
                                first_pos=w.first_pos, ratio=w.ratio)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _check(w, got, rows, lists=None):
    lists = w.lists if lists is None else lists
    q = indexer.upcast(w.q[rows], "bf16")
    # only the cache pages the rows attend, upcast once (the same data under a compacted
    # page numbering: logical block -> its page's slot in the subset)
    used = set()
    for r in rows:
        pos = attention.attended_positions(lists[r], w.first_pos, r, w.ratio)
        used.update(np.unique(pos // w.block_size).tolist())
    logical = np.array(sorted(used), dtype=np.int64)
    pages = w.block_table[logical] if logical.size else np.zeros(0, np.int64)
    k = indexer.upcast(w.k_cache[pages], "bf16")
    v = indexer.upcast(w.v_cache[pages], "bf16")
    bt = np.zeros(w.block_table.shape, dtype=np.int64)
    bt[logical] = np.arange(logical.size)
    for i, r in enumerate(rows):   # one row at a time: its own position
        a = (bt, lists[r:r + 1], w.first_pos + r, w.ratio, w.block_size, w.nkv, w.hd ** -0.5)
        ref = attention.prefill_attn(q[i:i + 1], k, v, *a)[0]
        mag = attention.prefill_attn(q[i:i + 1], k, np.abs(v), *a)[0]
        tol = 4 * 2.0 ** -12 * mag + 1e-6
        err = np.abs(got[r] - ref)
        assert np.all(err <= tol), f"row {r}: max err {err.max()} (tol {tol.max()})"


@pytest.mark.parametrize("nq,nkv,hd,ratio,block_size,topk", [(8, 2, 128, 16, 64, 16), (16, 1, 64, 8, 7, 9),
                                                             (12, 3, 128, 4, 16, 40), (4, 4, 64, 16, 32, 5)])
def test_prefill_attn_reduced(nq, nkv, hd, ratio, block_size, topk):
    """Grouped heads from 1 to 16 per KV head, both head widths, pages not a multiple of
    the block, rows with padded lists and with entries that must be skipped."""
    w = make_attention(f"attn_{nq}_{nkv}_{hd}", [44, nq, hd], rows=40, first_pos=ratio * 60 + 3, ratio=ratio,
                       block_size=block_size, nq=nq, nkv=nkv, hd=hd, topk=topk, pad_frac=0.3, junk=True)
    got = _run(w)
    _check(w, got, list(range(w.rows)))


def test_prefill_attn_tail_only_and_empty_rows():
    """topk 0: every row attends its tail alone; a row whose position completes a block
    attends nothing and gets zeros."""
    w = make_attention("attn_tail", [45], rows=20, first_pos=31, ratio=16, block_size=16, nq=8, nkv=2, hd=128, topk=1)
    empty = np.zeros((w.rows, 0), dtype=np.int32)
    got = _run(w, empty)
    _check(w, got, list(range(w.rows)), empty)
    assert np.all(got[0] == 0.0)          # position 31: blocks 0, 1 complete, no tail
    assert np.all(got[16] == 0.0)         # position 47


def test_prefill_attn_full_size_sampled_rows():
    """The QSA prefill shape (2048 rows, top 256 blocks of 16 positions, 32 over 4 heads):
    sampled rows against the oracle."""
    w = qsa_prefill_attention()
    got = _run(w)
    _check(w, got, [0, 1, 777, 1024, 2046, 2047])


def test_prefill_attn_of_the_selected_blocks():
    """The path's own selection as input: QSA block scores and their causal top-k on the
    GPU, then attention over those blocks of a K/V cache of the same length."""
    w5 = make(5, reduced=1)
    raw = bf16_tensor(w5.raw_keys).cuda()
    keys = torch.empty((w5.n_blocks, w5.hd), dtype=torch.float32, device="cuda")
    salb.qsa_block_pool(raw, torch.from_numpy(w5.k_norm_w).cuda(), keys, first_block=0, n_new=w5.n_blocks,
                        ratio=w5.ratio, rot=w5.rot, theta=w5.theta, eps=w5.eps)
    qp = salb.qsa_qprep_rows(bf16_tensor(w5.qk).cuda(), torch.from_numpy(w5.q_norm_w).cuda(), n_heads=w5.n_heads,
                             hd=w5.hd, first_pos=w5.first_pos, rot=w5.rot, theta=w5.theta, eps=w5.eps)
    sc = salb.qsa_score_rows(qp, keys, first_pos=w5.first_pos, ratio=w5.ratio, precision="mfma")
    sel, _ = salb.indexer_topk_select(sc, w5.top_k, first_pos=w5.first_pos, ratio=w5.ratio)
    lists = sel.cpu().numpy()
    w = make_attention("attn_chain", [46], rows=w5.rows, first_pos=w5.first_pos, ratio=w5.ratio, block_size=64, nq=8,
                       nkv=2, hd=128, topk=w5.top_k)
    got = _run(w, lists)
    _check(w, got, list(range(w.rows)), lists)
