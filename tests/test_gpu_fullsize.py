"""Parity at the full benchmark sizes, in the launch configuration the benchmark times
(indexer_score_rows on the MFMA path into an [T, n_cols] score matrix, then
indexer_topk_select with a zero-filled workspace), on rows the oracle computes one by
one.  Needs an MI355X."""

import numpy as np
import pytest
import torch

import sparse_attention_lightning_block_amd as salb
from oracle import indexer, qsa
from tests.parity import MFMA_ROWMAX, check_scores, check_topk, oracle_rows, oracle_rows_all, to_dev
from workloads import make, make_diag

pytestmark = pytest.mark.gpu


def _rows(w, cfg):
    if cfg == 4:
        return [w.T - 1, 2048, 513, 512, 511, 1, 0]     # causal rows across the k = 512 edge
    return list(range(w.T))                             # decode configs: every row


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_full_size_rows(cfg):
    w = make(cfg)
    d = to_dev(w)
    n_cols = w.max_lb * w.epb
    scores = torch.empty((w.T, n_cols), dtype=torch.float32, device="cuda")
    ws = torch.zeros(max(1, salb.indexer_topk_workspace_size(w.T, n_cols, w.top_k)), dtype=torch.uint8,
                     device="cuda")
    salb.indexer_score_rows(**d, n_cols=n_cols, precision="mfma", out=scores)
    idx, val = salb.indexer_topk_select(scores, w.top_k, valid_lens=d["valid_lens"], workspace=ws, with_scores=True)
    torch.cuda.synchronize()
    rows = _rows(w, cfg)
    ref, amag = oracle_rows_all(w, rows)
    for t in rows:
        g = scores[t].cpu().numpy()
        check_scores(g, ref[t], amag[t], "mfma", f"cfg{cfg} full t{t}")
        assert np.all(np.isneginf(g[int(w.valid_lens[t]):]))
        check_topk(idx[t].cpu().numpy(), val[t].cpu().numpy(), ref[t], amag[t], w.top_k, "mfma", f"cfg{cfg} full t{t}")
    # every row: the set rules that hold at any size
    gi = idx.cpu().numpy()
    for t in range(w.T):
        K = min(w.top_k, int(w.valid_lens[t]))
        assert np.all(gi[t, K:] == -1) and len(set(gi[t, :K].tolist())) == K
        assert np.all((gi[t, :K] >= 0) & (gi[t, :K] < w.valid_lens[t]))


def test_hbm_true_diagnostic_sampled_rows():
    """The diagnostic pool where every row reads its own pages (no page shared between
    the rows of a workgroup): sampled rows against the oracle, set rules on every row."""
    w = make_diag("hbm_true_T32_S262144")
    d = to_dev(w)
    n_cols = w.max_lb * w.epb
    scores = torch.empty((w.T, n_cols), dtype=torch.float32, device="cuda")
    ws = torch.zeros(max(1, salb.indexer_topk_workspace_size(w.T, n_cols, w.top_k)), dtype=torch.uint8,
                     device="cuda")
    salb.indexer_score_rows(**d, n_cols=n_cols, precision="mfma", out=scores)
    idx, val = salb.indexer_topk_select(scores, w.top_k, valid_lens=d["valid_lens"], workspace=ws, with_scores=True)
    torch.cuda.synchronize()
    order = np.argsort(w.valid_lens)
    rows = sorted({int(order[-1]), int(order[0])})
    ref, amag = oracle_rows(w, rows)
    for t in rows:
        g = scores[t].cpu().numpy()
        check_scores(g, ref[t], amag[t], "mfma", f"hbm_true t{t}")
        assert np.all(np.isneginf(g[int(w.valid_lens[t]):]))
        check_topk(idx[t].cpu().numpy(), val[t].cpu().numpy(), ref[t], amag[t], w.top_k, "mfma", f"hbm_true t{t}")
    gi = idx.cpu().numpy()
    for t in range(w.T):
        K = min(w.top_k, int(w.valid_lens[t]))
        assert np.all(gi[t, K:] == -1) and len(set(gi[t, :K].tolist())) == K


@pytest.mark.parametrize("cfg", [2, 3])
def test_full_size_fused_matches_split(cfg):
    """indexer_score_topk (the fused entry) returns what the two calls return."""
    w = make(cfg)
    d = to_dev(w)
    n_cols = w.max_lb * w.epb
    a_idx, a_val = salb.indexer_score_topk(**d, top_k=w.top_k, precision="mfma", with_scores=True)
    scores = salb.indexer_score_rows(**d, n_cols=n_cols, precision="mfma")
    b_idx, b_val = salb.indexer_topk_select(scores, w.top_k, valid_lens=d["valid_lens"], with_scores=True)
    assert torch.equal(a_idx, b_idx) and torch.equal(a_val, b_val)


def test_qsa_full_size_sampled():
    """QSA at full size: every block pooled and every row prepared on the GPU; sampled
    blocks, rows and row scores against the oracle; the causal top-k of sampled rows."""
    w = make(5)
    raw = torch.from_numpy(w.raw_keys.view(np.int16).copy()).view(torch.bfloat16).cuda()
    kw = torch.from_numpy(w.k_norm_w).cuda()
    keys_d = torch.empty((w.n_blocks, w.hd), dtype=torch.float32, device="cuda")
    salb.qsa_block_pool(raw, kw, keys_d, first_block=0, n_new=w.n_blocks, ratio=w.ratio, rot=w.rot, theta=w.theta,
                        eps=w.eps)
    qk = torch.from_numpy(w.qk.view(np.int16).copy()).view(torch.bfloat16).cuda()
    q_d = salb.qsa_qprep_rows(qk, torch.from_numpy(w.q_norm_w).cuda(), n_heads=w.n_heads, hd=w.hd,
                              first_pos=w.first_pos, rot=w.rot, theta=w.theta, eps=w.eps)
    sc = salb.qsa_score_rows(q_d, keys_d, first_pos=w.first_pos, ratio=w.ratio, precision="mfma")
    idx, val = salb.indexer_topk_select(sc, w.top_k, first_pos=w.first_pos, ratio=w.ratio, with_scores=True)
    torch.cuda.synchronize()
    keys = keys_d.cpu().numpy().astype(np.float64)
    q = q_d.cpu().numpy().astype(np.float64)
    # pooled keys: sampled blocks against the oracle from the bf16 raw keys
    raw64 = indexer.upcast(w.raw_keys, "bf16")
    for b0 in (0, 1, w.n_blocks // 2, w.n_blocks - 1):
        ref = qsa.block_pool(raw64, w.k_norm_w, b0, 1, w.ratio, w.rot, w.theta, w.eps)
        assert np.all(np.abs(keys[b0] - ref[0]) <= 1e-5 * np.max(np.abs(ref[0])))
    # prepared queries: sampled rows
    for r in (0, w.rows - 1):
        qr = qsa.qprep_rows(indexer.upcast(w.qk[r:r + 1], "bf16"), w.q_norm_w, 1, w.first_pos + r, w.n_heads * w.hd,
                            w.n_heads, w.hd, w.rot, w.theta, w.eps)[0]
        assert np.all(np.abs(q[r] - qr) <= 1e-5 * np.max(np.abs(qr), axis=-1, keepdims=True))
    # scores and top-k of sampled rows against the oracle's own chain (pooled keys from the
    # bf16 raw keys, prepared queries from the bf16 projections), not the GPU's intermediates
    keys_o = qsa.block_pool(raw64, w.k_norm_w, 0, w.n_blocks, w.ratio, w.rot, w.theta, w.eps)
    del raw64
    got = sc.cpu().numpy()
    gi, gv = idx.cpu().numpy(), val.cpu().numpy()
    for r in (0, 1, w.rows // 3, w.rows // 2, w.rows - 2, w.rows - 1):
        q_o = qsa.qprep_rows(indexer.upcast(w.qk[r:r + 1], "bf16"), w.q_norm_w, 1, w.first_pos + r,
                             w.n_heads * w.hd, w.n_heads, w.hd, w.rot, w.theta, w.eps)
        ref, valid = qsa.score_rows(q_o, keys_o, w.first_pos + r, w.ratio)
        v = int(valid[0])
        tol = np.full(v, MFMA_ROWMAX * np.max(np.abs(ref[0, :v])))
        err = np.abs(got[r, :v].astype(np.float64) - ref[0, :v])
        assert np.all(err <= tol), f"qsa full row {r}: max err {err.max()} tol {tol[0]}"
        assert np.all(np.isneginf(got[r, v:]))
        check_topk(gi[r], gv[r], ref[0, :v], None, w.top_k, "mfma", f"qsa full row {r}", tol=tol)
