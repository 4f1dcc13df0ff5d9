"""The hot path captured into HIP graphs: every replay, with eager work and
synchronisations between the replays, returns exactly what the eager calls return
(every call zeroes the workspace counters it needs inside its own launches, so nothing
needs clearing between replays).  Needs an MI355X."""

import numpy as np
import pytest
import torch

import sparse_attention_lightning_block_amd as salb
from tests.parity import to_dev
from workloads import make

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg,reduced", [(2, 0), (3, 1), (4, 1)])
def test_graph_replays_match_eager(cfg, reduced):
    w = make(cfg, reduced)
    d = to_dev(w)
    n_cols = w.max_lb * w.epb
    scores = torch.empty((w.T, n_cols), dtype=torch.float32, device="cuda")
    idx = torch.empty((w.T, w.top_k), dtype=torch.int32, device="cuda")
    val = torch.empty((w.T, w.top_k), dtype=torch.float32, device="cuda")
    ws = torch.full((max(256, salb.indexer_topk_workspace_size(w.T, n_cols, w.top_k)),), 0xA5, dtype=torch.uint8,
                    device="cuda")

    def path():
        salb.indexer_score_rows(**d, n_cols=n_cols, precision="mfma", out=scores)
        salb.indexer_topk_select(scores, w.top_k, valid_lens=d["valid_lens"], workspace=ws, out_idx=idx,
                                 out_scores=val)

    path()
    torch.cuda.synchronize()
    ref_s, ref_i, ref_v = scores.clone(), idx.clone(), val.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        path()
    other = make(2, 1)
    od = to_dev(other)
    for rep in range(4):
        scores.fill_(7.0)
        idx.fill_(-5)
        val.fill_(3.0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(scores.view(torch.int32), ref_s.view(torch.int32)), rep
        assert torch.equal(idx, ref_i), rep
        assert torch.equal(val.view(torch.int32), ref_v.view(torch.int32)), rep
        # eager work between replays, on other buffers (its own workspace)
        salb.indexer_score_topk(**od, top_k=other.top_k, precision="mfma")
        torch.cuda.synchronize()


def test_qsa_graph_replays_match_eager():
    w = make(5, reduced=1)
    raw = torch.from_numpy(w.raw_keys.view(np.int16).copy()).view(torch.bfloat16).cuda()
    kw = torch.from_numpy(w.k_norm_w).cuda()
    qk = torch.from_numpy(w.qk.view(np.int16).copy()).view(torch.bfloat16).cuda()
    qw = torch.from_numpy(w.q_norm_w).cuda()
    keys = torch.empty((w.n_blocks, w.hd), dtype=torch.float32, device="cuda")
    q = torch.empty((w.rows, w.n_heads, w.hd), dtype=torch.float32, device="cuda")
    sc = torch.empty((w.rows, w.n_blocks), dtype=torch.float32, device="cuda")
    idx = torch.empty((w.rows, w.top_k), dtype=torch.int32, device="cuda")
    ws = torch.zeros(salb.indexer_topk_workspace_size(w.rows, w.n_blocks, w.top_k), dtype=torch.uint8, device="cuda")

    def path():
        salb.qsa_block_pool(raw, kw, keys, first_block=0, n_new=w.n_blocks, ratio=w.ratio, rot=w.rot, theta=w.theta,
                            eps=w.eps)
        salb.qsa_qprep_rows(qk, qw, n_heads=w.n_heads, hd=w.hd, first_pos=w.first_pos, rot=w.rot, theta=w.theta,
                            eps=w.eps, out=q)
        salb.qsa_score_rows(q, keys, first_pos=w.first_pos, ratio=w.ratio, precision="mfma", out=sc)
        salb.indexer_topk_select(sc, w.top_k, first_pos=w.first_pos, ratio=w.ratio, workspace=ws, out_idx=idx)

    path()
    torch.cuda.synchronize()
    ref_k, ref_q, ref_s, ref_i = keys.clone(), q.clone(), sc.clone(), idx.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        path()
    for rep in range(3):
        for t in (keys, q, sc):
            t.fill_(1.5)
        idx.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(keys, ref_k) and torch.equal(q, ref_q), rep
        assert torch.equal(sc.view(torch.int32), ref_s.view(torch.int32)), rep
        assert torch.equal(idx, ref_i), rep
        path()  # eager work between replays
        torch.cuda.synchronize()


def test_qsa_fp16_score_select_graph_replays_match_eager():
    """The QSA prefill on fp16 storage with the fused score + sub-tile select captured once:
    every replay (workspace and outputs overwritten between replays, eager work between
    them) equals the eager call bit for bit."""
    w = make(5, reduced=1)
    raw = torch.from_numpy(w.raw_keys.view(np.int16).copy()).view(torch.bfloat16).cuda()
    kw = torch.from_numpy(w.k_norm_w).cuda()
    qk = torch.from_numpy(w.qk.view(np.int16).copy()).view(torch.bfloat16).cuda()
    qw = torch.from_numpy(w.q_norm_w).cuda()
    keys = torch.empty((w.n_blocks, w.hd), dtype=torch.float16, device="cuda")
    q = torch.empty((w.rows, w.n_heads, w.hd), dtype=torch.float16, device="cuda")
    idx = torch.empty((w.rows, w.top_k), dtype=torch.int32, device="cuda")
    val = torch.empty((w.rows, w.top_k), dtype=torch.float32, device="cuda")
    ws = torch.zeros(salb.qsa_score_select_f16_workspace_size(w.rows, w.n_blocks, w.top_k), dtype=torch.uint8,
                     device="cuda")

    def path():
        salb.qsa_block_pool(raw, kw, keys, first_block=0, n_new=w.n_blocks, ratio=w.ratio, rot=w.rot, theta=w.theta,
                            eps=w.eps)
        salb.qsa_qprep_rows(qk, qw, n_heads=w.n_heads, hd=w.hd, first_pos=w.first_pos, rot=w.rot, theta=w.theta,
                            eps=w.eps, out=q)
        salb.qsa_score_select_f16(q, keys, w.top_k, first_pos=w.first_pos, ratio=w.ratio, workspace=ws,
                                  out_idx=idx, out_scores=val)

    path()
    torch.cuda.synchronize()
    ref_i, ref_v = idx.clone(), val.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        path()
    for rep in range(3):
        ws.fill_(0xFF)
        idx.fill_(-7)
        val.fill_(1.5)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_i), rep
        assert torch.equal(val.view(torch.int32), ref_v.view(torch.int32)), rep
        path()  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("cfg,reduced", [(2, 0), (3, 1)])
def test_fused_entry_graph_replays_match_eager(cfg, reduced):
    """indexer_score_topk captured whole (scorer, select stages; the scorer launch zeroes
    the select counters): replays on a workspace left with another call's data between
    replays equal the eager result."""
    w = make(cfg, reduced)
    d = to_dev(w)
    nbytes = salb.indexer_score_topk_workspace_size(w.T, w.max_lb, w.epb, w.top_k)
    ws = torch.full((nbytes,), 0x5A, dtype=torch.uint8, device="cuda")
    idx = torch.empty((w.T, w.top_k), dtype=torch.int32, device="cuda")
    val = torch.empty((w.T, w.top_k), dtype=torch.float32, device="cuda")

    def path():
        salb.indexer_score_topk(**d, top_k=w.top_k, precision="mfma", workspace=ws, out_idx=idx, out_scores=val)

    path()
    torch.cuda.synchronize()
    ref_i, ref_v = idx.clone(), val.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        path()
    other = make(2, 1)
    od = to_dev(other)
    for rep in range(3):
        idx.fill_(-5)
        val.fill_(3.0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_i), rep
        assert torch.equal(val.view(torch.int32), ref_v.view(torch.int32)), rep
        # eager work between replays, on the same workspace (another shape)
        salb.indexer_score_topk(**od, top_k=other.top_k, precision="mfma", workspace=ws)
        torch.cuda.synchronize()


@pytest.mark.parametrize("n_blocks", [700, 32768])
def test_qsa_decode_step_graph_replays_match_eager(n_blocks):
    """One QSA decode step (the new block pooled and the query prepared in one launch,
    then qsa_score_topk: its scores over all blocks on the matrix cores and the top-k,
    through the long-row select when the row is long, its counters cleared by the score
    launch) captured once and replayed: bit-equal to the eager step every time."""
    w = make(5, reduced=0 if n_blocks > 700 else 1)
    nb = min(n_blocks, w.n_blocks)
    raw = torch.from_numpy(w.raw_keys.view(np.int16).copy()).view(torch.bfloat16).cuda()
    kw = torch.from_numpy(w.k_norm_w).cuda()
    qw = torch.from_numpy(w.q_norm_w).cuda()
    q_in = torch.from_numpy(w.qk[w.rows - 1].view(np.int16).copy()).view(torch.bfloat16).cuda()
    pos = nb * w.ratio - 1
    keys = torch.empty((w.n_blocks, w.hd), dtype=torch.float32, device="cuda")
    salb.qsa_block_pool(raw, kw, keys, first_block=0, n_new=nb, ratio=w.ratio, rot=w.rot, theta=w.theta, eps=w.eps)
    q = torch.empty((w.n_heads, w.hd), dtype=torch.float32, device="cuda")
    idx = torch.empty((1, w.top_k), dtype=torch.int32, device="cuda")
    val = torch.empty((1, w.top_k), dtype=torch.float32, device="cuda")
    ws = torch.full((max(256, salb.qsa_score_topk_workspace_size(nb, w.top_k)),), 0x5A, dtype=torch.uint8,
                    device="cuda")

    def step():  # the new block and the query in one launch, as the benchmark's step
        salb.qsa_decode_prep(raw, kw, keys, q_in.view(1, -1), qw, first_block=nb - 1, n_new=1, ratio=w.ratio,
                             n_heads=w.n_heads, hd=w.hd, first_pos=pos, rot=w.rot, theta=w.theta, eps=w.eps,
                             out=q.view(1, w.n_heads, w.hd))
        salb.qsa_score_topk(q, keys, w.top_k, n_blocks=nb, workspace=ws, out_idx=idx[0], out_scores=val[0])

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (keys, q, idx, val)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in (q, val):
            t.fill_(2.5)
        idx.fill_(-3)
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((keys, q, idx, val), ref):
            assert torch.equal(got.view(torch.int32), want.view(torch.int32)), rep
        step()  # eager work between replays
        torch.cuda.synchronize()
