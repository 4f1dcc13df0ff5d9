"""GPU parity of the QSA variant (block pooling, query prep, row scores, causal top-k)
through the C ABI against the float64 oracle.  Needs an MI355X."""

import numpy as np
import pytest
import torch

import sparse_attention_lightning_block_amd as salb
from oracle import indexer, qsa
from tests.parity import MFMA_ROWMAX, check_topk
from workloads import make
from workloads.configs import qsa as qsa_workload

pytestmark = pytest.mark.gpu

# Pooled keys and prepared queries: each element within VEC_REL of the vector's
# largest magnitude.  The GPU forms a 16-term mean, a sum of squares, one rsqrt and a
# rotation in fp32 (angles in fp64, cos/sin rounded to fp32): each element carries a
# few fp32 roundings (~1e-7 relative to the vector's scale); 1e-5 leaves a wide margin.
VEC_REL = 1e-5
# Row scores on the FP32 path from the same fp32 inputs: |dS| <= 1e-5 |S| + 1e-6 A,
# A = sum_h sum_d |q_hd k_d| / sqrt(hd) (the FP32 tolerance of the CSA scores).
# End to end from the bf16 inputs, the fp32 roundings of the pooled keys and the
# prepared queries enter every product: the A term grows to 1e-5.
S_REL, S_ABS_A, CHAIN_ABS_A = 1e-5, 1e-6, 1e-5


def _bf16(bits):
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)


def _pool_all(w, dev="cuda"):
    raw = _bf16(w.raw_keys).to(dev)
    kw = torch.from_numpy(w.k_norm_w).to(dev)
    keys = torch.full((w.n_blocks, w.hd), float("nan"), dtype=torch.float32, device=dev)
    salb.qsa_block_pool(raw, kw, keys, first_block=0, n_new=w.n_blocks, ratio=w.ratio, rot=w.rot, theta=w.theta,
                        eps=w.eps)
    return keys


def _qprep(w, dev="cuda"):
    qk = _bf16(w.qk).to(dev)
    qw = torch.from_numpy(w.q_norm_w).to(dev)
    return salb.qsa_qprep_rows(qk, qw, n_heads=w.n_heads, hd=w.hd, first_pos=w.first_pos, rot=w.rot, theta=w.theta,
                               eps=w.eps)


def _check_vectors(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    scale = np.max(np.abs(ref), axis=-1, keepdims=True)
    err = np.abs(got - ref)
    bad = np.argwhere(err > VEC_REL * scale)
    assert bad.size == 0, f"{what}: {len(bad)} elements out of tolerance, first {bad[:3].tolist()}"


def _abs_sum(q, keys, valid):
    """A[r, b] = sum_h sum_d |q[r,h,d] k[b,d]| / sqrt(hd), for b < valid[r]."""
    hd = q.shape[2]
    return [np.abs(q[r]).sum(axis=0) @ np.abs(keys[: int(valid[r])]).T / np.sqrt(hd) for r in range(q.shape[0])]


def test_block_pool_reduced():
    w = make(5, reduced=1)
    keys = _pool_all(w).cpu().numpy()
    ref = qsa.block_pool(indexer.upcast(w.raw_keys, "bf16"), w.k_norm_w, 0, w.n_blocks, w.ratio, w.rot, w.theta,
                         w.eps)
    _check_vectors(keys, ref, "block pool")


def test_block_pool_partial_range_and_empty():
    """Only rows first_block .. first_block + n_new - 1 are written; n_new == 0 writes nothing."""
    w = make(5, reduced=1)
    raw = _bf16(w.raw_keys).cuda()
    kw = torch.from_numpy(w.k_norm_w).cuda()
    keys = torch.full((w.n_blocks, w.hd), 7.0, dtype=torch.float32, device="cuda")
    salb.qsa_block_pool(raw, kw, keys, first_block=100, n_new=37, ratio=w.ratio, rot=w.rot, theta=w.theta, eps=w.eps)
    salb.qsa_block_pool(raw, kw, keys, first_block=5, n_new=0, ratio=w.ratio, rot=w.rot, theta=w.theta, eps=w.eps)
    got = keys.cpu().numpy()
    assert np.all(got[:100] == 7.0) and np.all(got[137:] == 7.0)
    ref = qsa.block_pool(indexer.upcast(w.raw_keys, "bf16"), w.k_norm_w, 100, 37, w.ratio, w.rot, w.theta, w.eps)
    _check_vectors(got[100:137], ref, "block pool range")


def test_qprep_rows_reduced():
    w = make(5, reduced=1)
    q = _qprep(w).cpu().numpy()
    ref = qsa.qprep_rows(indexer.upcast(w.qk, "bf16"), w.q_norm_w, w.rows, w.first_pos, w.n_heads * w.hd, w.n_heads,
                         w.hd, w.rot, w.theta, w.eps)
    _check_vectors(q, ref, "qprep")


# (n_heads, hd, rot, ratio, rows, qkw padding, first_pos): every head size, rotations
# narrower than hd and none, odd ratios, head counts that leave a slice of the query
# prep partly empty, and enough rows for both slice widths (256 chunks once the rows
# fill 1024 workgroups, else 128)
_SHAPES = [
    (3, 64, 64, 4, 5, 8, 17),
    (5, 256, 128, 7, 9, 0, 500000),
    (1, 128, 0, 16, 3, 0, 40),
    (64, 128, 96, 3, 300, 0, 262000),
    (40, 64, 62, 16, 7, 16, 123457),
    (24, 128, 128, 2, 2000, 0, 9),
]


@pytest.mark.parametrize("n_heads,hd,rot,ratio,rows,pad,first_pos", _SHAPES)
def test_pool_and_qprep_shapes(n_heads, hd, rot, ratio, rows, pad, first_pos):
    """Block pool and query prep against the oracle over head sizes, rotation widths and
    slicings; projection rows padded with NaN bits (a read past n_heads * hd shows); the
    one-launch decode prep and the fp16 outputs bit-identical to the fp32 calls."""
    nb = 37
    w = qsa_workload("qsa_shapes", [11, n_heads, hd, rows], n_tok=nb * ratio, hd=hd, ratio=ratio, rows=rows,
                     n_heads=n_heads, top_k=1, rot=rot, first_pos=first_pos)
    qk_bits = np.concatenate([w.qk, np.full((rows, pad), 0x7FC0, dtype=np.uint16)], axis=1)
    raw, kw = _bf16(w.raw_keys).cuda(), torch.from_numpy(w.k_norm_w).cuda()
    qk, qw = _bf16(qk_bits).cuda(), torch.from_numpy(w.q_norm_w).cuda()
    kwargs = dict(ratio=ratio, rot=rot, theta=w.theta, eps=w.eps)
    keys = torch.full((nb, hd), 7.0, dtype=torch.float32, device="cuda")
    salb.qsa_block_pool(raw, kw, keys, first_block=2, n_new=nb - 2, **kwargs)
    q = salb.qsa_qprep_rows(qk, qw, n_heads=n_heads, hd=hd, first_pos=first_pos, rot=rot, theta=w.theta, eps=w.eps)
    got_keys, got_q = keys.cpu().numpy(), q.cpu().numpy()
    assert np.all(got_keys[:2] == 7.0)
    ref_keys = qsa.block_pool(indexer.upcast(w.raw_keys, "bf16"), w.k_norm_w, 2, nb - 2, ratio, rot, w.theta, w.eps)
    _check_vectors(got_keys[2:], ref_keys, "block pool")
    ref_q = qsa.qprep_rows(indexer.upcast(qk_bits, "bf16"), w.q_norm_w, rows, first_pos, n_heads * hd + pad,
                           n_heads, hd, rot, w.theta, w.eps)
    _check_vectors(got_q, ref_q, "qprep")
    # the fused decode prep and the fp16 outputs give the same bits
    keys2 = torch.full((nb, hd), 7.0, dtype=torch.float32, device="cuda")
    q2 = salb.qsa_decode_prep(raw, kw, keys2, qk, qw, first_block=2, n_new=nb - 2, n_heads=n_heads, hd=hd,
                              first_pos=first_pos, **kwargs)
    assert torch.equal(keys2.view(torch.int32), keys.view(torch.int32))
    assert torch.equal(q2.view(torch.int32), q.view(torch.int32))
    keys16 = torch.zeros((nb, hd), dtype=torch.float16, device="cuda")
    salb.qsa_block_pool(raw, kw, keys16, first_block=2, n_new=nb - 2, **kwargs)
    q16 = salb.qsa_qprep_rows(qk, qw, n_heads=n_heads, hd=hd, first_pos=first_pos, rot=rot, theta=w.theta,
                              eps=w.eps, dtype=torch.float16)
    assert torch.equal(keys16[2:].view(torch.int16), keys[2:].half().view(torch.int16))
    assert torch.equal(q16.view(torch.int16), q.half().view(torch.int16))


@pytest.mark.parametrize("first_block,n_new,rows", [(100, 1, 1), (3, 45, 7), (0, 0, 2), (60, 33, 1)])
def test_decode_prep_is_pool_and_qprep_bit_for_bit(first_block, n_new, rows):
    """The one-launch decode prep writes exactly what qsa_block_pool and qsa_qprep_rows
    write (one new block and one query, many blocks and rows, no new block), leaves the
    other blocks untouched, and matches the oracle."""
    w = make(5, reduced=1)
    raw = _bf16(w.raw_keys).cuda()
    kw = torch.from_numpy(w.k_norm_w).cuda()
    qw = torch.from_numpy(w.q_norm_w).cuda()
    qk = _bf16(w.qk[:rows]).cuda() if rows else torch.empty((0, w.qk.shape[1]), dtype=torch.bfloat16, device="cuda")
    fp = w.first_pos + 5
    a_keys = torch.full((w.n_blocks, w.hd), 7.0, dtype=torch.float32, device="cuda")
    b_keys = a_keys.clone()
    a_q = salb.qsa_decode_prep(raw, kw, a_keys, qk, qw, first_block=first_block, n_new=n_new, ratio=w.ratio,
                               n_heads=w.n_heads, hd=w.hd, first_pos=fp, rot=w.rot, theta=w.theta, eps=w.eps)
    salb.qsa_block_pool(raw, kw, b_keys, first_block=first_block, n_new=n_new, ratio=w.ratio, rot=w.rot,
                        theta=w.theta, eps=w.eps)
    b_q = (salb.qsa_qprep_rows(qk, qw, n_heads=w.n_heads, hd=w.hd, first_pos=fp, rot=w.rot, theta=w.theta, eps=w.eps)
           if rows else torch.empty((0, w.n_heads, w.hd), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(a_keys.view(torch.int32), b_keys.view(torch.int32))
    assert torch.equal(a_q.view(torch.int32), b_q.view(torch.int32))
    got = a_keys.cpu().numpy()
    assert np.all(got[:first_block] == 7.0) and np.all(got[first_block + n_new:] == 7.0)
    if n_new:
        ref = qsa.block_pool(indexer.upcast(w.raw_keys, "bf16"), w.k_norm_w, first_block, n_new, w.ratio, w.rot,
                             w.theta, w.eps)
        _check_vectors(got[first_block:first_block + n_new], ref, "decode prep pool")
    if rows:
        ref = qsa.qprep_rows(indexer.upcast(w.qk[:rows], "bf16"), w.q_norm_w, rows, fp, w.n_heads * w.hd, w.n_heads,
                             w.hd, w.rot, w.theta, w.eps)
        _check_vectors(a_q.cpu().numpy(), ref, "decode prep qprep")


@pytest.mark.parametrize("nb", [0, 5, 700, 32768])
def test_score_topk_is_score_then_select_bit_for_bit(nb):
    """qsa_score_topk (scores in the workspace, the select's counters cleared by the score
    launch) against qsa_score followed by indexer_topk_select: the same indices and
    scores, bit for bit, from a workspace full of garbage, twice in a row; fewer blocks
    than top_k pads with -1 / -inf."""
    w = make(5, reduced=0 if nb > 1000 else 1)
    nb = min(nb, w.n_blocks)
    keys = _pool_all(w)
    r = w.rows - 1
    q = salb.qsa_qprep(_bf16(w.qk[r]).cuda(), torch.from_numpy(w.q_norm_w).cuda(), n_heads=w.n_heads, hd=w.hd,
                       pos=w.first_pos + r, rot=w.rot, theta=w.theta, eps=w.eps)
    ws = torch.full((max(256, salb.qsa_score_topk_workspace_size(nb, w.top_k)),), 0x5A, dtype=torch.uint8,
                    device="cuda")
    for _ in range(2):
        a_idx, a_val = salb.qsa_score_topk(q, keys, w.top_k, n_blocks=nb, with_scores=True, workspace=ws)
        if nb:
            sc = salb.qsa_score(q, keys, n_blocks=nb)
            b_idx, b_val = salb.indexer_topk_select(sc.view(1, nb), w.top_k, with_scores=True)
        torch.cuda.synchronize()
        if nb:
            assert torch.equal(a_idx, b_idx[0]) and torch.equal(a_val.view(torch.int32), b_val[0].view(torch.int32))
        k = min(nb, w.top_k)
        assert torch.all(a_idx[k:] == -1) and torch.all(torch.isneginf(a_val[k:]))
        assert torch.all(a_idx[:k] >= 0) and torch.all(a_idx[:k] < max(nb, 1))
        ws.fill_(0xA5)


# (rows, n_blocks, first_pos, ratio, n_heads, hd, top_k, keys): valid counts below and
# above top_k, fewer sub-tiles than top_k, top_k at the sub-tile select's limit (512) and
# past it (600: the general select), n_blocks not a multiple of 16, and rows of equal
# scores (every block key the same vector: the candidate list overflows and the select
# falls back to passes over the whole row)
_SCORE_SELECT = [
    (300, 300, 0, 1, 16, 64, 64, "normal"),
    (300, 2300, 2000, 1, 16, 64, 64, "normal"),
    (260, 5003, 4700, 1, 64, 128, 512, "normal"),
    (64, 32768, 40000, 1, 64, 128, 512, "normal"),
    (64, 3000, 2900, 1, 32, 128, 600, "normal"),
    (300, 4000, 3800, 1, 16, 64, 256, "equal"),
    (50, 2000, 31000, 16, 32, 128, 256, "normal"),
]


@pytest.mark.parametrize("rows,nb,first_pos,ratio,n_heads,hd,k,keys", _SCORE_SELECT)
def test_score_select_is_score_rows_then_select_bit_for_bit(rows, nb, first_pos, ratio, n_heads, hd, k, keys):
    """qsa_score_select_f16 gives the indices and scores of qsa_score_rows (fp16 inputs) then
    indexer_topk_select with the causal count, bit for bit, from a workspace full of
    garbage, twice in a row."""
    rng = np.random.default_rng(rows * 7 + nb + k)
    q = torch.from_numpy(rng.standard_normal((rows, n_heads, hd)).astype(np.float16)).cuda()
    if keys == "equal":
        kv = rng.standard_normal((1, hd)).astype(np.float16)
        kb = torch.from_numpy(np.repeat(kv, nb, axis=0)).cuda()
    else:
        kb = torch.from_numpy(rng.standard_normal((nb, hd)).astype(np.float16)).cuda()
    scores = salb.qsa_score_rows(q, kb, first_pos=first_pos, ratio=ratio)
    idx_ref, val_ref = salb.indexer_topk_select(scores, k, first_pos=first_pos, ratio=ratio, with_scores=True)
    ws = torch.full((salb.qsa_score_select_f16_workspace_size(rows, nb, k),), 0xFF, dtype=torch.uint8, device="cuda")
    for _ in range(2):
        idx, val = salb.qsa_score_select_f16(q, kb, k, first_pos=first_pos, ratio=ratio, with_scores=True,
                                             workspace=ws)
        assert torch.equal(idx, idx_ref)
        assert torch.equal(val.view(torch.int32), val_ref.view(torch.int32))
    # the two halves: the same scores, and (where the sub-tile select takes the shape) the
    # same selection
    sc, tm = salb.qsa_score_rows_f16_tmax(q, kb, first_pos=first_pos, ratio=ratio)
    assert torch.equal(sc[:, :nb].view(torch.int32), scores.view(torch.int32))
    ref_max = torch.full((rows, (nb + 15) // 16 * 16), -float("inf"), device="cuda")
    ref_max[:, :nb] = scores
    keys_u = ref_max.view(torch.int32).to(torch.int64) & 0xFFFFFFFF
    neg = keys_u >= 0x80000000
    ok = torch.where(neg, 0xFFFFFFFF - keys_u, keys_u | 0x80000000)     # order keys (no NaN, no -0 here)
    ok[:, nb:] = 0
    want = ok.view(rows, -1, 16).amax(dim=2)
    assert torch.equal(tm.to(torch.int64) & 0xFFFFFFFF, want)
    if k <= 512:
        idx2, val2 = salb.qsa_select_tiles(sc, tm, k, n_cols=nb, first_pos=first_pos, ratio=ratio, with_scores=True)
        assert torch.equal(idx2, idx_ref)
        assert torch.equal(val2.view(torch.int32), val_ref.view(torch.int32))


def test_score_select_full_size_matches_the_two_calls():
    """The QSA prefill (2048 rows x 32768 blocks, top_k 256, fp16 storage): the fused call's
    selection equals the two calls' for every row."""
    w = make(5)
    raw = _bf16(w.raw_keys).cuda()
    kw = torch.from_numpy(w.k_norm_w).cuda()
    keys = torch.empty((w.n_blocks, w.hd), dtype=torch.float16, device="cuda")
    salb.qsa_block_pool(raw, kw, keys, first_block=0, n_new=w.n_blocks, ratio=w.ratio, rot=w.rot, theta=w.theta,
                        eps=w.eps)
    qk = _bf16(w.qk).cuda()
    qw = torch.from_numpy(w.q_norm_w).cuda()
    q = salb.qsa_qprep_rows(qk, qw, n_heads=w.n_heads, hd=w.hd, first_pos=w.first_pos, rot=w.rot, theta=w.theta,
                            eps=w.eps, dtype=torch.float16)
    scores = salb.qsa_score_rows(q, keys, first_pos=w.first_pos, ratio=w.ratio)
    idx_ref, val_ref = salb.indexer_topk_select(scores, w.top_k, first_pos=w.first_pos, ratio=w.ratio,
                                                with_scores=True)
    del scores
    idx, val = salb.qsa_score_select_f16(q, keys, w.top_k, first_pos=w.first_pos, ratio=w.ratio, with_scores=True)
    assert torch.equal(idx, idx_ref)
    assert torch.equal(val.view(torch.int32), val_ref.view(torch.int32))


@pytest.mark.parametrize("n_heads,hd,nb,k", [(64, 128, 32768, 512), (48, 128, 5000, 256), (32, 128, 40001, 256),
                                             (16, 64, 3000, 600), (32, 64, 20000, 1)])
def test_score_topk_shapes_bit_for_bit(n_heads, hd, nb, k):
    """qsa_score_topk on the sub-tile select (matrix-core scorer, <= 32768 blocks, top_k <=
    512) and off it (48 heads: the vector scorer; 40001 blocks; top_k 600): the indices and
    scores of qsa_score then indexer_topk_select, bit for bit."""
    rng = np.random.default_rng(n_heads + hd + nb + k)
    q = torch.from_numpy(rng.standard_normal((n_heads, hd)).astype(np.float32)).cuda()
    keys = torch.from_numpy(rng.standard_normal((nb, hd)).astype(np.float32)).cuda()
    ws = torch.full((max(256, salb.qsa_score_topk_workspace_size(nb, k)),), 0x5A, dtype=torch.uint8, device="cuda")
    a_idx, a_val = salb.qsa_score_topk(q, keys, k, with_scores=True, workspace=ws)
    sc = salb.qsa_score(q, keys)
    b_idx, b_val = salb.indexer_topk_select(sc.view(1, nb), k, with_scores=True)
    assert torch.equal(a_idx, b_idx[0])
    assert torch.equal(a_val.view(torch.int32), b_val[0].view(torch.int32))


@pytest.mark.parametrize("precision", ["fp32", "mfma"])
def test_score_rows_and_topk_reduced(precision):
    """Scores from the GPU's own pooled keys and prepared queries (the same fp32 inputs on
    both sides), then the causal top-k on those scores."""
    w = make(5, reduced=1)
    keys_d = _pool_all(w)
    q_d = _qprep(w)
    sc = salb.qsa_score_rows(q_d, keys_d, first_pos=w.first_pos, ratio=w.ratio, precision=precision)
    idx, val = salb.indexer_topk_select(sc, w.top_k, first_pos=w.first_pos, ratio=w.ratio, with_scores=True)
    torch.cuda.synchronize()
    q, keys = q_d.cpu().numpy().astype(np.float64), keys_d.cpu().numpy().astype(np.float64)
    ref, valid = qsa.score_rows(q, keys, w.first_pos, w.ratio)
    A = _abs_sum(q, keys, valid)
    got, gi, gv = sc.cpu().numpy(), idx.cpu().numpy(), val.cpu().numpy()
    for r in range(w.rows):
        v = int(valid[r])
        assert np.all(np.isneginf(got[r, v:])), f"row {r}: blocks past the complete count must be -inf"
        if precision == "fp32":
            tol = S_REL * np.abs(ref[r, :v]) + S_ABS_A * A[r]
        else:
            tol = np.full(v, MFMA_ROWMAX * np.max(np.abs(ref[r, :v])))
        err = np.abs(got[r, :v].astype(np.float64) - ref[r, :v])
        assert np.all(err <= tol), f"row {r}: max err {err.max()}"
        check_topk(gi[r], gv[r], ref[r, :v], None, w.top_k, precision, f"qsa row {r}", tol=tol)


def test_chain_end_to_end_reduced():
    """bf16 raw keys and projections -> pooled keys, prepared q, scores, top-k; against the
    oracle chain in float64."""
    w = make(5, reduced=1)
    keys_d = _pool_all(w)
    q_d = _qprep(w)
    sc = salb.qsa_score_rows(q_d, keys_d, first_pos=w.first_pos, ratio=w.ratio, precision="fp32")
    idx, val = salb.indexer_topk_select(sc, w.top_k, first_pos=w.first_pos, ratio=w.ratio, with_scores=True)
    keys = qsa.block_pool(indexer.upcast(w.raw_keys, "bf16"), w.k_norm_w, 0, w.n_blocks, w.ratio, w.rot, w.theta,
                          w.eps)
    q = qsa.qprep_rows(indexer.upcast(w.qk, "bf16"), w.q_norm_w, w.rows, w.first_pos, w.n_heads * w.hd, w.n_heads,
                       w.hd, w.rot, w.theta, w.eps)
    ref, valid = qsa.score_rows(q, keys, w.first_pos, w.ratio)
    A = _abs_sum(q, keys, valid)
    got, gi, gv = sc.cpu().numpy(), idx.cpu().numpy(), val.cpu().numpy()
    for r in range(w.rows):
        v = int(valid[r])
        tol = S_REL * np.abs(ref[r, :v]) + CHAIN_ABS_A * A[r]
        err = np.abs(got[r, :v].astype(np.float64) - ref[r, :v])
        assert np.all(err <= tol), f"row {r}: max err {err.max()}"
        check_topk(gi[r], gv[r], ref[r, :v], None, w.top_k, "fp32", f"qsa chain row {r}", tol=tol)


# ------------------------------------------------------------------ decode (one query)

def _decode_case(w, r, keys_d):
    """Prepared query of projection row r as a decode query at position first_pos + r, its
    scores over the complete blocks and their top-k, all on the GPU."""
    pos = w.first_pos + r
    nb = min(w.n_blocks, (pos + 1) // w.ratio)
    q_in = _bf16(w.qk[r]).cuda()
    q = salb.qsa_qprep(q_in, torch.from_numpy(w.q_norm_w).cuda(), n_heads=w.n_heads, hd=w.hd, pos=pos, rot=w.rot,
                       theta=w.theta, eps=w.eps)
    sc = salb.qsa_score(q, keys_d, n_blocks=nb)
    idx, val = salb.indexer_topk_select(sc[None, :], w.top_k, with_scores=True)
    torch.cuda.synchronize()
    return pos, nb, q.cpu().numpy().astype(np.float64), sc.cpu().numpy(), idx[0].cpu().numpy(), val[0].cpu().numpy()


@pytest.mark.parametrize("r", [0, 17, 39])
def test_decode_query_reduced(r):
    """qsa_qprep, qsa_score and the top-k of one decode query: the prepared query against
    the oracle; the scores against the oracle on the GPU's own pooled keys and query (FP32
    rule), and end to end against the oracle chain from the bf16 inputs."""
    w = make(5, reduced=1)
    keys_d = _pool_all(w)
    pos, nb, q, sc, gi, gv = _decode_case(w, r, keys_d)
    qo = qsa.qprep(indexer.upcast(w.qk[r], "bf16"), w.q_norm_w, w.n_heads, w.hd, w.rot, pos, w.theta, w.eps)
    _check_vectors(q, qo, "decode qprep")
    keys = keys_d.cpu().numpy().astype(np.float64)
    ref = qsa.score_blocks(q, keys, nb)
    A = np.abs(q).sum(axis=0) @ np.abs(keys[:nb]).T / np.sqrt(w.hd)
    err = np.abs(sc.astype(np.float64) - ref)
    assert np.all(err <= S_REL * np.abs(ref) + S_ABS_A * A), f"max err {err.max()}"
    check_topk(gi, gv, ref, None, w.top_k, "fp32", f"decode {r}", tol=S_REL * np.abs(ref) + S_ABS_A * A)
    keys_o = qsa.block_pool(indexer.upcast(w.raw_keys, "bf16"), w.k_norm_w, 0, w.n_blocks, w.ratio, w.rot, w.theta,
                            w.eps)
    ref_o = qsa.score_blocks(qo, keys_o, nb)
    A_o = np.abs(qo).sum(axis=0) @ np.abs(keys_o[:nb]).T / np.sqrt(w.hd)
    assert np.all(np.abs(sc - ref_o) <= S_REL * np.abs(ref_o) + CHAIN_ABS_A * A_o)


def test_decode_query_full_size():
    """The last prefill position of the QSA workload as a decode query: 32768 complete
    blocks, top 256, against the oracle chain from the bf16 inputs."""
    w = make(5)
    keys_d = _pool_all(w)
    r = w.rows - 1
    pos, nb, q, sc, gi, gv = _decode_case(w, r, keys_d)
    assert nb == w.n_blocks
    qo = qsa.qprep(indexer.upcast(w.qk[r], "bf16"), w.q_norm_w, w.n_heads, w.hd, w.rot, pos, w.theta, w.eps)
    _check_vectors(q, qo, "decode qprep full")
    keys_o = qsa.block_pool(indexer.upcast(w.raw_keys, "bf16"), w.k_norm_w, 0, w.n_blocks, w.ratio, w.rot, w.theta,
                            w.eps)
    ref = qsa.score_blocks(qo, keys_o, nb)
    A = np.abs(qo).sum(axis=0) @ np.abs(keys_o).T / np.sqrt(w.hd)
    tol = S_REL * np.abs(ref) + CHAIN_ABS_A * A
    err = np.abs(sc.astype(np.float64) - ref)
    assert np.all(err <= tol), f"max err {err.max()}"
    check_topk(gi, gv, ref, None, w.top_k, "fp32", "decode full", tol=tol)


def test_decode_score_partial_table_and_empty():
    """Only the n_blocks given are scored (the table may be longer); n_blocks = 0 launches
    nothing."""
    w = make(5, reduced=1)
    keys_d = _pool_all(w)
    q = torch.randn(w.n_heads, w.hd, dtype=torch.float32, device="cuda")
    out = torch.full((w.n_blocks,), 9.0, dtype=torch.float32, device="cuda")
    salb.qsa_score(q, keys_d, n_blocks=100, out=out[:100])
    salb.qsa_score(q, keys_d, n_blocks=0, out=out[:0])
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(got[100:] == 9.0)
    ref = qsa.score_blocks(q.cpu().numpy().astype(np.float64), keys_d.cpu().numpy().astype(np.float64), 100)
    assert np.allclose(got[:100], ref, rtol=1e-5, atol=1e-5 * np.abs(ref).max())


@pytest.mark.parametrize("n_heads,hd,nb", [(16, 64, 1000), (48, 128, 777), (64, 128, 40001), (32, 128, 32785),
                                           (5, 128, 300), (32, 256, 129), (16, 128, 7)])
def test_decode_score_shapes(n_heads, hd, nb):
    """qsa_score over the shapes of both kernels (matrix-core tiles for 16..64 heads in
    steps of 16 at hd 64/128, one and two 16-block units per wave; the VALU kernel
    otherwise), ragged block counts, seeded N(0, 1) inputs: the FP32 rule against the
    oracle."""
    rng = np.random.default_rng([5, n_heads, hd, nb])
    q = rng.standard_normal((n_heads, hd)).astype(np.float32)
    keys = rng.standard_normal((nb + 3, hd)).astype(np.float32)
    out = torch.full((nb + 16,), 7.0, dtype=torch.float32, device="cuda")
    salb.qsa_score(torch.from_numpy(q).cuda(), torch.from_numpy(keys).cuda(), n_blocks=nb, out=out[:nb])
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(got[nb:] == 7.0)
    q64, k64 = q.astype(np.float64), keys.astype(np.float64)
    ref = qsa.score_blocks(q64, k64, nb)
    A = np.abs(q64).sum(axis=0) @ np.abs(k64[:nb]).T / np.sqrt(hd)
    err = np.abs(got[:nb].astype(np.float64) - ref)
    assert np.all(err <= S_REL * np.abs(ref) + S_ABS_A * A), f"max err {err.max()}"


@pytest.mark.parametrize("reduced,n_heads,hd", [(1, 32, 128), (1, 16, 64), (1, 64, 128), (0, 32, 128)])
def test_fp16_storage_is_the_mfma_path_bit_for_bit(reduced, n_heads, hd):
    """qsa_block_pool_f16 and qsa_qprep_rows_f16 store exactly the fp16 roundings of the
    fp32 results (torch's round-to-nearest-even .half()), and qsa_score_rows_f16 on them
    returns the fp32-input matrix-core scores bit for bit."""
    w = make(5, reduced=reduced)
    rng = np.random.default_rng([5, 16, n_heads, hd])
    if (n_heads, hd) != (w.n_heads, w.hd):      # other shapes: seeded bf16 projections and raw keys
        raw_np = rng.standard_normal((w.n_blocks * w.ratio, hd)).astype(np.float32)
        qk_np = rng.standard_normal((w.rows, n_heads * hd)).astype(np.float32)
        raw = torch.from_numpy(raw_np).to(torch.bfloat16).cuda()
        qk = torch.from_numpy(qk_np).to(torch.bfloat16).cuda()
        kw = torch.from_numpy(rng.normal(0, 0.1, hd).astype(np.float32)).cuda()
        qw = torch.from_numpy(rng.normal(0, 0.1, hd).astype(np.float32)).cuda()
        rot = min(w.rot, hd)
    else:
        raw = _bf16(w.raw_keys).cuda()
        qk = _bf16(w.qk).cuda()
        kw = torch.from_numpy(w.k_norm_w).cuda()
        qw = torch.from_numpy(w.q_norm_w).cuda()
        rot = w.rot
    k32 = torch.empty((w.n_blocks, hd), dtype=torch.float32, device="cuda")
    k16 = torch.empty((w.n_blocks, hd), dtype=torch.float16, device="cuda")
    for keys in (k32, k16):
        salb.qsa_block_pool(raw, kw, keys, first_block=0, n_new=w.n_blocks, ratio=w.ratio, rot=rot, theta=w.theta,
                            eps=w.eps)
    kwargs = dict(n_heads=n_heads, hd=hd, first_pos=w.first_pos, rot=rot, theta=w.theta, eps=w.eps)
    q32 = salb.qsa_qprep_rows(qk, qw, **kwargs)
    q16 = salb.qsa_qprep_rows(qk, qw, dtype=torch.float16, **kwargs)
    torch.cuda.synchronize()
    assert torch.equal(k16.view(torch.int16), k32.half().view(torch.int16))
    assert torch.equal(q16.view(torch.int16), q32.half().view(torch.int16))
    s32 = salb.qsa_score_rows(q32, k32, first_pos=w.first_pos, ratio=w.ratio, precision="mfma")
    s16 = salb.qsa_score_rows(q16, k16, first_pos=w.first_pos, ratio=w.ratio, precision="mfma")
    torch.cuda.synchronize()
    assert torch.equal(s16.view(torch.int32), s32.view(torch.int32))
