"""GPU parity: the HIP path through the C ABI against the CPU oracle.  Needs an MI355X."""

import numpy as np
import pytest
import torch

import sparse_attention_lightning_block_amd as salb
from oracle import indexer, nvfp4
from tests.parity import check_scores, check_topk, oracle_rows, to_dev
from workloads import make
from workloads.configs import csa, e4m3_encode_rne

pytestmark = pytest.mark.gpu


def _row(t):
    return t.cpu().numpy()


# ------------------------------------------------------------------ dequant

def _exhaustive_pool():
    """Every byte in every nibble position and every scale byte (NaN codes excluded)."""
    scales = np.array([c for c in range(256) if (c & 0x7f) != 0x7f], dtype=np.uint8)   # 254 codes
    D, epb = 64, 16
    n = len(scales) * 8                   # 8 keys per scale code, 32 bytes each = all 256 byte values
    keys = np.zeros((n, D // 2), dtype=np.uint8)
    sc = np.zeros((n, D // 16), dtype=np.uint8)
    for i, s in enumerate(scales):
        for j in range(8):
            keys[i * 8 + j] = np.arange(32 * j, 32 * j + 32, dtype=np.uint8)
            sc[i * 8 + j] = s
    P = n // epb
    g = np.linspace(0.5, 2.0, P).astype(np.float32)
    return keys.reshape(P, epb, D // 2), sc.reshape(P, epb, D // 16), g, epb


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_dequant_bit_exact_exhaustive(mode):
    keys, sc, g, epb = _exhaustive_pool()
    P = keys.shape[0]
    bt = np.random.default_rng(0).permutation(P).astype(np.int32)
    n = P * epb
    out = salb.indexer_debug_dequant(torch.from_numpy(keys).cuda(), torch.from_numpy(sc).cuda(),
                                     torch.from_numpy(g).cuda(), torch.from_numpy(bt).cuda(), n, mode)
    c, gg = nvfp4.dequant_row(keys, sc, g, bt, n, epb)
    ref = nvfp4.dequant_f32(c, gg) if mode == 1 else c.astype(np.float32)
    got = out.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))   # bit-exact, -0.0 included


@pytest.mark.parametrize("cfg", [1, 2])
def test_dequant_bit_exact_configs(cfg):
    w = make(cfg, reduced=1 if cfg != 1 else 0)
    d = to_dev(w)
    for t in range(min(w.T, 2)):
        n = int(w.valid_lens[t])
        c, gg = nvfp4.dequant_row(w.keys_fp4, w.key_scale, w.key_gscale, w.block_table[t], n, w.epb)
        for mode, ref in ((0, c.astype(np.float32)), (1, nvfp4.dequant_f32(c, gg)), (2, c.astype(np.float32))):
            got = salb.indexer_debug_dequant(d["keys_fp4"], d["key_scale"], d["key_gscale"], d["block_table"][t], n,
                                             mode).cpu().numpy()
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (cfg, t, mode)


# ------------------------------------------------------------------ scores

CASES = [(1, 0), (2, 1), (3, 1), (4, 1)]


@pytest.mark.parametrize("precision", ["fp32", "mfma"])
@pytest.mark.parametrize("cfg,reduced", CASES)
def test_score_rows(cfg, reduced, precision):
    w = make(cfg, reduced)
    d = to_dev(w)
    n_cols = w.max_lb * w.epb
    out = salb.indexer_score_rows(**d, n_cols=n_cols, precision=precision)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref, amag = oracle_rows(w)
    for t in range(w.T):
        v = int(w.valid_lens[t])
        check_scores(got[t], ref[t], amag[t], precision, f"cfg{cfg} t{t}")
        assert np.all(np.isneginf(got[t, v:])), "tail must be -inf"


@pytest.mark.parametrize("precision", ["fp32", "mfma"])
@pytest.mark.parametrize("cfg,reduced", CASES)
def test_score_topk(cfg, reduced, precision):
    w = make(cfg, reduced)
    d = to_dev(w)
    idx, val = salb.indexer_score_topk(**d, top_k=w.top_k, precision=precision, with_scores=True)
    torch.cuda.synchronize()
    gi, gv = idx.cpu().numpy(), val.cpu().numpy()
    ref, amag = oracle_rows(w)
    for t in range(w.T):
        check_topk(gi[t], gv[t], ref[t], amag[t], w.top_k, precision, f"cfg{cfg} t{t}")


def test_tiny_config_exact_topk_fp32():
    """Config 1 on the FP32 path: the selected sets equal the oracle's exactly except within tolerance;
    the short row (valid 17 < k) selects every key, zero scores ordered by index."""
    w = make(1)
    d = to_dev(w)
    idx, val = salb.indexer_score_topk(**d, top_k=w.top_k, precision="fp32", with_scores=True)
    gi = _row(idx)
    ref, _ = oracle_rows(w)
    o_idx, _ = indexer.topk(ref[3], w.top_k)
    assert gi[3].tolist() == o_idx.tolist()


def test_determinism():
    w = make(2, reduced=1)
    d = to_dev(w)
    a = salb.indexer_score_topk(**d, top_k=w.top_k, precision="mfma", with_scores=True)
    b = salb.indexer_score_topk(**d, top_k=w.top_k, precision="mfma", with_scores=True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))


@pytest.mark.parametrize("precision", ["fp32", "mfma"])
def test_edge_valid_lens_and_tables(precision):
    """valid_len in {0, 1, < k, not a multiple of epb, = capacity}; per-row tables; -1 in unread slots;
    a duplicated page (equal scores: the lower index wins)."""
    T, epb, max_lb, k = 6, 64, 40, 100
    w = csa("edges", [77], T=T, H=64, D=128, epb=epb, P=64, max_lb=max_lb, top_k=k,
            valid_lens=np.array([0, 1, 99, 1000, max_lb * epb, 333]), dist="gauss", w_scale=1 / 64, table="per_row")
    bt = w.block_table.copy()
    for t in range(T):
        used = -(-int(w.valid_lens[t]) // epb)
        bt[t, used:] = -1
    bt[5, 3] = bt[5, 1]          # duplicate page inside row 5's valid range (333 > 4*64)
    w.block_table = bt
    d = to_dev(w)
    idx, val = salb.indexer_score_topk(**d, top_k=k, precision=precision, with_scores=True)
    rows = salb.indexer_score_rows(**d, n_cols=max_lb * epb, precision=precision)
    torch.cuda.synchronize()
    gi, gv, gr = _row(idx), _row(val), _row(rows)
    ref, amag = oracle_rows(w)
    for t in range(T):
        check_scores(gr[t], ref[t], amag[t], precision, f"edge t{t}")
        check_topk(gi[t], gv[t], ref[t], amag[t], k, precision, f"edge t{t}")
    assert np.all(gi[0] == -1)
    assert gi[1][0] == 0 and np.all(gi[1][1:] == -1)
    # duplicated page: bit-equal scores at both logical positions
    assert np.array_equal(gr[5, 3 * epb:4 * epb], gr[5, 1 * epb:2 * epb])


def test_epb_not_multiple_of_16():
    w = csa("odd_epb", [78], T=3, H=16, D=64, epb=7, P=50, max_lb=40, top_k=20,
            valid_lens=np.array([280, 45, 7]), dist="tiny", table="per_row")
    d = to_dev(w)
    ref, amag = oracle_rows(w)
    for precision in ("fp32", "mfma"):
        rows = salb.indexer_score_rows(**d, n_cols=280, precision=precision)
        idx, val = salb.indexer_score_topk(**d, top_k=20, precision=precision, with_scores=True)
        gr, gi, gv = _row(rows), _row(idx), _row(val)
        for t in range(3):
            check_scores(gr[t], ref[t], amag[t], precision, f"odd epb t{t} {precision}")
            check_topk(gi[t], gv[t], ref[t], amag[t], 20, precision, f"odd epb t{t} {precision}")


# ------------------------------------------------------------------ select on given scores

@pytest.mark.parametrize("n_cols,k", [(1000, 32), (4096, 512), (70000, 2048), (300000, 2048), (40000, 256)])
def test_topk_select_exact(n_cols, k):
    """Selection alone on fixed fp32 scores is exact: indices equal the oracle's, ties included."""
    rng = np.random.default_rng(n_cols)
    rows = 3
    s = rng.standard_normal((rows, n_cols)).astype(np.float32)
    s[0, ::7] = 1.5                      # heavy ties
    s[1] = np.round(s[1] * 4) / 4         # coarse values: ties at the threshold
    s[2, : n_cols // 2] = 0.0
    s[2, 5] = -0.0
    valid = np.array([n_cols, n_cols - 17, max(0, k - 5)], dtype=np.int32)
    idx, val = salb.indexer_topk_select(torch.from_numpy(s).cuda(), k, valid_lens=torch.from_numpy(valid).cuda(),
                                        with_scores=True)
    gi, gv = _row(idx), _row(val)
    for r in range(rows):
        o_idx, o_val = indexer.topk(s[r, : valid[r]].astype(np.float64), k)
        assert gi[r].tolist() == o_idx.tolist(), r
        kk = min(k, int(valid[r]))
        assert np.array_equal(gv[r][:kk], o_val[:kk].astype(np.float32))


@pytest.mark.parametrize("n_cols,k", [(12000, 256), (30000, 256), (30002, 256), (32768, 2048), (20000, 1), (32768, 512)])
def test_topk_select_many_long_rows(n_cols, k):
    """Many rows (one workgroup per row: 1024 threads with 16 entries each in registers up
    to 16384 columns, 512 threads with 64 each up to 32768; a row of one repeated value
    overflows the candidate list and takes the radix passes over the row): exact against
    the oracle on sampled rows, with ties, empty rows, rows shorter than k, a row of
    k + 1 entries and full rows; set rules on every row."""
    rng = np.random.default_rng(n_cols + 7 * k)
    rows = 300
    s = rng.standard_normal((rows, n_cols)).astype(np.float32)
    s[0, ::7] = 1.5                          # heavy ties
    s[1] = np.round(s[1] * 4) / 4             # coarse values: ties at the threshold
    s[2, :] = 0.25                            # one value everywhere
    s[3, ::3] = -np.inf
    valid = rng.integers(0, n_cols + 1, rows).astype(np.int32)
    valid[:4] = n_cols
    valid[4], valid[5], valid[6], valid[7] = 0, max(0, k - 3), k, k + 1
    idx, val = salb.indexer_topk_select(torch.from_numpy(s).cuda(), k, valid_lens=torch.from_numpy(valid).cuda(),
                                        with_scores=True)
    gi, gv = _row(idx), _row(val)
    for r in list(range(8)) + [rows // 2, rows - 1]:
        o_idx, o_val = indexer.topk(s[r, : valid[r]].astype(np.float64), k)
        assert gi[r].tolist() == o_idx.tolist(), r
        kk = min(k, int(valid[r]))
        assert np.array_equal(gv[r][:kk], o_val[:kk].astype(np.float32)), r
    for r in range(rows):
        kk = min(k, int(valid[r]))
        assert np.all(gi[r, kk:] == -1) and len(set(gi[r, :kk].tolist())) == kk, r
        if kk:   # the k-th value bounds every unselected entry
            sel = np.zeros(int(valid[r]), bool)
            sel[gi[r, :kk]] = True
            assert np.all(s[r, : valid[r]][~sel] <= gv[r, kk - 1]), r


@pytest.mark.parametrize("rows,n_cols,k", [(8, 4096, 512), (300, 12000, 256), (300, 30000, 256), (4, 65536, 2048)])
def test_topk_select_unaligned_rows(rows, n_cols, k):
    """Rows that start 4 bytes past a 16-byte boundary with a stride of n_cols + 3 (the
    scalar-load kernels: short rows, wide rows, register rows, long-row pipeline) select
    exactly what the aligned rows (16-byte loads) select, and match the oracle."""
    rng = np.random.default_rng(rows + n_cols + k)
    s = rng.standard_normal((rows, n_cols)).astype(np.float32)
    s[0, ::5] = 0.75                                    # ties
    valid = rng.integers(k // 2, n_cols + 1, rows).astype(np.int32)
    valid[0] = n_cols
    base = torch.zeros((rows, n_cols + 3), dtype=torch.float32, device="cuda")
    base[:, 1:1 + n_cols] = torch.from_numpy(s).cuda()
    view = base[:, 1:1 + n_cols]
    assert view.data_ptr() % 16 == 4 and view.stride(0) == n_cols + 3
    vl = torch.from_numpy(valid).cuda()
    # the Python binding takes contiguous tensors only: the strided rows go through the C ABI
    from sparse_attention_lightning_block_amd import _lib
    lib = _lib.load()
    ws_bytes = max(int(lib.indexer_topk_workspace_size(rows, n_cols, k)), 256)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    gi_u = torch.empty((rows, k), dtype=torch.int32, device="cuda")
    gv_u = torch.empty((rows, k), dtype=torch.float32, device="cuda")
    _lib.check(lib.indexer_topk_select(view.data_ptr(), view.stride(0), vl.data_ptr(), 0, 0, rows, n_cols, k,
                                       gi_u.data_ptr(), gv_u.data_ptr(), ws.data_ptr(), ws_bytes,
                                       torch.cuda.current_stream().cuda_stream))
    gi_a, gv_a = salb.indexer_topk_select(torch.from_numpy(s).cuda(), k, valid_lens=vl, with_scores=True)
    assert torch.equal(gi_u, gi_a)
    assert torch.equal(gv_u.view(torch.int32), gv_a.view(torch.int32))
    gi = _row(gi_u)
    for r in (0, rows - 1):
        o_idx, _ = indexer.topk(s[r, : valid[r]].astype(np.float64), k)
        assert gi[r].tolist() == o_idx.tolist(), r


def test_topk_select_causal_rule():
    rng = np.random.default_rng(9)
    rows, nb, ratio, first = 5, 64, 16, 900
    s = rng.standard_normal((rows, nb)).astype(np.float32)
    idx, _ = salb.indexer_topk_select(torch.from_numpy(s).cuda(), 10, first_pos=first, ratio=ratio)
    gi = _row(idx)
    for r in range(rows):
        v = min(nb, (first + r + 1) // ratio)
        o_idx, _ = indexer.topk(s[r, :v].astype(np.float64), 10)
        assert gi[r].tolist() == o_idx.tolist()


@pytest.mark.parametrize("n_cols,k", [(5000, 2048), (100000, 2048), (8192, 8192), (20000, 1)])
def test_topk_select_degenerate(n_cols, k):
    """Rows whose winners crowd one score value (sorting-network fallback), rows of
    one repeated value (every entry a candidate), rows of exactly k entries."""
    rng = np.random.default_rng(n_cols + k)
    rows = 4
    s = (rng.standard_normal((rows, n_cols)) * 0.01).astype(np.float32)
    s[0, :] = 0.5                                     # one value everywhere
    big = rng.choice(n_cols, 100, replace=False)
    s[1, rng.choice(n_cols, min(3000, n_cols), replace=False)] = 1.0
    s[1, big] = 1e6                                   # winners: 100 large + many equal ones
    s[3, ::3] = -np.inf
    valid = np.array([n_cols, n_cols, min(k, n_cols), n_cols], dtype=np.int32)
    idx, val = salb.indexer_topk_select(torch.from_numpy(s).cuda(), k, valid_lens=torch.from_numpy(valid).cuda(),
                                        with_scores=True)
    gi, gv = _row(idx), _row(val)
    for r in range(rows):
        o_idx, o_val = indexer.topk(s[r, : valid[r]].astype(np.float64), k)
        assert gi[r].tolist() == o_idx.tolist(), r
        kk = min(k, int(valid[r]))
        assert np.array_equal(gv[r][:kk], o_val[:kk].astype(np.float32)), r


def test_topk_select_workspace_reuse():
    """One workspace, never cleared by the caller, serves consecutive calls of one shape."""
    rows, n_cols, k = 5, 90000, 2048
    ws = torch.full((salb.indexer_topk_workspace_size(rows, n_cols, k),), 0x3C, dtype=torch.uint8, device="cuda")
    for it in range(3):
        rng = np.random.default_rng(500 + it)
        s = rng.standard_normal((rows, n_cols)).astype(np.float32)
        if it == 1:
            s[:, ::5] = 2.0                  # ties at the threshold
        valid = rng.integers(0, n_cols + 1, rows).astype(np.int32)
        valid[0] = n_cols
        idx, val = salb.indexer_topk_select(torch.from_numpy(s).cuda(), k, valid_lens=torch.from_numpy(valid).cuda(),
                                            with_scores=True, workspace=ws)
        gi = _row(idx)
        for r in range(rows):
            o_idx, _ = indexer.topk(s[r, : valid[r]].astype(np.float64), k)
            assert gi[r].tolist() == o_idx.tolist(), (it, r)


GROUP_SHAPES = [
    # T, H, D, epb, table
    (5, 16, 64, 16, "shared"),      # four-row groups, one head tile
    (11, 16, 64, 16, "shared"),     # eight-row groups (ragged), eight-dim staging slices
    (13, 48, 128, 64, "shared"),    # three head tiles
    (16, 64, 256, 32, "shared"),    # four head tiles, widest keys
    (9, 32, 128, 7, "shared"),      # pages not a multiple of 16 keys
    (12, 64, 128, 64, "per_row"),   # rows of different sequences in one group
    (20, 64, 64, 16, "per_row"),
    (256, 16, 64, 16, "shared"),    # the most rows of the balanced split
    (257, 16, 64, 16, "shared"),    # one more: the chunked split
    (40, 32, 128, 1, "shared"),     # one key per page: short balanced segments
]


@pytest.mark.parametrize("T,H,D,epb,table", GROUP_SHAPES)
def test_group_scorer_shapes(T, H, D, epb, table):
    """Rows grouped four or eight to a workgroup, over every key width and head-tile count;
    valid lengths spread so that rows of one group end in different tiles and chunks."""
    max_lb = -(-(3000 if T < 200 else 700) // epb)
    P = max_lb + 8
    w = csa(f"group_{T}_{D}_{epb}_{table}", [91, T, D], T=T, H=H, D=D, epb=epb, P=P, max_lb=max_lb, top_k=64,
            valid_lens=lambda rng, n: rng.integers(0, max_lb * epb + 1, size=n), dist="gauss", w_scale=1 / H,
            table=table)
    d = to_dev(w)
    n_cols = max_lb * epb
    rows = salb.indexer_score_rows(**d, n_cols=n_cols, precision="mfma")
    idx, val = salb.indexer_score_topk(**d, top_k=64, precision="mfma", with_scores=True)
    torch.cuda.synchronize()
    gr, gi, gv = _row(rows), _row(idx), _row(val)
    ref, amag = oracle_rows(w)
    for t in range(T):
        v = int(w.valid_lens[t])
        check_scores(gr[t], ref[t], amag[t], "mfma", f"group shape t{t}")
        assert np.all(np.isneginf(gr[t, v:])), "tail must be -inf"
        check_topk(gi[t], gv[t], ref[t], amag[t], 64, "mfma", f"group shape t{t}")


def test_fused_entry_balanced_split():
    """The fused entry at 40 rows (the balanced split, no -inf tails written): equal to
    indexer_score_rows + indexer_topk_select, and to the oracle within tolerance."""
    T, epb = 40, 64
    max_lb = 50
    w = csa("fused_balanced", [92], T=T, H=64, D=128, epb=epb, P=max_lb + 8, max_lb=max_lb, top_k=256,
            valid_lens=lambda rng, n: rng.integers(0, max_lb * epb + 1, size=n), dist="gauss", w_scale=1 / 64)
    d = to_dev(w)
    a_idx, a_val = salb.indexer_score_topk(**d, top_k=256, precision="mfma", with_scores=True)
    rows = salb.indexer_score_rows(**d, n_cols=max_lb * epb, precision="mfma")
    b_idx, b_val = salb.indexer_topk_select(rows, 256, valid_lens=d["valid_lens"], with_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(a_idx, b_idx) and torch.equal(a_val.view(torch.int32), b_val.view(torch.int32))
    ref, amag = oracle_rows(w)
    gi, gv = _row(a_idx), _row(a_val)
    for t in range(T):
        check_topk(gi[t], gv[t], ref[t], amag[t], 256, "mfma", f"fused balanced t{t}")


# ------------------------------------------------------------------ FP32 path shapes

FP32_SHAPES = [
    # T, H, D, epb, table, q dtype: the FP32 kernel each one reaches
    (5, 16, 64, 16, "shared", "f32"),      # fp32 matrix cores, one head tile, hd 64
    (3, 48, 128, 7, "shared", "bf16"),     # three head tiles, steps crossing pages, bf16 q
    (9, 32, 128, 64, "per_row", "f32"),    # two head tiles, rows on their own pages
    (4, 64, 256, 32, "shared", "f32"),     # hd 256: the vector kernel
    (2, 5, 256, 16, "per_row", "bf16"),    # vector kernel, a partial head group
]


@pytest.mark.parametrize("T,H,D,epb,table,qdt", FP32_SHAPES)
def test_fp32_path_shapes(T, H, D, epb, table, qdt):
    """IDX_PREC_FP32 over the head counts and key widths of both of its kernels (the fp32
    matrix cores at hd 64/128, the vector ALUs at 256), fp32 and bf16 q, shared and
    per-row tables: scores by the FP32 rule and the top-k against the oracle."""
    max_lb = -(-1700 // epb)
    w = csa(f"fp32_{T}_{H}_{D}_{table}", [97, T, H, D], T=T, H=H, D=D, epb=epb, P=max_lb * 2 + 3, max_lb=max_lb,
            top_k=40, valid_lens=lambda rng, n: rng.integers(1, max_lb * epb + 1, size=n), dist="gauss",
            q_dtype=qdt, w_scale=1 / H, table=table)
    d = to_dev(w)
    n_cols = max_lb * epb
    rows = salb.indexer_score_rows(**d, n_cols=n_cols, precision="fp32")
    idx, val = salb.indexer_score_topk(**d, top_k=40, precision="fp32", with_scores=True)
    torch.cuda.synchronize()
    gr, gi, gv = _row(rows), _row(idx), _row(val)
    ref, amag = oracle_rows(w)
    for t in range(T):
        check_scores(gr[t], ref[t], amag[t], "fp32", f"fp32 shape T{T} H{H} D{D} t{t}")
        assert np.all(np.isneginf(gr[t, int(w.valid_lens[t]):]))
        check_topk(gi[t], gv[t], ref[t], amag[t], 40, "fp32", f"fp32 shape T{T} H{H} D{D} t{t}")


# ------------------------------------------------------------------ signs of g and w

SIGN_SHAPES = [
    # T, table, epb: the kernel each one reaches on the MFMA path
    (2, "shared", 64),     # fewer than four rows: the one-row split scorer (page-uniform steps)
    (3, "per_row", 7),     # split scorer, steps crossing pages
    (6, "shared", 64),     # four-row groups, each tile decoded once into LDS
    (6, "per_row", 64),    # four-row groups whose rows read different pages: per-wave streams
    (24, "shared", 64),    # eight-row groups, balanced split
    (24, "per_row", 16),   # eight-row groups, per-wave streams
    (260, "shared", 16),   # more than 256 rows: chunked eight-row groups
]


@pytest.mark.parametrize("precision", ["mfma", "fp32"])
@pytest.mark.parametrize("T,table,epb", SIGN_SHAPES)
def test_negative_gscale_and_weights(T, table, epb, precision):
    """Global scales negative on every third page and head weights negative on some heads
    (the header allows any sign): ReLU acts on g * dot, so the sign of g is folded into
    the decoded code values and |g| applied after the ReLU on the MFMA path.  Every
    kernel shape against the oracle, scores and top-k."""
    if precision == "fp32" and T > 24:
        pytest.skip("the fp32 scorer has one shape; covered by the smaller cases")
    n_keys = 1500 if T < 200 else 400
    max_lb = -(-n_keys // epb)
    w = csa(f"signs_{T}_{table}", [93, T, epb], T=T, H=64, D=128, epb=epb, P=max_lb * 2 + 3, max_lb=max_lb,
            top_k=48, valid_lens=lambda rng, n: rng.integers(1, max_lb * epb + 1, size=n), dist="gauss",
            w_scale=1 / 64, table=table)
    w.key_gscale = w.key_gscale.copy()
    w.key_gscale[::3] *= -1.0
    w.w = w.w.copy()
    w.w[:, 1::5] *= -1.0
    w.w[: T // 2, 0] = -0.5
    d = to_dev(w)
    n_cols = max_lb * epb
    rows = salb.indexer_score_rows(**d, n_cols=n_cols, precision=precision)
    idx, val = salb.indexer_score_topk(**d, top_k=48, precision=precision, with_scores=True)
    torch.cuda.synchronize()
    gr, gi, gv = _row(rows), _row(idx), _row(val)
    ref, amag = oracle_rows(w)
    assert any(np.any(r < 0) for r in ref.values()), "the case must produce negative scores"
    for t in range(T):
        check_scores(gr[t], ref[t], amag[t], precision, f"signs T{T} {table} t{t}")
        assert np.all(np.isneginf(gr[t, int(w.valid_lens[t]):]))
        check_topk(gi[t], gv[t], ref[t], amag[t], 48, precision, f"signs T{T} {table} t{t}")


# ------------------------------------------------------------------ streaming tails

@pytest.mark.parametrize("T,table,epb", [(8, "disjoint", 64), (3, "disjoint", 16), (2, "shared", 7)])
def test_stream_tails(T, table, epb):
    """The streaming scorers run whole eight-step trips and store four 16-key steps at a
    time: valid lengths cover every count of steps modulo eight (and a partial last step)
    for per-wave streams of eight rows on their own pages, and for the one-row split
    scorer (its four waves take every fourth step)."""
    lens = [16 * k + r for k, r in zip(range(T), (1, 16, 15, 7, 16, 3, 9, 16))]
    if T < 4:
        lens = [1000, 61, 16][:T]
    max_lb = -(-max(lens) // epb) + 1
    w = csa(f"tails_{T}_{epb}", [94, T, epb], T=T, H=64, D=128, epb=epb, P=max_lb * T + 3, max_lb=max_lb,
            top_k=8, valid_lens=np.array(lens), dist="gauss", w_scale=1 / 64, table=table)
    d = to_dev(w)
    n_cols = max_lb * epb
    rows = salb.indexer_score_rows(**d, n_cols=n_cols, precision="mfma")
    torch.cuda.synchronize()
    gr = _row(rows)
    ref, amag = oracle_rows(w)
    for t in range(T):
        check_scores(gr[t], ref[t], amag[t], "mfma", f"tails T{T} t{t}")
        assert np.all(np.isneginf(gr[t, lens[t]:])), t


# ------------------------------------------------------------------ IDX_F_VALIDATE

def test_validate_accepts_in_range_data():
    w = make(2, reduced=1)
    d = to_dev(w)
    a_idx, a_val = salb.indexer_score_topk(**d, top_k=w.top_k, precision="mfma", with_scores=True, validate=True)
    b_idx, b_val = salb.indexer_score_topk(**d, top_k=w.top_k, precision="mfma", with_scores=True)
    assert torch.equal(a_idx, b_idx) and torch.equal(a_val.view(torch.int32), b_val.view(torch.int32))
    n_cols = w.max_lb * w.epb
    a = salb.indexer_score_rows(**d, n_cols=n_cols, precision="mfma", validate=True)
    b = salb.indexer_score_rows(**d, n_cols=n_cols, precision="mfma")
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_validate_rejects_bad_metadata_before_scoring():
    """A page id outside the pool inside a row's valid range, or a valid length past the
    table: IDX_ERR_DATA names it and nothing else is launched (the outputs keep their
    contents).  Only the check kernel runs on such data, and it reads valid_lens and the
    block table alone."""
    w = make(2, reduced=1)
    d = to_dev(w)
    bt = d["block_table"].clone()
    bt[1, 5] = w.P            # row 1 reads logical block 5 (valid 2000 > 5 * 64)
    idx = torch.full((w.T, w.top_k), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(salb.IndexerError) as e:
        salb.indexer_score_topk(**dict(d, block_table=bt), top_k=w.top_k, precision="mfma", validate=True,
                                out_idx=idx)
    assert e.value.code == salb.IDX_ERR_DATA and "block_table[1][5]" in str(e.value)
    assert torch.all(idx == -7)
    vl = d["valid_lens"].clone()
    vl[2] = w.max_lb * w.epb + 1
    with pytest.raises(salb.IndexerError) as e:
        salb.indexer_score_topk(**dict(d, valid_lens=vl), top_k=w.top_k, precision="mfma", validate=True,
                                out_idx=idx)
    assert e.value.code == salb.IDX_ERR_DATA and "valid_lens[2]" in str(e.value)
    assert torch.all(idx == -7)
    # the split entry: its scores buffer only carries the check's status word
    n_cols = w.max_lb * w.epb
    out = torch.full((w.T, n_cols), 2.5, dtype=torch.float32, device="cuda")
    with pytest.raises(salb.IndexerError) as e:
        salb.indexer_score_rows(**dict(d, block_table=bt), n_cols=n_cols, precision="mfma", validate=True, out=out)
    assert e.value.code == salb.IDX_ERR_DATA
    assert torch.all(out.view(-1)[4:] == 2.5)
    # entries past a row's valid keys are never read, so -1 there is accepted
    bt2 = d["block_table"].clone()
    for t in range(w.T):
        bt2[t, -(-int(w.valid_lens[t]) // w.epb):] = -1
    a_idx, _ = salb.indexer_score_topk(**dict(d, block_table=bt2), top_k=w.top_k, precision="mfma", validate=True)
    b_idx, _ = salb.indexer_score_topk(**d, top_k=w.top_k, precision="mfma")
    assert torch.equal(a_idx, b_idx)


# ------------------------------------------------------------------ workspace as scratch

def test_one_workspace_serves_every_shape():
    """One workspace, filled with garbage first, serves selects and fused calls of
    different shapes in turn (each call initialises what it reads): every result equals
    the oracle's (selects on fixed scores are exact) or a fresh-workspace call's."""
    shapes = [(5, 90000, 2048), (3, 300000, 1024), (9, 20000, 512), (5, 90000, 2048), (40, 12000, 64)]
    need = max(salb.indexer_topk_workspace_size(r, n, k) for r, n, k in shapes)
    w2 = make(2, reduced=1)
    w3 = make(3, reduced=1)
    need = max(need, *(salb.indexer_score_topk_workspace_size(w.T, w.max_lb, w.epb, w.top_k) for w in (w2, w3)))
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    fused_ref = {}
    for w in (w2, w3):
        fused_ref[w.name] = salb.indexer_score_topk(**to_dev(w), top_k=w.top_k, precision="mfma")[0]
    for it, (rows, n_cols, k) in enumerate(shapes):
        rng = np.random.default_rng(700 + it)
        s = rng.standard_normal((rows, n_cols)).astype(np.float32)
        s[0, ::5] = 2.0                          # ties at the threshold
        valid = rng.integers(0, n_cols + 1, rows).astype(np.int32)
        valid[0] = n_cols
        idx, _ = salb.indexer_topk_select(torch.from_numpy(s).cuda(), k, valid_lens=torch.from_numpy(valid).cuda(),
                                          workspace=ws)
        gi = _row(idx)
        for r in range(rows):
            o_idx, _ = indexer.topk(s[r, : valid[r]].astype(np.float64), k)
            assert gi[r].tolist() == o_idx.tolist(), (it, r)
        w = (w2, w3)[it % 2]
        got = salb.indexer_score_topk(**to_dev(w), top_k=w.top_k, precision="mfma", workspace=ws)[0]
        assert torch.equal(got, fused_ref[w.name]), (it, w.name)


def test_nan_scores_rank_last_on_both_selects():
    """A NaN global scale makes every score of that page NaN.  The fused entry and the
    split entries must both rank NaN below every number: bit-equal indices and scores
    (NaN reported as the canonical quiet NaN), and no NaN entry selected while enough
    numbers remain."""
    w = make(3, reduced=1)
    w.key_gscale = w.key_gscale.copy()
    page = int(w.block_table[0, 3])
    w.key_gscale[page] = np.nan
    d = to_dev(w)
    a_idx, a_val = salb.indexer_score_topk(**d, top_k=w.top_k, precision="mfma", with_scores=True)
    rows = salb.indexer_score_rows(**d, n_cols=w.max_lb * w.epb, precision="mfma")
    b_idx, b_val = salb.indexer_topk_select(rows, w.top_k, valid_lens=d["valid_lens"], with_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(a_idx, b_idx)
    assert torch.equal(a_val.view(torch.int32), b_val.view(torch.int32))
    gi = _row(a_idx)
    nan_entries = set(range(3 * w.epb, 4 * w.epb))
    for t in range(w.T):
        v = int(w.valid_lens[t])
        if v - w.epb >= w.top_k:     # enough finite scores: none of the NaN page is chosen
            assert not (set(gi[t].tolist()) & nan_entries), t
    ref, amag = oracle_rows(w)
    for t in range(w.T):
        fin = np.isfinite(ref[t])
        assert np.isnan(ref[t][~fin]).all()
