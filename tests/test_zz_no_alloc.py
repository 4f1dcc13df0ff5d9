"""indexer_score_topk_noalloc (the library's own per-GPU scratch instead of a workspace)
against indexer_score_topk with a caller workspace: bit-identical indices and scores on
two calls in a row, the second smaller than the first, and a call too large for the
scratch rejected before any launch.  Needs an MI355X."""

import numpy as np
import pytest
import torch

import sparse_attention_lightning_block_amd as salb
from sparse_attention_lightning_block_amd import _lib
from workloads import make
from workloads.device import to_dev

pytestmark = pytest.mark.gpu


def _both(w):
    d = to_dev(w)
    ref_i, ref_v = salb.indexer_score_topk(**d, top_k=w.top_k, precision="mfma", with_scores=True)
    got_i, got_v = salb.indexer_score_topk_noalloc(**d, top_k=w.top_k, precision="mfma", with_scores=True)
    torch.cuda.synchronize()
    return ref_i, ref_v, got_i, got_v


def test_noalloc_matches_workspace_entry_twice_shrinking():
    # long-context decode (100 MiB of scratch), then the decode configuration (7 MiB)
    for cfg in (3, 2):
        w = make(cfg)
        ref_i, ref_v, got_i, got_v = _both(w)
        assert torch.equal(got_i, ref_i), cfg
        assert torch.equal(got_v.view(torch.int32), ref_v.view(torch.int32)), cfg
        K = np.minimum(w.top_k, w.valid_lens)
        gi = got_i.cpu().numpy()
        for t in range(w.T):
            assert np.all(gi[t, K[t]:] == -1) and len(set(gi[t, :K[t]].tolist())) == K[t]


def test_noalloc_rejects_a_call_larger_than_its_scratch():
    lib = _lib.load()
    need = lib.indexer_score_topk_workspace_size(64, 4096, 64, 2048)
    assert need > _lib.IDX_NOALLOC_SCRATCH_BYTES
    w = make(2, reduced=1)
    d = to_dev(w)
    idx = torch.full((64, 2048), -9, dtype=torch.int32, device="cuda")
    # the size rule is checked on the host before anything else: nothing is read or launched
    rc = lib.indexer_score_topk_noalloc(d["q"].data_ptr(), 0, d["w"].data_ptr(), d["keys_fp4"].data_ptr(),
                                        d["key_scale"].data_ptr(), d["key_gscale"].data_ptr(),
                                        d["block_table"].data_ptr(), 4096, d["valid_lens"].data_ptr(), 64, 64, 128,
                                        64, 4096, 8192, 2048, 1, 0, idx.data_ptr(), None, None)
    assert rc == _lib.IDX_ERR_WORKSPACE
    assert b"no-alloc" in lib.indexer_last_error()
    torch.cuda.synchronize()
    assert torch.all(idx == -9)
