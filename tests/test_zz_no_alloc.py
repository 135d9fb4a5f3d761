"""sparsesam_block_noalloc (the block entry point that allocates nothing, for callers
that cannot allocate) against sparsesam_block, through the C ABI.

Both run the same kernels in the same order, so the outputs must be bitwise equal.
Two calls in a row share the library's per-GPU scratch; the second takes a smaller
batch than the first, so it runs on scratch that still holds the first call's data.
"""
import sys

import numpy as np
import pytest
import torch

import structured_sparse_vit_amd as ss
from synth import block_weights, synthetic_images, token_features
from tests.gpu_cases import config

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _inputs(cfg, batch, seed):
    c = cfg.with_(batch=batch)
    img = torch.from_numpy(synthetic_images(c, seed)).to(DEV)
    x = torch.from_numpy(token_features(c, seed)).to(DEV)
    return img, x


@pytest.mark.parametrize("key", ["c2", "ragged"])
def test_block_noalloc_matches_block_twice_shrinking(key):
    cfg = config(key)
    plan = ss.Plan.from_config(cfg, max_batch=2)
    wd = ss.weights_to_device(block_weights(cfg, 0), plan)
    for call, (batch, seed) in enumerate(((2, 0), (1, 1))):  # second call: smaller input
        _say("block_noalloc", key, "call", call, "batch", batch)
        img, x = _inputs(cfg, batch, seed)
        imp = ss.importance(img, cfg.patch)
        perm, _, routed = ss.permute(plan, imp)
        want = x.clone()
        ss.block(plan, wd, want, perm, routed)
        got = x.clone()
        ss.block_noalloc(plan, wd, got, perm, routed)
        torch.cuda.synchronize()
        g, w = got.cpu().numpy(), want.cpu().numpy()
        assert np.isfinite(g).all()
        assert np.array_equal(g.view(np.uint32), w.view(np.uint32)), "call %d differs from sparsesam_block" % call
        assert not np.array_equal(g, x.cpu().numpy())


def test_block_noalloc_rejects_work_beyond_its_scratch():
    """The windowed ViT-B block at batch 4 needs about 150 MB of workspace: more than the
    fixed scratch, so the call fails before any launch and x is untouched."""
    _say("block_noalloc too large")
    cfg = config("c3")
    plan = ss.Plan.from_config(cfg)
    assert plan.info["block_workspace_bytes"] > ss.noalloc_scratch_bytes()
    wd = ss.weights_to_device(block_weights(cfg, 0), plan)
    img, x = _inputs(cfg, cfg.batch, 0)
    perm, _, routed = ss.permute(plan, ss.importance(img, cfg.patch))
    x0 = x.clone()
    with pytest.raises(ss.SparseSAMError) as e:
        ss.block_noalloc(plan, wd, x, perm, routed)
    assert e.value.status == 3  # SPARSESAM_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.equal(x, x0)
