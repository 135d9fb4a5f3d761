"""GPU parity of the dynamic MLP routing and the merge (through the C ABI).

- sparsesam_route_topk: the keep-set of arbitrary fp32 scores (with forced ties, -0.0,
  NaN, window pads) is bit-exact against the oracle's top_k_by_score.
- sparsesam_block_dynamic: the block's scores match the oracle's within the bf16 branch
  bar; its keep-set is exactly the selection of its own scores; under the oracle's
  scores it is a valid top-K up to the score error (any swap is explained by it); and
  the block output matches the oracle block run with that keep-set at the contract bar.
- mlp_merge plans (static and dynamic routing): block output against the oracle.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import structured_sparse_vit_amd as ss
from tests.gpu_cases import check_close, config, images, oracle_importance, rel_l2

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SCORE_REL = {"bf16": 1.5e-2, "f32": 1e-4}


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _oracle_topk(cfg, score):
    """The keep-set of every segment by score, in the library's layout."""
    tm = oracle.segments_for_image(cfg.grid, cfg.grid, cfg.window)
    tokens = cfg.grid * cfg.grid
    out = []
    for b in range(score.shape[0]):
        for row in tm:
            valid = row >= 0
            k = oracle.routed_count(cfg.mlp_density, int(valid.sum()))
            s = np.where(valid, score[b][np.maximum(row, 0)], np.float32(0.0)).astype(np.float32)
            out.append(row[oracle.top_k_by_score(s, valid, k)] + b * tokens)
    return np.concatenate(out)


@pytest.mark.parametrize("key", ["c1", "c2", "c3", "ragged"])
def test_route_topk_bit_exact(key):
    _say("route_topk", key)
    cfg = config(key).with_(batch=3)
    plan = ss.Plan.from_config(cfg)
    rng = np.random.default_rng(11)
    t = cfg.grid * cfg.grid
    score = np.stack([
        rng.uniform(size=t).astype(np.float32),
        (rng.integers(0, 3, t) * 0.5).astype(np.float32),   # many ties
        rng.exponential(size=t).astype(np.float32),
    ])
    score[1, ::7] = -0.0
    score[2, ::53] = np.nan
    got = ss.route_topk(plan, torch.from_numpy(score).to(DEV)).cpu().numpy()
    assert np.array_equal(got, _oracle_topk(cfg, score))


def _dynamic_case(key, merge=False, seed=0):
    from synth import block_weights, token_features
    cfg = config(key).with_(routing="update", mlp_merge=merge)
    plan = ss.Plan.from_config(cfg)
    x = token_features(cfg, seed)
    w = block_weights(cfg, seed)
    img = torch.from_numpy(images(key, seed)).to(DEV)
    imp_d = ss.importance(img, cfg.patch)
    perm, _, _ = ss.permute(plan, imp_d)
    xd = torch.from_numpy(x.copy()).to(DEV)
    _, routed, score = ss.block_dynamic(plan, ss.weights_to_device(w, plan), xd, perm)
    torch.cuda.synchronize()
    return cfg, x, w, oracle_importance(key, seed), xd.cpu().numpy(), routed.cpu().numpy(), score.cpu().numpy()


@pytest.mark.parametrize("key,merge", [("c1", False), ("c2", False), ("c3b1", False), ("ragged", False),
                                       ("c2", True), ("c3b1", True), ("ragged", True)])
def test_block_dynamic_parity(key, merge):
    _say("block_dynamic", key, "merge", merge)
    cfg, x, w, imp, got, routed, score = _dynamic_case(key, merge)
    # the keep-set is exactly the selection of the block's own scores
    assert np.array_equal(routed, _oracle_topk(cfg, score))
    # scores against the oracle's fp64 ones
    want, parts = oracle.block_forward(x, imp, w, cfg, return_parts=True)
    ref_score = np.stack(parts["score"])
    srel = rel_l2(score, ref_score)
    assert srel <= SCORE_REL[cfg.dtype], "score rel-L2 %.3e" % srel
    # under the oracle's scores the chosen set is a valid top-K up to the score error
    tm = oracle.segments_for_image(cfg.grid, cfg.grid, cfg.window)
    tokens = cfg.grid * cfg.grid
    chosen = set(routed.tolist())
    swaps = 0
    for b in range(cfg.batch):
        for row in tm:
            toks = row[row >= 0]
            rows = toks + b * tokens
            ins = np.array([r in chosen for r in rows])
            so, sg = ref_score[b][toks], score[b][toks]
            margin = 2.0 * float(np.abs(sg - so).max())
            if ins.all() or not ins.any():
                continue
            assert so[ins].min() >= so[~ins].max() - margin, "keep-set not a top-K under the oracle's scores"
            want_set = set((toks[oracle.top_k_by_score(so, np.ones(toks.size, bool), int(ins.sum()))]).tolist())
            swaps += len(want_set ^ set(toks[ins].tolist())) // 2
    _say("  score rel-L2 %.3e, keep-set swaps against the oracle's own choice: %d of %d" % (srel, swaps, routed.size))
    # the block, with the GPU's keep-set
    per_img = [routed[b * (routed.size // cfg.batch):(b + 1) * (routed.size // cfg.batch)] - b * tokens
               for b in range(cfg.batch)]
    want = oracle.block_forward(x, imp, w, cfg, routed_override=per_img)
    mx, rel = check_close(got, want, what="dynamic block " + key)
    _say("  block max-abs %.3e rel-L2 %.3e" % (mx, rel))


@pytest.mark.parametrize("key", ["c1", "c2", "c3b1", "ragged"])
def test_block_merge_parity(key):
    """Static routing with the merge: the segment's other tokens get the keep-set's mean update."""
    from synth import block_weights, token_features
    _say("block merge", key)
    cfg = config(key).with_(mlp_merge=True)
    plan = ss.Plan.from_config(cfg)
    x = token_features(cfg)
    w = block_weights(cfg)
    imp_d = ss.importance(torch.from_numpy(images(key)).to(DEV), cfg.patch)
    perm, _, routed = ss.permute(plan, imp_d)
    xd = torch.from_numpy(x.copy()).to(DEV)
    ss.block(plan, ss.weights_to_device(w, plan), xd, perm, routed)
    got = xd.cpu().numpy()
    want = oracle.block_forward(x, oracle_importance(key), w, cfg)
    mx, rel = check_close(got, want, what="merge block " + key)
    plain = oracle.block_forward(x, oracle_importance(key), w, cfg.with_(mlp_merge=False))
    assert rel_l2(got, plain) > 10 * rel, "the merge must change the result here"
    _say("  merge block max-abs %.3e rel-L2 %.3e" % (mx, rel))


def test_plan_kind_checks():
    cfg = config("c1")
    dyn = ss.Plan.from_config(cfg.with_(routing="update"))
    sta = ss.Plan.from_config(cfg)
    from synth import block_weights
    w = ss.weights_to_device(block_weights(cfg), sta)
    x = torch.zeros(1, 16, 16, 64, device=DEV)
    perm = torch.zeros(1, 256, dtype=torch.int32, device=DEV)
    routed = torch.zeros(dyn.info["routed_per_image"], dtype=torch.int32, device=DEV)
    with pytest.raises(ss.SparseSAMError) as e:
        ss.block(dyn, w, x, perm, routed)
    assert e.value.status == 1
    with pytest.raises(ValueError):
        ss.block_dynamic(sta, w, x, perm)
    merge = ss.Plan.from_config(cfg.with_(mlp_merge=True))
    with pytest.raises(ss.SparseSAMError) as e:
        ss.mlp(merge, x.view(-1, 64), routed, w["ln2_g"], w["ln2_b"], w["w1"], w["b1"], w["w2"], w["b2"])
    assert e.value.status == 2
    assert torch.count_nonzero(x) == 0
