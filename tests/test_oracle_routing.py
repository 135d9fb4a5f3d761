"""Pins for the oracle's dynamic MLP routing and residual correction (fp64).

- top_k_by_score: numpy's stable argsort on distinct scores, hand-worked ties (lower
  slot first), invalid slots last, k = all valid slots.
- update_score: a single moved token gives exactly its squared shift.
- the block with routing "update" equals an independent torch block: x1 from torch's
  masked SDPA (the pinned pattern per segment), the keep-set as the K largest
  ||x1 - x||^2 per segment by numpy's stable argsort, the MLP on those rows.
- merging: with fc2 = 0 and bias c every keep-set update is c, so every real token
  ends at x1 + c (closed form); a brute-force per-segment mean on a windowed block.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import (block_forward, importance, routed_count, segments_for_image, top_k_by_score, update_score)
from synth import block_weights, get_config, synthetic_images, token_features
from tests.test_oracle_encoder import _segment_parts, _t


def test_top_k_by_score_is_stable_argsort_on_distinct_scores():
    rng = np.random.default_rng(0)
    s = rng.uniform(size=500).astype(np.float32)
    for k in (1, 7, 200, 500):
        assert np.array_equal(top_k_by_score(s, np.ones(500, bool), k), np.argsort(-s, kind="stable")[:k])


def test_top_k_by_score_ties_invalid_and_full():
    s = np.array([1.0, 3.0, 3.0, 0.0, 3.0, 2.0])
    assert top_k_by_score(s, np.ones(6, bool), 2).tolist() == [1, 2]        # ties: lower slot first
    assert top_k_by_score(s, np.ones(6, bool), 4).tolist() == [1, 2, 4, 5]
    valid = np.array([True, True, False, True, False, True])
    assert top_k_by_score(s, valid, 3).tolist() == [1, 5, 0]                # invalid slots never chosen
    assert sorted(top_k_by_score(s, valid, 4).tolist()) == [0, 1, 3, 5]     # k = all valid slots
    # scores that differ only below fp32 resolution tie (ranked in fp32)
    t = np.array([1.0, 1.0 + 1e-12, 0.5])
    assert top_k_by_score(t, np.ones(3, bool), 1).tolist() == [0]


def test_update_score_single_moved_token():
    rng = np.random.default_rng(1)
    x = rng.normal(size=(10, 8))
    x1 = x.copy()
    x1[3, 5] += 0.25
    x1[7] += np.array([3.0, 4.0] + [0.0] * 6)
    sc = update_score(x, x1)
    assert sc[3] == 0.0625 and sc[7] == 25.0
    assert np.count_nonzero(sc) == 2


def _torch_dynamic_block(x, imp, w, cfg):
    """Independent torch fp64 block with dynamic routing (and merging when cfg says so)."""
    b, gh, gw, C = x.shape
    H = cfg.heads
    D = C // H
    out = np.empty((b, gh, gw, C))
    for i in range(b):
        xi = _t(x[i].reshape(gh * gw, C))
        h = F.layer_norm(xi, (C,), _t(w["ln1_g"]), _t(w["ln1_b"]), eps=1e-6)
        attn = torch.zeros_like(xi)
        segs = _segment_parts(imp[i], cfg, gh, gw)
        for row, mask, _ in segs:
            real = torch.from_numpy(row >= 0)
            idx = torch.from_numpy(np.maximum(row, 0))
            hs = torch.where(real[:, None], h[idx], torch.zeros(()))
            qkv = F.linear(hs, _t(w["w_qkv"]), _t(w["b_qkv"]))
            q, k, v = qkv.view(-1, 3, H, D).permute(1, 2, 0, 3)
            o = F.scaled_dot_product_attention(q, k, v, attn_mask=torch.from_numpy(mask)[None])
            attn[idx[real]] = o.transpose(0, 1).reshape(-1, C)[real]
        x1 = xi + F.linear(attn, _t(w["w_proj"]), _t(w["b_proj"]))
        score = ((x1 - xi) ** 2).sum(-1).numpy().astype(np.float32)
        h2 = F.layer_norm(x1, (C,), _t(w["ln2_g"]), _t(w["ln2_b"]), eps=1e-6)
        y = F.linear(F.gelu(F.linear(h2, _t(w["w1"]), _t(w["b1"]))), _t(w["w2"]), _t(w["b2"]))
        x2 = x1.clone()
        for row, _, _ in segs:
            toks = row[row >= 0]
            k = routed_count(cfg.mlp_density, toks.size)
            keep = toks[np.argsort(-score[toks], kind="stable")[:k]]
            rest = np.setdiff1d(toks, keep)
            kt, rt = torch.from_numpy(keep), torch.from_numpy(rest)
            x2[kt] = x1[kt] + y[kt]
            if cfg.mlp_merge and rest.size:
                x2[rt] = x1[rt] + y[kt].mean(0)
        out[i] = x2.view(gh, gw, C).numpy()
    return out


def _small(key, **over):
    cfg = get_config(key)
    if key == "c3":
        cfg = cfg.with_(batch=1, channels=64, heads=2, head_dim=32, mlp_hidden=128, image=288)  # 18 x 18, 4 windows
    cfg = cfg.with_(**over)
    imgs = synthetic_images(cfg)
    imp = np.stack([importance(im, cfg.patch) for im in imgs])
    return cfg, imp, token_features(cfg), block_weights(cfg)


@pytest.mark.parametrize("key", ["c1", "c3"])
@pytest.mark.parametrize("merge", [False, True])
def test_dynamic_block_is_torch_dynamic_block(key, merge):
    cfg, imp, x, w = _small(key, routing="update", mlp_merge=merge)
    got, parts = block_forward(x, imp, w, cfg, return_parts=True)
    want = _torch_dynamic_block(x, imp, w, cfg)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-10)
    # the dynamic keep-set differs from the importance one here
    static = block_forward(x, imp, w, cfg.with_(routing="importance"), return_parts=True)[1]
    assert not np.array_equal(parts["routed"][0], static["routed"][0])


def test_dynamic_routing_at_full_mlp_density_is_static():
    cfg, imp, x, w = _small("c1", mlp_density=1.0)
    a = block_forward(x, imp, w, cfg.with_(routing="update"))
    b = block_forward(x, imp, w, cfg)
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("key", ["c1", "c3"])
def test_merge_with_constant_updates_moves_every_real_token_by_the_constant(key):
    cfg, imp, x, w = _small(key)
    w = dict(w)
    w["w2"] = np.zeros_like(w["w2"])
    c = np.linspace(-0.5, 0.5, w["b2"].size).astype(np.float32)
    w["b2"] = c
    plain, parts = block_forward(x, imp, w, cfg, return_parts=True)
    merged = block_forward(x, imp, w, cfg.with_(mlp_merge=True))
    C = x.shape[-1]
    routed = parts["routed"][0]
    d = (merged - plain).reshape(-1, C)
    other = np.setdiff1d(np.arange(d.shape[0]), routed)
    np.testing.assert_array_equal(d[routed], 0.0)                       # keep-set unchanged by merging
    np.testing.assert_allclose(d[other], np.tile(c, (other.size, 1)), rtol=0, atol=1e-12)


def test_merge_brute_force_per_window_mean():
    cfg, imp, x, w = _small("c3")
    plain, parts = block_forward(x, imp, w, cfg, return_parts=True)
    merged = block_forward(x, imp, w, cfg.with_(mlp_merge=True))
    # x1 (the block input plus its attention update) is the block with fc2 = 0, b2 = 0
    w0 = dict(w)
    w0["w2"], w0["b2"] = np.zeros_like(w["w2"]), np.zeros_like(w["b2"])
    C = x.shape[-1]
    x1 = block_forward(x, imp, w0, cfg).reshape(-1, C)
    p, m = plain.reshape(-1, C), merged.reshape(-1, C)
    routed = set(parts["routed"][0].tolist())
    for row in segments_for_image(cfg.grid, cfg.grid, cfg.window):
        toks = [t for t in row.tolist() if t >= 0]
        kept = [t for t in toks if t in routed]
        rest = [t for t in toks if t not in routed]
        mean = [sum(p[t, c] - x1[t, c] for t in kept) / len(kept) for c in range(C)]
        for t in rest:
            np.testing.assert_allclose(m[t], [x1[t, c] + mean[c] for c in range(C)], rtol=0, atol=1e-12)
        for t in kept:
            np.testing.assert_array_equal(m[t], p[t])
