"""Pins for the oracle's encoder (a stack of global and windowed blocks, fp64).

The encoder is pinned against an independent torch fp64 statement of SAM's
encoder layout: pre-LN blocks, global attention at the given layers, zero-padded
14 x 14 windows (SAM's window partition) elsewhere.
- At density 1 every block is dense, so the oracle encoder must equal the dense
  torch encoder (torch SDPA, F.layer_norm, F.linear, F.gelu).
- At density < 1 the torch encoder applies the pattern as a boolean SDPA mask per
  segment and the MLP as a row mask; the mask and keep-set come from the pinned
  pattern and order functions, once per block type and image (one permutation set
  per type, reused by every layer of that type).
- The layer placement matters: moving the global layer changes the result.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import (band_radius, encoder_forward, importance, routed_tokens, segment_order, segments_for_image,
                    stripe_sort, token_mask)
from synth import block_weights, get_config, synthetic_images, token_features
from synth.configs import global_variant, window_variant


def _t(a):
    return torch.from_numpy(np.asarray(a, np.float64))


def _cfgs(density, batch=2):
    # 16 x 16 grid: one global segment of 256 tokens, or four 14 x 14 windows over the
    # grid padded to 28 x 28 (one full window, three partial)
    base = get_config("c4").with_(batch=batch, image=256, channels=64, heads=2, head_dim=32, mlp_hidden=128,
                                  attn_density=density, mlp_density=density, layers=3)
    return base, global_variant(base).with_(block=16, global_tokens=16), window_variant(base)


def _segment_parts(imp_img, cfg, gh, gw):
    """Per segment of one image: its token map row, pattern mask in token order and
    keep-set (image token ids), from the pinned order / stripe-sort / pattern functions."""
    tmap = segments_for_image(gh, gw, cfg.window)
    n = tmap.shape[1]
    r = band_radius(n, cfg.stripes, cfg.block, cfg.global_tokens, cfg.attn_density)
    side_h, side_w = (gh, gw) if cfg.window == 0 else (cfg.window, cfg.window)
    out = []
    for row in tmap:
        s = segment_order("importance", imp_img, row, side_h, side_w)
        _, inv = stripe_sort(s, cfg.stripes)
        out.append((row, token_mask(inv, cfg.stripes, cfg.block, cfg.global_tokens, r),
                    routed_tokens(s, row, cfg.mlp_density)))
    return out


def _torch_block(x, w, cfg, parts):
    """One pre-LN block in torch fp64 on x [b, gh, gw, C]; parts[i] = the segments of image i."""
    b, gh, gw, C = x.shape
    H = cfg.heads
    D = C // H
    out = x.clone()
    for i in range(b):
        xi = x[i].reshape(gh * gw, C)
        h = F.layer_norm(xi, (C,), _t(w["ln1_g"]), _t(w["ln1_b"]), eps=1e-6)
        attn = torch.zeros_like(xi)
        keep = torch.zeros(gh * gw, dtype=torch.bool)
        for row, mask, routed in parts[i]:
            real = torch.from_numpy(row >= 0)
            idx = torch.from_numpy(np.maximum(row, 0))
            hs = torch.where(real[:, None], h[idx], torch.zeros(()))   # zero-padded window
            qkv = F.linear(hs, _t(w["w_qkv"]), _t(w["b_qkv"]))
            q, k, v = qkv.view(-1, 3, H, D).permute(1, 2, 0, 3)
            o = F.scaled_dot_product_attention(q, k, v, attn_mask=torch.from_numpy(mask)[None])
            o = o.transpose(0, 1).reshape(-1, C)
            attn[idx[real]] = o[real]
            keep[torch.from_numpy(routed)] = True
        x1 = xi + F.linear(attn, _t(w["w_proj"]), _t(w["b_proj"]))
        h2 = F.layer_norm(x1, (C,), _t(w["ln2_g"]), _t(w["ln2_b"]), eps=1e-6)
        y = F.linear(F.gelu(F.linear(h2, _t(w["w1"]), _t(w["b1"]))), _t(w["w2"]), _t(w["b2"]))
        out[i] = torch.where(keep[:, None], x1 + y, x1).view(gh, gw, C)
    return out


def _torch_encoder(x, imp, ws, global_layers, cg, cw):
    b, gh, gw, _ = x.shape
    # one permutation set per block type and image, reused by every layer of that type
    pg = [_segment_parts(imp[i], cg, gh, gw) for i in range(b)]
    pw = [_segment_parts(imp[i], cw, gh, gw) for i in range(b)]
    h = _t(x)
    for l, w in enumerate(ws):
        g = l in global_layers
        h = _torch_block(h, w, cg if g else cw, pg if g else pw)
    return h.numpy()


def _inputs(base):
    imgs = synthetic_images(base)
    imp = np.stack([importance(im, base.patch) for im in imgs])
    x = token_features(base)
    ws = [block_weights(base, 0, layer=l) for l in range(base.layers)]
    return imp, x, ws


@pytest.mark.parametrize("global_layers", [[1], [0, 2]])
def test_encoder_at_density_one_is_dense_torch_encoder(global_layers):
    base, cg, cw = _cfgs(1.0)
    imp, x, ws = _inputs(base)
    got = encoder_forward(x, imp, ws, global_layers, cg, cw)
    b, gh, gw, C = x.shape
    # fully dense: no mask at all, every row through the MLP
    ones_g = [[(np.arange(gh * gw), np.ones((gh * gw, gh * gw), bool), np.arange(gh * gw))] for _ in range(b)]
    tm = segments_for_image(gh, gw, 14)
    ones_w = [[(row, np.ones((row.size, row.size), bool), row[row >= 0]) for row in tm] for _ in range(b)]
    h = _t(x)
    for l, w in enumerate(ws):
        g = l in global_layers
        h = _torch_block(h, w, cg if g else cw, ones_g if g else ones_w)
    np.testing.assert_allclose(got, h.numpy(), rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("density", [0.4, 0.3])
def test_sparse_encoder_is_masked_torch_encoder(density):
    base, cg, cw = _cfgs(density)
    imp, x, ws = _inputs(base)
    got = encoder_forward(x, imp, ws, [1], cg, cw)
    want = _torch_encoder(x, imp, ws, [1], cg, cw)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-10)
    # sparse really differs from dense here
    dense = encoder_forward(x, imp, ws, [1], cg.with_(attn_density=1.0, mlp_density=1.0),
                            cw.with_(attn_density=1.0, mlp_density=1.0))
    assert np.abs(got - dense).max() > 1e-3


def test_encoder_layer_placement_matters():
    base, cg, cw = _cfgs(0.4, batch=1)
    imp, x, ws = _inputs(base)
    a = encoder_forward(x, imp, ws, [1], cg, cw)
    b = encoder_forward(x, imp, ws, [2], cg, cw)
    assert np.abs(a - b).max() > 1e-3
    np.testing.assert_allclose(b, _torch_encoder(x, imp, ws, [2], cg, cw), rtol=1e-10, atol=1e-10)


def test_encoder_of_zero_layers_is_identity_and_one_layer_is_a_block():
    from oracle import block_forward
    base, cg, cw = _cfgs(0.4, batch=1)
    imp, x, ws = _inputs(base)
    np.testing.assert_array_equal(encoder_forward(x, imp, [], [], cg, cw), x.astype(np.float64))
    np.testing.assert_allclose(encoder_forward(x, imp, ws[:1], [], cg, cw), block_forward(x, imp, ws[0], cw),
                               rtol=0, atol=0)
