"""Pins for the oracle's attention, routed MLP and whole block (fp64)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import (block_forward, descending_order, gelu, importance, layer_norm, masked_attention,
                    position_keep, routed_mlp, stripe_sort, token_mask, window_token_map)
from synth import block_weights, get_config, synthetic_images, token_features


def _t(a):
    return torch.from_numpy(np.asarray(a, np.float64))


def test_attention_full_mask_is_torch_sdpa():
    rng = np.random.default_rng(0)
    q, k, v = (rng.normal(size=(200, 64)) for _ in range(3))
    got = masked_attention(q, k, v, np.ones((200, 200), bool), 64 ** -0.5)
    want = F.scaled_dot_product_attention(_t(q)[None], _t(k)[None], _t(v)[None])[0].numpy()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_attention_with_mask_is_torch_sdpa_with_bool_mask():
    rng = np.random.default_rng(1)
    n = 196
    q, k, v = (rng.normal(size=(n, 64)) for _ in range(3))
    inv = rng.permutation(n)
    M = token_mask(inv, 4, 16, 16, 0)
    got = masked_attention(q, k, v, M, 0.125)
    want = F.scaled_dot_product_attention(_t(q)[None], _t(k)[None], _t(v)[None],
                                          attn_mask=torch.from_numpy(M)[None])[0].numpy()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_attention_zero_query_is_mean_over_kept_keys():
    rng = np.random.default_rng(2)
    n = 256
    k, v = rng.normal(size=(n, 64)), rng.normal(size=(n, 64))
    M = position_keep(n, 2, 16, 16, 1)
    got = masked_attention(np.zeros((n, 64)), k, v, M, 0.125)
    for i in range(0, n, 17):
        np.testing.assert_allclose(got[i], v[M[i]].mean(axis=0), rtol=1e-12, atol=1e-12)


def test_attention_constant_values_give_constant_output():
    rng = np.random.default_rng(3)
    n = 64
    q, k = rng.normal(size=(n, 16)), rng.normal(size=(n, 16))
    v = np.tile(rng.normal(size=(1, 16)), (n, 1))
    got = masked_attention(q, k, v, position_keep(n, 4, 4, 4, 0), 0.25)
    np.testing.assert_allclose(got, v, rtol=1e-12, atol=1e-12)


def test_attention_brute_force_16_tokens():
    rng = np.random.default_rng(4)
    n, D = 16, 8
    q, k, v = (rng.normal(size=(n, D)) for _ in range(3))
    keep = position_keep(n, 4, 1, 1, 0)
    got = masked_attention(q, k, v, keep, D ** -0.5)
    for i in range(n):
        keys = [j for j in range(n) if keep[i, j]]
        sc = [sum(q[i, d] * k[j, d] for d in range(D)) / np.sqrt(D) for j in keys]
        mx = max(sc)
        w = [np.exp(x - mx) for x in sc]
        tot = sum(w)
        out = [sum(w[t] * v[keys[t], d] for t in range(len(keys))) / tot for d in range(D)]
        np.testing.assert_allclose(got[i], out, rtol=1e-12, atol=1e-12)


def test_layer_norm_and_gelu_match_torch():
    rng = np.random.default_rng(5)
    x = rng.normal(size=(10, 96)) * 3 + 1
    g, b = rng.normal(size=96), rng.normal(size=96)
    want = F.layer_norm(_t(x), (96,), _t(g), _t(b), eps=1e-6).numpy()
    np.testing.assert_allclose(layer_norm(x, g, b), want, rtol=1e-12, atol=1e-12)
    z = np.linspace(-6, 6, 101)
    np.testing.assert_allclose(gelu(z), F.gelu(_t(z), approximate="none").numpy(), rtol=1e-12, atol=1e-14)


def _torch_mlp(x, w):
    h = F.layer_norm(x, (x.shape[-1],), _t(w["ln2_g"]), _t(w["ln2_b"]), eps=1e-6)
    h = F.gelu(F.linear(h, _t(w["w1"]), _t(w["b1"])))
    return x + F.linear(h, _t(w["w2"]), _t(w["b2"]))


def test_routed_mlp_all_rows_is_dense_mlp_and_others_unchanged():
    cfg = get_config("c1")
    w = block_weights(cfg)
    rng = np.random.default_rng(6)
    x = rng.normal(size=(50, 64)).astype(np.float32)
    dense = _torch_mlp(_t(x), w).numpy()
    np.testing.assert_allclose(routed_mlp(x, np.arange(50), w), dense, rtol=1e-12, atol=1e-12)
    routed = np.array([3, 7, 8, 40])
    out = routed_mlp(x, routed, w)
    np.testing.assert_allclose(out[routed], dense[routed], rtol=1e-12, atol=1e-12)
    other = np.setdiff1d(np.arange(50), routed)
    assert np.array_equal(out[other], x[other].astype(np.float64))


def _torch_dense_block(x, w, heads, window):
    """Dense pre-LN ViT block (SAM-style zero-padded windows when window > 0), fp64."""
    b, gh, gw, C = x.shape
    D = C // heads
    xt = _t(x)
    h = F.layer_norm(xt, (C,), _t(w["ln1_g"]), _t(w["ln1_b"]), eps=1e-6)
    if window:
        ph, pw = -gh % window, -gw % window
        h = F.pad(h, (0, 0, 0, pw, 0, ph))
        Hp, Wp = gh + ph, gw + pw
        h = h.view(b, Hp // window, window, Wp // window, window, C).permute(0, 1, 3, 2, 4, 5)
        h = h.reshape(-1, window * window, C)
    else:
        h = h.reshape(b, gh * gw, C)
    qkv = F.linear(h, _t(w["w_qkv"]), _t(w["b_qkv"]))
    q, k, v = qkv.view(h.shape[0], h.shape[1], 3, heads, D).permute(2, 0, 3, 1, 4)
    o = F.scaled_dot_product_attention(q, k, v).transpose(1, 2).reshape(h.shape[0], h.shape[1], C)
    if window:
        o = o.view(b, Hp // window, Wp // window, window, window, C).permute(0, 1, 3, 2, 4, 5)
        o = o.reshape(b, Hp, Wp, C)[:, :gh, :gw]
    else:
        o = o.view(b, gh, gw, C)
    x1 = xt + F.linear(o, _t(w["w_proj"]), _t(w["b_proj"]))
    return _torch_mlp(x1, w).numpy()


@pytest.mark.parametrize("key,window", [("c1", 0), ("c3", 14)])
def test_block_at_density_one_is_dense_block(key, window):
    cfg = get_config(key).with_(attn_density=1.0, mlp_density=1.0, batch=1)
    if key == "c3":
        cfg = cfg.with_(channels=128, heads=2, mlp_hidden=256, image=448)  # 28 x 28 grid, 4 windows
    imgs = synthetic_images(cfg)
    imp = np.stack([importance(im, cfg.patch) for im in imgs])
    x = token_features(cfg)
    w = block_weights(cfg)
    got = block_forward(x, imp, w, cfg)
    want = _torch_dense_block(x, w, cfg.heads, window)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-10)


def test_block_window_pads_do_not_leak_and_sparse_differs():
    cfg = get_config("c3").with_(batch=1, channels=64, heads=1, mlp_hidden=128, image=288)  # 18 x 18 grid
    imgs = synthetic_images(cfg)
    imp = np.stack([importance(im, cfg.patch) for im in imgs])
    x = token_features(cfg)
    w = block_weights(cfg)
    out, parts = block_forward(x, imp, w, cfg, return_parts=True)
    assert out.shape == x.shape
    assert np.isfinite(out).all()
    assert parts["radius"] == 0
    n_routed = len(parts["routed"][0])
    # 4 windows: 14x14 (196 real), 14x4, 4x14, 4x4 -> K = 78, 22, 22, 6
    assert n_routed == 78 + 22 + 22 + 6
    dense = block_forward(x, imp, w, cfg.with_(attn_density=1.0, mlp_density=1.0))
    assert not np.allclose(out, dense)


def test_block_unrouted_rows_get_attention_only():
    cfg = get_config("c1")
    imgs = synthetic_images(cfg)
    imp = np.stack([importance(im, cfg.patch) for im in imgs])
    x = token_features(cfg)
    w = block_weights(cfg)
    out, parts = block_forward(x, imp, w, cfg, return_parts=True)
    # Re-derive x1 for unrouted rows with the mlp switched off via an empty-looking keep-set:
    # rows outside the keep-set must equal x + attention branch, i.e. equal between d_mlp=0.4
    # and the tiniest d_mlp whose keep-set is a subset.
    small = block_forward(x, imp, w, cfg.with_(mlp_density=0.001))
    routed = set(parts["routed"][0].tolist())
    flat_o, flat_s = out.reshape(-1, 64), small.reshape(-1, 64)
    s = descending_order(imp[0])
    top1 = s[0]
    for t in range(256):
        if t not in routed:
            assert np.array_equal(flat_o[t], flat_s[t])
    assert top1 in routed
    # the top token is routed in both (BLAS may block a 1-row product differently)
    np.testing.assert_allclose(flat_o[top1], flat_s[top1], rtol=1e-12, atol=1e-12)
