"""GPU parity: every C-ABI entry point against the oracle on the same seeded inputs.

Integer outputs (importance bits, perm, inv, keep-set) must match bit for bit;
floating-point outputs within max-abs 1e-2 and relative L2 5e-3.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import structured_sparse_vit_amd as ss
from synth import round_to_bf16
from tests.gpu_cases import check_close, config, images, oracle_block, oracle_importance, rel_l2

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _plan(cfg, **over):
    return ss.Plan.from_config(cfg.with_(**over) if over else cfg)


def _oracle_perm(cfg, imp):
    """Oracle perm / inv / keep-set (segment by segment, rank order) for a batch of maps."""
    tm = oracle.segments_for_image(cfg.grid, cfg.grid, cfg.window)
    side = cfg.window or cfg.grid
    perms, invs, routed = [], [], []
    tokens = cfg.grid * cfg.grid
    for b in range(imp.shape[0]):
        rs = []
        for row in tm:
            s = oracle.segment_order(cfg.ordering, imp[b], row, side, side, cfg.order_seed)
            p, i = oracle.stripe_sort(s, cfg.stripes)
            perms.append(p)
            invs.append(i)
            rs.append(oracle.routed_rank_order(s, row, cfg.mlp_density))
        routed.append(np.concatenate(rs) + b * tokens)
    return np.stack(perms), np.stack(invs), np.concatenate(routed)


# ------------------------------------------------------------------ importance

@pytest.mark.parametrize("key,noise", [("c1", 0.05), ("c2", 0.05), ("c3", 0.05), ("c2", 0.0)])
def test_importance_bit_exact(key, noise):
    _say("importance", key, noise)
    img = images(key, 0, noise)
    got = ss.importance(torch.from_numpy(img).to(DEV), config(key).patch).cpu().numpy()
    want = oracle_importance(key, 0, noise)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_importance_edge_images():
    _say("importance edges")
    rng = np.random.default_rng(1)
    imgs = np.stack([
        np.zeros((64, 96), np.float32),
        np.full((64, 96), 0.5, np.float32),
        rng.integers(0, 256, (64, 96)).astype(np.float32),
        (rng.normal(size=(64, 96)) * 1e-20).astype(np.float32),   # tiny values, subnormal squares
        (rng.normal(size=(64, 96)) * 1e15).astype(np.float32),    # large values
    ])
    got = ss.importance(torch.from_numpy(imgs).to(DEV), 16).cpu().numpy()
    want = np.stack([oracle.importance(im, 16) for im in imgs])
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    got8 = ss.importance(torch.from_numpy(imgs[:, :, :96]).to(DEV), 8).cpu().numpy()
    want8 = np.stack([oracle.importance(im, 8) for im in imgs])
    assert np.array_equal(got8.view(np.uint32), want8.view(np.uint32))


# ------------------------------------------------------------------ permute

@pytest.mark.parametrize("key", ["c1", "c2", "c3", "ragged"])
def test_permute_bit_exact(key):
    _say("permute", key)
    cfg = config(key)
    plan = _plan(cfg)
    imp = oracle_importance(key)
    perm, inv, routed = ss.permute(plan, torch.from_numpy(imp).to(DEV))
    wp, wi, wr = _oracle_perm(cfg, imp)
    assert np.array_equal(perm.cpu().numpy(), wp)
    assert np.array_equal(inv.cpu().numpy(), wi)
    assert np.array_equal(routed.cpu().numpy(), wr)


@pytest.mark.parametrize("ordering", ["zorder", "hilbert", "random"])
@pytest.mark.parametrize("key", ["c1", "c2", "c3", "ragged"])
def test_permute_orderings_bit_exact(key, ordering):
    """The other token orders (Z-order, Hilbert, seeded random): perm, inv and keep-set
    bit-exact against the oracle, windows with pads included."""
    _say("permute", key, ordering)
    cfg = config(key).with_(ordering=ordering, order_seed=12345)
    plan = _plan(cfg)
    imp = oracle_importance(key)
    perm, inv, routed = ss.permute(plan, torch.from_numpy(imp).to(DEV))
    wp, wi, wr = _oracle_perm(cfg, imp)
    assert np.array_equal(perm.cpu().numpy(), wp)
    assert np.array_equal(inv.cpu().numpy(), wi)
    assert np.array_equal(routed.cpu().numpy(), wr)


@pytest.mark.parametrize("key", ["c2", "c3"])
def test_permute_ties_zero_nan(key):
    _say("permute ties", key)
    cfg = config(key).with_(batch=3)
    plan = _plan(cfg)
    rng = np.random.default_rng(7)
    t = cfg.grid * cfg.grid
    imp = np.stack([
        np.zeros(t, np.float32),                                        # all ties
        rng.integers(0, 4, t).astype(np.float32) * np.float32(0.25),    # many ties
        rng.uniform(size=t).astype(np.float32),
    ])
    imp[1, ::5] = -0.0
    imp[2, ::97] = np.nan
    imp[2, 3] = np.inf
    perm, inv, routed = ss.permute(plan, torch.from_numpy(imp).to(DEV))
    wp, wi, wr = _oracle_perm(cfg, imp)
    assert np.array_equal(perm.cpu().numpy(), wp)
    assert np.array_equal(inv.cpu().numpy(), wi)
    assert np.array_equal(routed.cpu().numpy(), wr)


# ------------------------------------------------------------------ attention

def _attn_case(key, seed=0, **over):
    cfg = config(key)
    if over:
        cfg = cfg.with_(**over)
    plan = _plan(cfg)
    n, H, D = plan.info["seq_len"], cfg.heads, cfg.head_dim
    segs = cfg.batch * plan.info["segments_per_image"]
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((segs, H, n, D), dtype=np.float32) for _ in range(3))
    if cfg.dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    n_pad = (n + 7) // 8 * 8
    vt = np.full((segs, H, D, n_pad), np.nan, np.float32)  # pad columns must never be read
    vt[..., :n] = v.transpose(0, 1, 3, 2)
    dt = plan.torch_dtype
    dev = [torch.from_numpy(a).to(DEV, dt).contiguous() for a in (q, k, vt)]
    o = ss.attn(plan, *dev).float().cpu().numpy()
    keep = oracle.position_keep(n, cfg.stripes, cfg.block, cfg.global_tokens, plan.info["band_radius"])
    want = np.empty((segs, n, H * D))
    for s in range(segs):
        for h in range(H):
            want[s, :, h * D:(h + 1) * D] = oracle.masked_attention(q[s, h], k[s, h], v[s, h], keep, D ** -0.5)
    return o, want


@pytest.mark.parametrize("key", ["c1", "c2", "c3b1", "c5g", "c5w", "ragged"])
def test_attention_parity(key):
    _say("attention", key)
    o, want = _attn_case(key)
    check_close(o, want, what="attention " + key)


@pytest.mark.parametrize("key", ["c2", "c3b1", "c1"])
def test_attention_density_one_is_dense(key):
    _say("attention dense", key)
    o, want = _attn_case(key, seed=3, attn_density=1.0)
    check_close(o, want, what="dense attention " + key)


def test_attention_single_stripe_and_wide_band():
    _say("attention stripes=1")
    o, want = _attn_case("c2", seed=4, stripes=1, band_radius=2)
    check_close(o, want, what="stripes=1")


# ------------------------------------------------------------------ MLP

@pytest.mark.parametrize("key", ["c1", "c2", "c3b1"])
def test_mlp_parity_and_unrouted_rows_untouched(key):
    _say("mlp", key)
    x, w, imp, _, parts = oracle_block(key)
    cfg = config(key)
    plan = _plan(cfg)
    rows = x.reshape(-1, cfg.channels)
    routed = np.concatenate(parts["routed"]).astype(np.int32)
    wd = ss.weights_to_device(w, plan)
    xd = torch.from_numpy(rows.copy()).to(DEV)
    rd = torch.from_numpy(routed).to(DEV)
    ss.mlp(plan, xd, rd, wd["ln2_g"], wd["ln2_b"], wd["w1"], wd["b1"], wd["w2"], wd["b2"])
    got = xd.cpu().numpy()
    want = oracle.routed_mlp(rows, routed, w)
    check_close(got, want, what="mlp " + key)
    other = np.setdiff1d(np.arange(rows.shape[0]), routed)
    assert np.array_equal(got[other].view(np.uint32), rows[other].view(np.uint32))


def test_mlp_empty_keep_set_is_noop():
    cfg = config("c1")
    plan = _plan(cfg)
    w = ss.weights_to_device(oracle_block("c1")[1], plan)
    x = torch.randn(256, 64, device=DEV)
    x0 = x.clone()
    ss.mlp(plan, x, torch.empty(0, dtype=torch.int32, device=DEV), w["ln2_g"], w["ln2_b"], w["w1"], w["b1"],
           w["w2"], w["b2"])
    assert torch.equal(x, x0)


# ------------------------------------------------------------------ whole block

def _run_block(key, seed=0, gain=1.0):
    x, w, imp, want, parts = oracle_block(key, seed, gain)
    cfg = config(key)
    plan = _plan(cfg)
    img = torch.from_numpy(images(key, seed)).to(DEV)
    imp_d = ss.importance(img, cfg.patch)
    perm, inv, routed = ss.permute(plan, imp_d)
    wd = ss.weights_to_device(w, plan)
    xd = torch.from_numpy(x.copy()).to(DEV)
    ss.block(plan, wd, xd, perm, routed)
    torch.cuda.synchronize()
    return dict(x=x, want=want, parts=parts, imp=imp, got=xd.cpu().numpy(), imp_d=imp_d.cpu().numpy(),
                perm=perm.cpu().numpy(), inv=inv.cpu().numpy(), routed=routed.cpu().numpy(), plan=plan, wd=wd,
                img=img)


# Branch bars: the attention branch alone (x2 - x on rows outside the keep-set) and the
# whole block delta, relative L2 against the oracle's. bf16 operands give about 2^-9
# relative rounding per stage; fp32 runs are held far tighter.
BRANCH_REL = {"bf16": 1.5e-2, "f32": 1e-4}


def _check_block(key, r, gain):
    cfg = config(key)
    C = cfg.channels
    assert np.array_equal(r["imp_d"].view(np.uint32), r["imp"].view(np.uint32))
    assert np.array_equal(r["perm"], np.stack(r["parts"]["perm"]))
    assert np.array_equal(r["inv"], np.stack(r["parts"]["inv"]))
    # same keep-set (the library lists it in rank order, the oracle block ascending)
    assert np.array_equal(np.sort(r["routed"]), np.concatenate(r["parts"]["routed"]))
    got, want, x = (a.reshape(-1, C) for a in (r["got"], r["want"], r["x"]))
    routed = np.concatenate(r["parts"]["routed"])
    other = np.setdiff1d(np.arange(got.shape[0]), routed)
    err = np.abs(got - want)
    attn_rel = rel_l2(got[other] - x[other], want[other] - x[other])
    delta_rel = rel_l2(got - x, want - x)
    _say("  block %s gain %g: max err routed %.3e other %.3e | rel-L2 attention branch %.3e, block delta %.3e" % (
        key, gain, err[routed].max(), err[other].max() if other.size else 0.0, attn_rel, delta_rel))
    if gain == 1.0:
        check_close(got, want, what="block " + key)
    bar = BRANCH_REL[cfg.dtype]
    assert attn_rel <= bar, "block %s: attention branch rel-L2 %.3e > %.1e" % (key, attn_rel, bar)
    assert delta_rel <= bar, "block %s: block delta rel-L2 %.3e > %.1e" % (key, delta_rel, bar)


@pytest.mark.parametrize("key", ["c1", "c2", "c3", "ragged", "c4g", "c4w", "c1:zorder", "c3b1:hilbert",
                                 "c2:random"])
def test_block_parity(key):
    _say("block", key)
    _check_block(key, _run_block(key), 1.0)


@pytest.mark.parametrize("key,gain", [("c1", 10.0), ("c2", 3.0), ("c3b1", 3.0), ("ragged", 3.0)])
def test_block_parity_high_gain(key, gain):
    """Projection weights scaled up: the attention and MLP branches dominate the residual.
    (bf16 runs use a gain of 3 so the softmax stays far from one-hot.)"""
    _say("block high gain", key)
    _check_block(key, _run_block(key, gain=gain), gain)


@pytest.mark.parametrize("key,kind", [("c4", "global"), ("c4", "window"), ("c5", "global"), ("c5", "window")])
def test_block_full_batch_sampled(key, kind):
    """One block of the ViT-L / ViT-H encoder configs at their full batch (8 and 16
    images: the launch shapes the encoder benchmark times, with the large-tile GEMM
    paths) against the oracle on sampled images: the first and the last. Images are
    independent, so the oracle runs each sampled image alone."""
    from synth import block_weights, token_features
    from synth.configs import global_variant, window_variant
    _say("block full batch", key, kind)
    base = config(key)
    cfg = global_variant(base) if kind == "global" else window_variant(base)
    b = cfg.batch
    plan = _plan(cfg)
    img = images(key)
    assert img.shape[0] == b
    x = token_features(cfg, 0)
    w = block_weights(cfg, 0)
    imp_d = ss.importance(torch.from_numpy(img).to(DEV), cfg.patch)
    perm, inv, routed = ss.permute(plan, imp_d)
    xd = torch.from_numpy(x.copy()).to(DEV)
    ss.block(plan, ss.weights_to_device(w, plan), xd, perm, routed)
    got = xd.cpu().numpy()
    imp = imp_d.cpu().numpy()
    one = cfg.with_(batch=1)
    for i in (0, b - 1):
        want_imp = oracle.importance(img[i], cfg.patch)
        assert np.array_equal(imp[i].view(np.uint32), want_imp.view(np.uint32)), "importance of image %d" % i
        want = oracle.block_forward(x[i:i + 1], imp[i:i + 1], w, one)
        mx, rel = check_close(got[i:i + 1], want, what="block %s %s image %d of %d" % (key, kind, i, b))
        _say("  image %d of %d: max-abs %.3e rel-L2 %.3e" % (i, b, mx, rel))


def test_block_is_deterministic():
    _say("block determinism")
    cfg = config("c2")
    r = _run_block("c2")
    plan, wd = r["plan"], r["wd"]
    perm = torch.from_numpy(r["perm"]).to(DEV)
    routed = torch.from_numpy(r["routed"]).to(DEV)
    outs = []
    for _ in range(2):
        xd = torch.from_numpy(r["x"].copy()).to(DEV)
        ss.block(plan, wd, xd, perm, routed)
        outs.append(xd.cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    assert np.array_equal(outs[0].view(np.uint32), r["got"].view(np.uint32))


def test_block_density_one_matches_dense_oracle():
    _say("block dense c1")
    import oracle as O
    from synth import block_weights, token_features
    cfg = config("c1").with_(attn_density=1.0, mlp_density=1.0)
    plan = _plan(cfg)
    img = images("c1")
    imp = np.stack([O.importance(im, cfg.patch) for im in img])
    x, w = token_features(cfg), block_weights(cfg)
    want = O.block_forward(x, imp, w, cfg)
    imp_d = ss.importance(torch.from_numpy(img).to(DEV), cfg.patch)
    perm, inv, routed = ss.permute(plan, imp_d)
    xd = torch.from_numpy(x.copy()).to(DEV)
    ss.block(plan, ss.weights_to_device(w, plan), xd, perm, routed)
    check_close(xd.cpu().numpy(), want, max_abs=1e-4, rel_l2=1e-5, what="dense fp32 block")


# ------------------------------------------------------------------ encoder

def test_encoder_matches_block_by_block_and_oracle():
    """An 8-block stack of the c4 (ViT-L) layout at reduced width, batch 2: global blocks
    at layers 1, 3, 5, 7, windowed elsewhere, one permutation set per block type. The
    native encoder equals the same blocks called one by one (deterministic kernels:
    bit-equal) and the fp64 oracle encoder to the per-block bar scaled by sqrt(8) (each
    block adds its own independent bf16 rounding)."""
    _say("encoder 8 layers")
    import math

    from synth import block_weights, encoder_global_layers, token_features
    from synth.configs import global_variant, window_variant
    layers, b = 8, 2
    base = config("c4").with_(batch=b, channels=256, heads=4, mlp_hidden=512, layers=layers)
    cg, cw = global_variant(base).with_(batch=b), window_variant(base).with_(batch=b)
    pg, pw = _plan(cg), _plan(cw)
    imgs = np.stack([images("c4")[0], images("c4")[1]])
    imp = np.stack([oracle.importance(im, base.patch) for im in imgs])
    x0 = token_features(base, 0)
    gl = encoder_global_layers(layers)
    kinds = [1 if l in gl else 0 for l in range(layers)]
    ws = [block_weights(base, 0, layer=l) for l in range(layers)]
    wd = [ss.weights_to_device(w, pg) for w in ws]
    imp_d = torch.from_numpy(imp).to(DEV)
    perm_g, _, routed_g = ss.permute(pg, imp_d)
    perm_w, _, routed_w = ss.permute(pw, imp_d)
    x_enc = torch.from_numpy(x0.copy()).to(DEV)
    ss.encoder(pg, pw, wd, kinds, x_enc, (perm_g, routed_g), (perm_w, routed_w))
    x_seq = torch.from_numpy(x0.copy()).to(DEV)
    for l in range(layers):
        if kinds[l]:
            ss.block(pg, wd[l], x_seq, perm_g, routed_g)
        else:
            ss.block(pw, wd[l], x_seq, perm_w, routed_w)
    got = x_enc.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), x_seq.cpu().numpy().view(np.uint32))
    want = oracle.encoder_forward(x0, imp, ws, gl, cg, cw)
    s = math.sqrt(layers)
    _say("  encoder max-abs %.3e rel-L2 %.3e" % (np.abs(got - want).max(), rel_l2(got, want)))
    check_close(got, want, max_abs=1e-2 * s, rel_l2=5e-3 * s, what="encoder")


def test_encoder_full_size_matches_block_by_block():
    """The ViT-L encoder config at full size (24 blocks, batch 8, global at layers 5, 11,
    17, 23), one random layer's weights reused by every block: sparsesam_encoder equals
    the same blocks called one by one, bit for bit (each block is checked against the
    oracle by the sampled full-batch tests)."""
    _say("encoder full size c4")
    from synth import block_weights, encoder_global_layers, token_features
    from synth.configs import global_variant, window_variant
    base = config("c4")
    cg, cw = global_variant(base), window_variant(base)
    pg, pw = _plan(cg), _plan(cw)
    gl = encoder_global_layers(base.layers)
    kinds = [1 if l in gl else 0 for l in range(base.layers)]
    wd = ss.weights_to_device(block_weights(base, 0), pg)
    imp_d = ss.importance(torch.from_numpy(images("c4")).to(DEV), base.patch)
    perm_g, _, routed_g = ss.permute(pg, imp_d)
    perm_w, _, routed_w = ss.permute(pw, imp_d)
    x0 = token_features(base, 0)
    x_enc = torch.from_numpy(x0.copy()).to(DEV)
    ss.encoder(pg, pw, [wd] * base.layers, kinds, x_enc, (perm_g, routed_g), (perm_w, routed_w))
    x_seq = torch.from_numpy(x0.copy()).to(DEV)
    for l in range(base.layers):
        if kinds[l]:
            ss.block(pg, wd, x_seq, perm_g, routed_g)
        else:
            ss.block(pw, wd, x_seq, perm_w, routed_w)
    got, ref = x_enc.cpu().numpy(), x_seq.cpu().numpy()
    assert np.isfinite(got).all()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
