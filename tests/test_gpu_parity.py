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

def _attn_case(key, seed=0, heads_checked=None, **over):
    """sparsesam_attn on seeded N(0, 1) q, k, v against the oracle's masked dense
    attention; heads_checked samples the heads the oracle computes (all by default)."""
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
    hs = list(range(H)) if heads_checked is None else list(heads_checked)
    want = np.empty((segs, n, len(hs) * D))
    got = np.empty_like(want)
    for i, h in enumerate(hs):
        got[:, :, i * D:(i + 1) * D] = o[:, :, h * D:(h + 1) * D]
        for s in range(segs):
            want[s, :, i * D:(i + 1) * D] = oracle.masked_attention(q[s, h], k[s, h], v[s, h], keep, D ** -0.5)
    return got, want


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


@pytest.mark.parametrize("density", [0.4, 1.0])
def test_attention_head_dim_80_global(density):
    """The ViT-H global grid (head_dim 80, 16 heads) at density 0.4 (r = 3) and 1.0 (every
    query tile keeps all 64 key tiles): the head_dim-80 long-segment kernel."""
    _say("attention c5g density", density)
    o, want = _attn_case("c5g", seed=5, heads_checked=(0, 7, 15), attn_density=density)
    check_close(o, want, what="c5g attention d=%g" % density)


def _max_row_tiles(cfg):
    rp, _ = _plan(cfg).tile_list()
    return int(np.diff(rp).max())


@pytest.mark.parametrize("head_dim,density", [(64, 0.4), (64, 1.0), (80, 0.4), (80, 1.0)])
def test_attention_split_rows_and_combine(head_dim, density):
    """An 80 x 80 token grid (N = 6400, 25 tiles per stripe, 100 tiles): the global row
    (and at density 1 every row) keeps more than 64 key tiles, so its work is split into
    pieces that write partial results, merged by the combine kernel."""
    heads = 2 if head_dim == 64 else 8  # channels a multiple of 128
    over = dict(image=1280, heads=heads, head_dim=head_dim, channels=heads * head_dim, attn_density=density)
    cfg = config("c2").with_(**over)
    assert _max_row_tiles(cfg) > 64, "the plan must split rows"
    _say("attention split rows D", head_dim, "density", density)
    o, want = _attn_case("c2", seed=6, heads_checked=(0, heads - 1), **over)
    check_close(o, want, what="split-row attention D%d d=%g" % (head_dim, density))


@pytest.mark.parametrize("key,over", [
    ("c2", dict(block=32, global_tokens=32)),      # B = 32 over a 64 x 64 grid
    ("ragged", dict(window=0, block=16)),          # 18 x 18 global grid: stripes of 81, ragged tiles
])
def test_attention_bf16_simt_fallback(key, over):
    """bf16 plans the matrix-core kernels do not take (long segments with B != 64 or
    stripes not a multiple of 64) run the SIMT kernel on bf16 storage."""
    _say("attention bf16 simt", key, over)
    cfg = config(key).with_(**over)
    hc = (0, cfg.heads - 1)
    o, want = _attn_case(key, seed=7, heads_checked=hc, **over)
    check_close(o, want, what="bf16 SIMT attention %s %s" % (key, over))


@pytest.mark.parametrize("head_dim,block", [(32, 16), (80, 16), (128, 16), (80, 32), (128, 64)])
def test_attention_fp32_simt_head_dims(head_dim, block):
    """The fp32 SIMT kernel at every head_dim it takes and at the three tile lengths that
    set its threads per query: 16 threads (16-token tiles), 2 (32) and 1 (64; K rows by
    scalar loads); head_dim 128 stages 32-key chunks."""
    over = dict(heads=2, head_dim=head_dim, channels=2 * head_dim, block=block, global_tokens=block)
    _say("attention fp32 simt", over)
    o, want = _attn_case("c1", seed=8, **over)
    check_close(o, want, what="fp32 SIMT attention D%d B%d" % (head_dim, block))


# A short global segment (16 x 16 tokens, one stripe of sixteen 16-token tiles): every
# key tile has its own kept column, so the window kernel stores sixteen key classes in
# its 256 LDS slots (one 16-key block each), and the 32 x 32 window kernel would need two
# mask k-steps (17 classes with its pad keys).
SHORT_TWO_KSTEPS = dict(dtype="bf16", stripes=1, block=16, global_tokens=16, heads=2, mlp_hidden=256,
                        attn_density=0.3)


def mask_classes(cfg, plan):
    """Distinct kept columns of the plan's token mask (the key classes the plan's mask
    k-steps must tell apart, pads not counted)."""
    n = plan.info["seq_len"]
    keep = oracle.position_keep(n, cfg.stripes, cfg.block, cfg.global_tokens, plan.info["band_radius"])
    return len({keep[:, k].tobytes() for k in range(n)})


@pytest.mark.parametrize("head_dim", [64, 80])
def test_attention_short_segment_sixteen_classes(head_dim):
    _say("attention short segment, sixteen key classes, head_dim", head_dim)
    heads = 2 if head_dim == 64 else 8  # bf16 plans take channels in multiples of 128
    over = dict(SHORT_TWO_KSTEPS, heads=heads, head_dim=head_dim, channels=heads * head_dim)
    cfg = config("c1").with_(**over)
    plan = _plan(cfg)
    assert plan.info["seq_len"] <= 256 and mask_classes(cfg, plan) + 1 > 16
    o, want = _attn_case("c1", seed=11, **over)
    check_close(o, want, what="short segment, sixteen key classes, D %d" % head_dim)


@pytest.mark.parametrize("grid_h,grid_w,block,head_dim,ksteps", [
    (16, 15, 8, 64, 2), (16, 15, 8, 80, 2), (15, 17, 17, 64, 1), (15, 17, 17, 80, 1)])
def test_attention_window_slots_overflow(grid_h, grid_w, block, head_dim, ksteps):
    """Short global segments whose key classes do not fit 256 LDS slots in 16-key blocks
    (30 classes of 8 tokens; 15 classes of 17): these run the 32 x 32-block window kernel
    with its mask in one or two matrix-core k-steps."""
    heads = 2 if head_dim == 64 else 8  # bf16 plans take channels in multiples of 128
    plan = ss.Plan(grid_h, grid_w, 0, 1, block, block, -1, 0.3, 0.4, heads * head_dim, heads, head_dim, 256, 1,
                   "bf16")
    n = plan.info["seq_len"]
    _say("attention window slot overflow", grid_h, grid_w, block, head_dim)
    rng = np.random.default_rng(12)
    q, k, v = (round_to_bf16(rng.standard_normal((1, heads, n, head_dim), dtype=np.float32)) for _ in range(3))
    n_pad = (n + 7) // 8 * 8
    vt = np.full((1, heads, head_dim, n_pad), np.nan, np.float32)
    vt[..., :n] = v.transpose(0, 1, 3, 2)
    dev = [torch.from_numpy(a).to(DEV, torch.bfloat16).contiguous() for a in (q, k, vt)]
    o = ss.attn(plan, *dev).float().cpu().numpy()
    keep = oracle.position_keep(n, 1, block, block, plan.info["band_radius"])
    assert len({keep[:, j].tobytes() for j in range(n)}) + 1 > 16 * (ksteps - 1)
    want = np.concatenate([oracle.masked_attention(q[0, h], k[0, h], v[0, h], keep, head_dim ** -0.5)
                           for h in range(heads)], axis=1)
    check_close(o[0], want, what="window slot overflow %dx%d B%d D%d" % (grid_h, grid_w, block, head_dim))


@pytest.mark.parametrize("over", [
    dict(window=8, stripes=4, block=4, global_tokens=4, heads=2, head_dim=64, channels=128),
    dict(image=448, window=14, stripes=7, block=4, global_tokens=0, attn_density=0.5, heads=2, head_dim=64,
         channels=128),
    dict(image=192, window=0, stripes=2, block=12, global_tokens=12, heads=8, head_dim=80, channels=640),
    dict(window=0, stripes=4, block=8, global_tokens=8, attn_density=0.2, heads=2, head_dim=64, channels=128),
])
def test_attention_window_kernel_shapes(over):
    """Short segments of other shapes: on the window kernel's 16-key blocks, 64-token
    windows of 4-token tiles, seven stripes of 4-token tiles without global tokens (many
    classes, partly empty blocks) and a 144-token global segment at head_dim 80; and a
    256-token segment of 8-token tiles at density 0.2, whose classes need more than 256
    slots (the 32 x 32-block kernel)."""
    over = dict(over, dtype="bf16", mlp_hidden=256)
    _say("attention window kernel shape", over)
    o, want = _attn_case("c1", seed=14, **over)
    check_close(o, want, what="window kernel shape %s" % over)


@pytest.mark.parametrize("key,batch", [("c2", 4), ("c5g", 16)])
def test_attention_schedule_independent(key, batch):
    """Every work unit is computed the same whichever workgroup runs it, so attention over
    a batch (several rounds of units: the snake order, or at ViT-H global batch 16 the
    head-major order) equals, bit for bit, attention run one segment at a time (one round,
    XCD-grouped units)."""
    _say("attention schedule", key, batch)
    cfg = config(key).with_(batch=batch)
    plan = _plan(cfg)
    n, H, D = plan.info["seq_len"], cfg.heads, cfg.head_dim
    n_pad = (n + 7) // 8 * 8
    g = torch.Generator(device=DEV).manual_seed(21)
    q = torch.randn(batch, H, n, D, device=DEV, generator=g).to(torch.bfloat16)
    k = torch.randn(batch, H, n, D, device=DEV, generator=g).to(torch.bfloat16)
    vt = torch.randn(batch, H, D, n_pad, device=DEV, generator=g).to(torch.bfloat16)
    full = ss.attn(plan, q, k, vt)
    for s in range(batch):
        one = ss.attn(plan, q[s:s + 1].contiguous(), k[s:s + 1].contiguous(), vt[s:s + 1].contiguous())
        assert torch.equal(one[0], full[s]), "segment %d differs" % s


def test_attention_single_stripe_and_wide_band():
    _say("attention stripes=1")
    o, want = _attn_case("c2", seed=4, stripes=1, band_radius=2)
    check_close(o, want, what="stripes=1")


# ------------------------------------------------------------------ MLP

@pytest.mark.parametrize("key", ["c1", "c1odd", "c2", "c3b1"])
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


@pytest.mark.parametrize("key", ["c1", "c1odd", "c2", "c3", "ragged", "c4g", "c4w", "c1:zorder", "c3b1:hilbert",
                                 "c2:random"])
def test_block_parity(key):
    _say("block", key)
    _check_block(key, _run_block(key), 1.0)


@pytest.mark.parametrize("key,rel_pos", [("c2", False), ("c4g", False), ("c5g", False), ("c3", False),
                                         ("c1", False), ("c2:zorder", False), ("c2", True), ("c3b1", True)])
def test_forward_equals_the_three_calls(key, rel_pos):
    """sparsesam_forward (importance, permutation and block in one call; on the ViT global
    grids the permutation kernel also writes the block's first LayerNorm rows) against
    sparsesam_importance + sparsesam_permute + sparsesam_block on the same inputs: every
    output bit for bit, with and without the relative-position bias (whose tables read
    the permutation the same call writes)."""
    from synth import block_weights, token_features
    from synth.generate import rel_pos_tables
    _say("forward", key, "rel_pos" if rel_pos else "")
    cfg = config(key)
    plan = ss.Plan.from_config(cfg, rel_pos=True) if rel_pos else _plan(cfg)
    img = torch.from_numpy(images(key.split(":")[0])).to(DEV)
    x0 = torch.from_numpy(token_features(cfg, 0)).to(DEV)
    wh = block_weights(cfg, 0)
    if rel_pos:
        wh["rel_h"], wh["rel_w"] = rel_pos_tables(cfg, 0)
    w = ss.weights_to_device(wh, plan)
    imp = ss.importance(img, cfg.patch)
    perm, inv, routed = ss.permute(plan, imp)
    x1 = x0.clone()
    ss.block(plan, w, x1, perm, routed)
    x2 = x0.clone()
    imp2, perm2, inv2, routed2 = ss.forward(plan, w, img, x2, patch=cfg.patch)
    assert torch.equal(imp.view(torch.int32), imp2.view(torch.int32))
    assert torch.equal(perm, perm2) and torch.equal(inv, inv2) and torch.equal(routed, routed2)
    assert torch.equal(x1.view(torch.int32), x2.view(torch.int32)), "block output of %s" % key


def test_forward_argument_checks():
    """sparsesam_forward rejects an image whose size is not the plan's grid times the
    patch, a null inv and a dynamic plan, before any launch (x is left untouched)."""
    import ctypes
    from synth import block_weights, token_features
    from structured_sparse_vit_amd import _lib
    cfg = config("c1")
    plan = _plan(cfg)
    w = ss.weights_to_device(block_weights(cfg, 0), plan)
    img = torch.from_numpy(images("c1")).to(DEV)
    x = torch.from_numpy(token_features(cfg, 0)).to(DEV)
    x0 = x.clone()
    imp = torch.empty(cfg.batch, cfg.grid * cfg.grid, dtype=torch.float32, device=DEV)
    n, rpi = plan.info["seq_len"], plan.info["routed_per_image"]
    perm = torch.empty(cfg.batch, n, dtype=torch.int32, device=DEV)
    inv = torch.empty_like(perm)
    routed = torch.empty(cfg.batch * rpi, dtype=torch.int32, device=DEV)
    ws = torch.empty(plan.info["block_workspace_bytes"], dtype=torch.uint8, device=DEV)
    bw = ss._block_weights(plan, w)
    lib = _lib.load()
    P = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)
    H, W = img.shape[1], img.shape[2]
    call = lambda plan_h, h, inv_t: lib.sparsesam_forward(plan_h, ctypes.byref(bw), P(img), cfg.batch, h, W,
                                                          cfg.patch, P(x), P(imp), P(perm), P(inv_t), P(routed),
                                                          P(ws), ws.numel(), None)
    assert call(plan.handle, H + cfg.patch, inv) == 1  # height is not grid_h * patch
    assert call(plan.handle, H, None) == 1             # inv missing
    dyn = ss.Plan.from_config(cfg.with_(routing="update"))
    assert call(dyn.handle, H, inv) == 1               # the plan chooses its keep-set per block
    torch.cuda.synchronize()
    assert torch.equal(x, x0)
    assert call(plan.handle, H, inv) == 0


@pytest.mark.parametrize("key,gain", [("c1", 10.0), ("c2", 3.0), ("c3b1", 3.0), ("ragged", 3.0)])
def test_block_parity_high_gain(key, gain):
    """Projection weights scaled up: the attention and MLP branches dominate the residual.
    (bf16 runs use a gain of 3 so the softmax stays far from one-hot.)"""
    _say("block high gain", key)
    _check_block(key, _run_block(key, gain=gain), gain)


@pytest.mark.parametrize("key,kind,density", [("c4", "global", None), ("c4", "window", None),
                                              ("c5", "global", None), ("c5", "window", None),
                                              ("c5", "global", 0.4), ("c5", "window", 0.4),
                                              ("c5", "global", 1.0), ("c5", "window", 1.0)])
def test_block_full_batch_sampled(key, kind, density):
    """One block of the ViT-L / ViT-H encoder configs at their full batch (8 and 16
    images: the launch shapes the encoder benchmark times, with the large-tile GEMM
    paths) against the oracle on sampled images: the first and the last. Images are
    independent, so the oracle runs each sampled image alone."""
    from synth import block_weights, token_features
    from synth.configs import global_variant, window_variant
    _say("block full batch", key, kind, density)
    base = config(key)
    if density is not None:  # the ViT-H sweep's other densities (attention and MLP alike)
        base = base.with_(attn_density=density, mlp_density=density)
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

@pytest.mark.parametrize("key,over", [
    ("c4", dict(channels=256, heads=4, mlp_hidden=512)),                 # ViT-L layout, head_dim 64
    ("c5", dict(channels=640, heads=8, mlp_hidden=1280)),                # ViT-H layout, head_dim 80
])
def test_encoder_matches_block_by_block_and_oracle(key, over):
    """An 8-block stack of an encoder config's layout at reduced width: global blocks at
    layers 1, 3, 5, 7, windowed elsewhere, one permutation set per block type. The native
    encoder equals the same blocks called one by one (deterministic kernels: bit-equal)
    and matches the fp64 oracle encoder at the contract bar (max-abs 1e-2, rel-L2 5e-3)."""
    _say("encoder 8 layers", key, over)
    from synth import block_weights, encoder_global_layers, token_features
    from synth.configs import global_variant, window_variant
    layers, b = 8, (2 if key == "c4" else 1)
    base = config(key).with_(batch=b, layers=layers, **over)
    cg, cw = global_variant(base).with_(batch=b), window_variant(base).with_(batch=b)
    pg, pw = _plan(cg), _plan(cw)
    imgs = np.stack([images(key)[i] for i in range(b)])
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
    mx, rel = check_close(got, want, what="encoder " + key)
    _say("  encoder %s max-abs %.3e rel-L2 %.3e" % (key, mx, rel))


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


def _encoder_pair(key, over, layers, b, rel_pos=False, full_weights=False):
    """The same encoder run with the raster-order stream (sparsesam_encoder) and with the
    stream kept in stripe-sorted order (sparsesam_encoder_permuted)."""
    from synth import block_weights, encoder_global_layers, token_features
    from synth.configs import global_variant, window_variant
    from synth.generate import rel_pos_tables
    base = config(key).with_(batch=b, layers=layers, **over)
    cg, cw = global_variant(base).with_(batch=b), window_variant(base).with_(batch=b)
    pg, pw = ss.Plan.from_config(cg, rel_pos=rel_pos), ss.Plan.from_config(cw, rel_pos=rel_pos)
    gl = encoder_global_layers(layers)
    kinds = [1 if l in gl else 0 for l in range(layers)]
    ws = [block_weights(base, 0, layer=0 if full_weights else l) for l in range(layers)]
    wd = []
    for l, w in enumerate(ws):
        if rel_pos:
            w = dict(w)
            w["rel_h"], w["rel_w"] = rel_pos_tables(cg if kinds[l] else cw, 0, layer=l)
        wd.append(ss.weights_to_device(w, pg))
    imp_d = ss.importance(torch.from_numpy(images(key)[:b].copy()).to(DEV), base.patch)
    perm_g, inv_g, routed_g = ss.permute(pg, imp_d)
    perm_w, inv_w, routed_w = ss.permute(pw, imp_d)
    x0 = token_features(base, 0)
    xa = torch.from_numpy(x0.copy()).to(DEV)
    ss.encoder(pg, pw, wd, kinds, xa, (perm_g, routed_g), (perm_w, routed_w))
    xb = torch.from_numpy(x0.copy()).to(DEV)
    ss.encoder(pg, pw, wd, kinds, xb, (perm_g, inv_g), (perm_w, inv_w), sorted_stream=True)
    torch.cuda.synchronize()
    return xa.cpu().numpy(), xb.cpu().numpy(), x0, imp_d.cpu().numpy(), ws, gl, cg, cw


@pytest.mark.parametrize("key,over,layers,b,rel_pos", [
    ("c4", dict(channels=256, heads=4, mlp_hidden=512), 8, 2, False),     # ViT-L layout
    ("c5", dict(channels=640, heads=8, mlp_hidden=1280), 8, 1, False),    # ViT-H layout, head_dim 80
    ("ragged", dict(), 8, 2, False),                                      # 18 x 18 grid: padded windows
    ("c4", dict(channels=256, heads=4, mlp_hidden=512), 8, 1, True),      # with the relative-position bias
])
def test_encoder_sorted_stream_equals_raster_stream(key, over, layers, b, rel_pos):
    """The residual stream kept in stripe-sorted order between blocks (one composed gather
    at each change of block type) gives the raster-order encoder's result bit for bit."""
    _say("encoder sorted stream", key, over, "rel_pos", rel_pos)
    a, s, x0, imp, ws, gl, cg, cw = _encoder_pair(key, over, layers, b, rel_pos)
    assert np.isfinite(s).all()
    assert np.array_equal(a.view(np.uint32), s.view(np.uint32))
    if not rel_pos and key == "ragged":
        mx, rel = check_close(s, oracle.encoder_forward(x0, imp, ws, gl, cg, cw), what="sorted-stream encoder")
        _say("  against the oracle: max-abs %.3e rel-L2 %.3e" % (mx, rel))


def test_encoder_sorted_stream_full_size():
    """The ViT-L encoder at full size (24 blocks, batch 8), one layer's weights reused."""
    _say("encoder sorted stream full size c4")
    a, s = _encoder_pair("c4", {}, 24, 8, full_weights=True)[:2]
    assert np.isfinite(s).all()
    assert np.array_equal(a.view(np.uint32), s.view(np.uint32))
