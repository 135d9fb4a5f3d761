"""GPU parity of the decomposed relative-position bias against the oracle.

sparsesam_attn_relpos on random q, k, v and a random slot permutation: the full ViT-B
global grid (bf16, matrix-core kernel), ViT-B and ViT-H windows and ragged windows
(bf16, the window kernel on 16-key blocks; the 32 x 32-block kernel for segments
whose key classes overflow its slots), the ViT-H global grid (head_dim 80: fp16 tables,
matrix-core kernel attn_d80_rel_kernel) and the fp32 tiny config (fp32 tables, SIMT
kernel); and blocks of rel_pos plans on the image pipeline. Bars as in test_gpu_parity: max-abs 1e-2 and relative L2 5e-3.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import structured_sparse_vit_amd as ss
from synth import block_weights, round_to_bf16, token_features
from synth.generate import rel_pos_tables
from tests.gpu_cases import check_close, config, images, rel_l2

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# Values at the scale of a ViT-B block's (LayerNorm output times N(0, 0.02) weights over
# 768 channels: std ~0.55). The bias sharpens the softmax, so an output approaches single
# value rows; with N(0, 1) values it reaches |o| ~ 4, where storing o in bf16 alone rounds
# by up to 2^-7 -- most of the 1e-2 bar. q and k stay N(0, 1) (logits sharper than a
# block's).
V_STD = 0.55


def _attn_relpos_case(key, seed=0, std=0.1, **over):
    cfg = config(key)
    if over:
        cfg = cfg.with_(**over)
    plan = ss.Plan.from_config(cfg)
    n, H, D = plan.info["seq_len"], cfg.heads, cfg.head_dim
    side = cfg.window or cfg.grid
    segs = cfg.batch * plan.info["segments_per_image"]
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((segs, H, n, D), dtype=np.float32) for _ in range(3))
    v = (v * np.float32(V_STD)).astype(np.float32)
    if cfg.dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    perm = np.stack([rng.permutation(n) for _ in range(segs)]).astype(np.int32)
    rh, rw = rel_pos_tables(cfg, seed, std=std)
    n_pad = (n + 7) // 8 * 8
    vt = np.full((segs, H, D, n_pad), np.nan, np.float32)  # pad columns must never be read
    vt[..., :n] = v.transpose(0, 1, 3, 2)
    dt = plan.torch_dtype
    dev = [torch.from_numpy(a).to(DEV, dt).contiguous() for a in (q, k, vt)]
    o = ss.attn_relpos(plan, *dev, torch.from_numpy(perm).to(DEV), torch.from_numpy(rh).to(DEV),
                       torch.from_numpy(rw).to(DEV)).float().cpu().numpy()
    keep = oracle.position_keep(n, cfg.stripes, cfg.block, cfg.global_tokens, plan.info["band_radius"])
    want = np.empty((segs, n, H * D))
    for s in range(segs):
        for h in range(H):
            q_slot = np.empty((n, D))
            q_slot[perm[s]] = q[s, h]  # position p holds slot perm[s, p]
            bias = oracle.rel_pos_bias(q_slot, side, side, rh, rw)[np.ix_(perm[s], perm[s])]
            want[s, :, h * D:(h + 1) * D] = oracle.masked_attention(q[s, h], k[s, h], v[s, h], keep, D ** -0.5,
                                                                    bias)
    return o, want, plan


@pytest.mark.parametrize("key", ["c2", "c1", "ragged", "c3b1", "c5w", "c5g"])
def test_attn_relpos_parity(key):
    _say("attention + relative position", key)
    o, want, plan = _attn_relpos_case(key)
    _say("  max-abs %.3e rel-L2 %.3e" % (np.abs(o - want).max(), rel_l2(o, want)))
    check_close(o, want, what="attention relpos " + key)


def test_attn_relpos_short_segment_sixteen_classes():
    """The bias on a 16 x 16 bf16 segment of sixteen key classes (one stripe of sixteen
    16-token tiles; the window kernel's 256 slots hold one 16-key block per class)."""
    _say("attention + relative position, sixteen key classes")
    over = dict(dtype="bf16", stripes=1, block=16, global_tokens=16, heads=2, head_dim=64, channels=128,
                mlp_hidden=256, attn_density=0.3)
    o, want, plan = _attn_relpos_case("c1", seed=9, **over)
    _say("  max-abs %.3e rel-L2 %.3e" % (np.abs(o - want).max(), rel_l2(o, want)))
    check_close(o, want, what="attention relpos, sixteen key classes")


@pytest.mark.parametrize("grid_h,grid_w,block,head_dim", [(16, 15, 8, 64), (15, 17, 17, 80)])
def test_attn_relpos_window_slots_overflow(grid_h, grid_w, block, head_dim):
    """The bias on short global segments whose key classes do not fit the window kernel's
    256 LDS slots in 16-key blocks: the 32 x 32-block window kernel with two (30 classes)
    or one (15 classes) mask k-steps."""
    _say("attention + relative position, slot overflow", grid_h, grid_w, block, head_dim)
    heads = 2 if head_dim == 64 else 8  # bf16 plans take channels in multiples of 128
    plan = ss.Plan(grid_h, grid_w, 0, 1, block, block, -1, 0.3, 0.4, heads * head_dim, heads, head_dim, 256, 1,
                   "bf16", rel_pos=True)
    n, D = plan.info["seq_len"], head_dim
    rng = np.random.default_rng(13)
    q, k, v = (round_to_bf16(rng.standard_normal((1, heads, n, D), dtype=np.float32)) for _ in range(3))
    v = round_to_bf16((v * np.float32(V_STD)).astype(np.float32))
    perm = rng.permutation(n).astype(np.int32)[None]
    rh = (rng.standard_normal((2 * grid_h - 1, D), dtype=np.float32) * np.float32(0.1)).astype(np.float32)
    rw = (rng.standard_normal((2 * grid_w - 1, D), dtype=np.float32) * np.float32(0.1)).astype(np.float32)
    n_pad = (n + 7) // 8 * 8
    vt = np.full((1, heads, D, n_pad), np.nan, np.float32)
    vt[..., :n] = v.transpose(0, 1, 3, 2)
    dev = [torch.from_numpy(a).to(DEV, torch.bfloat16).contiguous() for a in (q, k, vt)]
    o = ss.attn_relpos(plan, *dev, torch.from_numpy(perm).to(DEV), torch.from_numpy(rh).to(DEV),
                       torch.from_numpy(rw).to(DEV)).float().cpu().numpy()
    keep = oracle.position_keep(n, 1, block, block, plan.info["band_radius"])
    want = np.empty((n, heads * D))
    for h in range(heads):
        q_slot = np.empty((n, D))
        q_slot[perm[0]] = q[0, h]
        bias = oracle.rel_pos_bias(q_slot, grid_h, grid_w, rh, rw)[np.ix_(perm[0], perm[0])]
        want[:, h * D:(h + 1) * D] = oracle.masked_attention(q[0, h], k[0, h], v[0, h], keep, D ** -0.5, bias)
    _say("  max-abs %.3e rel-L2 %.3e" % (np.abs(o[0] - want).max(), rel_l2(o[0], want)))
    check_close(o[0], want, what="attention relpos, slot overflow %dx%d B%d D%d" % (grid_h, grid_w, block, D))


def test_attn_relpos_bias_matters_and_zero_tables_match_plain():
    """At the synthetic tables' default scale (bias about 1.6 logits) the c2 outputs move
    far past the bar, and zero tables give the unbiased result."""
    o, want, plan = _attn_relpos_case("c2", seed=2, std=0.2)
    _say("  std 0.2: max-abs %.3e rel-L2 %.3e" % (np.abs(o - want).max(), rel_l2(o, want)))
    check_close(o, want, what="attention relpos c2 std 0.2")
    o0, want0, _ = _attn_relpos_case("c2", seed=2, std=0.0)
    check_close(o0, want0, what="attention relpos c2 zero tables")
    assert rel_l2(want, want0) > 0.1


def test_attn_relpos_dense_pattern():
    _say("attention + relative position, density 1")
    o, want, _ = _attn_relpos_case("c2", seed=5, attn_density=1.0)
    check_close(o, want, what="dense attention relpos c2")


@pytest.mark.parametrize("key", ["c1", "ragged", "c2"])
def test_block_relpos_parity(key):
    _say("block + relative position", key)
    cfg = config(key)
    seed = 0
    x = token_features(cfg, seed)
    w = block_weights(cfg, seed)
    rh, rw = rel_pos_tables(cfg, seed)
    wr = dict(w, rel_h=rh, rel_w=rw)
    imp = np.stack([oracle.importance(im, cfg.patch) for im in images(key, seed)])
    want = oracle.block_forward(x, imp, wr, cfg)
    plan = ss.Plan.from_config(cfg, rel_pos=True)
    img = torch.from_numpy(images(key, seed)).to(DEV)
    perm, inv, routed = ss.permute(plan, ss.importance(img, cfg.patch))
    wd = ss.weights_to_device(wr, plan)
    xd = torch.from_numpy(x.copy()).to(DEV)
    ss.block(plan, wd, xd, perm, routed)
    got = xd.cpu().numpy()
    check_close(got, want, what="block relpos " + key)
    plain = oracle.block_forward(x, imp, w, cfg)
    # the bias is visible in the result: the plain block is farther off than the bar
    assert rel_l2(got - x, plain - x) > 5 * max(rel_l2(got - x, want - x), 1e-4)


def test_block_relpos_plan_checks_tables():
    cfg = config("c1")
    plan = ss.Plan.from_config(cfg, rel_pos=True)
    w = ss.weights_to_device(block_weights(cfg, 0), plan)
    x = torch.zeros(cfg.batch, cfg.grid, cfg.grid, cfg.channels, device=DEV)
    perm = torch.zeros(cfg.batch, plan.info["seq_len"], dtype=torch.int32, device=DEV)
    routed = torch.zeros(cfg.batch * plan.info["routed_per_image"], dtype=torch.int32, device=DEV)
    with pytest.raises(TypeError):
        ss.block(plan, w, x, perm, routed)  # rel_pos_h missing
