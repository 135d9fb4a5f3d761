"""CPU-only checks of the C-ABI library: it loads, exports every declared symbol,
builds the static tile list on the host, and validates arguments before any launch."""
import ctypes
import os
import re

import numpy as np
import pytest

import structured_sparse_vit_amd as ss
from oracle import band_radius, position_keep, routed_count, window_token_map
from structured_sparse_vit_amd import _lib
from synth import get_config
from synth.configs import global_variant
from tests.conftest import ROOT

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libsparsesam.so not built")


def _declared_symbols():
    with open(os.path.join(ROOT, "include", "sparsesam.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sparsesam_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    declared = _declared_symbols()
    assert set(declared) == set(_lib.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


# The entry points the boundary table lists by name (plan lifecycle and queries, the
# five hot-path calls); this library exports each of them.
BOUNDARY_NAMES = ["sparsesam_plan_create", "sparsesam_plan_info_get", "sparsesam_plan_block_list",
                  "sparsesam_plan_destroy", "sparsesam_status_string", "sparsesam_last_error",
                  "sparsesam_importance", "sparsesam_permute", "sparsesam_attn", "sparsesam_mlp", "sparsesam_block"]


def test_library_exports_the_boundary_names():
    lib = _lib.load()
    declared = set(_declared_symbols())
    for name in BOUNDARY_NAMES:
        assert name in declared, name
        assert hasattr(lib, name), name


def test_boundary_aliases_agree():
    """sparsesam_plan_info_get / sparsesam_plan_block_list return what
    sparsesam_plan_get_info / sparsesam_plan_tile_list return."""
    import ctypes

    import numpy as np
    lib = _lib.load()
    d = _lib.PlanDesc(64, 64, 0, 4, 64, 64, -1, 0.4, 0.4, 768, 12, 64, 3072, 1, 1, 0, 0, 0)
    h = ctypes.c_void_p()
    assert lib.sparsesam_plan_create(ctypes.byref(d), ctypes.byref(h)) == 0
    try:
        a, b = _lib.PlanInfo(), _lib.PlanInfo()
        assert lib.sparsesam_plan_get_info(h, ctypes.byref(a)) == 0
        assert lib.sparsesam_plan_info_get(h, ctypes.byref(b)) == 0
        assert bytes(a) == bytes(b)
        assert a.tiles_kept == 1696
        rp1, rp2 = np.zeros(a.tiles + 1, np.int32), np.zeros(a.tiles + 1, np.int32)
        ci1, ci2 = np.zeros(a.tiles_kept, np.int32), np.zeros(a.tiles_kept, np.int32)
        vp = lambda v: v.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
        assert lib.sparsesam_plan_tile_list(h, vp(rp1), vp(ci1)) == 0
        assert lib.sparsesam_plan_block_list(h, vp(rp2), vp(ci2)) == 0
        assert np.array_equal(rp1, rp2) and np.array_equal(ci1, ci2)
        assert lib.sparsesam_plan_info_get(None, ctypes.byref(b)) == 1
        assert lib.sparsesam_plan_block_list(None, vp(rp2), vp(ci2)) == 1
    finally:
        lib.sparsesam_plan_destroy(h)


def test_status_strings():
    lib = _lib.load()
    for code in range(7):
        assert lib.sparsesam_status_string(code)
    assert lib.sparsesam_status_string(99) == b"unknown status"


def _tile_pairs_from_oracle(n, g, B, G, r):
    keep = position_keep(n, g, B, G, r)
    S = n // g
    nbs = -(-S // B)
    pos = np.arange(n)
    tile = (pos // S) * nbs + (pos % S) // B
    T = g * nbs
    kept = np.zeros((T, T), bool)
    qi, ki = np.nonzero(keep)
    kept[tile[qi], tile[ki]] = True
    return kept, int(keep.sum())


@pytest.mark.parametrize("key", ["c1", "c2", "c3", "c4", "c4g", "c5"])
def test_plan_matches_oracle_pattern(key):
    cfg = global_variant(get_config("c4")) if key == "c4g" else get_config(key)
    plan = ss.Plan.from_config(cfg)
    info = plan.info
    n = cfg.window ** 2 if cfg.window else cfg.grid ** 2
    r = band_radius(n, cfg.stripes, cfg.block, cfg.global_tokens, cfg.attn_density)
    assert info["seq_len"] == n
    assert info["band_radius"] == r
    kept, pairs = _tile_pairs_from_oracle(n, cfg.stripes, cfg.block, cfg.global_tokens, r)
    rp, ci = plan.tile_list()
    got = np.zeros_like(kept)
    for t in range(info["tiles"]):
        got[t, ci[rp[t]:rp[t + 1]]] = True
    assert np.array_equal(got, kept)
    assert info["tiles_kept"] == kept.sum()
    assert info["pairs_kept"] == pairs
    assert abs(info["realised_density"] - pairs / n ** 2) < 1e-15
    # keep-set size per image
    tm = window_token_map(cfg.grid, cfg.grid, cfg.window) if cfg.window else np.arange(n)[None]
    want = sum(routed_count(cfg.mlp_density, int((row >= 0).sum())) for row in tm)
    assert info["routed_per_image"] == want


def test_plan_known_values():
    info = ss.Plan.from_config(get_config("c2")).info
    assert (info["band_radius"], info["tiles_kept"], info["routed_per_image"]) == (3, 1696, 1638)
    assert abs(info["realised_density"] - 0.4140625) < 1e-12
    info = ss.Plan.from_config(get_config("c3")).info
    assert (info["band_radius"], info["tiles_kept"], info["pairs_kept"], info["routed_per_image"]) == (0, 88, 16528, 1634)
    info = ss.Plan.from_config(get_config("c1")).info
    assert (info["band_radius"], info["tiles_kept"], info["routed_per_image"]) == (1, 112, 102)


def test_plan_density_one_is_dense():
    cfg = get_config("c2").with_(attn_density=1.0, mlp_density=1.0)
    info = ss.Plan.from_config(cfg).info
    assert info["tiles_kept"] == info["tiles"] ** 2
    assert info["realised_density"] == 1.0
    assert info["routed_per_image"] == 4096


def _create(**over):
    cfg = get_config("c2")
    d = dict(grid_h=64, grid_w=64, window=0, stripes=4, block=64, global_tokens=64, band_radius=-1,
             attn_density=0.4, mlp_density=0.4, channels=768, heads=12, head_dim=64, mlp_hidden=3072,
             max_batch=1, dtype="bf16")
    d.update(over)
    return ss.Plan(**d)


@pytest.mark.parametrize("over,status", [
    (dict(stripes=3), 1),                # 4096 % 3 != 0
    (dict(block=0), 1),
    (dict(block=2000), 1),               # > S
    (dict(global_tokens=32), 1),         # not a multiple of block
    (dict(attn_density=0.0), 1),
    (dict(attn_density=1.5), 1),
    (dict(mlp_density=-0.1), 1),
    (dict(channels=700), 1),             # != heads * head_dim
    (dict(max_batch=0), 1),
    (dict(band_radius=-2), 1),
    (dict(head_dim=48, channels=576), 2),
    (dict(channels=1600, heads=20, head_dim=80), 2),
    (dict(window=128, grid_h=128, grid_w=128, block=64, global_tokens=64), 2),  # 16384 keys in LDS is fine ...
])
def test_plan_validation(over, status):
    if over.get("window") == 128:
        # 1 window of 16384 tokens: sort keys need 128 KiB + flags: accepted
        _create(**over)
        return
    with pytest.raises(ss.SparseSAMError) as ei:
        _create(**over)
    assert ei.value.status == status


def test_plan_rejects_sort_beyond_lds():
    with pytest.raises(ss.SparseSAMError) as ei:
        _create(grid_h=256, grid_w=256, block=64, global_tokens=64)
    assert ei.value.status == 2


def test_compute_calls_without_device_return_no_device():
    lib = _lib.load()
    plan = _create()
    if plan.info["has_device_copy"]:
        pytest.skip("a GPU is present")
    p = ctypes.c_void_p(16)
    st = lib.sparsesam_permute(plan.handle, p, 1, p, p, p, None)
    assert st == 6
    st = lib.sparsesam_attn(plan.handle, 1, p, p, p, p, ctypes.c_float(0.125), p, 1 << 20, None)
    assert st == 6
    assert b"no device copy" in lib.sparsesam_last_error()


def test_importance_argument_validation_before_launch():
    lib = _lib.load()
    p = ctypes.c_void_p(16)
    assert lib.sparsesam_importance(p, 1, 100, 64, 16, p, None) == 1   # 100 % 16
    assert lib.sparsesam_importance(p, 1, 64, 64, 64, p, None) == 2    # patch > 32
    assert lib.sparsesam_importance(None, 1, 64, 64, 16, p, None) == 1
    assert lib.sparsesam_importance(p, -1, 64, 64, 16, p, None) == 1
    assert lib.sparsesam_importance(None, 0, 64, 64, 16, None, None) == 0  # empty batch is a no-op


def test_null_plan_and_info():
    lib = _lib.load()
    assert lib.sparsesam_plan_create(None, None) == 1
    assert lib.sparsesam_plan_get_info(None, None) == 1
    lib.sparsesam_plan_destroy(None)


def test_encoder_validation_before_launch():
    """sparsesam_encoder rejects bad layer kinds, missing or mismatched plans before any
    launch (these checks come before the device check, so they run without a GPU)."""
    lib = _lib.load()
    g = _create()
    w_cfg = get_config("c3").with_(channels=g.desc.channels, heads=g.desc.heads, head_dim=g.desc.head_dim,
                                   mlp_hidden=g.desc.mlp_hidden)
    w = ss.Plan.from_config(w_cfg)
    layers = (_lib.BlockWeights * 2)()
    p = ctypes.c_void_p(16)

    def call(gp, wp, kinds, n=2):
        karr = (ctypes.c_uint8 * 2)(*kinds)
        return lib.sparsesam_encoder(gp, wp, layers, karr, n, p, 1, p, p, p, p, p, 1 << 30, None)

    assert call(g.handle, w.handle, [1, 0], n=0) == 0          # no layers: a no-op
    assert call(g.handle, w.handle, [1, 2]) == 1                # kinds outside {0, 1}
    assert call(None, w.handle, [1, 0]) == 1                    # a global layer without a global plan
    assert call(g.handle, None, [1, 0]) == 1                    # a windowed layer without a window plan
    assert lib.sparsesam_encoder(g.handle, w.handle, None, None, 2, p, 1, p, p, p, p, p, 1, None) == 1
    assert lib.sparsesam_encoder(g.handle, w.handle, layers, (ctypes.c_uint8 * 2)(1, 0), -1, p, 1, p, p, p, p, p,
                                 1, None) == 1
    other = ss.Plan.from_config(w_cfg.with_(channels=2 * g.desc.channels, heads=2 * g.desc.heads))
    assert call(g.handle, other.handle, [1, 0]) == 1            # plans of different shapes
    assert b"share grid" in lib.sparsesam_last_error()


# ------------------------------------------------------------------ relative-position bias

def test_relpos_plan_validation_and_workspace():
    # rel_pos is a flag
    lib = _lib.load()
    d = _create().desc
    d.rel_pos = 2
    h = ctypes.c_void_p()
    assert lib.sparsesam_plan_create(ctypes.byref(d), ctypes.byref(h)) == 1
    # segments above 64 x 64 and head_dim above 80 have no bias tables
    for over in (dict(grid_h=128, grid_w=128, block=64, global_tokens=64), dict(head_dim=128, heads=6, dtype="f32")):
        with pytest.raises(ss.SparseSAMError) as ei:
            _create(rel_pos=True, **over)
        assert ei.value.status == 2
        assert _create(**over).info["relpos_workspace_bytes"] == 0
    # the workspace is proportional to the segment count (callers scale it per segment)
    for over in (dict(), dict(window=14, stripes=4, block=16, global_tokens=16, max_batch=3)):
        plan = _create(rel_pos=True, **over)
        segs = plan.desc.max_batch * plan.info["segments_per_image"]
        total = plan.info["relpos_workspace_bytes"]
        assert total > 0 and total % segs == 0
        per_seg = total // segs
        n, tj = plan.info["seq_len"], 128 if not over else 32
        assert per_seg >= plan.desc.heads * n * tj * 4 + n * 4
        # a rel_pos plan's block workspace holds the tables on top of the plain block's
        assert plan.info["block_workspace_bytes"] > _create(**over).info["block_workspace_bytes"]


def test_attn_relpos_validation_before_launch():
    lib = _lib.load()
    plan = _create()
    p = ctypes.c_void_p(256)
    f = ctypes.c_float(0.125)
    if plan.info["has_device_copy"]:
        # argument checks that come before any launch
        assert lib.sparsesam_attn_relpos(plan.handle, 1, p, p, p, p, f, None, p, p, p, 1 << 30, None) == 1
        assert lib.sparsesam_attn_relpos(plan.handle, 1, p, p, p, p, f, p, ctypes.c_void_p(260), p, p, 1 << 30,
                                         None) == 1  # rel_h not 16-byte aligned
        assert lib.sparsesam_attn_relpos(plan.handle, 1, p, p, p, p, ctypes.c_float(0.0), p, p, p, p, 1 << 30,
                                         None) == 1
        assert lib.sparsesam_attn_relpos(plan.handle, 1, p, p, p, p, f, p, p, p, p, 16, None) == 3  # workspace
    else:
        assert lib.sparsesam_attn_relpos(plan.handle, 1, p, p, p, p, f, p, p, p, p, 1 << 30, None) == 6


# ------------------------------------------------------------------ dynamic routing and the merge

def test_routing_and_merge_plan_validation_and_workspace():
    base = _create()
    dyn = _create(routing="update")
    mrg = _create(mlp_merge=True)
    both = _create(routing="update", mlp_merge=True)
    # the dynamic plan adds the squared-update partials (one fp32 per 32 channels per token),
    # the merge the keep-set's fp32 updates; the pattern and keep-set size are unchanged
    assert dyn.info["block_workspace_bytes"] >= base.info["block_workspace_bytes"] + 4096 * 24 * 4
    assert mrg.info["block_workspace_bytes"] >= 1638 * (768 * 2 + 3072 * 2) + 1638 * 768 * 4
    assert both.info["block_workspace_bytes"] >= max(dyn.info["block_workspace_bytes"],
                                                     mrg.info["block_workspace_bytes"])
    for p in (dyn, mrg, both):
        assert p.info["tiles_kept"] == base.info["tiles_kept"]
        assert p.info["routed_per_image"] == base.info["routed_per_image"]
    lib = _lib.load()
    for field, val in (("routing", 2), ("routing", -1), ("mlp_merge", 2)):
        d = _lib.PlanDesc(64, 64, 0, 4, 64, 64, -1, 0.4, 0.4, 768, 12, 64, 3072, 1, 1, 0, 0, 0, 0, 0)
        setattr(d, field, val)
        h = ctypes.c_void_p()
        assert lib.sparsesam_plan_create(ctypes.byref(d), ctypes.byref(h)) == 1, field
    # the merge keeps a bit per slot of a segment in LDS: at most 16384 slots
    with pytest.raises(ss.SparseSAMError) as ei:
        _create(grid_h=160, grid_w=160, block=40, global_tokens=40, mlp_merge=True, channels=768)
    assert ei.value.status == 2


def test_routing_entry_points_check_the_plan_kind_first():
    """Block calls check the plan's routing before anything else (so without a GPU too):
    sparsesam_block and sparsesam_forward reject dynamic plans, sparsesam_block_dynamic
    static ones, and the encoder does not take dynamic plans."""
    lib = _lib.load()
    dyn, sta = _create(routing="update"), _create()
    w = _lib.BlockWeights()
    p = ctypes.c_void_p(16)
    assert lib.sparsesam_block(dyn.handle, ctypes.byref(w), p, 1, p, p, p, 1 << 30, None) == 1
    assert b"sparsesam_block_dynamic" in lib.sparsesam_last_error()
    assert lib.sparsesam_block_dynamic(sta.handle, ctypes.byref(w), p, 1, p, p, None, p, 1 << 30, None) == 1
    assert lib.sparsesam_forward(dyn.handle, ctypes.byref(w), p, 1, 1024, 1024, 16, p, p, p, p, p, p, 1 << 30,
                                 None) == 1
    assert b"sparsesam_block_dynamic" in lib.sparsesam_last_error()
    assert lib.sparsesam_block_noalloc(dyn.handle, ctypes.byref(w), p, 1, p, p, None) in (1, 6)
    layers = (_lib.BlockWeights * 1)()
    karr = (ctypes.c_uint8 * 1)(1)
    assert lib.sparsesam_encoder(dyn.handle, None, layers, karr, 1, p, 1, p, p, p, p, p, 1 << 30, None) == 2
    assert lib.sparsesam_route_topk(None, p, 1, p, None) == 1


def test_sorted_stream_encoder_workspace_and_checks():
    lib = _lib.load()
    g = _create()
    w_cfg = get_config("c3").with_(channels=g.desc.channels, heads=g.desc.heads, head_dim=g.desc.head_dim,
                                   mlp_hidden=g.desc.mlp_hidden)
    w = ss.Plan.from_config(w_cfg)
    need = ctypes.c_size_t()
    assert lib.sparsesam_encoder_permuted_workspace(g.handle, w.handle, 4, ctypes.byref(need)) == 0
    # two stream buffers of the windowed order (100 windows x 196 rows, larger than raster) + a block workspace
    assert need.value >= 2 * 4 * 25 * 196 * 768 * 4 + w.info["block_workspace_bytes"] * 4 // 4
    assert lib.sparsesam_encoder_permuted_workspace(None, None, 1, ctypes.byref(need)) == 1
    layers = (_lib.BlockWeights * 2)()
    karr = (ctypes.c_uint8 * 2)(1, 0)
    p = ctypes.c_void_p(16)
    assert lib.sparsesam_encoder_permuted(g.handle, w.handle, layers, karr, 0, p, 1, p, p, p, p, p, 1, None) == 0
    assert lib.sparsesam_encoder_permuted(None, w.handle, layers, karr, 2, p, 1, p, p, p, p, p, 1 << 40,
                                          None) == 1
    m = _create(mlp_merge=True)
    assert lib.sparsesam_encoder_permuted(m.handle, None, layers, (ctypes.c_uint8 * 2)(1, 1), 2, p, 1, p, p, p, p, p,
                                          1 << 40, None) == 2


def test_window_kernel_tables(tmp_path):
    """The window kernel's slot map, key blocks and query groups, checked on the host by
    tests/window_tables_check.cpp for ViT-B/H windows, partial windows, short global
    segments, two plans whose classes overflow the 256 slots, and a sweep of about 3500
    short-segment plan shapes."""
    import shutil
    import subprocess
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    exe = str(tmp_path / "window_tables_check")
    lib_dir = os.path.dirname(_lib.LIB_PATH)
    cmd = [hipcc, "-std=c++17", "-O1", "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "structured_sparse_vit_amd", "csrc"),
           os.path.join(ROOT, "tests", "window_tables_check.cpp"), "-L" + lib_dir, "-lsparsesam",
           "-Wl,-rpath," + lib_dir, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("all ok"), r.stdout[-2000:]

