"""Shared inputs and oracle results for the GPU parity tests (cached per process)."""
import functools

import numpy as np

import oracle
from synth import block_weights, get_config, synthetic_images, token_features
from synth.configs import global_variant, window_variant

# Floating-point bar for every float output, from the method's target tolerances.
MAX_ABS = 1e-2
REL_L2 = 5e-3


def config(key):
    """Named workloads of the tests: the configs plus reduced encoder blocks; "key:order"
    is workload `key` with another token ordering (seed 12345 for the random one)."""
    if ":" in key:
        base, ordering = key.split(":")
        return config(base).with_(ordering=ordering, order_seed=12345)
    if key == "c4g":
        return global_variant(get_config("c4")).with_(batch=1)
    if key == "c4w":
        return window_variant(get_config("c4")).with_(batch=1)
    if key == "c5g":
        return global_variant(get_config("c5")).with_(batch=1)
    if key == "c5w":
        return window_variant(get_config("c5")).with_(batch=1)
    if key == "c3b1":
        return get_config("c3").with_(batch=1)
    if key == "ragged":  # 18 x 18 grid: four windows, three of them partial; small channels
        return get_config("c3").with_(batch=2, image=288, channels=128, heads=2, mlp_hidden=256)
    if key == "c1odd":  # fp32, head_dim 32 (16 threads per query), MLP hidden 200: ragged GEMM K and N
        return get_config("c1").with_(channels=96, heads=3, head_dim=32, mlp_hidden=200)
    return get_config(key)


@functools.lru_cache(maxsize=None)
def images(key, seed=0, noise=0.05):
    return synthetic_images(config(key), seed, noise)


@functools.lru_cache(maxsize=None)
def oracle_importance(key, seed=0, noise=0.05):
    cfg = config(key)
    return np.stack([oracle.importance(im, cfg.patch) for im in images(key, seed, noise)])


@functools.lru_cache(maxsize=None)
def oracle_block(key, seed=0, gain=1.0):
    cfg = config(key)
    x = token_features(cfg, seed)
    w = block_weights(cfg, seed, gain=gain)
    imp = oracle_importance(key, seed)
    out, parts = oracle.block_forward(x, imp, w, cfg, return_parts=True)
    return x, w, imp, out, parts


def rel_l2(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    return float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30))


def check_close(got, want, max_abs=MAX_ABS, rel_l2=REL_L2, what=""):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.isfinite(got).all(), what + ": non-finite output"
    err = np.abs(got - want)
    mx = float(err.max()) if err.size else 0.0
    rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30))
    assert mx <= max_abs, "%s: max-abs %.3e > %.1e" % (what, mx, max_abs)
    assert rel <= rel_l2, "%s: rel-L2 %.3e > %.1e" % (what, rel, rel_l2)
    return mx, rel
