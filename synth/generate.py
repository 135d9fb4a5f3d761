"""Seeded generators for images, token features and block weights.

Every array comes from numpy's PCG64 generator seeded by (purpose, seed, index),
so the oracle side and the HIP side read identical bits. Nothing here computes
any step of the method.

Image recipe (a stand-in for the segmentation benchmarks the pages evaluate on,
which are not available here): a zero canvas; rectangles with a uniform top-left
corner and sides uniform in [H/16, H/2]; ellipses with a uniform centre and
semi-axes uniform in [H/32, H/4]; each shape filled with an intensity uniform in
[0, 1], painted in order over what is there; then i.i.d. N(0, noise) per pixel,
no clipping; stored as fp32.
"""
import numpy as np

_PURPOSE = {"image": 1, "features": 2, "weights": 3, "rel_pos": 4}


def _rng(purpose: str, seed: int, index: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([_PURPOSE[purpose], int(seed), int(index)]))


def synthetic_image(size: int, n_rect: int, n_ellipse: int, seed: int, index: int = 0,
                    noise: float = 0.05) -> np.ndarray:
    """One grayscale image [size, size] fp32 of filled rectangles and ellipses plus noise.

    ``noise = 0`` gives the noise-free variant, whose flat regions produce exact ties.
    """
    rng = _rng("image", seed, index)
    img = np.zeros((size, size), np.float32)
    yy, xx = np.mgrid[0:size, 0:size]
    for _ in range(n_rect):
        y0, x0 = rng.integers(0, size, size=2)
        h, w = rng.integers(size // 16, size // 2 + 1, size=2)
        val = np.float32(rng.uniform(0.0, 1.0))
        img[y0:y0 + h, x0:x0 + w] = val
    for _ in range(n_ellipse):
        cy, cx = rng.uniform(0, size, size=2)
        ry, rx = rng.uniform(size / 32, size / 4, size=2)
        val = np.float32(rng.uniform(0.0, 1.0))
        inside = ((yy - cy) / ry) ** 2 + ((xx - cx) / rx) ** 2 <= 1.0
        img[inside] = val
    if noise > 0:
        img = img + rng.normal(0.0, noise, size=(size, size)).astype(np.float32)
    return img.astype(np.float32)


def synthetic_images(cfg, seed: int = 0, noise: float = 0.05) -> np.ndarray:
    """[batch, image, image] fp32, one independent image per batch element."""
    return np.stack([synthetic_image(cfg.image, cfg.shapes_rect, cfg.shapes_ellipse, seed, i, noise)
                     for i in range(cfg.batch)])


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bfloat16 (ties to even), returned as fp32."""
    a = np.ascontiguousarray(a, np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32).reshape(a.shape)


def token_features(cfg, seed: int = 0) -> np.ndarray:
    """Residual-stream input x ~ N(0, 1), fp32 [batch, grid, grid, C]."""
    rng = _rng("features", seed)
    g = cfg.grid
    return rng.standard_normal((cfg.batch, g, g, cfg.channels), dtype=np.float32)


def block_weights(cfg, seed: int = 0, layer: int = 0, gain: float = 1.0) -> dict:
    """Parameters of one pre-LN ViT block, matrices in [out, in] layout.

    Matrices and biases ~ N(0, 0.02); LayerNorm gamma = 1 + N(0, 0.02), beta ~ N(0, 0.02).
    ``gain`` scales the projection matrices (w_qkv, w_proj, w1, w2): tests use gain > 1 so
    the attention and MLP branches are large next to the residual and a mistake in either
    stands out.
    For bf16 configs every matrix and bias is rounded to bf16 values (still stored as
    fp32 here), so that both sides read exactly the same numbers.
    """
    rng = _rng("weights", seed, layer)
    C, Hm = cfg.channels, cfg.mlp_hidden

    def n(*shape):
        return (rng.standard_normal(shape, dtype=np.float32) * np.float32(0.02)).astype(np.float32)

    w = {
        "ln1_g": (1.0 + n(C)).astype(np.float32),
        "ln1_b": n(C),
        "w_qkv": n(3 * C, C),
        "b_qkv": n(3 * C),
        "w_proj": n(C, C),
        "b_proj": n(C),
        "ln2_g": (1.0 + n(C)).astype(np.float32),
        "ln2_b": n(C),
        "w1": n(Hm, C),
        "b1": n(Hm),
        "w2": n(C, Hm),
        "b2": n(C),
    }
    if gain != 1.0:
        for k in ("w_qkv", "w_proj", "w1", "w2"):
            w[k] = (w[k] * np.float32(gain)).astype(np.float32)
    if cfg.dtype == "bf16":
        for k in ("w_qkv", "b_qkv", "w_proj", "b_proj", "w1", "b1", "w2", "b2"):
            w[k] = round_to_bf16(w[k])
    return w


def rel_pos_tables(cfg, seed: int = 0, layer: int = 0, std: float = 0.2) -> tuple:
    """Decomposed relative-position tables of one block: rel_h [2 Sh - 1, D] and rel_w
    [2 Sw - 1, D] fp32 ~ N(0, std), Sh x Sw the segment shape (the grid for global
    attention, the window otherwise). SAM starts them at zero; a trained encoder's are
    not, so the synthetic ones are drawn at a scale where the bias moves the logits by
    about one unit.
    """
    rng = _rng("rel_pos", seed, layer)
    side = cfg.window if cfg.window else cfg.grid
    D = cfg.head_dim
    rh = (rng.standard_normal((2 * side - 1, D), dtype=np.float32) * np.float32(std)).astype(np.float32)
    rw = (rng.standard_normal((2 * side - 1, D), dtype=np.float32) * np.float32(std)).astype(np.float32)
    return rh, rw


def encoder_global_layers(layers: int) -> list:
    """Indices of the global-attention blocks in an encoder of ``layers`` blocks.

    Four equally spaced global blocks, the last block among them: (k + 1) * L / 4 - 1.
    """
    return [(k + 1) * layers // 4 - 1 for k in range(4)]
