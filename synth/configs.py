"""Workload definitions: one SAM-shaped encoder block or encoder per entry.

Sizes follow SAM's image encoder: a 1024 x 1024 input cut into 16 x 16 patches
gives a 64 x 64 token grid; windowed blocks use 14 x 14 windows over the grid
padded to 70 x 70; global blocks attend over all 4096 tokens. The tiny entry is
a 256 x 256 image (16 x 16 grid) used where the oracle must finish quickly.

Pattern fields: ``stripes`` is the number g of stripes the stripe-sort produces
(the pages' 4 x 4 mosaic means g = 4), ``block`` the pattern tile B in tokens,
``global_tokens`` the size G of the global keep-set, ``band_radius`` -1 asks
for the smallest band whose realised density reaches ``attn_density``.
"""
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Config:
    name: str
    batch: int
    image: int            # square image side in pixels
    patch: int            # pixels per token side
    shapes_rect: int      # rectangles painted into the synthetic image
    shapes_ellipse: int   # ellipses painted into the synthetic image
    channels: int
    heads: int
    head_dim: int
    mlp_hidden: int
    window: int           # 0 = global attention, w = w x w windows
    stripes: int
    block: int
    global_tokens: int
    band_radius: int
    attn_density: float
    mlp_density: float
    dtype: str            # "f32" or "bf16": weights and matrix-engine operands
    layers: int = 1       # encoder depth (1 = a single block)
    ordering: str = "importance"  # token order ahead of the stripe-sort (see oracle.ORDERINGS)
    order_seed: int = 0           # seed of the "random" ordering
    routing: str = "importance"   # MLP keep-set: the importance order, or "update" (this block's attention update)
    mlp_merge: bool = False       # the keep-set's mean MLP update added to the segment's other tokens

    @property
    def grid(self) -> int:
        return self.image // self.patch

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


CONFIGS = {
    # Tiny single block, fp32: 16 x 16 grid, C 64, one head, 2 stripes (2 x 2 mosaic),
    # B = G = 16, density 0.4, MLP 256 on 40 % of tokens.
    "c1": Config("c1_tiny_f32", 1, 256, 16, 8, 0, 64, 1, 64, 256, 0, 2, 16, 16, -1, 0.4, 0.4, "f32"),
    # SAM ViT-B global-attention block, bf16, batch 1.
    "c2": Config("c2_vitb_global_b1", 1, 1024, 16, 8, 8, 768, 12, 64, 3072, 0, 4, 64, 64, -1, 0.4, 0.4, "bf16"),
    # SAM ViT-B windowed block, bf16, batch 4: 25 windows of 14 x 14 per image.
    "c3": Config("c3_vitb_window_b4", 4, 1024, 16, 8, 8, 768, 12, 64, 3072, 14, 4, 16, 16, -1, 0.4, 0.4, "bf16"),
    # SAM ViT-L-shaped encoder, bf16, batch 8, 24 blocks (4 global), density 0.3.
    "c4": Config("c4_vitl_encoder_b8", 8, 1024, 16, 8, 8, 1024, 16, 64, 4096, 14, 4, 16, 16, -1, 0.3, 0.3, "bf16", 24),
    # SAM ViT-H-shaped encoder, bf16, batch 16, 32 blocks (4 global), head_dim 80.
    "c5": Config("c5_vith_encoder_b16", 16, 1024, 16, 8, 8, 1280, 16, 80, 5120, 14, 4, 16, 16, -1, 0.3, 0.3, "bf16", 32),
}


def get_config(key: str) -> Config:
    return CONFIGS[key]


def global_variant(cfg: Config) -> Config:
    """The global-attention block of an encoder config (B = G = 64 over N = 4096)."""
    return cfg.with_(window=0, block=64, global_tokens=64, layers=1)


def window_variant(cfg: Config) -> Config:
    """The windowed block of an encoder config (14 x 14 windows, B = G = 16)."""
    return cfg.with_(window=14, block=16, global_tokens=16, layers=1)
