"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This package holds data recipes only (shapes, seeds, value distributions) and
none of the method's arithmetic: no Sobel, no sort, no permutation, no mask,
no attention and no MLP. Both `oracle/` and the tests or bench that drive the
HIP library read the arrays it returns.
"""
from .configs import CONFIGS, Config, get_config
from .generate import (
    synthetic_image,
    synthetic_images,
    token_features,
    block_weights,
    round_to_bf16,
    encoder_global_layers,
)

__all__ = [
    "CONFIGS",
    "Config",
    "get_config",
    "synthetic_image",
    "synthetic_images",
    "token_features",
    "block_weights",
    "round_to_bf16",
    "encoder_global_layers",
]
