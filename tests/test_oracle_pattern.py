"""Pins for the oracle's static block pattern, band radius and mask."""
import json
import os

import numpy as np
import pytest

from oracle import band_radius, descending_order, position_keep, stripe_sort, token_mask
from tests.conftest import GOLDEN


def _tile_count_closed_form(g, nb, r):
    """Kept tiles when S is a multiple of B and G = B (inclusion-exclusion).

    band: g^2 sub-maps, each with nb(2r+1) - r(r+1) tiles within radius r;
    plus the global tile's row and column (g*nb each, sharing one tile), minus
    the 2*g*(r+1) of them already inside the band.
    """
    r = min(r, nb - 1)
    band = g * g * (nb * (2 * r + 1) - r * (r + 1))
    return band + 2 * g * (nb - r - 1)


def _tiles_kept(keep, n, g, B):
    S = n // g
    nbs = -(-S // B)
    tile = (np.arange(n) // S) * nbs + (np.arange(n) % S) // B
    T = g * nbs
    kept = np.zeros((T, T), bool)
    qi, ki = np.nonzero(keep)
    kept[tile[qi], tile[ki]] = True
    return kept


@pytest.mark.parametrize("n,g,B,r,want", [(4096, 4, 64, 3, 1696), (4096, 4, 64, 2, 1288),
                                          (4096, 4, 64, 15, 4096), (256, 2, 16, 1, 112),
                                          (256, 4, 16, 1, 176), (4096, 4, 64, 0, None)])
def test_tile_counts_closed_form(n, g, B, r, want):
    keep = position_keep(n, g, B, B, r)
    kept = _tiles_kept(keep, n, g, B)
    nb = n // g // B
    assert kept.sum() == _tile_count_closed_form(g, nb, r)
    if want is not None:
        assert kept.sum() == want
    # whole tiles only: every tile is all-kept or all-dropped (no in-tile masking)
    assert keep.sum() == kept.sum() * B * B


def test_window_pattern_token_density():
    keep = position_keep(196, 4, 16, 16, 0)
    # band: 16 sub-maps x (3 * 16^2 + 1^2); global rows/cols 16 x 196 each; overlaps
    band = 16 * (3 * 256 + 1)
    want = band + 2 * 16 * 196 - 256 - 2 * 16 * 64 + 256
    assert keep.sum() == want == 16528
    assert abs(keep.sum() / 196 ** 2 - 0.4302) < 1e-4
    kept_tiles = _tiles_kept(keep, 196, 4, 16)
    assert kept_tiles.sum() == 88


@pytest.mark.parametrize("n,g,B,d,want_r", [(4096, 4, 64, 0.4, 3), (4096, 4, 64, 0.3, 2),
                                            (4096, 4, 64, 1.0, 15), (256, 2, 16, 0.4, 1),
                                            (196, 4, 16, 0.4, 0), (196, 4, 16, 0.3, 0),
                                            (196, 4, 16, 1.0, 3), (256, 4, 16, 0.4, 1)])
def test_band_radius_is_smallest_reaching_density(n, g, B, d, want_r):
    r = band_radius(n, g, B, B, d)
    assert r == want_r
    dens = position_keep(n, g, B, B, r).mean()
    assert dens >= np.float32(d) or r == (n // g - 1) // B
    if r > 0:
        assert position_keep(n, g, B, B, r - 1).mean() < np.float32(d)


def test_density_one_keeps_everything():
    for n, g, B in [(4096, 4, 64), (196, 4, 16), (256, 2, 16)]:
        r = band_radius(n, g, B, B, 1.0)
        assert position_keep(n, g, B, B, r).all()


@pytest.mark.parametrize("n,g,B,G,r", [(256, 2, 16, 16, 1), (196, 4, 16, 16, 0), (64, 4, 4, 8, 1)])
def test_pattern_symmetric_with_diagonal(n, g, B, G, r):
    keep = position_keep(n, g, B, G, r)
    assert np.array_equal(keep, keep.T)
    assert keep.diagonal().all()
    assert keep.any(axis=1).all()


@pytest.mark.parametrize("n,g,B,G,r", [(256, 2, 16, 16, 1), (196, 4, 16, 16, 0), (4096, 4, 64, 64, 3)])
def test_rank_form_equals_position_form(n, g, B, G, r):
    rng = np.random.default_rng(n + r)
    imp = rng.uniform(size=n).astype(np.float32)
    s = descending_order(imp)
    perm, inv = stripe_sort(s, g)
    M = token_mask(inv, g, B, G, r)
    rank = np.empty(n, np.int64)
    rank[s] = np.arange(n)
    a = rank % g
    blk = (rank // g) // B
    glob = (a == 0) & (rank // g < G)
    M2 = (np.abs(blk[:, None] - blk[None, :]) <= r) | glob[:, None] | glob[None, :]
    assert np.array_equal(M, M2)


def test_hand_worked_16_token_mask():
    with open(os.path.join(GOLDEN, "stripe_sort_4x4.json")) as f:
        ex = json.load(f)
    with open(os.path.join(GOLDEN, "mask_16_tokens.json")) as f:
        gm = json.load(f)
    s = descending_order(np.array(ex["importance"], np.float32))
    perm, inv = stripe_sort(s, gm["stripes"])
    M = token_mask(inv, gm["stripes"], gm["block"], gm["global_tokens"], gm["radius"])
    assert M.sum() == gm["kept_total"]
    for tok, keys in gm["kept_keys"].items():
        assert np.nonzero(M[int(tok)])[0].tolist() == keys
