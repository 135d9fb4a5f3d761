"""Plain CPU statement of the SparseSAM encoder-block hot path (the oracle).

TEST INFRASTRUCTURE ONLY: used by tests/, by ``__graft_entry__.smoke()`` and by
the ``cpu_baseline`` leg of ``bench.py``; never by the product path.

What it computes, step by step, with the passage each step follows:

* importance -- a parameter-free Sobel operator gives a local gradient
  magnitude per pixel as a proxy for information density ("Technische
  Samenvatting: SparseSAM", Methodologie, 1. Stripe-Sort Attention, the
  gradient-based ordering bullet; the same step in "技術概要：SparseSAM", 手法).
  Reading: unnormalised [1,2,1] x [-1,0,1] kernels, zero border, L2 magnitude,
  mean over each 16 x 16 patch in a fixed order (the token grid is SAM's).
  These steps are fp32 with one rounding per operation in the order written,
  because the sort below turns them into integers.
* descending order -- tokens sorted by importance, highest first (same page,
  stripe-sort bullet: a plain sort would put the foreground first). Ties go to
  the lower token index; -0.0 equals +0.0; NaN sorts after every number.
* stripe-sort -- the sorted list is read as a matrix of g columns, transposed
  and flattened (same bullet). g = 4 from the 4 x 4 mosaic of the static
  pattern bullet.
* static pattern -- a 4 x 4 mosaic of sub-maps, each banded along its
  diagonal, plus a small global keep-set (same page, static pattern bullet).
  Reading: the same band of radius r (in B-token blocks of each stripe) in
  every sub-map; the global set is the first G positions of stripe 0 and is
  symmetric; r is the smallest radius whose kept share of the N x N map
  reaches the requested density.
* attention -- ordinary softmax attention restricted to the kept pairs, built
  densely with an explicit mask in the original token order.
* routed MLP -- the top K tokens of the importance order form the keep-set,
  the MLP runs on them only, every other token keeps its residual value
  unchanged ("Technische Samenvatting: SparseSAM", Methodologie,
  2. Residual-Consistency MLP, token routing / selective computation /
  residual propagation bullets). Reading: the undefined correction on the
  residual set is zero; K = floor(d * n_real + 1/2), at least 1.
* one permutation per image (global blocks) or per window (windowed blocks),
  reused by every block of that type (the closing paragraph of that section).
* dynamic routing (optional) -- the same bullet on selective computation says
  the keep-set tokens are those with high feature dissimilarity or update
  magnitude. Reading: per segment, the K tokens whose update by this block's
  attention sub-block, x1 - x, has the largest squared L2 norm (ranked in fp32,
  the kernels' precision; ties to the lower slot, pads never chosen), with the
  same K as the static keep-set.
* residual correction (optional) -- the residual-propagation bullet writes the
  bypassing tokens as y_i = x_i + eps_i while calling them unchanged, and the
  registry API names an ``mlp_merge`` flag. Reading: eps_i = 0 by default (the
  tokens stay bitwise unchanged); with merging on, every real token of a segment
  outside its keep-set receives the mean of the MLP updates of that segment's
  keep-set, the keep-set's updates merged into one shared update.
* relative-position bias (optional) -- the pages name fused "FA2 + rel-pos"
  kernels in the SparseSAM repository's kernel folder (the README's repository
  layout) but never define the term. Reading: SAM's image encoder's decomposed
  relative position (Kirillov et al., "Segment Anything", 2023, after Li et al.,
  MViTv2, CVPR 2022): a query at segment coordinates (y, x) adds
  <q, Rh[y - y' + Sh - 1]> + <q, Rw[x - x' + Sw - 1]> to its logit for the key at
  (y', x'), with the unscaled query, tables shared by the heads of a block and
  Sh x Sw the segment shape (the grid, or the padded window).

Block structure (not on the pages; SAM encoder conventions): pre-LN block,
LayerNorm eps 1e-6 with biased variance, biases on qkv/proj/fc1/fc2, exact-erf
GELU, softmax scale head_dim ** -0.5, matrices in [out, in] layout.

Floating point: importance in fp32 (it decides integers, so both sides take it
in the same precision); the block arithmetic in fp64.

Parity status: every function here is pinned by tests in tests/test_oracle_*.py
against brute force, closed forms, library special cases or hand-worked
examples. The exact pattern semantics (which band, which global set, how r is
chosen) are readings of the pages, which print no mask, no density table and no
value: they are pinned only to their own written definitions (the hand-worked
examples under tests/golden/ are derived from those definitions), so for the
pattern rule itself parity is unpinned by the pages.
"""
import math

import numpy as np
from scipy.special import erf

__all__ = [
    "sobel_magnitude",
    "patch_mean",
    "importance",
    "window_token_map",
    "segment_importance",
    "descending_order",
    "ORDERINGS",
    "morton_code",
    "hilbert_index",
    "splitmix64",
    "order_key",
    "ascending_order",
    "segment_order",
    "stripe_sort",
    "routed_count",
    "routed_tokens",
    "routed_rank_order",
    "position_keep",
    "band_radius",
    "token_mask",
    "masked_attention",
    "rel_pos_bias",
    "layer_norm",
    "gelu",
    "routed_mlp",
    "ROUTINGS",
    "update_score",
    "top_k_by_score",
    "merged_update",
    "segments_for_image",
    "block_forward",
    "encoder_forward",
]

F32 = np.float32


# ----------------------------------------------------------------------------
# Importance (fp32, fixed operation order)
# ----------------------------------------------------------------------------

def sobel_magnitude(img: np.ndarray) -> np.ndarray:
    """L2 Sobel gradient magnitude of a grayscale image, zero outside the image.

    gx = ((P[y-1,x+1] + 2 P[y,x+1]) + P[y+1,x+1]) - ((P[y-1,x-1] + 2 P[y,x-1]) + P[y+1,x-1])
    gy = ((P[y+1,x-1] + 2 P[y+1,x]) + P[y+1,x+1]) - ((P[y-1,x-1] + 2 P[y-1,x]) + P[y-1,x+1])
    m  = sqrt(gx*gx + gy*gy)
    Each operation rounds once to fp32 in exactly this order (no fused multiply-add).
    """
    img = np.asarray(img, dtype=F32)
    H, W = img.shape
    P = np.zeros((H + 2, W + 2), F32)
    P[1:-1, 1:-1] = img

    def at(dy, dx):
        return P[1 + dy:1 + dy + H, 1 + dx:1 + dx + W]

    two = F32(2.0)
    gx = ((at(-1, 1) + two * at(0, 1)) + at(1, 1)) - ((at(-1, -1) + two * at(0, -1)) + at(1, -1))
    gy = ((at(1, -1) + two * at(1, 0)) + at(1, 1)) - ((at(-1, -1) + two * at(-1, 0)) + at(-1, 1))
    sq = gx * gx
    sq = sq + gy * gy
    return np.sqrt(sq).astype(F32)


def patch_mean(mag: np.ndarray, patch: int) -> np.ndarray:
    """Mean of each patch x patch tile, tokens in raster order -> fp32 [Hg * Wg].

    Fixed order: each pixel row of a tile is summed left to right starting from 0,
    the row sums are added top to bottom starting from 0, then the total is divided
    by patch * patch (one correctly rounded fp32 division).
    """
    mag = np.asarray(mag, dtype=F32)
    H, W = mag.shape
    Hg, Wg = H // patch, W // patch
    t = mag[:Hg * patch, :Wg * patch].reshape(Hg, patch, Wg, patch)
    rows = np.zeros((Hg, patch, Wg), F32)
    for c in range(patch):
        rows = rows + t[:, :, :, c]
    total = np.zeros((Hg, Wg), F32)
    for r in range(patch):
        total = total + rows[:, r, :]
    return (total / F32(patch * patch)).astype(F32).reshape(-1)


def importance(img: np.ndarray, patch: int = 16) -> np.ndarray:
    """Per-token importance of one image: Sobel magnitude pooled per patch."""
    return patch_mean(sobel_magnitude(img), patch)


# ----------------------------------------------------------------------------
# Segments: one global segment per image, or w x w windows
# ----------------------------------------------------------------------------

def window_token_map(grid_h: int, grid_w: int, window: int) -> np.ndarray:
    """[n_windows, window*window] image token id of each window-local slot, -1 for pad.

    The grid is padded at the bottom and right up to multiples of ``window``;
    windows are taken in raster order and the slots of a window in raster order.
    """
    nwy = -(-grid_h // window)
    nwx = -(-grid_w // window)
    out = np.full((nwy * nwx, window * window), -1, np.int64)
    for wy in range(nwy):
        for wx in range(nwx):
            for ly in range(window):
                for lx in range(window):
                    y, x = wy * window + ly, wx * window + lx
                    if y < grid_h and x < grid_w:
                        out[wy * nwx + wx, ly * window + lx] = y * grid_w + x
    return out


def segments_for_image(grid_h: int, grid_w: int, window: int) -> np.ndarray:
    """Token map of the attention segments of one image: [segments, N] ids or -1."""
    if window == 0:
        return np.arange(grid_h * grid_w, dtype=np.int64)[None, :]
    return window_token_map(grid_h, grid_w, window)


def segment_importance(imp: np.ndarray, token_map: np.ndarray) -> np.ndarray:
    """Importance of each segment slot (pad slots read as 0; their order is set apart)."""
    out = np.where(token_map >= 0, imp[np.maximum(token_map, 0)], F32(0.0))
    return out.astype(F32)


# ----------------------------------------------------------------------------
# Ordering and stripe-sort
# ----------------------------------------------------------------------------

def descending_order(imp: np.ndarray, valid: np.ndarray = None) -> np.ndarray:
    """Slot ids sorted by importance, highest first, written as a rank count.

    Slot j precedes slot i when imp[j] > imp[i], or when they are equal and j < i.
    -0.0 and +0.0 are equal; a NaN is below every number and equal to every NaN.
    Slots with valid == False (window padding) come after every valid slot, in
    index order. rank[i] = number of slots preceding i; s[rank[i]] = i.
    """
    v = np.asarray(imp, dtype=F32).astype(np.float64)
    v = np.where(v == 0.0, 0.0, v)
    nan = np.isnan(v)
    n = v.shape[0]
    ok = np.ones(n, bool) if valid is None else np.asarray(valid, bool)
    idx = np.arange(n)
    vi, vj = v[:, None], v[None, :]
    ni, nj = nan[:, None], nan[None, :]
    oi, oj = ok[:, None], ok[None, :]
    with np.errstate(invalid="ignore"):
        j_higher = (~nj) & (ni | (vj > vi))
        same = (ni & nj) | ((~ni) & (~nj) & (vj == vi))
    by_value = j_higher | (same & (idx[None, :] < idx[:, None]))
    precedes = (oj & ~oi) | (oj & oi & by_value) | (~oj & ~oi & (idx[None, :] < idx[:, None]))
    rank = precedes.sum(axis=1)
    s = np.empty(n, np.int64)
    s[rank] = idx
    return s


def stripe_sort(s: np.ndarray, stripes: int):
    """Stripe-sort of a sorted token list: (perm, inv).

    The sorted list is viewed as a matrix with ``stripes`` columns (row k holds
    ranks k*g .. k*g+g-1), transposed, and flattened. perm[p] is the token at
    position p of the new sequence; inv[perm[p]] = p.
    """
    s = np.asarray(s, dtype=np.int64)
    n = s.shape[0]
    if n % stripes != 0:
        raise ValueError("sequence length must be a multiple of the stripe count")
    perm = s.reshape(n // stripes, stripes).T.reshape(-1).copy()
    inv = np.empty(n, np.int64)
    inv[perm] = np.arange(n)
    return perm, inv


def routed_count(mlp_density: float, n_real: int) -> int:
    """K = floor(d * n_real + 1/2) in double precision, at least 1 (d given as fp32)."""
    d = float(np.float32(mlp_density))
    return max(1, int(math.floor(d * n_real + 0.5)))


def routed_tokens(s: np.ndarray, token_map_row: np.ndarray, mlp_density: float) -> np.ndarray:
    """Image token ids of the keep-set of one segment, ascending.

    The keep-set is the first K entries of the importance order; pad slots sort
    after every real slot and K <= number of real slots, so none is taken.
    """
    n_real = int((token_map_row >= 0).sum())
    k = routed_count(mlp_density, n_real)
    picked = token_map_row[s[:k]]
    assert (picked >= 0).all()
    return np.sort(picked)


def routed_rank_order(s: np.ndarray, token_map_row: np.ndarray, mlp_density: float) -> np.ndarray:
    """The keep-set of one segment as image token ids in importance order (the first K
    entries of the order itself, most important first). Same set as routed_tokens."""
    n_real = int((token_map_row >= 0).sum())
    k = routed_count(mlp_density, n_real)
    picked = token_map_row[s[:k]]
    assert (picked >= 0).all()
    return picked


# ----------------------------------------------------------------------------
# Ordering variants (the pages' other names for the token order)
# ----------------------------------------------------------------------------
#
# "Technische Samenvatting: SparseSAM" (abstract) and its method section call the
# permutation a Z-order (Morton) ordering, and the README's method registry lists
# random and Hilbert-curve orders next to the importance order. Reading: each
# variant replaces only the sort key of a segment's slots -- ascending key instead
# of descending importance, ties to the lower slot, window pads after every real
# slot -- and everything downstream (stripe-sort, pattern, keep-set = the first K of
# the same order) is unchanged. Keys come from the slot's position inside its
# segment: (y, x) on the token grid for a global segment, (ly, lx) inside the window
# for a windowed one.

ORDERINGS = ("importance", "zorder", "hilbert", "random")


def morton_code(y: int, x: int) -> int:
    """Z-order (Morton) code of cell (y, x): bit b of x goes to bit 2b, bit b of y to
    bit 2b + 1, so x varies fastest inside every 2 x 2 block."""
    code = 0
    for b in range(16):
        code |= ((x >> b) & 1) << (2 * b)
        code |= ((y >> b) & 1) << (2 * b + 1)
    return code


def hilbert_index(side: int, y: int, x: int) -> int:
    """Position of cell (y, x) along the Hilbert curve that fills a side x side square
    (side a power of two), written from its recursive construction: the square splits
    into quadrants visited in the order (x, y) = (low, low), (low, high), (high, high),
    (high, low); the curves inside the first and last quadrants are the half-size curve
    mirrored in the main diagonal and in the anti-diagonal respectively, so that each
    sub-curve starts next to where the previous one ended. The curve starts at (0, 0)
    and ends at (x, y) = (side - 1, 0)."""
    if side == 1:
        return 0
    h = side // 2
    qx, qy = int(x >= h), int(y >= h)
    lx, ly = x - h * qx, y - h * qy
    if qy == 0 and qx == 0:
        q, cx, cy = 0, ly, lx                    # mirrored in the main diagonal
    elif qy == 1 and qx == 0:
        q, cx, cy = 1, lx, ly
    elif qy == 1 and qx == 1:
        q, cx, cy = 2, lx, ly
    else:
        q, cx, cy = 3, h - 1 - ly, h - 1 - lx    # mirrored in the anti-diagonal
    return q * h * h + hilbert_index(h, cy, cx)


def splitmix64(state: int) -> int:
    """First output of the SplitMix64 generator started at `state` (Steele, Lea and
    Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014, with the
    mixing constants of its widely used 64-bit variant): the state advances by the
    golden-ratio increment and the result goes through two xor-shift-multiply rounds
    and a final xor-shift."""
    m = (1 << 64) - 1
    z = (state + 0x9E3779B97F4A7C15) & m
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & m
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & m
    return z ^ (z >> 31)


def order_key(ordering: str, slot: int, seg_h: int, seg_w: int, seed: int = 0) -> int:
    """Ascending sort key of a segment slot (slot = ly * seg_w + lx) for a non-importance
    ordering. Hilbert keys use the smallest power-of-two square covering the segment;
    random keys are the top 31 bits of splitmix64(seed * 2^32 + slot), the same order in
    every segment and image."""
    y, x = divmod(slot, seg_w)
    if ordering == "zorder":
        return morton_code(y, x)
    if ordering == "hilbert":
        side = 1
        while side < max(seg_h, seg_w):
            side *= 2
        return hilbert_index(side, y, x)
    if ordering == "random":
        return splitmix64(((seed & 0xFFFFFFFF) << 32) | slot) >> 33
    raise ValueError("unknown ordering %r" % (ordering,))


def ascending_order(keys, valid=None) -> np.ndarray:
    """Slot ids sorted by key ascending, ties to the lower slot, slots with valid ==
    False after every valid slot in index order."""
    n = len(keys)
    ok = np.ones(n, bool) if valid is None else np.asarray(valid, bool)
    return np.array(sorted(range(n), key=lambda i: (0 if ok[i] else 1, int(keys[i]) if ok[i] else 0, i)),
                    dtype=np.int64)


def segment_order(ordering: str, imp: np.ndarray, token_map_row: np.ndarray, seg_h: int, seg_w: int,
                  seed: int = 0) -> np.ndarray:
    """The sorted slot list of one segment under `ordering` (see ORDERINGS)."""
    valid = token_map_row >= 0
    if ordering == "importance":
        return descending_order(segment_importance(imp, token_map_row), valid=valid)
    keys = [order_key(ordering, s, seg_h, seg_w, seed) for s in range(token_map_row.shape[0])]
    return ascending_order(keys, valid=valid)


# ----------------------------------------------------------------------------
# Static pattern
# ----------------------------------------------------------------------------

def position_keep(n: int, stripes: int, block: int, global_tokens: int, radius: int) -> np.ndarray:
    """Kept (query position, key position) pairs of the stripe-sorted sequence, [n, n] bool.

    Position p lies in stripe a = p // S at offset u = p % S (S = n / stripes), in
    stripe-local block j = u // block. A pair is kept when the blocks are within
    ``radius`` of each other (the band, the same in every stripe pair), or when either
    position is global (stripe 0, u < global_tokens).
    """
    S = n // stripes
    p = np.arange(n)
    u = p % S
    a = p // S
    j = u // block
    glob = (a == 0) & (u < global_tokens)
    band = np.abs(j[:, None] - j[None, :]) <= radius
    return band | glob[:, None] | glob[None, :]


def band_radius(n: int, stripes: int, block: int, global_tokens: int, attn_density: float) -> int:
    """Smallest radius r >= 0 whose kept share of the n x n map reaches the density."""
    d = float(np.float32(attn_density))
    S = n // stripes
    last = (S - 1) // block
    for r in range(last + 1):
        kept = int(position_keep(n, stripes, block, global_tokens, r).sum())
        if kept / float(n * n) >= d:
            return r
    return last


def token_mask(inv: np.ndarray, stripes: int, block: int, global_tokens: int, radius: int) -> np.ndarray:
    """The pattern in original token order: M[i, k] = keep(inv[i], inv[k])."""
    n = inv.shape[0]
    keep = position_keep(n, stripes, block, global_tokens, radius)
    return keep[np.ix_(inv, inv)]


# ----------------------------------------------------------------------------
# Block arithmetic (fp64)
# ----------------------------------------------------------------------------

def masked_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray,
                     scale: float, bias: np.ndarray = None) -> np.ndarray:
    """softmax(q k^T * scale + bias) v with pairs outside ``mask`` removed (score -inf).

    q, k, v: [n, D]; mask: [n, n] bool (every row keeps at least one key); bias:
    [n, n] added to the logits (None: no bias).
    """
    s = (q.astype(np.float64) @ k.astype(np.float64).T) * scale
    if bias is not None:
        s = s + bias
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return (e / e.sum(axis=1, keepdims=True)) @ v.astype(np.float64)


def rel_pos_bias(q: np.ndarray, seg_h: int, seg_w: int, rel_h: np.ndarray, rel_w: np.ndarray) -> np.ndarray:
    """Decomposed relative-position bias [n, n] of one segment and head (n = seg_h * seg_w).

    q: [n, D] queries in segment slot order (slot = y * seg_w + x), unscaled; rel_h:
    [2 seg_h - 1, D], rel_w: [2 seg_w - 1, D]. The steps of SAM's encoder: the table
    rows for every (query row, key row) offset, Rh[y, y'] = rel_h[y - y' + seg_h - 1];
    the per-query row terms B_h[i, y'] = <q_i, Rh[y_i, y']> (likewise B_w with columns);
    the bias of the pair (i, k) is B_h[i, y_k] + B_w[i, x_k].
    """
    q = q.astype(np.float64)
    n, D = q.shape
    assert n == seg_h * seg_w
    assert rel_h.shape == (2 * seg_h - 1, D) and rel_w.shape == (2 * seg_w - 1, D)
    yy = np.arange(seg_h)
    xx = np.arange(seg_w)
    Rh = rel_h.astype(np.float64)[yy[:, None] - yy[None, :] + seg_h - 1]  # [seg_h, seg_h, D]
    Rw = rel_w.astype(np.float64)[xx[:, None] - xx[None, :] + seg_w - 1]  # [seg_w, seg_w, D]
    slot = np.arange(n)
    y, x = slot // seg_w, slot % seg_w
    b_h = np.einsum("id,ikd->ik", q, Rh[y])  # [n, seg_h]: query i against key row k
    b_w = np.einsum("id,ikd->ik", q, Rw[x])  # [n, seg_w]
    return b_h[:, y] + b_w[:, x]


def layer_norm(x: np.ndarray, gamma: np.ndarray, beta: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """LayerNorm over the last axis with the biased variance."""
    x = x.astype(np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * gamma.astype(np.float64) + beta.astype(np.float64)


def gelu(z: np.ndarray) -> np.ndarray:
    """GELU with the exact Gaussian CDF: z * (1 + erf(z / sqrt 2)) / 2."""
    return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))


def _linear(x, w, b):
    return x @ w.astype(np.float64).T + b.astype(np.float64)


def routed_mlp(x: np.ndarray, routed: np.ndarray, w: dict) -> np.ndarray:
    """Residual-Consistency MLP on rows of x [rows, C]: only routed rows change.

    x2[t] = x[t] + fc2(GELU(fc1(LN2(x[t])))) for t in routed; x2[t] = x[t] otherwise.
    """
    out = x.astype(np.float64).copy()
    xr = out[routed]
    h = gelu(_linear(layer_norm(xr, w["ln2_g"], w["ln2_b"]), w["w1"], w["b1"]))
    out[routed] = xr + _linear(h, w["w2"], w["b2"])
    return out


# ----------------------------------------------------------------------------
# Dynamic routing and the residual correction (optional readings)
# ----------------------------------------------------------------------------

ROUTINGS = ("importance", "update")


def update_score(x: np.ndarray, x1: np.ndarray) -> np.ndarray:
    """Squared L2 norm of each row's update, ||x1[t] - x[t]||^2 (fp64): how far this
    block's attention sub-block moved token t."""
    d = np.asarray(x1, np.float64) - np.asarray(x, np.float64)
    return (d * d).sum(axis=-1)


def top_k_by_score(score: np.ndarray, valid: np.ndarray, k: int) -> np.ndarray:
    """Slot ids of the k largest scores, largest first: the importance order's rank
    count applied to the scores rounded to fp32 (ties to the lower slot, slots with
    valid == False after every valid slot)."""
    return descending_order(np.asarray(score, np.float64).astype(F32), valid=valid)[:k]


def merged_update(x1_rows: np.ndarray, x2_rows: np.ndarray) -> np.ndarray:
    """The keep-set's MLP updates merged into one: their mean, [C] (fp64)."""
    return (np.asarray(x2_rows, np.float64) - np.asarray(x1_rows, np.float64)).mean(axis=0)


def block_forward(x: np.ndarray, imp: np.ndarray, w: dict, cfg, radius: int = None,
                  return_parts: bool = False, routed_override: list = None):
    """One SparseSAM encoder block on x [batch, gh, gw, C] (fp32 in, fp64 out).

    imp: [batch, gh*gw] fp32 importance. The pattern and keep-set come from
    ``cfg`` (window, stripes, block, global_tokens, band_radius, attn_density,
    mlp_density, heads, head_dim). Attention is dense with an explicit mask in the
    original token order, per segment; window pad slots carry h = 0 as keys and
    queries and their outputs are dropped. With w["rel_h"] and w["rel_w"] set, every
    head adds the relative-position bias (rel_pos_bias) of its segment to its logits;
    pads have their padded-window coordinates.

    cfg.routing "update" chooses each segment's keep-set by update_score instead of the
    importance order (same K); cfg.mlp_merge adds merged_update of a segment's keep-set
    to its other real tokens. routed_override (one array of image token ids per image)
    replaces the chosen keep-sets, e.g. by a set another implementation chose.
    """
    routing = getattr(cfg, "routing", "importance")
    merge = bool(getattr(cfg, "mlp_merge", False))
    if routing not in ROUTINGS:
        raise ValueError("unknown routing %r" % (routing,))
    b, gh, gw, C = x.shape
    H, D = cfg.heads, cfg.head_dim
    tmap = segments_for_image(gh, gw, cfg.window)
    n = tmap.shape[1]
    if radius is None:
        radius = cfg.band_radius if cfg.band_radius >= 0 else band_radius(
            n, cfg.stripes, cfg.block, cfg.global_tokens, cfg.attn_density)
    scale = D ** -0.5
    xf = x.reshape(b, gh * gw, C).astype(np.float64)
    out = np.empty_like(xf)
    parts = {"perm": [], "inv": [], "routed": [], "radius": radius, "score": [], "routed_seg": []}
    for i in range(b):
        h = layer_norm(xf[i], w["ln1_g"], w["ln1_b"])
        attn_out = np.zeros((gh * gw, C))
        routed_img = []
        orders = []
        for seg in range(tmap.shape[0]):
            row = tmap[seg]
            real = row >= 0
            seg_h, seg_w = (gh, gw) if cfg.window == 0 else (cfg.window, cfg.window)
            s = segment_order(getattr(cfg, "ordering", "importance"), imp[i], row, seg_h, seg_w,
                              getattr(cfg, "order_seed", 0))
            perm, inv = stripe_sort(s, cfg.stripes)
            parts["perm"].append(perm)
            parts["inv"].append(inv)
            orders.append(s)
            hs = np.zeros((n, C))
            hs[real] = h[row[real]]
            qkv = _linear(hs, w["w_qkv"], w["b_qkv"])
            mask = token_mask(inv, cfg.stripes, cfg.block, cfg.global_tokens, radius)
            o = np.empty((n, C))
            rel = w.get("rel_h") is not None
            for hd in range(H):
                q = qkv[:, hd * D:(hd + 1) * D]
                k = qkv[:, C + hd * D:C + (hd + 1) * D]
                v = qkv[:, 2 * C + hd * D:2 * C + (hd + 1) * D]
                bias = rel_pos_bias(q, seg_h, seg_w, w["rel_h"], w["rel_w"]) if rel else None
                o[:, hd * D:(hd + 1) * D] = masked_attention(q, k, v, mask, scale, bias)
            attn_out[row[real]] = o[real]
        x1 = xf[i] + _linear(attn_out, w["w_proj"], w["b_proj"])
        score = update_score(xf[i], x1)
        parts["score"].append(score)
        for seg in range(tmap.shape[0]):
            row = tmap[seg]
            if routing == "importance":
                routed_img.append(routed_tokens(orders[seg], row, cfg.mlp_density))
            else:
                real = row >= 0
                k = routed_count(cfg.mlp_density, int(real.sum()))
                slots = top_k_by_score(np.where(real, score[np.maximum(row, 0)], 0.0), real, k)
                routed_img.append(np.sort(row[slots]))
        if routed_override is not None:
            routed_img = [np.sort(np.asarray(routed_override[i], np.int64))]
        parts["routed_seg"].append(routed_img)
        routed = np.sort(np.concatenate(routed_img))
        parts["routed"].append(routed + i * gh * gw)
        x2 = routed_mlp(x1, routed, w)
        if merge:
            # every real token of a segment outside its keep-set gets the mean MLP update of
            # that segment's keep-set (the keep-sets of an override are split by segment)
            in_keep = np.zeros(gh * gw, bool)
            in_keep[routed] = True
            for seg in range(tmap.shape[0]):
                row = tmap[seg]
                toks = row[row >= 0]
                kept = toks[in_keep[toks]]
                rest = toks[~in_keep[toks]]
                if kept.size and rest.size:
                    x2[rest] = x1[rest] + merged_update(x1[kept], x2[kept])
        out[i] = x2
    out = out.reshape(b, gh, gw, C)
    if return_parts:
        return out, parts
    return out


def encoder_forward(x: np.ndarray, imp: np.ndarray, layer_weights: list, global_layers: list,
                    cfg_global, cfg_window):
    """A stack of blocks: global-attention blocks at ``global_layers``, windowed elsewhere.

    Each block recomputes nothing of the ordering that depends on activations: the
    permutation depends on the image only, so every block of a type sees the same one.
    """
    h = x.astype(np.float64)
    for l, w in enumerate(layer_weights):
        cfg = cfg_global if l in global_layers else cfg_window
        h = block_forward(h, imp, w, cfg)
    return h
