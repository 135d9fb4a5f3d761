"""Pins of the oracle's decomposed relative-position bias (SAM's image encoder, after
MViTv2): logit(i, k) += <q_i, Rh[y_i - y_k + Sh - 1]> + <q_i, Rw[x_i - x_k + Sw - 1]>.

Each test fixes a value the definition forces by construction, independent of how
the oracle evaluates it: a neighbour picked out by a one-hot table, a 3 : 1 softmax
split, invariance under a per-query constant, and reduction to plain attention.
"""
import math

import numpy as np
import pytest

from oracle import sparsesam_oracle as O
from synth.configs import get_config
from synth.generate import block_weights, rel_pos_tables, synthetic_images, token_features

BIG = 80.0  # exp(-80) ~ 2e-35: a key pushed down by BIG carries no weight at fp64


def _select_tables(seg_h, seg_w, D, dy, dx):
    """Tables whose bias is 0 for the offset (dy, dx) = (y_q - y_k, x_q - x_k) and
    -BIG per mismatching axis when q = e_0."""
    rh = np.zeros((2 * seg_h - 1, D))
    rw = np.zeros((2 * seg_w - 1, D))
    rh[:, 0] = -BIG
    rw[:, 0] = -BIG
    rh[dy + seg_h - 1, 0] = 0.0
    rw[dx + seg_w - 1, 0] = 0.0
    return rh, rw


@pytest.mark.parametrize("dy,dx", [(1, 0), (0, 1), (-2, 1), (1, -3)])
def test_one_hot_tables_pick_the_neighbour(dy, dx):
    """q = e_0 and k = 0: only the bias separates keys, and it is 0 exactly for the key
    at (y - dy, x - dx); every query with that neighbour returns its value row."""
    seg_h, seg_w, D = 5, 6, 4
    n = seg_h * seg_w
    rng = np.random.default_rng(3)
    q = np.zeros((n, D))
    q[:, 0] = 1.0
    k = np.zeros((n, D))
    v = rng.standard_normal((n, D))
    rh, rw = _select_tables(seg_h, seg_w, D, dy, dx)
    bias = O.rel_pos_bias(q, seg_h, seg_w, rh, rw)
    out = O.masked_attention(q, k, v, np.ones((n, n), bool), 0.125, bias)
    checked = 0
    for i in range(n):
        y, x = divmod(i, seg_w)
        yk, xk = y - dy, x - dx
        if 0 <= yk < seg_h and 0 <= xk < seg_w:
            np.testing.assert_allclose(out[i], v[yk * seg_w + xk], rtol=0, atol=1e-12)
            checked += 1
    assert checked >= n // 3


def test_bias_values_on_a_tiny_segment():
    """2 x 3 segment, D = 1: the bias of a pair is q_i * (Rh[dy + 1] + Rw[dx + 2])."""
    seg_h, seg_w = 2, 3
    q = np.array([[1.0], [2.0], [-1.0], [0.5], [3.0], [-2.0]])
    rh = np.array([[10.0], [20.0], [30.0]])               # dy = -1, 0, 1
    rw = np.array([[1.0], [2.0], [3.0], [4.0], [5.0]])    # dx = -2 .. 2
    b = O.rel_pos_bias(q, seg_h, seg_w, rh, rw)
    # query 4 sits at (1, 1); key 0 at (0, 0): dy = 1, dx = 1 -> 3 * (30 + 4)
    assert b[4, 0] == 3.0 * 34.0
    # query 0 at (0, 0); key 5 at (1, 2): dy = -1, dx = -2 -> 1 * (10 + 1)
    assert b[0, 5] == 11.0
    # query 2 at (0, 2); key 3 at (1, 0): dy = -1, dx = 2 -> -1 * (10 + 5)
    assert b[2, 3] == -15.0
    # the diagonal: dy = dx = 0 -> q_i * (20 + 3)
    np.testing.assert_array_equal(np.diag(b), q[:, 0] * 23.0)


def test_bias_enters_unscaled_logits():
    """Two kept keys whose biases differ by ln 3 (q . k = 0) share the weight 3 : 1,
    whatever the softmax scale: the bias is added after the scaling."""
    seg_h, seg_w, D = 1, 3, 2
    q = np.array([[1.0, 0.0]] * 3)
    k = np.array([[0.0, 1.0]] * 3)
    v = np.array([[1.0, 0.0], [0.0, 1.0], [5.0, 5.0]])
    rh = np.zeros((1, D))
    rw = np.zeros((5, D))
    rw[2, 0] = math.log(3.0)  # dx = 0: the query itself (slot 0) gets ln 3
    mask = np.eye(3, dtype=bool)
    mask[0, 1] = True
    for scale in (0.125, 1.0, 4.0):
        out = O.masked_attention(q, k, v, mask, scale, O.rel_pos_bias(q, seg_h, seg_w, rh, rw))
        np.testing.assert_allclose(out[0], [0.75, 0.25], rtol=0, atol=1e-15)


def test_per_query_constant_leaves_output_unchanged():
    """Adding c * e_1 to every row of both tables adds 2 c q_i1 to all logits of query i:
    softmax is invariant, so the output is too."""
    rng = np.random.default_rng(11)
    seg_h, seg_w, D = 4, 5, 8
    n = seg_h * seg_w
    q, k, v = (rng.standard_normal((n, D)) for _ in range(3))
    rh = rng.standard_normal((2 * seg_h - 1, D))
    rw = rng.standard_normal((2 * seg_w - 1, D))
    mask = rng.random((n, n)) < 0.5
    mask[np.arange(n), np.arange(n)] = True
    base = O.masked_attention(q, k, v, mask, D ** -0.5, O.rel_pos_bias(q, seg_h, seg_w, rh, rw))
    rh2, rw2 = rh.copy(), rw.copy()
    rh2[:, 1] += 7.0
    rw2[:, 1] -= 2.5
    moved = O.masked_attention(q, k, v, mask, D ** -0.5, O.rel_pos_bias(q, seg_h, seg_w, rh2, rw2))
    np.testing.assert_allclose(moved, base, rtol=1e-11, atol=1e-12)


def test_bias_is_translation_invariant():
    """The bias depends on the offset only: pairs with the same (dy, dx) share it for a
    shared query vector."""
    rng = np.random.default_rng(5)
    seg_h, seg_w, D = 4, 4, 3
    n = seg_h * seg_w
    q = np.tile(rng.standard_normal(D), (n, 1))
    rh = rng.standard_normal((2 * seg_h - 1, D))
    rw = rng.standard_normal((2 * seg_w - 1, D))
    b = O.rel_pos_bias(q, seg_h, seg_w, rh, rw)
    # (1, 1) -> (0, 0) and (3, 2) -> (2, 1): both dy = 1, dx = 1
    assert b[1 * 4 + 1, 0] == b[3 * 4 + 2, 2 * 4 + 1]
    # (0, 3) -> (3, 0) and (0, 3) against itself differ
    assert b[3, 12] != b[3, 3]


def _block_case(cfg):
    x = token_features(cfg, 4)[:1]
    w = block_weights(cfg, 4)
    imp = np.stack([O.importance(im, cfg.patch) for im in synthetic_images(cfg, 4)[:1]])
    return x, imp, w


@pytest.mark.parametrize("window", [0, 6])
def test_zero_tables_reduce_to_plain_attention(window):
    cfg = get_config("c1").with_(window=window)
    x, imp, w = _block_case(cfg)
    plain = O.block_forward(x, imp, w, cfg)
    side = window or cfg.grid
    w0 = dict(w)
    w0["rel_h"] = np.zeros((2 * side - 1, cfg.head_dim))
    w0["rel_w"] = np.zeros((2 * side - 1, cfg.head_dim))
    np.testing.assert_array_equal(O.block_forward(x, imp, w0, cfg), plain)


def test_block_bias_changes_only_the_attention_branch():
    """With random tables the block output moves (the bias is used), and at attention
    density 1 it is the same for every token ordering (the bias follows each token's
    own coordinates, not its position in the sorted sequence)."""
    cfg = get_config("c1").with_(attn_density=1.0, mlp_density=1.0)
    x, imp, w = _block_case(cfg)
    rh, rw = rel_pos_tables(cfg, 4)
    wr = dict(w, rel_h=rh, rel_w=rw)
    plain = O.block_forward(x, imp, w, cfg)
    biased = O.block_forward(x, imp, wr, cfg)
    assert np.abs(biased - plain).max() > 1e-3
    for ordering in ("zorder", "random"):
        other = O.block_forward(x, imp, wr, cfg.with_(ordering=ordering, order_seed=9))
        np.testing.assert_allclose(other, biased, rtol=1e-10, atol=1e-10)
