"""Pins for the oracle's ordering, stripe-sort and keep-set routing."""
import itertools
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import (descending_order, routed_count, routed_rank_order, routed_tokens, segment_importance,
                    stripe_sort, window_token_map)
from tests.conftest import GOLDEN


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_order_matches_numpy_stable_argsort():
    rng = np.random.default_rng(0)
    imp = rng.uniform(0, 1, 4096).astype(np.float32)
    imp[::7] = imp[3]  # many exact ties
    want = np.argsort(-imp, kind="stable")
    assert np.array_equal(descending_order(imp), want)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6])
def test_order_brute_force_every_tie_pattern(n):
    for vals in itertools.product([0.0, 1.0, 2.0], repeat=n):
        v = np.array(vals, np.float32)
        want = sorted(range(n), key=lambda i: (-vals[i], i))
        assert list(descending_order(v)) == want


def test_order_negative_zero_equals_zero():
    v = np.array([-0.0, 0.0, -0.0, 1.0], np.float32)
    assert list(descending_order(v)) == [3, 0, 1, 2]


def test_order_invalid_slots_last_even_after_nan():
    v = np.array([np.nan, 5.0, -1.0, 0.0, 2.0], np.float32)
    valid = np.array([True, False, True, False, True])
    assert list(descending_order(v, valid)) == [4, 2, 0, 1, 3]


def test_order_nan_after_every_number():
    v = np.array([np.nan, -1.0, 2.0, np.nan, -np.inf, 0.5], np.float32)
    assert list(descending_order(v)) == [2, 5, 1, 4, 0, 3]


@settings(max_examples=60, deadline=None)
@given(st.lists(st.sampled_from([0.0, -0.0, 0.25, 0.5, 3.0, -1.0]), min_size=1, max_size=40))
def test_order_is_a_bijection_and_sorted(vals):
    v = np.array(vals, np.float32)
    s = descending_order(v)
    assert sorted(s.tolist()) == list(range(len(v)))
    for x, y in zip(s[:-1], s[1:]):
        assert v[x] > v[y] or (v[x] == v[y] and x < y)


def test_stripe_sort_hand_worked_4x4():
    g = _golden("stripe_sort_4x4.json")
    imp = np.array(g["importance"], np.float32)
    s = descending_order(imp)
    assert s.tolist() == g["sorted"]
    perm, inv = stripe_sort(s, g["stripes"])
    assert perm.tolist() == g["perm"]
    assert inv.tolist() == g["inv"]
    tmap = np.arange(16)
    assert routed_count(g["mlp_density"], 16) == g["routed_k"]
    assert routed_tokens(s, tmap, g["mlp_density"]).tolist() == g["routed"]
    # in rank order the keep-set is the head of the hand-worked order itself
    assert routed_rank_order(s, tmap, g["mlp_density"]).tolist() == g["sorted"][:g["routed_k"]]
    # keep-set positions in the stripe-sorted sequence: one contiguous run per stripe
    pos = sorted(inv[g["routed"]].tolist())
    runs = [list(range(a, b)) for a, b in g["routed_positions_per_stripe"]]
    assert pos == sorted(sum(runs, []))


@pytest.mark.parametrize("n,g", [(16, 4), (256, 2), (4096, 4), (196, 4), (12, 3)])
def test_stripe_sort_closed_form_and_bijection(n, g):
    rng = np.random.default_rng(n)
    s = rng.permutation(n)
    perm, inv = stripe_sort(s, g)
    S = n // g
    p = np.arange(n)
    assert np.array_equal(perm, s[g * (p % S) + p // S])
    assert np.array_equal(perm[inv], np.arange(n))
    assert np.array_equal(inv[perm], np.arange(n))


def test_stripe_sort_degenerate_group_sizes():
    s = np.array([3, 1, 4, 0, 5, 2, 7, 6])
    assert np.array_equal(stripe_sort(s, 1)[0], s)
    assert np.array_equal(stripe_sort(s, 8)[0], s)


def test_stripe_sort_rejects_ragged():
    with pytest.raises(ValueError):
        stripe_sort(np.arange(10), 4)


@pytest.mark.parametrize("d,n,k", [(0.4, 4096, 1638), (0.3, 4096, 1229), (0.4, 196, 78), (0.4, 112, 45),
                                   (0.4, 64, 26), (0.3, 196, 59), (0.3, 112, 34), (0.3, 64, 19),
                                   (0.4, 256, 102), (1.0, 196, 196), (0.001, 10, 1)])
def test_routed_count_values(d, n, k):
    assert routed_count(d, n) == k


@pytest.mark.parametrize("n,g,d", [(4096, 4, 0.4), (196, 4, 0.3), (256, 2, 0.4)])
def test_routed_positions_are_stripe_runs(n, g, d):
    rng = np.random.default_rng(5)
    imp = rng.uniform(size=n).astype(np.float32)
    s = descending_order(imp)
    perm, inv = stripe_sort(s, g)
    k = routed_count(d, n)
    routed = routed_tokens(s, np.arange(n), d)
    S = n // g
    want = sorted(a * S + u for a in range(g) for u in range(-(-(k - a) // g)))
    assert sorted(inv[routed].tolist()) == want


def test_window_token_map_padding():
    tm = window_token_map(64, 64, 14)
    assert tm.shape == (25, 196)
    reals = (tm >= 0).sum(axis=1)
    assert sorted(set(reals.tolist())) == [64, 112, 196]
    assert (reals == 196).sum() == 16 and (reals == 112).sum() == 8 and (reals == 64).sum() == 1
    ids = tm[tm >= 0]
    assert np.array_equal(np.sort(ids), np.arange(4096))
    assert tm[0, 15] == 64 + 1  # window 0, local (1, 1) -> token (1, 1)
    assert tm[4, 0] == 56       # window (0, 4) starts at column 56
    assert tm[4, 8] == -1       # column 64 is padding


def test_window_pads_never_routed_and_sort_last():
    rng = np.random.default_rng(9)
    imp = rng.uniform(size=4096).astype(np.float32)
    tm = window_token_map(64, 64, 14)
    seg = segment_importance(imp, tm[24])  # the corner window: 8 x 8 real
    s = descending_order(seg, valid=tm[24] >= 0)
    n_real = int((tm[24] >= 0).sum())
    assert n_real == 64
    assert np.all(tm[24][s[:n_real]] >= 0)
    assert np.all(tm[24][s[n_real:]] < 0)
    # pads keep index order among themselves
    assert np.all(np.diff(s[n_real:]) > 0)
    r = routed_tokens(s, tm[24], 0.4)
    assert len(r) == 26 and np.all(r >= 0)
    rr = routed_rank_order(s, tm[24], 0.4)
    assert sorted(rr.tolist()) == r.tolist()
    assert np.all(np.diff(imp[rr]) <= 0)  # most important first
    assert imp[rr[0]] == imp[tm[24][tm[24] >= 0]].max()
