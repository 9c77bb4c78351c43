"""Window membership and indexing (BASA paper, §3.1: cyclic shift by -Delta, then a
partition into non-overlapping windows; App. A.1: the partition is a reshape/permute of
a grid exactly divisible by the window).

The oracle's membership table is built from the inverse map (window, local slot) ->
original position. These tests check it against an independently derived forward map,
position -> (window, local slot), and against structural facts of the partition.
"""
import json
import os

import numpy as np
import pytest

from oracle import basa_oracle as O
from sparse_attention_dit_amd.configs import WORKLOADS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def forward_map(grid, window, shift):
    """Per axis: r = (p - s) mod n is the position in the rolled grid; the window
    coordinate is r // w and the local coordinate r % w. Combined row-major."""
    T, H, W = grid
    wt, wh, ww = window
    N = T * H * W
    p = np.arange(N)
    pt, ph, pw = p // (H * W), (p // W) % H, p % W
    rt, rh, rw = (pt - shift[0]) % T, (ph - shift[1]) % H, (pw - shift[2]) % W
    win = ((rt // wt) * (H // wh) + rh // wh) * (W // ww) + rw // ww
    loc = ((rt % wt) * wh + rh % wh) * ww + rw % ww
    return win, loc


CASES = [
    ((1, 16, 16), (1, 8, 8), (0, 4, 4)),
    ((1, 64, 64), (1, 16, 16), (0, 8, 8)),
    ((1, 128, 128), (1, 32, 32), (0, 16, 16)),
    ((1, 256, 256), (1, 32, 32), (0, 16, 0)),
    ((21, 30, 52), (7, 15, 26), (3, 7, 13)),
    ((21, 30, 52), (21, 15, 26), (0, 7, 13)),
    ((6, 6, 6), (3, 2, 3), (-1, -5, 8)),
]


@pytest.mark.parametrize("grid,window,shift", CASES)
def test_table_is_a_permutation_and_agrees_with_forward_map(grid, window, shift):
    table = O.window_members(grid, window, shift)
    N = int(np.prod(grid))
    assert table.shape == (N // int(np.prod(window)), int(np.prod(window)))
    assert np.array_equal(np.sort(table.ravel()), np.arange(N))
    win, loc = forward_map(grid, window, O.reduce_shift(grid, shift))
    assert np.array_equal(table[win, loc], np.arange(N))


@pytest.mark.parametrize("w", WORKLOADS, ids=lambda w: w.name)
def test_workload_shift_cycles(w):
    for s in w.shifts:
        table = O.window_members(w.grid, w.window, s)
        assert table.shape == (w.num_windows, w.window_tokens)
        assert np.array_equal(np.sort(table.ravel()), np.arange(w.tokens))


def test_shift_reduction_handles_negative_and_large():
    assert O.reduce_shift((21, 30, 52), (-3, -7, -13)) == (18, 23, 39)
    assert O.reduce_shift((21, 30, 52), (21 * 5 + 3, -30 * 2, 52 * 7 - 1)) == (3, 0, 51)
    g, w = (21, 30, 52), (7, 15, 26)
    assert np.array_equal(O.window_members(g, w, (-3, -7, -13)), O.window_members(g, w, (18, 23, 39)))


def _partition_sets(grid, window, shift):
    return {frozenset(r.tolist()) for r in O.window_members(grid, window, shift)}


def test_half_window_shifts_are_sign_independent():
    for grid, window, s in [((1, 16, 16), (1, 8, 8), (0, 4, 4)),
                            ((1, 64, 64), (1, 16, 16), (0, 8, 8)),
                            ((1, 256, 256), (1, 32, 32), (0, 16, 16))]:
        neg = tuple(-x for x in s)
        assert _partition_sets(grid, window, s) == _partition_sets(grid, window, neg)


def test_video_shift_sign_changes_membership():
    g, w = (21, 30, 52), (7, 15, 26)
    assert _partition_sets(g, w, (3, 7, 13)) != _partition_sets(g, w, (-3, -7, -13))
    # the w-axis offset 13 is half of 26, so on that axis alone the sign does not matter
    assert _partition_sets(g, w, (0, 0, 13)) == _partition_sets(g, w, (0, 0, -13))
    assert _partition_sets(g, w, (3, 0, 0)) != _partition_sets(g, w, (-3, 0, 0))
    assert _partition_sets(g, w, (0, 7, 0)) != _partition_sets(g, w, (0, -7, 0))


def test_window_rows_are_contiguous_runs_with_at_most_one_wrap():
    """Inside one window row (fixed t, h) the members are consecutive grid columns, with
    at most one wrap-around per row: what lets a kernel read them with wide loads."""
    g, w, s = (21, 30, 52), (7, 15, 26), (3, 7, 13)
    table = O.window_members(g, w, s)
    W = g[2]
    for row in table.reshape(-1, w[2]):
        cols = row % W
        breaks = np.count_nonzero(np.diff(cols) != 1)
        assert breaks <= 1


def test_table3_density_golden():
    """Table 3 of the paper prints attention sparsity for the Wan2.1 workload. With
    M = window tokens (full temporal extent), one routed window (K = 1) and G pooled
    tokens, density = (2M + G) / N. The partition helper must give M / N = 1/16 for the
    15x26 windows on the 60x104 latent grid, which reproduces the printed values."""
    with open(os.path.join(GOLDEN, "wan_table3_density.json")) as f:
        gold = json.load(f)
    T, H, W = gold["latent_grid"]
    for row in gold["rows"]:
        wh, ww = row["window"]
        ph, pw = row["pool"]
        table = O.window_members((T, H, W), (T, wh, ww), (0, 0, 0))
        n_win, M = table.shape
        N = T * H * W
        G = T * (-(-H // ph)) * (-(-W // pw))
        sparsity = 1.0 - (2 * M + G) / N
        assert round(100 * sparsity, 2) == row["sparsity_percent"], row
        assert n_win == 16


def test_members_of_agrees_with_table():
    for grid, window, s in [((21, 30, 52), (7, 15, 26), (3, 7, 13)), ((1, 64, 64), (1, 16, 16), (0, 8, 8)),
                            ((6, 6, 6), (3, 2, 3), (-1, -5, 8))]:
        table = O.window_members(grid, window, s)
        win, _ = forward_map(grid, window, O.reduce_shift(grid, s))
        for p in np.random.default_rng(0).choice(int(np.prod(grid)), 50, replace=False):
            assert np.array_equal(O.members_of(grid, window, s, p), table[win[p]])
