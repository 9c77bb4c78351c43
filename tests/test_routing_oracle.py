"""Pins for the true-window routing reference (BASA §3.3, Eq. 6; App. A.2: K = 1, radius 1).

Each test checks it against something other than itself:
  * window descriptors against means over the tokens labelled by a numpy.roll-ed window
    grid;
  * candidate sets against a broadcast Chebyshev-distance matrix on window coordinates;
  * the top-1 choice against numpy.argmax over the score matrix with non-candidates set
    to -inf (argmax returns the first maximum, i.e. the lowest index on ties);
  * routed attention against dense attention with a mask allowing the own window, the
    routed window and the memory.
"""
import math

import numpy as np
import pytest
from scipy.special import logsumexp

from oracle import basa_oracle as O
from oracle import memory_oracle as M
from oracle import routing_oracle as R


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _labels(grid, window, shift):
    T, H, W = grid
    wt, wh, ww = window
    idx = np.arange(T * H * W).reshape(T, H, W)
    rolled = np.roll(idx, shift=(-shift[0], -shift[1], -shift[2]), axis=(0, 1, 2))
    wid = (np.arange(T)[:, None, None] // wt * (H // wh) + np.arange(H)[None, :, None] // wh) * (W // ww) \
        + np.arange(W)[None, None, :] // ww
    lab = np.empty(T * H * W, dtype=np.int64)
    lab[rolled.ravel()] = wid.ravel()
    return lab


CASES = [((1, 12, 12), (1, 4, 4), (0, 1, 2)), ((2, 8, 9), (1, 4, 3), (1, 2, 1)), ((3, 6, 8), (3, 2, 2), (0, 1, 3)),
         ((1, 4, 4), (1, 4, 4), (0, 0, 0))]


@pytest.mark.parametrize("grid,window,shift", CASES)
def test_window_means_match_labelled_means(grid, window, shift):
    N = int(np.prod(grid))
    x = _rand((2, 2, N, 8), 1)
    lab = _labels(grid, window, shift)
    got = R.window_means(x, grid, window, shift)
    for w_id in range(lab.max() + 1):
        assert np.allclose(got[:, :, w_id], x[:, :, lab == w_id].mean(axis=2), atol=1e-14)


@pytest.mark.parametrize("grid,window", [((1, 12, 12), (1, 4, 4)), ((3, 6, 8), (1, 2, 2)), ((1, 4, 4), (1, 4, 4)),
                                         ((21, 60, 104), (21, 15, 26))])
@pytest.mark.parametrize("radius", [1, 2])
def test_candidates_match_distance_matrix(grid, window, radius):
    nt, nh, nw = R.window_grid(grid, window)
    coords = np.stack(np.indices((nt, nh, nw)).reshape(3, -1), axis=1)
    dist = np.abs(coords[:, None, :] - coords[None, :, :]).max(axis=2)
    expect = [np.nonzero((dist[i] >= 1) & (dist[i] <= radius))[0].tolist() for i in range(len(coords))]
    assert R.candidates(grid, window, radius) == expect


def _masked_argmax(s, C):
    n = s.shape[-1]
    allowed = np.zeros((n, n), dtype=bool)
    for i, c in enumerate(C):
        allowed[i, c] = True
    masked = np.where(allowed, s, -np.inf)
    r = np.argmax(masked, axis=-1)
    return np.where(allowed.any(axis=1), r, -1)


@pytest.mark.parametrize("grid,window,shift", CASES)
def test_top1_matches_masked_argmax(grid, window, shift):
    N = int(np.prod(grid))
    q, k = _rand((2, 3, N, 16), 2), _rand((2, 3, N, 16), 3)
    qbar, kbar = R.window_means(q, grid, window, shift), R.window_means(k, grid, window, shift)
    s = np.einsum("bhid,bhjd->bhij", qbar, kbar) / 4.0
    got = R.route_top1(qbar, kbar, grid, window)
    C = R.candidates(grid, window)
    assert np.array_equal(got, _masked_argmax(s, C))


def test_ties_go_to_the_lowest_index():
    grid, window = (1, 12, 12), (1, 4, 4)   # 3 x 3 window grid: the centre window 4 has 8 candidates
    qbar = np.zeros((1, 1, 9, 4))
    kbar = np.zeros((1, 1, 9, 4))
    qbar[..., 0] = 1.0
    kbar[0, 0, [2, 6, 7], 0] = 5.0          # three equal best scores for window 4
    route = R.route_top1(qbar, kbar, grid, window)
    assert route[0, 0, 4] == 2
    assert route[0, 0, 0] == 1              # all of window 0's candidates (1, 3, 4) tie at 0
    one = R.route_top1(qbar[:, :, :1], kbar[:, :, :1], (1, 4, 4), (1, 4, 4))
    assert one[0, 0, 0] == -1               # a single window has no candidate


@pytest.mark.parametrize("grid,window,shift", CASES[:3])
@pytest.mark.parametrize("with_memory", [False, True])
def test_routed_attention_matches_masked_dense(grid, window, shift, with_memory):
    N = int(np.prod(grid))
    q, k, v = (_rand((1, 2, N, 8), s) for s in (4, 5, 6))
    qbar, kbar = R.window_means(q, grid, window, shift), R.window_means(k, grid, window, shift)
    route = R.route_top1(qbar, kbar, grid, window)
    km = vm = None
    if with_memory:
        km, vm = M.pool_kv(k, grid, (2, 2)), M.pool_kv(v, grid, (2, 2))
    got, lse = R.routed_attention(q, k, v, route, grid, window, shift, km, vm, return_lse=True)
    lab = _labels(grid, window, shift)
    d = q.shape[-1]
    for h in range(2):
        allowed = (lab[:, None] == lab[None, :]) | (route[0, h][lab][:, None] == lab[None, :])
        keys, vals = k[0, h], v[0, h]
        if with_memory:
            allowed = np.concatenate([allowed, np.ones((N, km.shape[2]), dtype=bool)], axis=1)
            keys, vals = np.concatenate([keys, km[0, h]]), np.concatenate([vals, vm[0, h]])
        S = np.where(allowed, q[0, h] @ keys.T / math.sqrt(d), -np.inf)
        ref_lse = logsumexp(S, axis=1)
        ref = np.exp(S - ref_lse[:, None]) @ vals
        assert np.allclose(got[0, h], ref, atol=1e-12, rtol=0)
        assert np.allclose(lse[0, h], ref_lse, atol=1e-12, rtol=0)


def test_no_route_and_no_memory_is_plain_windows():
    grid, window, shift = (2, 8, 9), (1, 4, 3), (1, 2, 1)
    q, k, v = (_rand((1, 2, 144, 8), s) for s in (7, 8, 9))
    route = np.full((1, 2, 12), -1)
    assert np.allclose(R.routed_attention(q, k, v, route, grid, window, shift),
                       O.window_attention(q, k, v, grid, window, shift), atol=1e-14, rtol=0)


def test_rows_match_whole_tensor():
    grid, window, shift = (2, 8, 9), (1, 4, 3), (1, 2, 1)
    q, k, v = (_rand((1, 2, 144, 8), s) for s in (10, 11, 12))
    route = R.route_top1(R.window_means(q, grid, window, shift), R.window_means(k, grid, window, shift), grid,
                         window)
    km, vm = M.pool_kv(k, grid, (4, 3)), M.pool_kv(v, grid, (4, 3))
    full, lse = R.routed_attention(q, k, v, route, grid, window, shift, km, vm, return_lse=True)
    rows = np.array([0, 17, 80, 143])
    o, l = R.routed_attention_rows(q, k, v, route, grid, window, shift, rows, km, vm)
    assert np.allclose(o, full[:, :, rows], atol=1e-13) and np.allclose(l, lse[:, :, rows], atol=1e-13)


def test_planted_mistakes_are_caught(monkeypatch):
    real = R.candidates

    def with_self(grid, window, radius=1):
        return [sorted(c + [i]) for i, c in enumerate(real(grid, window, radius))]
    monkeypatch.setattr(R, "candidates", with_self)
    with pytest.raises(AssertionError):
        test_candidates_match_distance_matrix((1, 12, 12), (1, 4, 4), 1)

    def wrapped(grid, window, radius=1):
        nt, nh, nw = R.window_grid(grid, window)
        out = []
        for i in range(nt * nh * nw):
            t, h, w = i // (nh * nw), (i // nw) % nh, i % nw
            c = {((t + a) % nt * nh + (h + b) % nh) * nw + (w + e) % nw
                 for a in (-1, 0, 1) for b in (-1, 0, 1) for e in (-1, 0, 1)}
            c.discard(i)
            out.append(sorted(c))
        return out
    monkeypatch.setattr(R, "candidates", wrapped)
    with pytest.raises(AssertionError):
        test_candidates_match_distance_matrix((1, 12, 12), (1, 4, 4), 1)
    monkeypatch.setattr(R, "candidates", real)

    def last_on_ties(qbar, kbar, grid, window, radius=1):  # ties to the highest index
        s = R.scores(qbar, kbar)
        C = real(grid, window, radius)
        out = np.full(s.shape[:3], -1)
        for i, c in enumerate(C):
            for b in range(s.shape[0]):
                for h in range(s.shape[1]):
                    if c:
                        vals = s[b, h, i, c]
                        out[b, h, i] = c[len(c) - 1 - int(np.argmax(vals[::-1]))]
        return out
    monkeypatch.setattr(R, "route_top1", last_on_ties)
    with pytest.raises(AssertionError):
        test_ties_go_to_the_lowest_index()
