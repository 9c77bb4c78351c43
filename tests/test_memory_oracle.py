"""Pins for the pooled-memory reference (BASA §3.2 Eq. 4-5, App. A.1 Eq. 9 and Eq. 12).

Each test checks it against something other than itself:
  * pooling against a scatter-add over every token (region = integer division), with
    partial regions at the far edges, and the p = 1 / p = whole-frame special cases;
  * window + memory attention against dense attention over [K; pooled K] with a
    block-diagonal mask built from a numpy.roll-ed index grid;
  * the page's own merge formula (Eq. 12) applied to a window-only and a memory-only
    result, each with its log-sum-exp;
  * closed forms (q = 0 averages window and memory values) and the log-sum-exp against
    scipy's logsumexp.
"""
import math

import numpy as np
import pytest
from scipy.special import logsumexp

from oracle import basa_oracle as O
from oracle import memory_oracle as M


def _rand(shape, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(shape)


def _scatter_pool(x, grid, pool):
    T, H, W = grid
    ph, pw = pool
    gh, gw = -(-H // ph), -(-W // pw)
    B, Hh, N, d = x.shape
    acc = np.zeros((B, Hh, T * gh * gw, d))
    cnt = np.zeros(T * gh * gw)
    for tok in range(N):
        t, h, w = tok // (H * W), (tok // W) % H, tok % W
        g = (t * gh + h // ph) * gw + w // pw
        acc[:, :, g] += x[:, :, tok]
        cnt[g] += 1
    return acc / cnt[None, None, :, None]


@pytest.mark.parametrize("grid,pool", [((1, 8, 8), (4, 4)), ((1, 10, 7), (4, 3)), ((3, 5, 9), (2, 4)),
                                       ((2, 6, 6), (1, 1)), ((2, 4, 6), (4, 6)), ((1, 3, 3), (5, 5))])
def test_pool_matches_scatter_add(grid, pool):
    x = _rand((2, 2, int(np.prod(grid)), 8), 3)
    got = M.pool_kv(x, grid, pool)
    assert got.shape[2] == M.pooled_count(grid, pool)
    assert np.allclose(got, _scatter_pool(x, grid, pool), atol=1e-13, rtol=0)


def test_pool_special_cases():
    grid = (2, 6, 10)
    x = _rand((1, 2, 120, 4), 4)
    assert np.array_equal(M.pool_kv(x, grid, (1, 1)), x)
    frame_means = x.reshape(1, 2, 2, 60, 4).mean(axis=3)
    assert np.allclose(M.pool_kv(x, grid, (6, 10)), frame_means, atol=1e-14)
    assert M.pooled_count((21, 60, 104), (4, 4)) == 21 * 15 * 26
    assert M.pooled_count((1, 128, 128), (4, 4)) == 1024


def _masked_dense(q, keys, vals, mask):
    d = q.shape[-1]
    S = np.einsum("bhid,bhjd->bhij", q, keys) / math.sqrt(d)
    S = np.where(mask, S, -np.inf)
    lse = logsumexp(S, axis=-1)
    P = np.exp(S - lse[..., None])
    return np.einsum("bhij,bhjd->bhid", P, vals), lse


def _window_mask(grid, window, shift):
    """[N, N] same-window mask from an index grid rolled by -shift and cut into blocks."""
    T, H, W = grid
    wt, wh, ww = window
    idx = np.arange(T * H * W).reshape(T, H, W)
    rolled = np.roll(idx, shift=(-shift[0], -shift[1], -shift[2]), axis=(0, 1, 2))
    lab = np.empty(T * H * W, dtype=np.int64)
    wid = (np.arange(T)[:, None, None] // wt * (H // wh) + np.arange(H)[None, :, None] // wh) * (W // ww) \
        + np.arange(W)[None, None, :] // ww
    lab[rolled.ravel()] = wid.ravel()
    return lab[:, None] == lab[None, :]


CASES = [((1, 8, 8), (1, 4, 4), (0, 2, 3), (4, 4)), ((2, 6, 9), (2, 3, 3), (1, 1, 2), (3, 4)),
         ((3, 4, 6), (1, 2, 3), (2, 3, 5), (2, 2))]


@pytest.mark.parametrize("grid,window,shift,pool", CASES)
def test_window_memory_matches_masked_dense(grid, window, shift, pool):
    N = int(np.prod(grid))
    q, k, v = (_rand((1, 2, N, 8), s) for s in (10, 11, 12))
    km, vm = M.pool_kv(k, grid, pool), M.pool_kv(v, grid, pool)
    got, lse = M.window_attention_memory(q, k, v, km, vm, grid, window, shift, return_lse=True)
    Mm = km.shape[2]
    mask = np.concatenate([_window_mask(grid, window, shift), np.ones((N, Mm), dtype=bool)], axis=1)
    ref, ref_lse = _masked_dense(q, np.concatenate([k, km], 2), np.concatenate([v, vm], 2), mask)
    assert np.allclose(got, ref, atol=1e-12, rtol=0)
    assert np.allclose(lse, ref_lse, atol=1e-12, rtol=0)


@pytest.mark.parametrize("grid,window,shift,pool", CASES)
def test_merge_formula_recovers_the_joint_softmax(grid, window, shift, pool):
    N = int(np.prod(grid))
    q, k, v = (_rand((1, 2, N, 8), s) for s in (20, 21, 22))
    km, vm = M.pool_kv(k, grid, pool), M.pool_kv(v, grid, pool)
    o_w, l_w = O.window_attention(q, k, v, grid, window, shift, return_lse=True)
    o_m, l_m = _masked_dense(q, km, vm, np.ones((N, km.shape[2]), dtype=bool))
    o, l = M.merge(o_w, l_w, o_m, l_m)
    joint, joint_lse = M.window_attention_memory(q, k, v, km, vm, grid, window, shift, return_lse=True)
    assert np.allclose(o, joint, atol=1e-12, rtol=0)
    assert np.allclose(l, joint_lse, atol=1e-12, rtol=0)


def test_closed_forms_and_empty_memory():
    grid, window, shift, pool = (1, 8, 8), (1, 4, 4), (0, 1, 2), (2, 2)
    k, v = _rand((1, 1, 64, 4), 30), _rand((1, 1, 64, 4), 31)
    km, vm = M.pool_kv(k, grid, pool), M.pool_kv(v, grid, pool)
    q0 = np.zeros_like(k)
    got = M.window_attention_memory(q0, k, v, km, vm, grid, window, shift)
    table = O.window_members(grid, window, shift)
    for members in table:
        expect = (v[0, 0, members].sum(0) + vm[0, 0].sum(0)) / (members.size + vm.shape[2])
        assert np.allclose(got[0, 0, members], expect, atol=1e-14)
    q = _rand((1, 1, 64, 4), 32)
    empty = np.zeros((1, 1, 0, 4))
    assert np.allclose(M.window_attention_memory(q, k, v, empty, empty, grid, window, shift),
                       O.window_attention(q, k, v, grid, window, shift), atol=1e-14, rtol=0)


def test_rows_match_whole_tensor():
    grid, window, shift, pool = (2, 6, 9), (2, 3, 3), (1, 4, 7), (3, 4)
    q, k, v = (_rand((1, 2, 108, 8), s) for s in (40, 41, 42))
    km, vm = M.pool_kv(k, grid, pool), M.pool_kv(v, grid, pool)
    full, lse = M.window_attention_memory(q, k, v, km, vm, grid, window, shift, return_lse=True)
    rows = np.array([0, 5, 33, 107])
    o, l = M.window_attention_memory_rows(q, k, v, km, vm, grid, window, shift, rows)
    assert np.allclose(o, full[:, :, rows], atol=1e-13) and np.allclose(l, lse[:, :, rows], atol=1e-13)


def test_planted_mistakes_are_caught(monkeypatch):
    # a pooling that drops the partial far-edge regions (floor instead of ceil)
    real_pool = M.pool_kv

    def floor_pool(x, grid, pool):
        T, H, W = grid
        ph, pw = pool
        full = real_pool(x, grid, pool)
        gh, gw = -(-H // ph), -(-W // pw)
        keep = [(t * gh + i) * gw + j for t in range(T) for i in range(H // ph) for j in range(W // pw)]
        return full[:, :, keep]
    monkeypatch.setattr(M, "pool_kv", floor_pool)
    with pytest.raises(AssertionError):
        test_pool_matches_scatter_add((1, 10, 7), (4, 3))
    monkeypatch.setattr(M, "pool_kv", real_pool)
    # a merge with the weight of the wrong branch
    real_merge = M.merge
    monkeypatch.setattr(M, "merge", lambda a, la, b, lb: real_merge(a, lb, b, la))
    with pytest.raises(AssertionError):
        test_merge_formula_recovers_the_joint_softmax(*CASES[0])
    monkeypatch.setattr(M, "merge", real_merge)
    # memory values not appended (keys only): values of the window stand in
    real_attn = M.window_attention_memory

    def keys_only(q, k, v, km, vm, *a, **kw):
        return real_attn(q, k, v, km, np.zeros_like(vm), *a, **kw)
    monkeypatch.setattr(M, "window_attention_memory", keys_only)
    with pytest.raises(AssertionError):
        test_window_memory_matches_masked_dense(*CASES[1])
