"""Pins for the fp64 oracle: each test checks it against something other than itself.

Pins used (BASA paper, §3.1 "Shifted Window Sparse Attention" and App. A.1 "Regular
execution with standard attention backends"):
  * brute force: dense N x N attention with a block-diagonal mask built in the shifted
    frame from an index grid rolled by numpy.roll;
  * the paper's own execution recipe: roll by -Delta, reshape/permute into windows,
    fold windows into the batch, library SDPA (torch, CPU, float64), undo the permute,
    roll back by +Delta;
  * identities: window == grid is dense attention for every shift; a shift by a whole
    window (or a whole grid) relabels windows and leaves the output bitwise unchanged;
  * closed forms: q = 0 gives the window mean of v; constant v rows give that constant;
    1x1x1 windows give v; a one-hot v probe reads back window membership;
  * softmax rows of the attention map sum to 1 and are non-negative;
  * a scalar-loop formulation of the same definition (no BLAS) on tiny inputs.
"""
import itertools
import math

import numpy as np
import pytest
import torch

from oracle import basa_oracle as O


def _rand_qkv(shape, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal(shape) for _ in range(3)]


def _dense_reference(q, k, v, mask=None):
    """Textbook masked softmax attention written from the definition, per head."""
    d = q.shape[-1]
    S = np.einsum("bhid,bhjd->bhij", q, k) / math.sqrt(d)
    if mask is not None:
        S = np.where(mask, S, -np.inf)
    S = S - S.max(axis=-1, keepdims=True)
    P = np.exp(S)
    P = P / P.sum(axis=-1, keepdims=True)
    return np.einsum("bhij,bhjd->bhid", P, v)


def _shifted_window_ids(grid, window, shift):
    """Window id of every original token, found by rolling an index grid by -shift
    with numpy.roll and cutting the rolled grid into blocks."""
    T, H, W = grid
    wt, wh, ww = window
    idx = np.arange(T * H * W).reshape(T, H, W)
    rolled = np.roll(idx, shift=(-shift[0], -shift[1], -shift[2]), axis=(0, 1, 2))
    it, ih, iw = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    block = ((it // wt) * (H // wh) + ih // wh) * (W // ww) + iw // ww
    win = np.empty(T * H * W, dtype=np.int64)
    win[rolled.ravel()] = block.ravel()
    return win


def _roll_reshape_sdpa(q, k, v, grid, window, shift):
    """The paper's App. A.1 recipe with library routines: numpy.roll, reshape/transpose,
    windows folded into the batch, torch SDPA (CPU float64), inverse permutation,
    roll back."""
    B, Hh, N, d = q.shape
    T, H, W = grid
    wt, wh, ww = window
    nt, nh, nw = T // wt, H // wh, W // ww

    def to_windows(x):
        x = x.reshape(B, Hh, T, H, W, d)
        x = np.roll(x, shift=(-shift[0], -shift[1], -shift[2]), axis=(2, 3, 4))
        x = x.reshape(B, Hh, nt, wt, nh, wh, nw, ww, d)
        x = x.transpose(0, 2, 4, 6, 1, 3, 5, 7, 8)  # B, nt, nh, nw, heads, wt, wh, ww, d
        return x.reshape(B * nt * nh * nw, Hh, wt * wh * ww, d)

    qw, kw, vw = (torch.from_numpy(np.ascontiguousarray(to_windows(x))) for x in (q, k, v))
    ow = torch.nn.functional.scaled_dot_product_attention(qw, kw, vw).numpy()
    x = ow.reshape(B, nt, nh, nw, Hh, wt, wh, ww, d).transpose(0, 4, 1, 5, 2, 6, 3, 7, 8)
    x = x.reshape(B, Hh, T, H, W, d)
    x = np.roll(x, shift=shift, axis=(2, 3, 4))
    return x.reshape(B, Hh, N, d)


SMALL_CASES = [
    # (grid, window)
    ((1, 8, 8), (1, 4, 4)),
    ((1, 8, 12), (1, 4, 3)),
    ((6, 6, 6), (3, 2, 3)),
    ((4, 6, 10), (4, 3, 5)),   # full temporal extent, the paper's video setting
]


@pytest.mark.parametrize("grid,window", SMALL_CASES)
def test_matches_block_diagonal_mask_all_shifts(grid, window):
    N = int(np.prod(grid))
    q, k, v = _rand_qkv((1, 2, N, 8), seed=11)
    T, H, W = grid
    # every shift on the two spatial axes, a few on the temporal axis, plus negatives
    shifts = [(st, sh, sw) for st in sorted({0, 1 % T, T - 1}) for sh in range(H) for sw in range(W)]
    shifts += [(-1, -3, -5), (-T - 1, -2 * H + 1, 7 * W + 2)]
    for s in shifts:
        win = _shifted_window_ids(grid, window, s)
        mask = (win[:, None] == win[None, :])[None, None]
        ref = _dense_reference(q, k, v, mask)
        got = O.window_attention(q, k, v, grid, window, s)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12, err_msg=f"shift {s}")


@pytest.mark.parametrize("grid,window", SMALL_CASES + [((1, 16, 16), (1, 8, 8))])
def test_matches_roll_reshape_sdpa_recipe(grid, window):
    N = int(np.prod(grid))
    q, k, v = _rand_qkv((2, 3, N, 16), seed=12)
    rng = np.random.default_rng(5)
    shifts = [(0, 0, 0)] + [tuple(int(x) for x in rng.integers(-40, 40, size=3)) for _ in range(6)]
    for s in shifts:
        ref = _roll_reshape_sdpa(q, k, v, grid, window, s)
        got = O.window_attention(q, k, v, grid, window, s)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12, err_msg=f"shift {s}")


def test_shift_sign_follows_roll_by_minus_delta():
    """Fix the sign reading: on a 3x6x6 grid with 3x3x3 windows a (1, 1, 2) shift is
    not its own negative modulo the window, so +s and -s give different partitions;
    the oracle must agree with numpy.roll(x, -Delta), not with numpy.roll(x, +Delta)."""
    grid, window = (3, 6, 6), (3, 3, 3)
    N = 108
    q, k, v = _rand_qkv((1, 1, N, 8), seed=13)
    s = (1, 1, 2)
    minus = _roll_reshape_sdpa(q, k, v, grid, window, s)
    plus = _roll_reshape_sdpa(q, k, v, grid, window, tuple(-x for x in s))
    got = O.window_attention(q, k, v, grid, window, s)
    np.testing.assert_allclose(got, minus, rtol=0, atol=1e-12)
    assert np.abs(got - plus).max() > 1e-3


@pytest.mark.parametrize("grid", [(1, 8, 8), (2, 3, 5), (5, 1, 7)])
def test_window_equal_grid_is_dense_for_every_shift(grid):
    N = int(np.prod(grid))
    q, k, v = _rand_qkv((1, 2, N, 8), seed=14)
    dense = _dense_reference(q, k, v)
    ranges = [range(n) for n in grid]
    for s in itertools.product(*ranges):
        got = O.window_attention(q, k, v, grid, grid, s)
        np.testing.assert_allclose(got, dense, rtol=0, atol=1e-12, err_msg=f"shift {s}")
    # the oracle's own dense path agrees with torch SDPA (library routine, CPU float64)
    sd = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x) for x in (q, k, v))).numpy()
    np.testing.assert_allclose(O.full_attention(q, k, v), sd, rtol=0, atol=1e-12)


def test_shift_by_whole_window_is_bitwise_identical():
    grid, window = (4, 8, 12), (2, 4, 3)
    q, k, v = _rand_qkv((1, 2, 384, 8), seed=15)
    base = (1, 2, 1)
    ref = O.window_attention(q, k, v, grid, window, base)
    for kt, kh, kw in [(1, 0, 0), (0, 1, 0), (0, 0, 1), (2, -3, 5), (-1, -1, -1)]:
        s = (base[0] + kt * window[0], base[1] + kh * window[1], base[2] + kw * window[2])
        got = O.window_attention(q, k, v, grid, window, s)
        assert np.array_equal(got, ref), s
    s = (base[0] + grid[0], base[1] - 2 * grid[1], base[2] + 3 * grid[2])
    assert np.array_equal(O.window_attention(q, k, v, grid, window, s), ref)
    # a shift that is not a multiple of the window changes the partition and the output
    other = O.window_attention(q, k, v, grid, window, (base[0], base[1] + 1, base[2]))
    assert np.abs(other - ref).max() > 1e-3


def test_softmax_rows_sum_to_one():
    grid, window = (2, 8, 8), (2, 4, 4)
    q, k, _ = _rand_qkv((1, 1, 128, 16), seed=16)
    for P in O.window_weights(q * 3.0, k, grid, window, (1, 2, 3)):
        assert (P >= 0).all()
        np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=P.shape[1] * 2.0 ** -52)


def test_window_weights_equal_masked_dense_attention_map():
    """Each window's weight matrix is the block of the dense softmax map, built with the
    block-diagonal mask of the shifted frame (numpy.roll of an index grid), that the
    window's members index; the map is zero between tokens of different windows. Scaled
    q makes the rows far from uniform, so a wrong scale or a transposed product fails."""
    grid, window, s = (2, 8, 8), (2, 4, 4), (1, 2, 3)
    N = 128
    q, k, _ = _rand_qkv((1, 1, N, 16), seed=17)
    q = q * 3.0
    win = _shifted_window_ids(grid, window, s)
    mask = win[:, None] == win[None, :]
    S = (q[0, 0] @ k[0, 0].T) / math.sqrt(16)
    S = np.where(mask, S, -np.inf)
    P = np.exp(S - S.max(axis=1, keepdims=True))
    P = P / P.sum(axis=1, keepdims=True)
    assert (P[~mask] == 0).all()
    table = O.window_members(grid, window, s)
    mats = O.window_weights(q, k, grid, window, s)
    assert len(mats) == len(table)
    for members, Pw in zip(table, mats):
        np.testing.assert_allclose(Pw, P[np.ix_(members, members)], rtol=0, atol=1e-14)


def test_closed_forms():
    grid, window, s = (2, 6, 8), (1, 3, 4), (1, 2, 3)
    N = 96
    q, k, v = _rand_qkv((2, 2, N, 8), seed=17)
    # q = 0: uniform weights -> mean of v over the window (membership by brute force)
    win = _shifted_window_ids(grid, window, s)
    got = O.window_attention(np.zeros_like(q), k, v, grid, window, s)
    for i in range(N):
        members = np.nonzero(win == win[i])[0]
        np.testing.assert_allclose(got[:, :, i], v[:, :, members].mean(axis=2), rtol=0, atol=1e-13)
    # constant v rows -> that constant, whatever q and k are
    c = np.random.default_rng(1).standard_normal(8)
    vc = np.broadcast_to(c, v.shape).copy()
    np.testing.assert_allclose(O.window_attention(q, k, vc, grid, window, s), vc, rtol=0, atol=1e-13)
    # 1x1x1 windows -> each token attends only to itself
    np.testing.assert_allclose(O.window_attention(q, k, v, grid, (1, 1, 1), s), v, rtol=0, atol=0)


def test_one_hot_probe_reads_membership():
    grid, window, s = (1, 8, 8), (1, 4, 4), (0, 2, 3)
    N, d = 64, 16
    rng = np.random.default_rng(18)
    probe = rng.choice(N, size=d, replace=False)
    v = np.zeros((1, 1, N, d))
    v[0, 0, probe, np.arange(d)] = 1.0
    zeros = np.zeros((1, 1, N, d))
    got = O.window_attention(zeros, zeros, v, grid, window, s)[0, 0]
    win = _shifted_window_ids(grid, window, s)
    expect = (win[:, None] == win[probe][None, :]) / 16.0
    np.testing.assert_array_equal(got, expect)


def test_scalar_loops_match_blas_mode():
    grid, window = (2, 4, 4), (2, 2, 2)
    q, k, v = _rand_qkv((1, 2, 32, 4), seed=19)
    for s in [(0, 0, 0), (1, 1, 1), (-1, 3, 2)]:
        np.testing.assert_allclose(O.window_attention_loops(q, k, v, grid, window, s),
                                   O.window_attention(q, k, v, grid, window, s), rtol=0, atol=1e-13)


def test_sampled_rows_match_whole_tensor():
    grid, window, s = (3, 8, 10), (3, 4, 5), (2, 5, 7)
    q, k, v = _rand_qkv((2, 2, 240, 8), seed=20)
    rows = np.array([0, 5, 77, 128, 239])
    full = O.window_attention(q, k, v, grid, window, s)
    np.testing.assert_allclose(O.window_attention_rows(q, k, v, grid, window, s, rows),
                               full[:, :, rows], rtol=0, atol=1e-14)
    dense = O.full_attention(q, k, v)
    np.testing.assert_allclose(O.full_attention_rows(q, k, v, rows), dense[:, :, rows], rtol=0, atol=1e-14)


def test_log_sum_exp_output():
    grid, window, s = (1, 8, 8), (1, 4, 4), (0, 1, 2)
    q, k, v = _rand_qkv((1, 1, 64, 8), seed=21)
    _, lse = O.window_attention(q, k, v, grid, window, s, return_lse=True)
    win = _shifted_window_ids(grid, window, s)
    S = (q[0, 0] @ k[0, 0].T) / math.sqrt(8)
    for i in range(64):
        row = S[i, win == win[i]]
        assert abs(lse[0, 0, i] - math.log(sum(math.exp(x) for x in row))) < 1e-12


def test_rejects_non_divisible_or_bad_sizes():
    q = np.zeros((1, 1, 64, 4))
    with pytest.raises(ValueError):
        O.window_attention(q, q, q, (1, 8, 8), (1, 3, 4), (0, 0, 0))
    with pytest.raises(ValueError):
        O.window_attention(q, q, q, (1, 8, 8), (1, 0, 4), (0, 0, 0))
    with pytest.raises(ValueError):
        O.window_attention(q, q, q, (1, 4, 8), (1, 4, 4), (0, 0, 0))  # 32 tokens != N


# --- planted mistakes: each plausible slip in the oracle must trip one of the pins above

def _pins_pass():
    """Run the brute-force, recipe and closed-form pins on a small non-square 3-D case
    with an asymmetric shift; True when the (possibly patched) oracle passes them all."""
    grid, window, s = (2, 6, 9), (2, 3, 3), (1, 1, 2)
    N = 108
    q, k, v = _rand_qkv((1, 2, N, 8), seed=23)
    got = O.window_attention(q, k, v, grid, window, s)
    win = _shifted_window_ids(grid, window, s)
    mask = (win[:, None] == win[None, :])[None, None]
    ok = np.allclose(got, _dense_reference(q, k, v, mask), rtol=0, atol=1e-10)
    ok &= np.allclose(got, _roll_reshape_sdpa(q, k, v, grid, window, s), rtol=0, atol=1e-10)
    ok &= np.allclose(O.window_attention(q, k, v, grid, grid, s), _dense_reference(q, k, v), rtol=0, atol=1e-10)
    return bool(ok)


def _members_variant(kind):
    orig = O.window_members

    def patched(grid, window, shift):
        (T, H, W), (wt, wh, ww) = O.check_partition(grid, window)
        st, sh, sw = O.reduce_shift(grid, shift)
        sgn = -1 if kind == "sign" else 1
        extra = 1 if kind == "off_by_one" else 0
        rows = []
        for mt in range(T // wt):
            for mh in range(H // wh):
                for mw in range(W // ww):
                    r = []
                    for lt in range(wt):
                        for lh in range(wh):
                            for lw in range(ww):
                                pt = (mt * wt + lt + sgn * st) % T
                                ph = (mh * wh + lh + sgn * sh) % H
                                pw = (mw * ww + lw + sgn * sw + extra) % W
                                if kind == "axes":
                                    r.append((pt * W + pw) * H + ph)
                                else:
                                    r.append((pt * H + ph) * W + pw)
                    rows.append(r)
        return np.array(rows, dtype=np.int64)
    return orig, patched


@pytest.mark.parametrize("kind", ["sign", "off_by_one", "axes"])
def test_planted_indexing_mistakes_are_caught(kind, monkeypatch):
    assert _pins_pass()
    _, patched = _members_variant(kind)
    monkeypatch.setattr(O, "window_members", patched)
    assert not _pins_pass()


@pytest.mark.parametrize("kind", ["no_scale", "wrong_axis", "k_as_v", "sqrt_d_times"])
def test_planted_arithmetic_mistakes_are_caught(kind, monkeypatch):
    assert _pins_pass()

    def attend(Qw, Kw, Vw, scale):
        if kind == "no_scale":
            scale = 1.0
        if kind == "sqrt_d_times":
            scale = 1.0 / (scale * scale) * scale  # sqrt(d) instead of 1/sqrt(d)
        S = (Qw @ Kw.T) * scale
        ax = 0 if kind == "wrong_axis" else 1
        P = np.exp(S - S.max(axis=ax, keepdims=True))
        P = P / P.sum(axis=ax, keepdims=True)
        Out = P @ (Kw if kind == "k_as_v" else Vw)
        return Out, np.zeros(Qw.shape[0])

    monkeypatch.setattr(O, "_attend", attend)
    assert not _pins_pass()
