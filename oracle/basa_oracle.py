"""fp64 CPU oracle for BASA shifted local-window attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls or links this
module; only the tests, the smoke check and the benchmark's CPU-baseline leg do. It
shares no code with the HIP library: it is written from the paper alone.

Source: "Backend-Agnostic Sparse Attention for Fast High-Resolution Visual Generation"
(Ma, Song, Wu, Liu, Zhao; arXiv 2610.08772).
  * §3.1 "Shifted Window Sparse Attention": the token grid is cyclically shifted by
    -Delta, cut into non-overlapping windows, each window gets ordinary scaled
    dot-product softmax attention, and the outputs are shifted back by +Delta.
  * §3.1 "Attention complexity" and App. A.1 "Regular execution with standard attention
    backends": the shift is a cyclic roll, the partition is a pure reshape/permute of
    a grid exactly divisible by the window, and all windows are folded into the batch.

Readings taken where the paper is silent (each is listed with its reason in the design
notes of this repository):
  * sign: "shift by -Delta" is a roll by -Delta, i.e. shifted[i] = x[(i + Delta) mod n],
    so window m along an axis holds the original positions (m*w + l + Delta) mod n;
  * windows that wrap the grid edge attend across it (a torus, no mask);
  * the partition is only defined for grids exactly divisible by the window;
  * the video case generalises the paper's 2-D (h, w) offset to (t, h, w); a window
    spanning the whole temporal axis (wt = T) is the paper's own video setting;
  * the softmax scale is 1/sqrt(head_dim);
  * windows are numbered row-major over (t, h, w) window coordinates and members in a
    window row-major over (t, h, w) local coordinates. The output does not depend on
    this order; the exported membership table does.

Arrays are [B, heads, N, head_dim] with N = T*H*W tokens flattened row-major over
(t, h, w). Everything is computed in float64.
"""
from __future__ import annotations

import math
from typing import Sequence, Tuple

import numpy as np

Triple = Tuple[int, int, int]


def _as_triple(x: Sequence[int], what: str) -> Triple:
    t = tuple(int(v) for v in x)
    if len(t) != 3:
        raise ValueError(f"{what} must have 3 entries (t, h, w), got {x!r}")
    return t  # type: ignore[return-value]


def check_partition(grid: Sequence[int], window: Sequence[int]) -> Tuple[Triple, Triple]:
    """Validate a grid/window pair: positive sizes, window divides the grid exactly
    (App. A.1: the reshape-only partition applies to exactly divisible resolutions)."""
    g = _as_triple(grid, "grid")
    w = _as_triple(window, "window")
    for n, m, ax in zip(g, w, "thw"):
        if n <= 0 or m <= 0:
            raise ValueError(f"axis {ax}: sizes must be positive (grid {n}, window {m})")
        if n % m:
            raise ValueError(f"axis {ax}: window {m} does not divide grid {n}")
    return g, w


def reduce_shift(grid: Sequence[int], shift: Sequence[int]) -> Triple:
    """Shift offsets reduced into [0, n) per axis: a cyclic roll by n is the identity."""
    g = _as_triple(grid, "grid")
    s = _as_triple(shift, "shift")
    return tuple(si % ni for si, ni in zip(s, g))  # type: ignore[return-value]


def window_members(grid: Sequence[int], window: Sequence[int], shift: Sequence[int]) -> np.ndarray:
    """Membership table of the shifted partition, shape [n_windows, window_tokens].

    Entry [m, l] is the flat index (in the original, unshifted grid) of the token that
    sits at local position l of window m after rolling the grid by -shift (§3.1).
    Per axis: original position = (m_a * w_a + l_a + s_a) mod n_a.
    """
    (T, H, W), (wt, wh, ww) = check_partition(grid, window)
    st, sh, sw = reduce_shift(grid, shift)
    nt, nh, nw = T // wt, H // wh, W // ww
    table = np.empty((nt * nh * nw, wt * wh * ww), dtype=np.int64)
    m = 0
    for mt in range(nt):
        for mh in range(nh):
            for mw in range(nw):
                l = 0
                for lt in range(wt):
                    pt = (mt * wt + lt + st) % T
                    for lh in range(wh):
                        ph = (mh * wh + lh + sh) % H
                        for lw in range(ww):
                            pw = (mw * ww + lw + sw) % W
                            table[m, l] = (pt * H + ph) * W + pw
                            l += 1
                m += 1
    return table


def members_of(grid: Sequence[int], window: Sequence[int], shift: Sequence[int], token: int) -> np.ndarray:
    """Members (flat original tokens, in local order) of the window holding ``token``:
    the rolled position of the token along each axis is (p - s) mod n, its window
    coordinate that position // w; the members then follow the same rule as
    ``window_members``. Lets huge grids be sampled without building the whole table."""
    (T, H, W), (wt, wh, ww) = check_partition(grid, window)
    st, sh, sw = reduce_shift(grid, shift)
    token = int(token)
    pt, ph, pw = token // (H * W), (token // W) % H, token % W
    mt, mh, mw = ((pt - st) % T) // wt, ((ph - sh) % H) // wh, ((pw - sw) % W) // ww
    out = []
    for lt in range(wt):
        for lh in range(wh):
            for lw in range(ww):
                out.append((((mt * wt + lt + st) % T) * H + (mh * wh + lh + sh) % H) * W + (mw * ww + lw + sw) % W)
    return np.array(out, dtype=np.int64)


def _attend(Qw: np.ndarray, Kw: np.ndarray, Vw: np.ndarray, scale: float):
    """Dense softmax(Q K^T * scale) V for one window, plus the per-row log-sum-exp of
    the scaled logits. Plain definition, with the usual max subtraction."""
    S = (Qw @ Kw.T) * scale
    mx = S.max(axis=1, keepdims=True)
    P = np.exp(S - mx)
    den = P.sum(axis=1, keepdims=True)
    O = (P / den) @ Vw
    lse = (mx + np.log(den))[:, 0]
    return O, lse


def _check_qkv(q, k, v, upcast=True):
    """Shape check; with ``upcast`` the arrays are converted to float64 as a whole. The
    sampled-row functions pass upcast=False and convert each gathered slice instead, so
    full-size float32 inputs are never copied in full (the arithmetic is float64 either
    way)."""
    if upcast:
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    if q.ndim != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError(f"q, k, v must share one [B, heads, N, d] shape: {q.shape} {k.shape} {v.shape}")
    return q, k, v


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def window_attention(q, k, v, grid, window, shift, *, return_lse: bool = False):
    """Shifted local-window attention (§3.1), explicit loop over (batch, head, window).

    For every window of the shifted partition, the member rows of q, k, v are gathered,
    given dense scaled dot-product softmax attention, and the result rows are written
    back at the members' original positions (the "shift back").
    Returns out [B, heads, N, d] (and the per-row log-sum-exp [B, heads, N] of the
    scaled logits when ``return_lse``).
    """
    q, k, v = _check_qkv(q, k, v)
    B, Hh, N, d = q.shape
    table = window_members(grid, window, shift)
    if table.size != N:
        raise ValueError(f"grid holds {table.size} tokens but q has N={N}")
    scale = 1.0 / math.sqrt(d)
    out = np.empty_like(q)
    lse = np.empty((B, Hh, N), dtype=np.float64)
    for b in range(B):
        for h in range(Hh):
            for members in table:
                O, l = _attend(q[b, h, members], k[b, h, members], v[b, h, members], scale)
                out[b, h, members] = O
                lse[b, h, members] = l
    return (out, lse) if return_lse else out


def window_attention_loops(q, k, v, grid, window, shift):
    """The same computation in scalar Python loops, for tiny cases only. Serves as a
    check of the BLAS formulation above (no numpy reductions or matmuls used)."""
    q, k, v = _check_qkv(q, k, v)
    B, Hh, N, d = q.shape
    table = window_members(grid, window, shift).tolist()
    scale = 1.0 / math.sqrt(d)
    out = np.zeros_like(q)
    for b in range(B):
        for h in range(Hh):
            for members in table:
                for i in members:
                    logits = []
                    for j in members:
                        acc = 0.0
                        for c in range(d):
                            acc += q[b, h, i, c] * k[b, h, j, c]
                        logits.append(acc * scale)
                    top = max(logits)
                    weights = [math.exp(x - top) for x in logits]
                    total = sum(weights)
                    for c in range(d):
                        acc = 0.0
                        for wgt, j in zip(weights, members):
                            acc += wgt * v[b, h, j, c]
                        out[b, h, i, c] = acc / total
    return out


def window_weights(q, k, grid, window, shift, b: int = 0, h: int = 0):
    """Per-window softmax weight matrices P (list of [W, W]) for one (batch, head):
    the attention map the window attention applies. Used to check its properties."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d)
    mats = []
    for members in window_members(grid, window, shift):
        S = (q[b, h, members] @ k[b, h, members].T) * scale
        P = np.exp(S - S.max(axis=1, keepdims=True))
        mats.append(P / P.sum(axis=1, keepdims=True))
    return mats


def window_attention_rows(q, k, v, grid, window, shift, rows):
    """Output rows ``rows`` (flat original token indices) of window attention, for all
    (batch, head); shape [B, heads, len(rows), d]. Each row is computed on its own from
    its window's keys and values, so full-size workloads can be sampled cheaply."""
    q, k, v = _check_qkv(q, k, v, upcast=False)
    B, Hh, N, d = q.shape
    table = window_members(grid, window, shift)
    owner = np.empty(N, dtype=np.int64)
    for m, members in enumerate(table):
        owner[members] = m
    rows = np.asarray(rows, dtype=np.int64)
    scale = 1.0 / math.sqrt(d)
    out = np.empty((B, Hh, rows.size, d), dtype=np.float64)
    for b in range(B):
        for h in range(Hh):
            for r_i, r in enumerate(rows):
                members = table[owner[r]]
                O, _ = _attend(_f64(q[b, h, r:r + 1]), _f64(k[b, h, members]), _f64(v[b, h, members]), scale)
                out[b, h, r_i] = O[0]
    return out


def full_attention(q, k, v, *, return_lse: bool = False):
    """Dense softmax attention over all N tokens: the baseline the paper's speedups
    are measured against (Tables 2 and 3, "Dense"/SDPA rows)."""
    q, k, v = _check_qkv(q, k, v)
    B, Hh, N, d = q.shape
    scale = 1.0 / math.sqrt(d)
    out = np.empty_like(q)
    lse = np.empty((B, Hh, N), dtype=np.float64)
    for b in range(B):
        for h in range(Hh):
            out[b, h], lse[b, h] = _attend(q[b, h], k[b, h], v[b, h], scale)
    return (out, lse) if return_lse else out


def full_attention_rows(q, k, v, rows):
    """Rows ``rows`` of dense attention, [B, heads, len(rows), d]."""
    q, k, v = _check_qkv(q, k, v, upcast=False)
    B, Hh, N, d = q.shape
    rows = np.asarray(rows, dtype=np.int64)
    scale = 1.0 / math.sqrt(d)
    out = np.empty((B, Hh, rows.size, d), dtype=np.float64)
    for b in range(B):
        for h in range(Hh):
            out[b, h], _ = _attend(_f64(q[b, h, rows]), _f64(k[b, h]), _f64(v[b, h]), scale)
    return out
