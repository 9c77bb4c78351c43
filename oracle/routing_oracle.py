"""fp64 reference for BASA's content-adaptive true-window routing.

TEST INFRASTRUCTURE ONLY. Only the tests use this module; it shares no code with the HIP
library and is written from the paper alone.

Source: "Backend-Agnostic Sparse Attention for Fast High-Resolution Visual Generation".
  * §3.3 "Content-Adaptive True-Window Routing": each query window i gets a descriptor
    q_i, the mean of its query tokens, and every candidate window j a descriptor k_j, the
    mean of its key tokens (the displayed equation, Eq. 6 here); their relevance is the
    scaled dot product s_ij = q_i . k_j / sqrt(d); the router keeps the TopK candidates
    of a restricted candidate set C_i, and window i then attends to its own tokens, the
    routed windows' original (uncompressed) tokens and the pooled memory.
  * App. A.2 "Video resolution extrapolation": K = 1 routed window, candidate windows
    within radius one of the query window.

Readings (the pages leave them open):
  * windows are those of the current shifted partition, numbered row-major over window
    coordinates (t, h, w) like everywhere else; "radius one" is Chebyshev distance <= 1
    on those coordinates (for the pages' video windows, which span the whole temporal
    axis, that is the spatial 3x3 neighbourhood), without wrap-around at the window-grid
    edges, and the query window itself is not a candidate (its tokens are always
    attended);
  * ties in s_ij go to the lowest window index; a window with no candidate routes to -1
    (nothing is added);
  * one softmax spans the window, the routed window and the memory (as §3.2 does for
    window and memory); the routed window's tokens are attended in their window's slot
    order.
"""
from __future__ import annotations

import math
from typing import List, Sequence

import numpy as np

from .basa_oracle import _attend, _check_qkv, _f64, check_partition, window_members


def window_grid(grid: Sequence[int], window: Sequence[int]):
    (T, H, W), (wt, wh, ww) = check_partition(grid, window)
    return T // wt, H // wh, W // ww


def window_means(x, grid, window, shift) -> np.ndarray:
    """Eq. 6 descriptors: mean of x over each window's members, [B, heads, n_win, d]."""
    x = _f64(x)
    table = window_members(grid, window, shift)
    return np.stack([x[:, :, members].mean(axis=2) for members in table], axis=2)


def candidates(grid, window, radius: int = 1) -> List[List[int]]:
    """C_i for every window i: windows at Chebyshev distance 1..radius on the window grid,
    no wrap-around, ascending index."""
    nt, nh, nw = window_grid(grid, window)
    out = []
    for i in range(nt * nh * nw):
        ti, hi, wi = i // (nh * nw), (i // nw) % nh, i % nw
        c = []
        for j in range(nt * nh * nw):
            tj, hj, wj = j // (nh * nw), (j // nw) % nh, j % nw
            dist = max(abs(ti - tj), abs(hi - hj), abs(wi - wj))
            if 1 <= dist <= radius:
                c.append(j)
        out.append(c)
    return out


def scores(qbar, kbar) -> np.ndarray:
    """s_ij = q_i . k_j / sqrt(d) for every pair, [B, heads, n_win, n_win]."""
    qbar, kbar = _f64(qbar), _f64(kbar)
    return np.einsum("bhid,bhjd->bhij", qbar, kbar) / math.sqrt(qbar.shape[-1])


def route_top1(qbar, kbar, grid, window, radius: int = 1) -> np.ndarray:
    """TopK with K = 1 over C_i (ties -> lowest index, empty C_i -> -1): [B, heads, n_win]."""
    s = scores(qbar, kbar)
    C = candidates(grid, window, radius)
    B, Hh, n, _ = s.shape
    route = np.full((B, Hh, n), -1, dtype=np.int64)
    for b in range(B):
        for h in range(Hh):
            for i in range(n):
                best = None
                for j in C[i]:  # ascending, strict > keeps the lowest index on ties
                    if best is None or s[b, h, i, j] > s[b, h, i, best]:
                        best = j
                route[b, h, i] = -1 if best is None else best
    return route


def routed_attention(q, k, v, route, grid, window, shift, kmem=None, vmem=None, *, return_lse: bool = False):
    """Window i's queries attend, in one softmax, to window i's tokens, the tokens of
    window route[b, h, i] (if >= 0) and the memory tokens (if given)."""
    q, k, v = _check_qkv(q, k, v)
    B, Hh, N, d = q.shape
    table = window_members(grid, window, shift)
    scale = 1.0 / math.sqrt(d)
    out = np.empty_like(q)
    lse = np.empty((B, Hh, N))
    for b in range(B):
        for h in range(Hh):
            for i, members in enumerate(table):
                keys = [k[b, h, members]]
                vals = [v[b, h, members]]
                j = int(route[b, h, i])
                if j >= 0:
                    keys.append(k[b, h, table[j]])
                    vals.append(v[b, h, table[j]])
                if kmem is not None:
                    keys.append(_f64(kmem[b, h]))
                    vals.append(_f64(vmem[b, h]))
                out[b, h, members], lse[b, h, members] = _attend(q[b, h, members], np.concatenate(keys),
                                                                 np.concatenate(vals), scale)
    return (out, lse) if return_lse else out


def routed_attention_rows(q, k, v, route, grid, window, shift, rows, kmem=None, vmem=None):
    """Rows ``rows`` of routed_attention, each on its own: (out, lse)."""
    from .basa_oracle import members_of
    q, k, v = _check_qkv(q, k, v, upcast=False)
    B, Hh, N, d = q.shape
    (T, H, W), (wt, wh, ww) = check_partition(grid, window)
    table = window_members(grid, window, shift)
    win_of = np.empty(N, dtype=np.int64)
    for i, members in enumerate(table):
        win_of[members] = i
    scale = 1.0 / math.sqrt(d)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((B, Hh, rows.size, d))
    lse = np.empty((B, Hh, rows.size))
    for n, r in enumerate(rows):
        i = int(win_of[r])
        own = members_of(grid, window, shift, int(r))
        for b in range(B):
            for h in range(Hh):
                idx = [own]
                j = int(route[b, h, i])
                if j >= 0:
                    idx.append(table[j])
                sel = np.concatenate(idx)
                keys, vals = [_f64(k[b, h, sel])], [_f64(v[b, h, sel])]
                if kmem is not None:
                    keys.append(_f64(kmem[b, h]))
                    vals.append(_f64(vmem[b, h]))
                o, l = _attend(_f64(q[b, h, r:r + 1]), np.concatenate(keys), np.concatenate(vals), scale)
                out[b, h, n], lse[b, h, n] = o[0], l[0]
    return out, lse
