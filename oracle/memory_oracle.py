"""fp64 reference for BASA's K/V-pooled global memory and the log-sum-exp merge.

TEST INFRASTRUCTURE ONLY. Only the tests (and the benchmark's CPU-baseline leg) use this
module; it shares no code with the HIP library and is written from the paper alone.

Source: "Backend-Agnostic Sparse Attention for Fast High-Resolution Visual Generation".
  * §3.2 "K/V-Pooled Global Memory", first displayed equation (Eq. 4 here): each pooled
    key (value) is the mean of the keys (values) of the tokens in its pooling region.
    Second displayed equation (Eq. 5): a window's keys and values are its own followed by
    all pooled ones, and its queries attend to that union (one softmax).
  * App. A.1, "Computational complexity" (Eq. 9): G = ceil(H/p_h) * ceil(W/p_w) pooled
    tokens, i.e. regions of p_h x p_w tokens with partial regions at the far edges; the
    video cost term carries G per frame, so pooling is spatial, one set per frame.
  * App. A.1, "Regular execution" (Eq. 12): two attention results over disjoint key
    sets merge as O = (1 - g) O_a + g O_b with g = sigmoid(l_b - l_a), l the per-row
    log-sum-exp of each part.

Readings (the pages leave them open):
  * pooling regions tile the original (unshifted) spatial grid from its origin,
    row-major (t, region h, region w); a region cut by the far edge averages only the
    tokens it holds;
  * pooled tokens are computed in fp64 here; the library rounds them to the tensor
    dtype (bf16 RNE), so a caller can store them.
"""
from __future__ import annotations

import math
from typing import Sequence

import numpy as np

from .basa_oracle import _attend, _check_qkv, _f64, window_members


def pooled_count(grid: Sequence[int], pool: Sequence[int]) -> int:
    """T * G with G = ceil(H/ph) * ceil(W/pw) (Eq. 9)."""
    T, H, W = (int(x) for x in grid)
    ph, pw = (int(x) for x in pool)
    if min(T, H, W, ph, pw) <= 0:
        raise ValueError("sizes must be positive")
    return T * (-(-H // ph)) * (-(-W // pw))


def pool_kv(x, grid: Sequence[int], pool: Sequence[int]) -> np.ndarray:
    """Eq. 4 for one tensor x [B, heads, T*H*W, d]: the mean over each region, returned as
    [B, heads, T*G, d] ordered (t, region row, region column)."""
    x = _f64(x)
    T, H, W = (int(v) for v in grid)
    ph, pw = (int(v) for v in pool)
    B, Hh, N, d = x.shape
    if N != T * H * W:
        raise ValueError(f"grid {grid} holds {T * H * W} tokens, x has {N}")
    gh, gw = -(-H // ph), -(-W // pw)
    xs = x.reshape(B, Hh, T, H, W, d)
    out = np.empty((B, Hh, T, gh, gw, d))
    for i in range(gh):
        for j in range(gw):
            region = xs[:, :, :, i * ph:(i + 1) * ph, j * pw:(j + 1) * pw, :]
            out[:, :, :, i, j, :] = region.mean(axis=(3, 4))
    return out.reshape(B, Hh, T * gh * gw, d)


def window_attention_memory(q, k, v, kmem, vmem, grid, window, shift, *, return_lse: bool = False):
    """Eq. 5: every window's queries attend jointly to the window's own keys/values and to
    all memory keys/values kmem, vmem [B, heads, M, d] (one softmax over the union)."""
    q, k, v = _check_qkv(q, k, v)
    kmem, vmem = _f64(kmem), _f64(vmem)
    B, Hh, N, d = q.shape
    if kmem.shape != vmem.shape or kmem.shape[:2] != (B, Hh) or kmem.shape[3] != d:
        raise ValueError("memory must be [B, heads, M, d] with q's B, heads and d")
    table = window_members(grid, window, shift)
    scale = 1.0 / math.sqrt(d)
    out = np.empty_like(q)
    lse = np.empty((B, Hh, N))
    for b in range(B):
        for h in range(Hh):
            for members in table:
                Kw = np.concatenate([k[b, h, members], kmem[b, h]], axis=0)
                Vw = np.concatenate([v[b, h, members], vmem[b, h]], axis=0)
                out[b, h, members], lse[b, h, members] = _attend(q[b, h, members], Kw, Vw, scale)
    return (out, lse) if return_lse else out


def window_attention_memory_rows(q, k, v, kmem, vmem, grid, window, shift, rows):
    """Rows ``rows`` of window_attention_memory, each computed on its own (for sampling
    large workloads); returns (out [B, heads, len(rows), d], lse [B, heads, len(rows)])."""
    from .basa_oracle import members_of
    q, k, v = _check_qkv(q, k, v, upcast=False)
    B, Hh, N, d = q.shape
    scale = 1.0 / math.sqrt(d)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((B, Hh, rows.size, d))
    lse = np.empty((B, Hh, rows.size))
    for i, r in enumerate(rows):
        members = members_of(grid, window, shift, int(r))
        for b in range(B):
            for h in range(Hh):
                Kw = np.concatenate([_f64(k[b, h, members]), _f64(kmem[b, h])], axis=0)
                Vw = np.concatenate([_f64(v[b, h, members]), _f64(vmem[b, h])], axis=0)
                o, l = _attend(_f64(q[b, h, r:r + 1]), Kw, Vw, scale)
                out[b, h, i], lse[b, h, i] = o[0], l[0]
    return out, lse


def merge(o_a, lse_a, o_b, lse_b):
    """Eq. 12: O = (1 - g) O_a + g O_b, g = sigmoid(lse_b - lse_a); the merged
    log-sum-exp is log(exp(lse_a) + exp(lse_b))."""
    o_a, o_b, lse_a, lse_b = (_f64(x) for x in (o_a, o_b, lse_a, lse_b))
    g = 1.0 / (1.0 + np.exp(lse_a - lse_b))
    o = (1.0 - g)[..., None] * o_a + g[..., None] * o_b
    return o, np.logaddexp(lse_a, lse_b)
