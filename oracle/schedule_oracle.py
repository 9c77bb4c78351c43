"""Reference for BASA's interleaved shift schedule (pure integers).

TEST INFRASTRUCTURE ONLY. Only the tests use this module; the library's schedule
function is written separately and is checked against it.

Source: "Backend-Agnostic Sparse Attention for Fast High-Resolution Visual Generation",
§3.1, "Interleaved shift schedule", the three displayed equations (numbered Eq. 1-3
here in order of appearance):
  Eq. 1: for a window side w and L sparse-attention layers, the offsets
         a_i = (i * delta) mod w with delta = max(1, floor(w / L)), i = 0 .. L-1;
  Eq. 2: the per-layer offsets b interleave the two halves of a:
         (b_0, .., b_{L-1}) = (a_0, a_K, a_1, a_{K+1}, .., a_{K-1}, a_{L-1});
  Eq. 3: the shift of layer l at denoising step s is
         Delta_{l,s} = ((b^h_l + c^h_s) mod w_h, (b^w_l + c^w_s) mod w_w),
         with b^h built for w = w_h and b^w for w = w_w.

Readings (the page leaves them open):
  * K = ceil(L / 2): the interleaving takes a_0, a_K, a_1, a_{K+1}, ... alternately from
    the first half (a_0 .. a_{K-1}) and the second half (a_K .. a_{L-1}). For even L this
    ends with a_{K-1}, a_{L-1} exactly as printed; for odd L the first half is one longer
    and the sequence ends with a_{K-1}.
  * c_s, the per-step offset, is not defined on the page: it is a caller-supplied pair of
    integers (any sign; reduced modulo the window side).
"""
from __future__ import annotations

from typing import List, Tuple


def offsets(w: int, L: int) -> List[int]:
    """Eq. 1: a_i = (i * delta) mod w, delta = max(1, floor(w / L))."""
    if w <= 0 or L <= 0:
        raise ValueError("window side and layer count must be positive")
    delta = max(1, w // L)
    return [(i * delta) % w for i in range(L)]


def interleave(a: List[int]) -> List[int]:
    """Eq. 2 with K = ceil(L / 2): first half and second half taken alternately."""
    L = len(a)
    K = (L + 1) // 2
    first, second = a[:K], a[K:]
    b = []
    for j in range(K):
        b.append(first[j])
        if j < len(second):
            b.append(second[j])
    return b


def layer_offsets(w: int, L: int) -> List[int]:
    """b for one axis: Eq. 2 applied to Eq. 1."""
    return interleave(offsets(w, L))


def shift_schedule(L: int, wh: int, ww: int, c: Tuple[int, int] = (0, 0)) -> List[Tuple[int, int]]:
    """Eq. 3: (Delta^h, Delta^w) for layers l = 0 .. L-1 at a step with offset c = (c^h, c^w)."""
    bh, bw = layer_offsets(wh, L), layer_offsets(ww, L)
    return [((bh[l] + c[0]) % wh, (bw[l] + c[1]) % ww) for l in range(L)]
