"""Interleaved shift schedule (BASA §3.1, Eq. 1-3): the reference pinned by hand-derived
cases and invariants, and the library's host function checked against it exactly."""
import ctypes

import numpy as np
import pytest

from oracle import schedule_oracle as S
from sparse_attention_dit_amd import _lib


def test_worked_case_w32_L32():
    # delta = max(1, 32 // 32) = 1, so a_i = i and K = 16: b = (0, 16, 1, 17, ..., 15, 31)
    b = S.layer_offsets(32, 32)
    assert b == [x for j in range(16) for x in (j, 16 + j)]


def test_printed_pattern_even_L():
    for w, L in [(32, 8), (16, 12), (26, 10), (15, 4)]:
        a, b = S.offsets(w, L), S.layer_offsets(w, L)
        K = L // 2
        assert b[:4] == [a[0], a[K], a[1], a[K + 1]]
        assert b[-2:] == [a[K - 1], a[L - 1]]


def test_delta_and_wrap():
    assert S.offsets(32, 8) == [0, 4, 8, 12, 16, 20, 24, 28]          # delta = 4
    assert S.offsets(16, 57) == [i % 16 for i in range(57)]          # delta = max(1, 0) = 1
    assert S.offsets(26, 4) == [0, 6, 12, 18]                         # delta = floor(26/4) = 6


@pytest.mark.parametrize("w,L", [(32, 32), (32, 7), (16, 57), (26, 5), (15, 1), (7, 2), (30, 19)])
def test_interleave_is_the_out_shuffle(w, L):
    """Independent derivation: with K = ceil(L/2), element a_i sits at position 2i (first
    half) or 2(i-K)+1 (second half); b is therefore a permutation of a."""
    a = S.offsets(w, L)
    K = (L + 1) // 2
    b = [None] * L
    for i, x in enumerate(a):
        b[2 * i if i < K else 2 * (i - K) + 1] = x
    assert S.layer_offsets(w, L) == b
    assert sorted(b) == sorted(a)


def test_step_offset_is_modular():
    base = S.shift_schedule(10, 15, 26)
    assert base == list(zip(S.layer_offsets(15, 10), S.layer_offsets(26, 10)))
    assert S.shift_schedule(10, 15, 26, (15, 26)) == base
    assert S.shift_schedule(10, 15, 26, (-1, 3)) == [((h - 1) % 15, (w + 3) % 26) for h, w in base]


def test_planted_mistakes_are_caught(monkeypatch):
    real = S.interleave

    def floor_half(a):  # K = L // 2 drops an element for odd L
        K = len(a) // 2
        return [x for j in range(K) for x in (a[j], a[K + j])]

    monkeypatch.setattr(S, "interleave", floor_half)
    with pytest.raises(AssertionError):
        test_interleave_is_the_out_shuffle(26, 5)
    monkeypatch.setattr(S, "interleave", lambda a: real(a[len(a) // 2:] + a[:len(a) // 2]))  # halves swapped
    with pytest.raises(AssertionError):
        test_worked_case_w32_L32()


@pytest.mark.parametrize("L,wh,ww,c", [(32, 32, 32, (0, 0)), (57, 16, 16, (3, -5)), (10, 15, 26, (7, 11)),
                                      (7, 32, 16, (-40, 100)), (1, 8, 8, (0, 0)), (19, 30, 52, (1, 1))])
def test_library_matches_reference(L, wh, ww, c):
    got = _lib.shift_schedule(L, (wh, ww), c)
    assert got == S.shift_schedule(L, wh, ww, c)


def test_library_argument_errors():
    lib = _lib.load()
    buf = (ctypes.c_int32 * 4)()
    assert lib.basa_shift_schedule(0, 8, 8, 0, 0, buf, buf) == 2
    assert lib.basa_shift_schedule(4, 0, 8, 0, 0, buf, buf) == 2
    assert lib.basa_shift_schedule(4, 8, 8, 0, 0, None, buf) == 1
