"""Concurrent calls on two HIP streams.

The bf16 kernels launch a persistent grid of one workgroup per CU, so two calls running
at once on different streams share the CUs. Each must still produce exactly what it
produces alone. Calls whose last round of work items is split keep the halves' partial
results in a workspace of their stream, so two such calls at once must not disturb each
other either. Both streams have the default priority.
"""
import pytest
import torch

from gpu_util import log_case
from sparse_attention_dit_amd import _lib

pytestmark = pytest.mark.gpu


def _inputs(shape, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return [torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16) for _ in range(3)]


def test_two_streams_match_serial_results():
    a_grid, a_win, a_shift = (1, 64, 64), (1, 16, 16), (0, 8, 8)
    b_grid, b_win, b_shift = (3, 30, 26), (3, 15, 13), (1, 7, 6)
    a = _inputs((1, 24, 64 * 64, 128), 11)
    b = _inputs((2, 6, 3 * 30 * 26, 64), 12)
    log_case("two streams", a_grid, a_win, b_grid, b_win)

    ref_a, ref_b = torch.empty_like(a[0]), torch.empty_like(b[0])
    _lib.window_attn_fwd(*a, ref_a, a_grid, a_win, a_shift)
    _lib.window_attn_fwd(*b, ref_b, b_grid, b_win, b_shift)
    torch.cuda.synchronize()

    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    out_a, out_b = torch.empty_like(ref_a), torch.empty_like(ref_b)
    for _ in range(3):
        with torch.cuda.stream(s1):
            for _ in range(4):
                _lib.window_attn_fwd(*a, out_a, a_grid, a_win, a_shift, stream=s1)
        with torch.cuda.stream(s2):
            for _ in range(4):
                _lib.window_attn_fwd(*b, out_b, b_grid, b_win, b_shift, stream=s2)
        torch.cuda.synchronize()
        assert torch.equal(out_a, ref_a), "stream 1 result differs from the serial one"
        assert torch.equal(out_b, ref_b), "stream 2 result differs from the serial one"


def test_two_streams_with_split_items():
    """Both streams run the per-item kernel with a split last round at the same time."""
    grid, win = (1, 48, 90), (1, 24, 45)  # 17-tile windows
    a_shift, b_shift = (0, 7, -11), (0, -5, 13)
    a = _inputs((1, 19, 48 * 90, 128), 21)  # 380 items: 124 split
    b = _inputs((1, 18, 48 * 90, 64), 22)   # 360 items: 104 split
    log_case("two streams, split items", grid, win, a_shift, b_shift)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    ref_a, ref_b = torch.empty_like(a[0]), torch.empty_like(b[0])
    with torch.cuda.stream(s1):
        _lib.window_attn_fwd(*a, ref_a, grid, win, a_shift, stream=s1)
    torch.cuda.synchronize()
    with torch.cuda.stream(s2):
        _lib.window_attn_fwd(*b, ref_b, grid, win, b_shift, stream=s2)
    torch.cuda.synchronize()
    out_a, out_b = torch.empty_like(ref_a), torch.empty_like(ref_b)
    for _ in range(3):
        with torch.cuda.stream(s1):
            for _ in range(4):
                _lib.window_attn_fwd(*a, out_a, grid, win, a_shift, stream=s1)
        with torch.cuda.stream(s2):
            for _ in range(4):
                _lib.window_attn_fwd(*b, out_b, grid, win, b_shift, stream=s2)
        torch.cuda.synchronize()
        assert torch.equal(out_a, ref_a), "stream 1 result differs from the serial one"
        assert torch.equal(out_b, ref_b), "stream 2 result differs from the serial one"
