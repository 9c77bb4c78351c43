"""GPU parity when each workgroup of the persistent bf16 kernels walks several work items.

The bf16 kernels launch at most one workgroup per CU and loop over the work items
(batch*head, window, query tile of 256 rows). The small parity cases have fewer items
than an MI355X has CUs (256), so each workgroup there runs one item; these cases have
several hundred items, so that most workgroups run two to four, in uneven numbers. Every
output element (and the log-sum-exp where written) is compared with the fp64 reference:
plain windows (both head dims, a ragged window), pooled memory, and a routed window with
memory. A second set has item counts just below, at and just above the CU count and twice
it (255, 256, 257, 513). A third set runs the per-item kernel with a last round of at most
half the grid, whose items are split in two along the key stream and merged by the half
that finishes second (the memory and 2-tile cases above are split as well). Bars as
everywhere: bf16 rel-L2 <= 5e-3 and max-abs <= 2e-2, LSE max-abs <= 3e-3.
"""
import math

import numpy as np
import pytest
import torch

from gpu_util import assert_parity, log_case, to_device, to_host
from oracle import basa_oracle as O
from oracle import memory_oracle as M
from oracle import routing_oracle as R
from sparse_attention_dit_amd import _lib, inputs

CUS = 256  # MI355X
BM = 256   # query rows per work item

# name, B, heads, head_dim, grid, window, shift, path, pool, seed
CASES = [
    ("plain-d128", 2, 20, 128, (1, 32, 32), (1, 8, 8), (0, 3, 5), "plain", None, 301),
    ("plain-d64-ragged", 1, 80, 64, (2, 20, 30), (2, 10, 15), (1, 4, -6), "plain", None, 302),
    ("memory-d128", 1, 100, 128, (1, 32, 32), (1, 8, 16), (0, 4, 8), "memory", (4, 4), 303),
    ("routed-memory-d64", 1, 100, 64, (1, 32, 32), (1, 8, 16), (0, 5, 3), "routed+memory", (4, 4), 304),
    # windows of 3, 8, 15 and 16 key tiles: the continuous-stream kernel, whose ring of row
    # offsets holds two items (3 and 16 tiles are its limits); 2 tiles: the per-item kernel
    ("plain-d128-w192-3tiles", 1, 40, 128, (1, 48, 64), (1, 12, 16), (0, 5, 7), "plain", None, 307),
    ("plain-d128-w512", 1, 80, 128, (1, 32, 64), (1, 16, 32), (0, 5, 9), "plain", None, 305),
    ("plain-d128-w960-ragged", 1, 40, 128, (1, 48, 80), (1, 24, 40), (0, 7, -11), "plain", None, 306),
    ("plain-d64-w1024-16tiles", 1, 24, 64, (1, 64, 128), (1, 32, 32), (0, 9, 21), "plain", None, 309),
    ("plain-d64-w128-2tiles", 1, 72, 64, (1, 32, 32), (1, 8, 16), (0, 3, 9), "plain", None, 308),
]


def work_items(B, heads, grid, window):
    n_win = int(np.prod([g // w for g, w in zip(grid, window)]))
    return B * heads * n_win * math.ceil(int(np.prod(window)) / BM)


# item counts just below, at and just above one and two per CU (plain windows, one query
# tile per window): name, heads, head_dim, grid, window, shift, seed
EDGE = [
    ("255-items", 51, 128, (1, 8, 40), (1, 8, 8), (0, 2, 3), 311),
    ("256-items", 64, 64, (1, 16, 16), (1, 8, 8), (0, 4, 1), 312),
    ("257-items", 257, 64, (1, 8, 8), (1, 8, 8), (0, 1, 1), 313),
    ("513-items", 19, 128, (3, 24, 24), (1, 8, 8), (1, 3, 5), 314),
]


# per-item kernel (windows of more than 16 or fewer than 3 key tiles), 256 < items <= 384:
# the last round is split. Ragged 17-tile windows (1080 keys), so the halves are 9 and 8
# tiles and the second half ends in a partial tile; and 2-tile windows with a last round of
# exactly half the grid (384 items: 256 halves of one tile each).
# name, heads, head_dim, grid, window, shift, seed
SPLIT = [
    ("split-d128-w1080", 19, 128, (1, 48, 90), (1, 24, 45), (0, 7, -11), 321),
    ("split-d64-w1080", 18, 64, (1, 48, 90), (1, 24, 45), (0, -5, 13), 322),
    ("split-d128-w128-half-grid", 48, 128, (1, 32, 32), (1, 8, 16), (0, 3, 5), 323),
]


def test_split_cases_have_a_short_last_round():
    for name, heads, d, grid, window, *_ in SPLIT:
        n = work_items(1, heads, grid, window)
        assert CUS < n <= CUS + CUS // 2, (name, n)
        tiles = math.ceil(int(np.prod(window)) / 64)
        assert tiles > 16 or 2 <= tiles < 3, name


@pytest.mark.gpu
@pytest.mark.parametrize("case", SPLIT, ids=[c[0] for c in SPLIT])
def test_split_items_every_element(case):
    name, heads, d, grid, window, shift, seed = case
    N = int(np.prod(grid))
    t = inputs.draw_qkv((1, heads, N, d), "bf16", seed)
    dev = to_device(t)
    log_case(name, "items", work_items(1, heads, grid, window), "grid", grid, "window", window, "shift", shift)
    outs = []
    for _ in range(2):
        out = torch.full_like(dev["q"], float("nan"))
        _lib.window_attn_fwd(dev["q"], dev["k"], dev["v"], out, grid, window, shift)
        torch.cuda.synchronize()
        outs.append(out)
    # the merged halves are added in a fixed order: the same result whichever half merges
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16)), name
    ref = O.window_attention(t.f64("q"), t.f64("k"), t.f64("v"), grid, window, shift)
    assert_parity(to_host(outs[0]), ref, "bf16", name)


def test_edge_item_counts():
    assert [work_items(1, c[1], c[3], c[4]) for c in EDGE] == [255, 256, 257, 513]


@pytest.mark.gpu
@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_item_counts_around_the_grid(case):
    name, heads, d, grid, window, shift, seed = case
    N = int(np.prod(grid))
    t = inputs.draw_qkv((1, heads, N, d), "bf16", seed)
    dev = to_device(t)
    out = torch.empty_like(dev["q"])
    log_case(name, "grid", grid, "window", window, "shift", shift)
    _lib.window_attn_fwd(dev["q"], dev["k"], dev["v"], out, grid, window, shift)
    torch.cuda.synchronize()
    ref = O.window_attention(t.f64("q"), t.f64("k"), t.f64("v"), grid, window, shift)
    assert_parity(to_host(out), ref, "bf16", name)


def test_cases_span_several_items_per_workgroup():
    """Every case has more than twice as many work items as CUs, and not a multiple of
    the CU count, so workgroups run different numbers of items."""
    for name, B, heads, d, grid, window, *_ in CASES:
        n = work_items(B, heads, grid, window)
        assert n > 2 * CUS, (name, n)
    assert any(work_items(*c[1:3], c[4], c[5]) % CUS for c in CASES)


def _dtype_tensor_bf16(x64):
    bits = inputs.round_to_bf16_bits(np.ascontiguousarray(x64, dtype=np.float32))
    exact = inputs.bf16_bits_to_float32(bits).astype(np.float64)
    return torch.from_numpy(bits.view(np.int16)).to("cuda").view(torch.bfloat16), exact


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_many_items_every_element(case):
    name, B, heads, d, grid, window, shift, path, pool, seed = case
    N = int(np.prod(grid))
    t = inputs.draw_qkv((B, heads, N, d), "bf16", seed)
    dev = to_device(t)
    q, k, v = t.f64("q"), t.f64("k"), t.f64("v")
    out = torch.empty_like(dev["q"])
    lse = torch.empty((B, heads, N), dtype=torch.float32, device="cuda")
    log_case(name, "items", work_items(B, heads, grid, window), "grid", grid, "window", window, "shift", shift)

    km_dev = vm_dev = km = vm = None
    if "memory" in path:
        km_dev, km = _dtype_tensor_bf16(M.pool_kv(k, grid, pool))
        vm_dev, vm = _dtype_tensor_bf16(M.pool_kv(v, grid, pool))

    ref_lse = None
    if path == "plain":
        _lib.window_attn_fwd(dev["q"], dev["k"], dev["v"], out, grid, window, shift)
        torch.cuda.synchronize()
        ref = O.window_attention(q, k, v, grid, window, shift)
    elif path == "memory":
        _lib.window_attn_mem_fwd(dev["q"], dev["k"], dev["v"], km_dev, vm_dev, out, grid, window, shift, lse=lse)
        torch.cuda.synchronize()
        ref, ref_lse = M.window_attention_memory(q, k, v, km, vm, grid, window, shift, return_lse=True)
    else:
        qbar, kbar = R.window_means(q, grid, window, shift), R.window_means(k, grid, window, shift)
        route = R.route_top1(qbar, kbar, grid, window)
        route_dev = torch.from_numpy(route.astype(np.int32)).cuda()
        _lib.window_attn_routed_fwd(dev["q"], dev["k"], dev["v"], route_dev, km_dev, vm_dev, out, grid, window,
                                    shift, lse=lse)
        torch.cuda.synchronize()
        ref, ref_lse = R.routed_attention(q, k, v, route, grid, window, shift, km, vm, return_lse=True)

    assert_parity(to_host(out), ref, "bf16", name)
    if ref_lse is not None:
        err = float(np.abs(lse.cpu().numpy().astype(np.float64) - ref_lse).max())
        assert err <= 3e-3, f"{name}: lse max-abs {err:.3e}"
