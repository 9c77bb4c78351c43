"""The entry points inside a captured HIP graph.

A DiT's denoising loop calls the attention once per layer and step with the same shapes,
which is what graph capture is for. Inside a capture the library's calls make no
allocation, no memset and no synchronisation: a call whose last round of work items is
split (per-item kernel) uses the workspace its stream got from an earlier call outside the
capture, and the no-allocation entry point uses the library's static array. Each test
captures a sequence of calls into a graph (`torch.cuda.graph`), then replays it several
times with new inputs copied into the captured tensors, with eager work and a
synchronisation between replays, and checks that every replay equals the eager result bit
for bit (a launch is deterministic: split items are merged in a fixed order).
"""
import pytest
import torch

from gpu_util import log_case
from sparse_attention_dit_amd import _lib

pytestmark = pytest.mark.gpu

GRID, WINDOW, SHIFTS = (2, 32, 48), (1, 16, 16), [(0, 0, 0), (1, 8, 8)]
REPLAYS = 3


def _new_inputs(shape, dtype, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return [torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(dtype) for _ in range(3)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_window_attention_graph_replays(dtype):
    N = GRID[0] * GRID[1] * GRID[2]
    shape = (1, 4, N, 128)
    q, k, v = _new_inputs(shape, dtype, 1)
    outs = [torch.empty_like(q) for _ in SHIFTS]
    log_case("graph window attention", dtype, shape, GRID, WINDOW, SHIFTS)

    # warm the library (first call reads the device's CU count) outside the capture
    for s, o in zip(SHIFTS, outs):
        _lib.window_attn_fwd(q, k, v, o, GRID, WINDOW, s)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for s, o in zip(SHIFTS, outs):
            _lib.window_attn_fwd(q, k, v, o, GRID, WINDOW, s)

    for r in range(REPLAYS):
        nq, nk, nv = _new_inputs(shape, dtype, 100 + r)
        q.copy_(nq)
        k.copy_(nk)
        v.copy_(nv)
        graph.replay()
        torch.cuda.synchronize()
        for s, o in zip(SHIFTS, outs):
            ref = torch.empty_like(q)
            _lib.window_attn_fwd(nq, nk, nv, ref, GRID, WINDOW, s)  # eager, on fresh tensors
            torch.cuda.synchronize()
            assert torch.equal(o, ref), f"replay {r}, shift {s}: graph output differs from eager"


def test_memory_path_graph_replays():
    """Pooling and attention with memory (and its log-sum-exp) captured together."""
    T, H, W = GRID
    pool = (4, 4)
    N = T * H * W
    n_mem = T * (H // pool[0]) * (W // pool[1])
    shape = (1, 4, N, 128)
    q, k, v = _new_inputs(shape, torch.bfloat16, 2)
    kmem = torch.empty((1, 4, n_mem, 128), dtype=torch.bfloat16, device="cuda")
    vmem = torch.empty_like(kmem)
    out = torch.empty_like(q)
    lse = torch.empty((1, 4, N), dtype=torch.float32, device="cuda")
    log_case("graph memory path", shape, GRID, WINDOW, pool)

    def chain(q_, k_, v_, km_, vm_, o_, l_):
        _lib.pool_kv(k_, v_, km_, vm_, GRID, pool)
        _lib.window_attn_mem_fwd(q_, k_, v_, km_, vm_, o_, GRID, WINDOW, SHIFTS[1], lse=l_)

    chain(q, k, v, kmem, vmem, out, lse)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        chain(q, k, v, kmem, vmem, out, lse)

    for r in range(REPLAYS):
        nq, nk, nv = _new_inputs(shape, torch.bfloat16, 200 + r)
        q.copy_(nq)
        k.copy_(nk)
        v.copy_(nv)
        graph.replay()
        torch.cuda.synchronize()
        rkm, rvm = torch.empty_like(kmem), torch.empty_like(vmem)
        rout, rlse = torch.empty_like(out), torch.empty_like(lse)
        chain(nq, nk, nv, rkm, rvm, rout, rlse)
        torch.cuda.synchronize()
        assert torch.equal(kmem, rkm) and torch.equal(vmem, rvm), f"replay {r}: pooled memory differs"
        assert torch.equal(out, rout), f"replay {r}: output differs from eager"
        assert torch.equal(lse, rlse), f"replay {r}: log-sum-exp differs from eager"


# 17-tile windows (per-item kernel), 19 heads: 380 work items, the last 124 split in two
SPLIT_GRID, SPLIT_WINDOW, SPLIT_SHIFT = (1, 48, 90), (1, 24, 45), (0, 7, -11)


def _replay_and_compare(graph, captured, outs, call, shape, seed0):
    q, k, v = captured
    for r in range(REPLAYS):
        nq, nk, nv = _new_inputs(shape, torch.bfloat16, seed0 + r)
        q.copy_(nq)
        k.copy_(nk)
        v.copy_(nv)
        graph.replay()
        torch.cuda.synchronize()
        ref = torch.empty_like(q)
        call(nq, nk, nv, ref)  # eager, on fresh tensors
        torch.cuda.synchronize()
        assert torch.equal(outs, ref), f"replay {r}: graph output differs from eager"


def test_split_items_graph_replays():
    """Captured on a stream that made its split workspace in an eager call before."""
    N = SPLIT_GRID[0] * SPLIT_GRID[1] * SPLIT_GRID[2]
    shape = (1, 19, N, 128)
    q, k, v = _new_inputs(shape, torch.bfloat16, 3)
    out = torch.empty_like(q)
    s = torch.cuda.Stream()
    log_case("graph split items", shape, SPLIT_GRID, SPLIT_WINDOW, SPLIT_SHIFT)

    def call(q_, k_, v_, o_):
        with torch.cuda.stream(s):
            _lib.window_attn_fwd(q_, k_, v_, o_, SPLIT_GRID, SPLIT_WINDOW, SPLIT_SHIFT, stream=s)

    call(q, k, v, out)  # outside the capture: the stream's workspace is made here
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        _lib.window_attn_fwd(q, k, v, out, SPLIT_GRID, SPLIT_WINDOW, SPLIT_SHIFT, stream=s)
    _replay_and_compare(graph, (q, k, v), out, call, shape, 300)


def test_noalloc_graph_replays():
    """The no-allocation entry point, captured on a stream it has never run on."""
    N = SPLIT_GRID[0] * SPLIT_GRID[1] * SPLIT_GRID[2]
    shape = (1, 19, N, 128)
    q, k, v = _new_inputs(shape, torch.bfloat16, 4)
    out = torch.empty_like(q)
    log_case("graph no-alloc", shape, SPLIT_GRID, SPLIT_WINDOW, SPLIT_SHIFT)

    def call(q_, k_, v_, o_):
        _lib.window_attn_fwd_noalloc(q_, k_, v_, o_, SPLIT_GRID, SPLIT_WINDOW, SPLIT_SHIFT)

    call(q, k, v, out)  # reads the CU count and the array's address, allocates nothing
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        _lib.window_attn_fwd_noalloc(q, k, v, out, SPLIT_GRID, SPLIT_WINDOW, SPLIT_SHIFT, stream=s)
    _replay_and_compare(graph, (q, k, v), out, call, shape, 400)


def test_split_call_captured_on_a_new_stream_runs_unsplit():
    """Captured on a stream with no workspace yet: the call cannot allocate inside the
    capture, so it runs without the split. Its replays agree with each other bit for bit and
    with the eager (split) result to the bf16 bar (a different summation order)."""
    from gpu_util import assert_parity, to_host
    N = SPLIT_GRID[0] * SPLIT_GRID[1] * SPLIT_GRID[2]
    shape = (1, 19, N, 128)
    q, k, v = _new_inputs(shape, torch.bfloat16, 5)
    out = torch.empty_like(q)
    log_case("graph, stream without workspace", shape, SPLIT_GRID, SPLIT_WINDOW, SPLIT_SHIFT)
    ref = torch.empty_like(q)
    _lib.window_attn_fwd(q, k, v, ref, SPLIT_GRID, SPLIT_WINDOW, SPLIT_SHIFT)  # eager, default stream
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        _lib.window_attn_fwd(q, k, v, out, SPLIT_GRID, SPLIT_WINDOW, SPLIT_SHIFT, stream=s)
    first = None
    for r in range(REPLAYS):
        graph.replay()
        torch.cuda.synchronize()
        if first is None:
            first = out.clone()
        assert torch.equal(out, first), f"replay {r} differs from the first"
    assert_parity(to_host(first), to_host(ref), "bf16", "graph without workspace vs eager")
