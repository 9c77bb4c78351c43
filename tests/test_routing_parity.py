"""GPU parity of true-window routing (BASA §3.3) through the C ABI against the fp64
reference on the same seeded inputs.

Bars:
  * window descriptors (fp32): within n * 2^-24 * mean|x| of the fp64 mean, where
    n = W/8 + 32 bounds the number of fp32 additions on any path of the kernel's sum
    (first-order floating-point summation bound);
  * routing decisions are an argmax decided in floating point. Fed the same fp32
    descriptors, the device must pick the reference's window wherever the reference's best
    score beats the runner-up by more than 1e-5 (well above fp32 dot-product rounding at
    these magnitudes); within that margin any candidate scoring within 1e-5 of the best
    is valid;
  * routed attention: the windowed-attention bars, with the reference's own route fed to
    both sides; log-sum-exp as for the pooled-memory path.
"""
import numpy as np
import pytest
import torch

from gpu_util import assert_parity, log_case, to_device, to_host
from oracle import basa_oracle as O
from oracle import memory_oracle as M
from oracle import routing_oracle as R
from sparse_attention_dit_amd import _lib, inputs

pytestmark = pytest.mark.gpu

LSE_TOL = {"bf16": 3e-3, "f32": 1e-5}
MARGIN = 1e-5


def _nwin(grid, window):
    return int(np.prod([g // w for g, w in zip(grid, window)]))


MEAN_CASES = [
    ("bf16", 128, (1, 32, 32), (1, 8, 8), (0, 4, 4)),
    ("bf16", 64, (3, 10, 12), (3, 5, 6), (1, 2, 3)),
    ("f32", 128, (2, 8, 12), (1, 4, 6), (1, 1, 2)),
    ("bf16", 128, (21, 30, 52), (7, 15, 26), (3, 7, 13)),
]


@pytest.mark.parametrize("dtype,d,grid,window,shift", MEAN_CASES)
def test_window_means_match_reference(dtype, d, grid, window, shift):
    N = int(np.prod(grid))
    heads = 2
    t = inputs.draw_qkv((1, heads, N, d), dtype, seed=800 + N)
    dev = to_device(t)
    n = _nwin(grid, window)
    qbar = torch.empty((1, heads, n, d), dtype=torch.float32, device="cuda")
    kbar = torch.empty_like(qbar)
    log_case("window means", dtype, d, grid, window, shift)
    _lib.window_means(dev["q"], dev["k"], qbar, kbar, grid, window, shift)
    torch.cuda.synchronize()
    W = int(np.prod(window))
    for name, got in (("q", qbar), ("k", kbar)):
        ref = R.window_means(t.f64(name), grid, window, shift)
        scale = R.window_means(np.abs(t.f64(name)), grid, window, shift)
        bound = (W / 8 + 32) * 2.0 ** -24 * scale
        assert np.all(np.abs(got.cpu().numpy() - ref) <= bound), name


ROUTE_CASES = [((1, 48, 48), (1, 8, 8)), ((21, 60, 104), (21, 15, 26)), ((4, 30, 52), (2, 15, 13)),
               ((1, 16, 16), (1, 16, 16))]


@pytest.mark.parametrize("grid,window", ROUTE_CASES)
@pytest.mark.parametrize("radius", [1, 2])
def test_route_decisions(grid, window, radius):
    """The decision kernel on reference descriptors (rounded to fp32), including planted
    exact ties."""
    rng = np.random.default_rng(900 + radius)
    n = _nwin(grid, window)
    d = 128
    qbar = rng.standard_normal((2, 3, n, d)).astype(np.float32)
    kbar = rng.standard_normal((2, 3, n, d)).astype(np.float32)
    if n >= 9:
        kbar[0, 0, 1] = kbar[0, 0, 2]          # exact ties for every window next to both
        kbar[1, 2, :] = kbar[1, 2, 0]          # a head where every candidate ties
    route = torch.empty((2, 3, n), dtype=torch.int32, device="cuda")
    log_case("route top1", grid, window, radius)
    _lib.route_top1(torch.from_numpy(qbar).cuda(), torch.from_numpy(kbar).cuda(), route, grid, window, radius)
    torch.cuda.synchronize()
    got = route.cpu().numpy()
    ref = R.route_top1(qbar.astype(np.float64), kbar.astype(np.float64), grid, window, radius)
    s = R.scores(qbar.astype(np.float64), kbar.astype(np.float64))
    C = R.candidates(grid, window, radius)
    for b in range(2):
        for h in range(3):
            for i in range(n):
                if not C[i]:
                    assert got[b, h, i] == -1
                    continue
                cand = s[b, h, i, C[i]]
                order = np.sort(cand)[::-1]
                exact_tie = cand.size > 1 and order[0] == order[1]
                clear = cand.size == 1 or order[0] - order[1] > MARGIN
                if clear or exact_tie:
                    assert got[b, h, i] == ref[b, h, i], (b, h, i)
                else:
                    assert got[b, h, i] in C[i] and s[b, h, i, got[b, h, i]] >= order[0] - MARGIN


ATTN_CASES = [
    # name, dtype, d, grid, window, shift, pool (None: no memory)
    ("2d-bf16-route", "bf16", 128, (1, 24, 24), (1, 8, 8), (0, 3, 5), None),
    ("2d-bf16-route-mem", "bf16", 128, (1, 24, 24), (1, 8, 8), (0, 3, 5), (4, 4)),
    ("video-bf16-route-mem", "bf16", 128, (4, 12, 15), (4, 6, 5), (0, 2, 3), (4, 4)),
    ("3d-bf16-d64-ragged", "bf16", 64, (3, 9, 12), (3, 3, 4), (1, 1, 2), (3, 4)),
    ("2d-f32-route-mem", "f32", 64, (1, 12, 18), (1, 6, 6), (0, 2, 4), (4, 4)),
]


def _ref_route(t, grid, window, shift):
    return R.route_top1(R.window_means(t.f64("q"), grid, window, shift),
                        R.window_means(t.f64("k"), grid, window, shift), grid, window)


def _to_dtype_tensor(x64, dtype):
    x32 = np.ascontiguousarray(x64, dtype=np.float32)
    if dtype == "bf16":
        bits = inputs.round_to_bf16_bits(x32)
        return (torch.from_numpy(bits.view(np.int16)).to("cuda").view(torch.bfloat16),
                inputs.bf16_bits_to_float32(bits).astype(np.float64))
    return torch.from_numpy(x32).to("cuda"), x32.astype(np.float64)


@pytest.mark.parametrize("case", ATTN_CASES, ids=[c[0] for c in ATTN_CASES])
def test_routed_attention_every_element(case):
    name, dtype, d, grid, window, shift, pool = case
    N = int(np.prod(grid))
    t = inputs.draw_qkv((1, 2, N, d), dtype, seed=1000 + N)
    dev = to_device(t)
    route = _ref_route(t, grid, window, shift)
    km_dev = vm_dev = km = vm = None
    if pool is not None:
        km_dev, km = _to_dtype_tensor(M.pool_kv(t.f64("k"), grid, pool), dtype)
        vm_dev, vm = _to_dtype_tensor(M.pool_kv(t.f64("v"), grid, pool), dtype)
    out = torch.empty_like(dev["q"])
    lse = torch.empty((1, 2, N), dtype=torch.float32, device="cuda")
    log_case(name, "basa_window_attn_routed_fwd", grid, window, shift, pool)
    _lib.window_attn_routed_fwd(dev["q"], dev["k"], dev["v"], torch.from_numpy(route.astype(np.int32)).cuda(),
                                km_dev, vm_dev, out, grid, window, shift, lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = R.routed_attention(t.f64("q"), t.f64("k"), t.f64("v"), route, grid, window, shift, km, vm,
                                      return_lse=True)
    assert_parity(to_host(out), ref, dtype, name)
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= LSE_TOL[dtype]


def test_route_minus_one_or_out_of_range_adds_nothing():
    grid, window, shift = (1, 16, 16), (1, 8, 8), (0, 4, 4)
    t = inputs.draw_qkv((1, 2, 256, 128), "bf16", seed=1100)
    dev = to_device(t)
    plain = torch.empty_like(dev["q"])
    _lib.window_attn_fwd(dev["q"], dev["k"], dev["v"], plain, grid, window, shift)
    for fill in (-1, 4, 1 << 30, -7):
        route = torch.full((1, 2, 4), fill, dtype=torch.int32, device="cuda")
        out = torch.empty_like(plain)
        log_case("route fill", fill)
        _lib.window_attn_routed_fwd(dev["q"], dev["k"], dev["v"], route, None, None, out, grid, window, shift)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), plain.view(torch.int16))


def test_wan_table3_shape_full_basa_sampled_rows():
    """The pages' full video configuration: 21x60x104 latent grid, windows 21x15x26, one
    routed window within radius one, pooled memory p = (4, 4); the whole chain on the
    device (descriptors, routing, pooling, attention). The device route is checked
    against the reference route by the margin rule, and the output on sampled rows of
    windows with clear decisions against the reference chain."""
    grid, window, shift, pool = (21, 60, 104), (21, 15, 26), (0, 7, 13), (4, 4)
    heads, N, d = 12, 131040, 128
    t = inputs.draw_qkv((1, heads, N, d), "bf16", seed=6)
    dev = to_device(t)
    n = _nwin(grid, window)
    qbar = torch.empty((1, heads, n, d), dtype=torch.float32, device="cuda")
    kbar = torch.empty_like(qbar)
    route = torch.empty((1, heads, n), dtype=torch.int32, device="cuda")
    G = M.pooled_count(grid, pool)
    km = torch.empty((1, heads, G, d), dtype=torch.bfloat16, device="cuda")
    vm = torch.empty_like(km)
    out = torch.empty_like(dev["q"])
    lse = torch.empty((1, heads, N), dtype=torch.float32, device="cuda")
    log_case("wan 21x60x104 full BASA chain")
    _lib.window_means(dev["q"], dev["k"], qbar, kbar, grid, window, shift)
    _lib.route_top1(qbar, kbar, route, grid, window, 1)
    _lib.pool_kv(dev["k"], dev["v"], km, vm, grid, pool)
    _lib.window_attn_routed_fwd(dev["q"], dev["k"], dev["v"], route, km, vm, out, grid, window, shift, lse=lse)
    torch.cuda.synchronize()
    qb = R.window_means(t.exact["q"], grid, window, shift)
    kb = R.window_means(t.exact["k"], grid, window, shift)
    ref_route = R.route_top1(qb, kb, grid, window)
    s = R.scores(qb, kb)
    C = R.candidates(grid, window)
    got_route = route.cpu().numpy()
    # decisions: equal to the reference where its margin is clear, a near-best candidate
    # otherwise (the descriptors' fp32 error moves scores by far less than 1e-6 here)
    clear = np.zeros((heads, n), dtype=bool)
    for h in range(heads):
        for i in range(n):
            cand = np.sort(s[0, h, i, C[i]])[::-1]
            clear[h, i] = cand[0] - cand[1] > 1e-6
            if clear[h, i]:
                assert got_route[0, h, i] == ref_route[0, h, i]
            else:
                assert got_route[0, h, i] in C[i] and s[0, h, i, got_route[0, h, i]] >= cand[0] - 1e-6
    # attention: rows of windows whose decision is clear in every head, so the reference
    # chain (its own route, its own pooled memory) determines every expected value
    table = O.window_members(grid, window, shift)
    ok_windows = [i for i in range(n) if clear[:, i].all()]
    assert len(ok_windows) >= n // 2
    rng = np.random.default_rng(1200)
    rows = np.array(sorted({int(rng.choice(table[i])) for i in ok_windows for _ in range(3)}))
    _, km_ref = _to_dtype_tensor(M.pool_kv(t.exact["k"], grid, pool), "bf16")
    _, vm_ref = _to_dtype_tensor(M.pool_kv(t.exact["v"], grid, pool), "bf16")
    ref, ref_lse = R.routed_attention_rows(t.exact["q"], t.exact["k"], t.exact["v"], ref_route, grid, window, shift,
                                           rows, km_ref, vm_ref)
    sel = torch.from_numpy(rows).cuda()
    assert_parity(to_host(out[:, :, sel]), ref, "bf16", "wan full BASA")
    assert np.abs(lse[:, :, sel].cpu().numpy() - ref_lse).max() <= LSE_TOL["bf16"]
