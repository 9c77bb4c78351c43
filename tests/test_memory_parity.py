"""GPU parity of the pooled global memory path (BASA §3.2) and the log-sum-exp output,
through the C ABI, against the fp64 reference on the same seeded inputs.

Bars:
  * pooling: bf16 results within one bf16 ulp of the reference mean rounded to nearest
    even (the kernel accumulates in fp32, so a sum can round differently once); fp32
    within 2^-20 of the region's mean magnitude (an fp32 sum of at most ph*pw terms);
  * attention with memory: the windowed-attention bars (bf16 rel-L2 <= 5e-3 and max-abs
    <= 2e-2, fp32 <= 1e-5); the memory fed to both sides is the reference's pooled
    tensor rounded to the tensor dtype, so both see identical values;
  * log-sum-exp: max-abs <= 3e-3 for bf16 (the row sum adds P rounded to bf16, relative
    error at most 2^-9 ~ 1.95e-3, plus fp32 rounding of the logits), 1e-5 for fp32.
"""
import numpy as np
import pytest
import torch

from gpu_util import assert_parity, log_case, to_device, to_host
from oracle import basa_oracle as O
from oracle import memory_oracle as M
from sparse_attention_dit_amd import _lib, inputs

pytestmark = pytest.mark.gpu

LSE_TOL = {"bf16": 3e-3, "f32": 1e-5}


def _to_dtype_tensor(x64, dtype):
    """fp64 array -> (device tensor in dtype, the same values as fp64)."""
    x32 = np.ascontiguousarray(x64, dtype=np.float32)
    if dtype == "bf16":
        bits = inputs.round_to_bf16_bits(x32)
        exact = inputs.bf16_bits_to_float32(bits).astype(np.float64)
        dev = torch.from_numpy(bits.view(np.int16)).to("cuda").view(torch.bfloat16)
    else:
        exact = x32.astype(np.float64)
        dev = torch.from_numpy(x32).to("cuda")
    return dev, exact


def _ulp_bf16_diff(got_bits, ref_bits):
    """Distance in bf16 ulps between two bf16 bit arrays (same-sign ordered integers)."""
    def ordered(b):
        b = b.astype(np.int32)
        return np.where(b & 0x8000, 0x8000 - (b & 0x7FFF), 0x8000 + b)
    return np.abs(ordered(got_bits) - ordered(ref_bits))


POOL_CASES = [
    ("bf16", 128, (1, 16, 16), (4, 4)),
    ("bf16", 128, (2, 10, 13), (4, 4)),     # ragged far-edge regions
    ("bf16", 64, (3, 9, 7), (2, 3)),
    ("f32", 64, (2, 10, 13), (4, 3)),
    ("f32", 128, (1, 6, 6), (6, 6)),       # one region per frame
    ("bf16", 128, (1, 5, 5), (1, 1)),      # identity pooling
]


@pytest.mark.parametrize("dtype,d,grid,pool", POOL_CASES)
def test_pool_matches_reference(dtype, d, grid, pool):
    N = int(np.prod(grid))
    t = inputs.draw_qkv((2, 3, N, d), dtype, seed=300 + d + N)
    dev = to_device(t)
    G = M.pooled_count(grid, pool)
    km = torch.empty((2, 3, G, d), dtype=dev["k"].dtype, device="cuda")
    vm = torch.empty_like(km)
    log_case("pool", dtype, d, grid, pool)
    _lib.pool_kv(dev["k"], dev["v"], km, vm, grid, pool)
    torch.cuda.synchronize()
    for name, got in (("k", km), ("v", vm)):
        ref = M.pool_kv(t.f64(name), grid, pool)
        if dtype == "bf16":
            ref_bits = inputs.round_to_bf16_bits(ref.astype(np.float32))
            got_bits = got.view(torch.int16).cpu().numpy().view(np.uint16)
            dist = _ulp_bf16_diff(got_bits, ref_bits)
            assert dist.max() <= 1, f"{name}: {int(dist.max())} ulp"
            assert (dist == 0).mean() > 0.95
        else:
            # fp32 sum of up to ph*pw terms: error below 2^-20 of the region's mean magnitude
            g = got.cpu().numpy().astype(np.float64)
            scale = M.pool_kv(np.abs(t.f64(name)), grid, pool)
            assert np.all(np.abs(g - ref) <= 2.0 ** -20 * scale)


ATTN_CASES = [
    # name, dtype, d, grid, window, shift, pool
    ("2d-bf16", "bf16", 128, (1, 16, 24), (1, 8, 12), (0, 3, 5), (4, 4)),
    ("3d-bf16-ragged", "bf16", 128, (3, 10, 12), (3, 5, 6), (1, 2, 3), (4, 5)),
    ("2d-bf16-d64", "bf16", 64, (1, 20, 20), (1, 10, 10), (0, 5, 5), (3, 3)),
    ("2d-f32", "f32", 64, (1, 12, 12), (1, 6, 6), (0, 3, 3), (4, 4)),
    ("3d-f32-d128", "f32", 128, (2, 6, 8), (2, 3, 4), (1, 1, 2), (2, 3)),
]


@pytest.mark.parametrize("case", ATTN_CASES, ids=[c[0] for c in ATTN_CASES])
def test_window_memory_every_element(case):
    name, dtype, d, grid, window, shift, pool = case
    N = int(np.prod(grid))
    t = inputs.draw_qkv((1, 2, N, d), dtype, seed=400 + N)
    dev = to_device(t)
    km_dev, km = _to_dtype_tensor(M.pool_kv(t.f64("k"), grid, pool), dtype)
    vm_dev, vm = _to_dtype_tensor(M.pool_kv(t.f64("v"), grid, pool), dtype)
    out = torch.empty_like(dev["q"])
    lse = torch.empty((1, 2, N), dtype=torch.float32, device="cuda")
    log_case(name, "basa_window_attn_mem_fwd", grid, window, shift, pool)
    _lib.window_attn_mem_fwd(dev["q"], dev["k"], dev["v"], km_dev, vm_dev, out, grid, window, shift, lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = M.window_attention_memory(t.f64("q"), t.f64("k"), t.f64("v"), km, vm, grid, window, shift,
                                             return_lse=True)
    assert_parity(to_host(out), ref, dtype, name)
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= LSE_TOL[dtype]


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_lse_of_plain_windows_and_no_memory_is_the_plain_path(dtype, d):
    grid, window, shift = (2, 12, 20), (2, 6, 10), (1, 4, 7)
    N = 480
    t = inputs.draw_qkv((1, 2, N, d), dtype, seed=500 + d)
    dev = to_device(t)
    out = torch.empty_like(dev["q"])
    lse = torch.empty((1, 2, N), dtype=torch.float32, device="cuda")
    log_case("no memory + lse", dtype, d)
    _lib.window_attn_mem_fwd(dev["q"], dev["k"], dev["v"], None, None, out, grid, window, shift, lse=lse)
    plain = torch.empty_like(out)
    _lib.window_attn_fwd(dev["q"], dev["k"], dev["v"], plain, grid, window, shift)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16) if dtype == "bf16" else out,
                       plain.view(torch.int16) if dtype == "bf16" else plain)
    _, ref_lse = O.window_attention(t.f64("q"), t.f64("k"), t.f64("v"), grid, window, shift, return_lse=True)
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= LSE_TOL[dtype]


def test_pool_then_attend_end_to_end():
    """Device pooling feeding device attention against the reference chain (pool in fp64,
    round to bf16, attend)."""
    grid, window, shift, pool = (1, 32, 32), (1, 16, 16), (0, 8, 8), (4, 4)
    N = 1024
    t = inputs.draw_qkv((1, 3, N, 128), "bf16", seed=600)
    dev = to_device(t)
    G = M.pooled_count(grid, pool)
    km = torch.empty((1, 3, G, 128), dtype=torch.bfloat16, device="cuda")
    vm = torch.empty_like(km)
    out = torch.empty_like(dev["q"])
    log_case("pool -> attend", grid, window, shift, pool)
    _lib.pool_kv(dev["k"], dev["v"], km, vm, grid, pool)
    _lib.window_attn_mem_fwd(dev["q"], dev["k"], dev["v"], km, vm, out, grid, window, shift)
    torch.cuda.synchronize()
    _, km_ref = _to_dtype_tensor(M.pool_kv(t.f64("k"), grid, pool), "bf16")
    _, vm_ref = _to_dtype_tensor(M.pool_kv(t.f64("v"), grid, pool), "bf16")
    ref = M.window_attention_memory(t.f64("q"), t.f64("k"), t.f64("v"), km_ref, vm_ref, grid, window, shift)
    assert_parity(to_host(out), ref, "bf16", "pool -> attend")


WORKLOAD_CASES = [
    # FLUX 2048^2 latent grid with the pages' default pooling factor p = 4 (1024 memory tokens)
    ("flux-2048-p4", 24, (1, 128, 128), (1, 32, 32), (0, 16, 16), (4, 4), 3),
    # Wan-shaped video, p = (4, 4) per frame: 21 x 8 x 13 = 2184 memory tokens
    ("wan-21x30x52-p4", 12, (21, 30, 52), (7, 15, 26), (3, 7, 13), (4, 4), 5),
]


@pytest.mark.parametrize("case", WORKLOAD_CASES, ids=[c[0] for c in WORKLOAD_CASES])
def test_workload_memory_sampled_rows(case):
    name, heads, grid, window, shift, pool, seed = case
    N = int(np.prod(grid))
    t = inputs.draw_qkv((1, heads, N, 128), "bf16", seed=seed)
    dev = to_device(t)
    G = M.pooled_count(grid, pool)
    km = torch.empty((1, heads, G, 128), dtype=torch.bfloat16, device="cuda")
    vm = torch.empty_like(km)
    out = torch.empty_like(dev["q"])
    lse = torch.empty((1, heads, N), dtype=torch.float32, device="cuda")
    log_case(name, "pool + basa_window_attn_mem_fwd", grid, window, shift, pool)
    _lib.pool_kv(dev["k"], dev["v"], km, vm, grid, pool)
    _lib.window_attn_mem_fwd(dev["q"], dev["k"], dev["v"], km, vm, out, grid, window, shift, lse=lse)
    torch.cuda.synchronize()
    # the pooled memory itself, whole tensor
    km_ref64 = M.pool_kv(t.exact["k"], grid, pool)
    vm_ref64 = M.pool_kv(t.exact["v"], grid, pool)
    for got, ref in ((km, km_ref64), (vm, vm_ref64)):
        dist = _ulp_bf16_diff(got.view(torch.int16).cpu().numpy().view(np.uint16),
                              inputs.round_to_bf16_bits(ref.astype(np.float32)))
        assert dist.max() <= 1
    _, km_ref = _to_dtype_tensor(km_ref64, "bf16")
    _, vm_ref = _to_dtype_tensor(vm_ref64, "bf16")
    rng = np.random.default_rng(700 + seed)
    rows = np.array(sorted(set(rng.choice(N, 48, replace=False).tolist()) | {0, N - 1}))
    ref, ref_lse = M.window_attention_memory_rows(t.exact["q"], t.exact["k"], t.exact["v"], km_ref, vm_ref, grid,
                                                  window, shift, rows)
    sel = torch.from_numpy(rows).cuda()
    assert_parity(to_host(out[:, :, sel]), ref, "bf16", name)
    assert np.abs(lse[:, :, sel].cpu().numpy() - ref_lse).max() <= LSE_TOL["bf16"]
