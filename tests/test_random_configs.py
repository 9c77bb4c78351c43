"""GPU parity on 40 seeded random configurations, through the C ABI, against the fp64 reference.

Each case draws the grid, window, shift, dtype, head_dim, batch and heads together, and
one of three paths:
  * plain shifted-window attention (BASA §3.1);
  * window + pooled memory (§3.2), with the log-sum-exp;
  * window + routed window (§3.3), with or without the memory, with the log-sum-exp.

Every output element is compared. The draws come from a fixed seed, so the cases are the same
on every run. They cover combinations the hand-picked cases do not: ragged windows with
memory and a routed window, head_dim 64 with 3-D windows, batch > 1, negative and
out-of-range shifts.

The memory and the route fed to the library are the reference's own: the pooled tokens
(fp64, rounded to the tensor dtype) and the top-1 choice. Both sides therefore attend to
the same keys, and the bar is the attention bar (bf16 rel-L2 <= 5e-3 and max-abs <= 2e-2,
fp32 <= 1e-5). The log-sum-exp bar is 3e-3 for bf16 (the row sum adds P rounded to bf16)
and 1e-5 for fp32.
"""
import numpy as np
import pytest
import torch

from gpu_util import assert_parity, log_case, to_device, to_host
from oracle import basa_oracle as O
from oracle import memory_oracle as M
from oracle import routing_oracle as R
from sparse_attention_dit_amd import _lib, inputs

LSE_TOL = {"bf16": 3e-3, "f32": 1e-5}
N_CASES = 40


def _draw_case(i):
    rng = np.random.default_rng(9000 + i)
    three_d = rng.random() < 0.5
    window = (int(rng.integers(1, 4)) if three_d else 1, int(rng.integers(2, 21)), int(rng.integers(2, 21)))
    counts = (int(rng.integers(1, 3)) if three_d else 1, int(rng.integers(1, 4)), int(rng.integers(1, 4)))
    grid = tuple(w * c for w, c in zip(window, counts))
    # keep the reference quick: at most ~2,400 tokens
    while np.prod(grid) > 2400:
        counts = tuple(max(1, c - 1) for c in counts)
        grid = tuple(w * c for w, c in zip(window, counts))
    shift = tuple(int(rng.integers(-n, 2 * n + 1)) for n in grid)
    dtype = "bf16" if rng.random() < 0.7 else "f32"
    d = int(rng.choice([64, 128]))
    B, heads = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    path = str(rng.choice(["plain", "memory", "routed", "routed+memory"], p=[0.3, 0.25, 0.2, 0.25]))
    pool = (int(rng.integers(1, 5)), int(rng.integers(1, 5)))
    return dict(grid=grid, window=window, shift=shift, dtype=dtype, d=d, B=B, heads=heads, path=path, pool=pool,
                seed=9100 + i)


def _dtype_tensor(x64, dtype):
    """fp64 array -> (device tensor in dtype, the same values as fp64)."""
    x32 = np.ascontiguousarray(x64, dtype=np.float32)
    if dtype == "bf16":
        bits = inputs.round_to_bf16_bits(x32)
        exact = inputs.bf16_bits_to_float32(bits).astype(np.float64)
        return torch.from_numpy(bits.view(np.int16)).to("cuda").view(torch.bfloat16), exact
    return torch.from_numpy(x32).to("cuda"), x32.astype(np.float64)


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CASES))
def test_random_configuration(i):
    c = _draw_case(i)
    grid, window, shift, dtype = c["grid"], c["window"], c["shift"], c["dtype"]
    N = int(np.prod(grid))
    t = inputs.draw_qkv((c["B"], c["heads"], N, c["d"]), dtype, seed=c["seed"])
    dev = to_device(t)
    q, k, v = t.f64("q"), t.f64("k"), t.f64("v")
    out = torch.empty_like(dev["q"])
    lse = torch.empty((c["B"], c["heads"], N), dtype=torch.float32, device="cuda")
    name = f"case{i}-{c['path']}-{dtype}-d{c['d']}-B{c['B']}h{c['heads']}"
    log_case(name, grid, window, shift, c["pool"] if "memory" in c["path"] else "")

    km_dev = vm_dev = km = vm = None
    if "memory" in c["path"]:
        km_dev, km = _dtype_tensor(M.pool_kv(k, grid, c["pool"]), dtype)
        vm_dev, vm = _dtype_tensor(M.pool_kv(v, grid, c["pool"]), dtype)

    if c["path"] == "plain":
        _lib.window_attn_fwd(dev["q"], dev["k"], dev["v"], out, grid, window, shift)
        torch.cuda.synchronize()
        ref = O.window_attention(q, k, v, grid, window, shift)
        ref_lse = None
    elif c["path"] == "memory":
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

    assert_parity(to_host(out), ref, dtype, name)
    if ref_lse is not None:
        err = float(np.abs(lse.cpu().numpy().astype(np.float64) - ref_lse).max())
        assert err <= LSE_TOL[dtype], f"{name}: lse max-abs {err:.3e}"


def test_draws_cover_the_combinations():
    """The seeded draws include every path, both dtypes and head dims, ragged windows, 3-D
    windows and batch > 1 (so a change to the generator cannot silently drop coverage)."""
    cases = [_draw_case(i) for i in range(N_CASES)]
    assert {c["path"] for c in cases} == {"plain", "memory", "routed", "routed+memory"}
    assert {c["dtype"] for c in cases} == {"bf16", "f32"} and {c["d"] for c in cases} == {64, 128}
    assert any(int(np.prod(c["window"])) % 64 for c in cases if c["dtype"] == "bf16")
    assert any(int(np.prod(c["window"])) > 128 for c in cases if c["dtype"] == "bf16")  # several K/V tiles
    assert any(c["window"][0] > 1 for c in cases) and any(c["B"] > 1 for c in cases)
    assert any(any(s < 0 or s >= n for s, n in zip(c["shift"], c["grid"])) for c in cases)
