"""GPU robustness: no writes outside `out`, bitwise determinism, argument errors on real
device tensors, and the extremes of the supported index range."""
import numpy as np
import pytest
import torch

from gpu_util import assert_parity, log_case, to_device, to_host
from oracle import basa_oracle as O
from sparse_attention_dit_amd import _lib, inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_guard_bands_untouched_and_deterministic(dtype, d):
    grid, window, s = (7, 30, 26), (7, 15, 26), (3, 7, 13)
    if dtype == "f32":
        grid, window, s = (3, 10, 14), (3, 5, 7), (1, 2, 3)
    N = int(np.prod(grid))
    t = inputs.draw_qkv((1, 2, N, d), dtype, seed=200)
    dev = to_device(t)
    guard = 4096
    numel = dev["q"].numel()
    buf = torch.empty(numel + 2 * guard, dtype=dev["q"].dtype, device="cuda")
    buf.fill_(12345.0)
    out = buf[guard:guard + numel].view(dev["q"].shape)
    log_case("guard bands", dtype, d, grid, window, s)
    _lib.window_attn_fwd(dev["q"], dev["k"], dev["v"], out, grid, window, s)
    torch.cuda.synchronize()
    assert torch.all(buf[:guard] == 12345.0) and torch.all(buf[guard + numel:] == 12345.0)
    again = torch.empty_like(out)
    _lib.window_attn_fwd(dev["q"], dev["k"], dev["v"], again, grid, window, s)
    torch.cuda.synchronize()
    assert torch.equal(out, again)
    ref = O.window_attention(t.f64("q"), t.f64("k"), t.f64("v"), grid, window, s)
    assert_parity(to_host(out), ref, dtype, "guarded output")


def test_argument_errors_on_device_tensors():
    t = inputs.draw_qkv((1, 2, 256, 64), "bf16", seed=201)
    dev = to_device(t)
    out = torch.zeros_like(dev["q"])
    with pytest.raises(_lib.BasaError) as e:
        _lib.window_attn_fwd(dev["q"], dev["k"], dev["v"], dev["q"], (1, 16, 16), (1, 8, 8), (0, 0, 0))
    assert e.value.status == 4
    with pytest.raises(_lib.BasaError) as e:
        _lib.window_attn_fwd(dev["q"], dev["k"], dev["v"], out, (1, 16, 16), (1, 6, 8), (0, 0, 0))
    assert e.value.status == 2
    misaligned = torch.empty(dev["q"].numel() + 8, dtype=torch.bfloat16, device="cuda")[1:1 + dev["q"].numel()]
    with pytest.raises(_lib.BasaError) as e:
        _lib.window_attn_fwd(dev["q"], dev["k"], dev["v"], misaligned.view(dev["q"].shape), (1, 16, 16),
                             (1, 8, 8), (0, 0, 0))
    assert e.value.status == 7
    torch.cuda.synchronize()
    assert torch.all(out == 0)


def test_offsets_beyond_2_pow_31_elements():
    """264 heads x 65536 tokens x 128 > 2^31 elements (and 2^32 bytes) per tensor: the
    last heads sit past the 32-bit element range, so the per-head base must be 64-bit."""
    shape = (1, 264, 65536, 128)
    grid, window, s = (1, 256, 256), (1, 32, 32), (0, 16, 16)
    log_case("64-bit offsets", shape)
    dev = inputs.draw_qkv_device(shape, "bf16", seed=202)
    out = torch.empty_like(dev["q"])
    _lib.window_attn_fwd(dev["q"], dev["k"], dev["v"], out, grid, window, s)
    torch.cuda.synchronize()
    rows = np.array([0, 12345, 65535])
    heads = [0, 255, 263]
    for h in heads:
        sub = {n: dev[n][:, h:h + 1].float().cpu().numpy() for n in "qkv"}
        ref = O.window_attention_rows(sub["q"], sub["k"], sub["v"], grid, window, s, rows)
        got = out[:, h:h + 1, torch.from_numpy(rows).cuda()].float().cpu().numpy()
        assert_parity(got, ref, "bf16", f"head {h}")


def test_largest_supported_head():
    """N * head_dim = 2^31 - 2^16 (just inside the 32-bit per-head range)."""
    grid, window, s = (1, 4096, 4095), (1, 16, 15), (0, 8, 7)
    N = 4096 * 4095
    shape = (1, 1, N, 128)
    log_case("largest head", shape)
    dev = inputs.draw_qkv_device(shape, "bf16", seed=203)
    out = torch.empty_like(dev["q"])
    _lib.window_attn_fwd(dev["q"], dev["k"], dev["v"], out, grid, window, s)
    torch.cuda.synchronize()
    rows = np.array([0, N // 2 + 17, N - 1])
    for r in rows:
        members = O.members_of(grid, window, s, r)
        idx = torch.from_numpy(members).cuda()
        sub = {n: dev[n][:, :, idx].float().cpu().numpy() for n in "qkv"}
        pos = int(np.nonzero(members == r)[0][0])
        local_grid = (1, 1, members.size)
        ref = O.window_attention_rows(sub["q"], sub["k"], sub["v"], local_grid, local_grid, (0, 0, 0), [pos])
        got = out[:, :, r:r + 1].float().cpu().numpy()
        assert_parity(got, ref, "bf16", f"row {r}")
