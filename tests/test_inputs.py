"""The seeded input generator: bf16 rounding is round-to-nearest-even (checked against
torch's float32 -> bfloat16 conversion) and draws are reproducible."""
import numpy as np
import torch

from sparse_attention_dit_amd import inputs


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000, dtype=np.float32) * 10.0 ** rng.integers(-6, 6, 200000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.0078125, 1.01171875, 3.0e38, -3.0e38,
                                  1e-40, -1e-40], dtype=np.float32)]).astype(np.float32)
    ours = inputs.round_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = inputs.bf16_bits_to_float32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_draws_are_seeded_and_shared():
    a = inputs.draw_qkv((1, 2, 64, 8), "bf16", seed=3)
    b = inputs.draw_qkv((1, 2, 64, 8), "bf16", seed=3)
    c = inputs.draw_qkv((1, 2, 64, 8), "bf16", seed=4)
    for n in "qkv":
        assert np.array_equal(a.dev[n], b.dev[n])
        assert np.array_equal(inputs.bf16_bits_to_float32(a.dev[n]), a.exact[n])
    assert not np.array_equal(a.dev["q"], c.dev["q"])
    f = inputs.draw_qkv((1, 1, 16, 8), "f32", seed=1)
    assert f.dev["q"].dtype == np.float32 and np.array_equal(f.dev["q"], f.exact["q"])
