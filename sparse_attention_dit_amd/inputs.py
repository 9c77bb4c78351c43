"""Seeded synthetic inputs shared by the GPU path's tests/bench and the CPU oracle.

This module holds none of the attention arithmetic: it only draws q, k, v and rounds
them to the storage type the device sees. Both sides consume exactly the same values:
the device gets the raw bits, the oracle gets the same values upcast to float64.

Recipe (the pages measure on FLUX.1-dev and Wan2.1 activations that are not available
here; these Gaussian tensors of the same shapes stand in for them):
  * ``numpy.random.default_rng(seed)``, one generator per workload;
  * q, k, v drawn in that order with ``standard_normal(shape, dtype=float32)``;
  * bf16 workloads round each float32 to bfloat16 with round-to-nearest-even.
"""
from __future__ import annotations

import numpy as np


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bfloat16 bit patterns, round-to-nearest-even.

    NaN is not expected (inputs are finite Gaussians); inf/overflow follow the usual
    RNE carry into the exponent.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = u + np.uint32(0x7FFF) + lsb
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_float32(bits: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


class Tensors:
    """One drawn tensor set: ``dev`` holds what goes to the device (float32 array, or
    uint16 bf16 bits); ``exact`` holds the identical values as float32 arrays (bf16
    values are exactly representable); ``f64(name)`` upcasts one of them to float64."""

    def __init__(self, dtype: str, dev: dict, exact: dict):
        self.dtype = dtype
        self.dev = dev
        self.exact = exact

    def f64(self, name: str) -> np.ndarray:
        return self.exact[name].astype(np.float64)


def draw_qkv(shape, dtype: str, seed: int, q_scale: float = 1.0) -> Tensors:
    """Draw q, k, v of ``shape`` = (B, heads, N, head_dim) from ``seed``.

    ``dtype`` is "f32" or "bf16". ``q_scale`` multiplies q before rounding (used for the
    peaky-logit robustness case); it is 1.0 for the standard workloads.
    """
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"dtype must be 'f32' or 'bf16', got {dtype!r}")
    rng = np.random.default_rng(seed)
    raw = {}
    for name in ("q", "k", "v"):
        raw[name] = rng.standard_normal(tuple(shape), dtype=np.float32)
    if q_scale != 1.0:
        raw["q"] = (raw["q"] * np.float32(q_scale)).astype(np.float32)
    dev, exact = {}, {}
    for name, a in raw.items():
        if dtype == "bf16":
            bits = round_to_bf16_bits(a)
            dev[name] = bits
            exact[name] = bf16_bits_to_float32(bits)
        else:
            dev[name] = a
            exact[name] = a
    return Tensors(dtype, dev, exact)


def from_float_arrays(arrays: dict, dtype: str) -> Tensors:
    """Wrap caller-built float arrays (structured probes: one-hot V, zero Q, ...) so that
    both sides again see identical values. Values are rounded to bf16 when dtype is bf16."""
    dev, exact = {}, {}
    for name, a in arrays.items():
        a32 = np.ascontiguousarray(a, dtype=np.float32)
        if dtype == "bf16":
            bits = round_to_bf16_bits(a32)
            dev[name] = bits
            exact[name] = bf16_bits_to_float32(bits)
        else:
            dev[name] = a32
            exact[name] = a32
    return Tensors(dtype, dev, exact)


def draw_qkv_device(shape, dtype: str, seed: int, device="cuda"):
    """Seeded q, k, v drawn directly in device memory (torch's generator, N(0,1)),
    for sizes whose host copies would not fit; callers copy back only the rows the
    oracle needs. Returns a dict of device tensors of ``dtype`` ("bf16" or "f32")."""
    import torch
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = {}
    for name in ("q", "k", "v"):
        out[name] = torch.randn(tuple(shape), generator=gen, device=device, dtype=torch.float32).to(tdt)
    return out
