"""Helpers shared by the GPU tests: device upload/download, tolerances, case logging."""
import sys

import numpy as np

# Floating-point parity bars: bf16 rel-L2 <= 5e-3 and max-abs <= 2e-2; fp32 <= 1e-5 for both.
TOL = {"bf16": (5e-3, 2e-2), "f32": (1e-5, 1e-5)}


def log_case(*parts):
    """Name the case on stdout before a GPU step, flushed, so a crash still names it."""
    print("[case]", *parts, flush=True)
    sys.stdout.flush()


def to_device(tensors):
    import torch
    out = {}
    for n, a in tensors.dev.items():
        if tensors.dtype == "bf16":
            out[n] = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda").view(torch.bfloat16)
        else:
            out[n] = torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    return out


def to_host(x):
    """Device tensor -> float64 numpy (bf16 values upcast exactly)."""
    return x.float().cpu().numpy().astype(np.float64)


def errors(got, ref):
    diff = np.asarray(got, dtype=np.float64) - np.asarray(ref, dtype=np.float64)
    rel = float(np.linalg.norm(diff) / np.linalg.norm(ref))
    mx = float(np.abs(diff).max())
    return rel, mx


def assert_parity(got, ref, dtype, what):
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    rel, mx = errors(got, ref)
    rtol, atol = TOL[dtype]
    print(f"[parity] {what}: rel_l2={rel:.3e} max_abs={mx:.3e}", flush=True)
    assert rel <= rtol and mx <= atol, f"{what}: rel_l2 {rel:.3e} (<= {rtol}), max_abs {mx:.3e} (<= {atol})"
