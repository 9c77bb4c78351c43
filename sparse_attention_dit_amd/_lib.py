"""ctypes binding of ``libbasa.so`` (declarations and contracts: include/basa.h).

Argument marshalling only: torch tensors supply device pointers and the current HIP
stream, every computation runs in the library's kernels. There is no fallback: if the
library is missing or a call fails, a ``BasaError`` is raised.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# Always the in-tree build: no environment variable or search path can substitute another
# library for the one the tests, the smoke check and the benchmark report on.
LIB_PATH = os.path.join(_PKG, "libbasa.so")

DTYPE_F32 = 0
DTYPE_BF16 = 1

# Exported C symbols, in header order.
SYMBOLS = ("basa_window_attn_fwd", "basa_window_attn_fwd_noalloc", "basa_full_attn_fwd", "basa_pool_kv", "basa_window_attn_mem_fwd",
           "basa_window_means", "basa_route_top1", "basa_window_attn_routed_fwd", "basa_window_perm",
           "basa_shift_schedule", "basa_status_string", "basa_version")


class BasaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({status_string(status)})")


_lib = None


def load() -> ctypes.CDLL:
    """Load the in-tree library once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise BasaError(-1, f"{LIB_PATH} is missing; build it with `python -m sparse_attention_dit_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i = ctypes.c_void_p, ctypes.c_int
    lib.basa_window_attn_fwd.argtypes = [vp, vp, vp, vp] + [i] * 13 + [vp]
    lib.basa_window_attn_fwd.restype = i
    lib.basa_window_attn_fwd_noalloc.argtypes = [vp, vp, vp, vp] + [i] * 13 + [vp]
    lib.basa_window_attn_fwd_noalloc.restype = i
    lib.basa_full_attn_fwd.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp]
    lib.basa_full_attn_fwd.restype = i
    lib.basa_pool_kv.argtypes = [vp, vp, vp, vp] + [i] * 9 + [vp]
    lib.basa_pool_kv.restype = i
    lib.basa_window_attn_mem_fwd.argtypes = [vp] * 5 + [i, vp, vp] + [i] * 13 + [vp]
    lib.basa_window_attn_mem_fwd.restype = i
    lib.basa_window_means.argtypes = [vp] * 4 + [i] * 13 + [vp]
    lib.basa_window_means.restype = i
    lib.basa_route_top1.argtypes = [vp] * 3 + [i] * 10 + [vp]
    lib.basa_route_top1.restype = i
    lib.basa_window_attn_routed_fwd.argtypes = [vp] * 6 + [i, vp, vp] + [i] * 13 + [vp]
    lib.basa_window_attn_routed_fwd.restype = i
    lib.basa_window_perm.argtypes = [i] * 9 + [vp, vp]
    lib.basa_window_perm.restype = i
    lib.basa_shift_schedule.argtypes = [i] * 5 + [vp, vp]
    lib.basa_shift_schedule.restype = i
    lib.basa_status_string.argtypes = [i]
    lib.basa_status_string.restype = ctypes.c_char_p
    lib.basa_version.argtypes = []
    lib.basa_version.restype = i
    _lib = lib
    return lib


def library_info() -> dict:
    """Which library is loaded: its path relative to the repository root and the first 16
    hex digits of the SHA-256 of its bytes (printed by the smoke check, recorded by the
    benchmark)."""
    import hashlib
    load()
    with open(LIB_PATH, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()[:16]
    return {"path": os.path.relpath(LIB_PATH, os.path.dirname(_PKG)), "sha256_16": digest}


def status_string(status: int) -> str:
    if status == -1:
        return "library not built"
    return load().basa_status_string(int(status)).decode()


def _stream_handle(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise BasaError(3, f"unsupported tensor dtype {t.dtype}")


def _check_tensors(q, k, v, out):
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if not t.is_cuda:
            raise BasaError(1, f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise BasaError(2, f"{name} must be contiguous")
        if t.dim() != 4:
            raise BasaError(2, f"{name} must be [B, heads, N, head_dim]")
        if t.shape != q.shape or t.dtype != q.dtype:
            raise BasaError(2, f"{name} shape/dtype {tuple(t.shape)}/{t.dtype} differs from q")
        if t.device != q.device:
            raise BasaError(2, f"{name} is on {t.device}, q on {q.device}")


def window_attn_fwd(q, k, v, out, grid, window, shift, stream=None) -> None:
    """Shifted local-window attention into ``out`` (all [B, heads, T*H*W, head_dim])."""
    _check_tensors(q, k, v, out)
    B, H_, N, d = q.shape
    T, H, W = (int(x) for x in grid)
    wt, wh, ww = (int(x) for x in window)
    st, sh, sw = (int(x) for x in shift)
    if T * H * W != N:
        raise BasaError(2, f"grid {grid} holds {T * H * W} tokens, tensors hold {N}")
    rc = load().basa_window_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H_, T, H, W,
                                     wt, wh, ww, st, sh, sw, d, _dtype_code(q), _stream_handle(stream))
    if rc != 0:
        raise BasaError(rc, "basa_window_attn_fwd")


def window_attn_fwd_noalloc(q, k, v, out, grid, window, shift, stream=None) -> None:
    """``window_attn_fwd`` through the entry point that allocates nothing (static scratch)."""
    _check_tensors(q, k, v, out)
    B, H_, N, d = q.shape
    T, H, W = (int(x) for x in grid)
    wt, wh, ww = (int(x) for x in window)
    st, sh, sw = (int(x) for x in shift)
    if T * H * W != N:
        raise BasaError(2, f"grid {grid} holds {T * H * W} tokens, tensors hold {N}")
    rc = load().basa_window_attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H_, T, H,
                                             W, wt, wh, ww, st, sh, sw, d, _dtype_code(q), _stream_handle(stream))
    if rc != 0:
        raise BasaError(rc, "basa_window_attn_fwd_noalloc")


def full_attn_fwd(q, k, v, out, stream=None) -> None:
    """Dense attention baseline (same kernel, window = whole sequence)."""
    _check_tensors(q, k, v, out)
    B, H_, N, d = q.shape
    rc = load().basa_full_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H_, N, d,
                                   _dtype_code(q), _stream_handle(stream))
    if rc != 0:
        raise BasaError(rc, "basa_full_attn_fwd")


def pooled_count(grid, pool) -> int:
    """Memory tokens per head: T * ceil(H/ph) * ceil(W/pw)."""
    T, H, W = (int(x) for x in grid)
    ph, pw = (int(x) for x in pool)
    return T * (-(-H // ph)) * (-(-W // pw))


def pool_kv(k, v, kmem, vmem, grid, pool, stream=None) -> None:
    """Pooled memory: kmem/vmem [B, heads, T*gh*gw, d] = region means of k/v."""
    for name, t in (("k", k), ("v", v), ("kmem", kmem), ("vmem", vmem)):
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise BasaError(2, f"{name} must be a contiguous 4-D device tensor")
        if t.dtype != k.dtype:
            raise BasaError(2, f"{name} dtype {t.dtype} differs from k")
    if v.shape != k.shape:
        raise BasaError(2, "k and v shapes differ")
    B, H_, N, d = k.shape
    T, H, W = (int(x) for x in grid)
    if T * H * W != N:
        raise BasaError(2, f"grid {grid} holds {T * H * W} tokens, tensors hold {N}")
    G = pooled_count(grid, pool)
    for name, t in (("kmem", kmem), ("vmem", vmem)):
        if tuple(t.shape) != (B, H_, G, d):
            raise BasaError(2, f"{name} must be {(B, H_, G, d)}, got {tuple(t.shape)}")
    ph, pw = (int(x) for x in pool)
    rc = load().basa_pool_kv(k.data_ptr(), v.data_ptr(), kmem.data_ptr(), vmem.data_ptr(), B, H_, T, H, W, ph, pw,
                             d, _dtype_code(k), _stream_handle(stream))
    if rc != 0:
        raise BasaError(rc, "basa_pool_kv")


def window_attn_mem_fwd(q, k, v, kmem, vmem, out, grid, window, shift, lse=None, stream=None) -> None:
    """Windowed attention whose keys/values are the window's plus the memory's (kmem,
    vmem: [B, heads, M, d]; None for no memory); lse: optional fp32 [B, heads, N]."""
    window_attn_routed_fwd(q, k, v, None, kmem, vmem, out, grid, window, shift, lse, stream)


def _n_win(grid, window):
    (T, H, W), (wt, wh, ww) = ((int(x) for x in grid), (int(x) for x in window))
    if min(T, H, W, wt, wh, ww) <= 0 or T % wt or H % wh or W % ww:
        raise BasaError(2, f"window {window} does not divide grid {grid}")
    return (T // wt) * (H // wh) * (W // ww)


def window_means(q, k, qbar, kbar, grid, window, shift, stream=None) -> None:
    """Window descriptors: qbar/kbar fp32 [B, heads, n_win, d] = means of q/k per window."""
    import torch
    if q.shape != k.shape or q.dtype != k.dtype or not (q.is_cuda and k.is_cuda) or q.dim() != 4:
        raise BasaError(2, "q and k must be device tensors of one [B, heads, N, d] shape and dtype")
    if not (q.is_contiguous() and k.is_contiguous()):
        raise BasaError(2, "q and k must be contiguous")
    B, H_, N, d = q.shape
    want = (B, H_, _n_win(grid, window), d)
    for name, t in (("qbar", qbar), ("kbar", kbar)):
        if not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != want:
            raise BasaError(2, f"{name} must be a contiguous float32 device tensor {want}")
    T, H, W = (int(x) for x in grid)
    if T * H * W != N:
        raise BasaError(2, f"grid {grid} holds {T * H * W} tokens, tensors hold {N}")
    wt, wh, ww = (int(x) for x in window)
    st, sh, sw = (int(x) for x in shift)
    rc = load().basa_window_means(q.data_ptr(), k.data_ptr(), qbar.data_ptr(), kbar.data_ptr(), B, H_, T, H, W, wt,
                                  wh, ww, st, sh, sw, d, _dtype_code(q), _stream_handle(stream))
    if rc != 0:
        raise BasaError(rc, "basa_window_means")


def route_top1(qbar, kbar, route, grid, window, radius=1, stream=None) -> None:
    """route int32 [B, heads, n_win]: best-scoring window within the radius (-1: none)."""
    import torch
    if qbar.shape != kbar.shape or qbar.dtype != torch.float32 or kbar.dtype != torch.float32 or qbar.dim() != 4:
        raise BasaError(2, "qbar and kbar must be float32 [B, heads, n_win, d] of one shape")
    B, H_, n_win, d = qbar.shape
    if n_win != _n_win(grid, window):
        raise BasaError(2, "descriptor count does not match the window grid")
    if not route.is_cuda or route.dtype != torch.int32 or not route.is_contiguous() or tuple(route.shape) != (B, H_,
                                                                                                               n_win):
        raise BasaError(2, "route must be a contiguous int32 device tensor [B, heads, n_win]")
    if not (qbar.is_cuda and kbar.is_cuda and qbar.is_contiguous() and kbar.is_contiguous()):
        raise BasaError(2, "qbar and kbar must be contiguous device tensors")
    T, H, W = (int(x) for x in grid)
    wt, wh, ww = (int(x) for x in window)
    rc = load().basa_route_top1(qbar.data_ptr(), kbar.data_ptr(), route.data_ptr(), B, H_, T, H, W, wt, wh, ww,
                                int(radius), d, _stream_handle(stream))
    if rc != 0:
        raise BasaError(rc, "basa_route_top1")


def window_attn_routed_fwd(q, k, v, route, kmem, vmem, out, grid, window, shift, lse=None, stream=None) -> None:
    """Windowed attention over the window's, the routed window's (route int32 [B, heads,
    n_win] or None) and the memory's keys/values (kmem, vmem or None); lse optional."""
    import torch
    _check_tensors(q, k, v, out)
    B, H_, N, d = q.shape
    n_mem = 0
    kp = vp_ = 0
    if kmem is not None or vmem is not None:
        for name, t in (("kmem", kmem), ("vmem", vmem)):
            if t is None or not t.is_cuda or not t.is_contiguous() or t.dim() != 4 or t.dtype != q.dtype:
                raise BasaError(2, f"{name} must be a contiguous 4-D device tensor of q's dtype")
            if t.shape[0] != B or t.shape[1] != H_ or t.shape[3] != d:
                raise BasaError(2, f"{name} must be [B, heads, M, d]")
        if kmem.shape != vmem.shape:
            raise BasaError(2, "kmem and vmem shapes differ")
        n_mem, kp, vp_ = int(kmem.shape[2]), kmem.data_ptr(), vmem.data_ptr()
    lp = 0
    if lse is not None:
        if not lse.is_cuda or lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (B, H_, N):
            raise BasaError(2, "lse must be a contiguous float32 device tensor [B, heads, N]")
        lp = lse.data_ptr()
    T, H, W = (int(x) for x in grid)
    if T * H * W != N:
        raise BasaError(2, f"grid {grid} holds {T * H * W} tokens, tensors hold {N}")
    wt, wh, ww = (int(x) for x in window)
    st, sh, sw = (int(x) for x in shift)
    rp = 0
    if route is not None:
        want = (B, H_, _n_win(grid, window))
        if not route.is_cuda or route.dtype != torch.int32 or not route.is_contiguous() or tuple(route.shape) != want:
            raise BasaError(2, f"route must be a contiguous int32 device tensor {want}")
        rp = route.data_ptr()
    rc = load().basa_window_attn_routed_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), rp or None, kp or None,
                                            vp_ or None, n_mem, out.data_ptr(), lp or None, B, H_, T, H, W, wt, wh,
                                            ww, st, sh, sw, d, _dtype_code(q), _stream_handle(stream))
    if rc != 0:
        raise BasaError(rc, "basa_window_attn_routed_fwd")


def window_perm(grid, window, shift, perm, stream=None) -> None:
    """Write the window membership table (int32 device tensor of T*H*W entries)."""
    import torch
    if not perm.is_cuda or perm.dtype != torch.int32 or not perm.is_contiguous():
        raise BasaError(2, "perm must be a contiguous int32 device tensor")
    T, H, W = (int(x) for x in grid)
    if perm.numel() != T * H * W:
        raise BasaError(2, f"perm holds {perm.numel()} entries, grid has {T * H * W}")
    wt, wh, ww = (int(x) for x in window)
    st, sh, sw = (int(x) for x in shift)
    rc = load().basa_window_perm(T, H, W, wt, wh, ww, st, sh, sw, perm.data_ptr(), _stream_handle(stream))
    if rc != 0:
        raise BasaError(rc, "basa_window_perm")


def shift_schedule(L, window_hw, c=(0, 0)):
    """Per-layer (dh, dw) shifts of the interleaved schedule for a step offset c."""
    L = int(L)
    if L <= 0:
        raise BasaError(2, "L must be positive")
    dh, dw = (ctypes.c_int32 * L)(), (ctypes.c_int32 * L)()
    wh, ww = (int(x) for x in window_hw)
    rc = load().basa_shift_schedule(L, wh, ww, int(c[0]), int(c[1]), dh, dw)
    if rc != 0:
        raise BasaError(rc, "basa_shift_schedule")
    return [(int(dh[l]), int(dw[l])) for l in range(L)]


def version() -> int:
    return int(load().basa_version())
