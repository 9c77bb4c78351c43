"""Host-side checks of the C ABI and of the library's index map (no GPU needed).

* the built library loads and exports every function include/basa.h declares;
* every argument error returns its status code before any HIP call is made;
* the index map header, compiled for the host, reproduces the oracle's membership table
  bit for bit, and its division by invariant integers matches '/'.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from oracle import basa_oracle as O
from sparse_attention_dit_amd import _lib
from sparse_attention_dit_amd.configs import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "basa.h")
CSRC = os.path.join(ROOT, "sparse_attention_dit_amd", "csrc")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(basa_\w+)\s*\(", text, flags=re.M)


def test_header_and_binding_agree():
    declared = _declared_functions()
    assert set(declared) == set(_lib.SYMBOLS), declared


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True, check=True)
    exported = set(re.findall(r"\sT\s(\w+)", nm.stdout))
    for name in _declared_functions():
        assert name in exported, name


def test_status_strings():
    for code in range(9):
        s = _lib.status_string(code)
        assert s and s != "unknown status"
    assert _lib.status_string(99) == "unknown status"
    assert _lib.version() >> 16 == 1


# fake, aligned, distinct device addresses: every call below must fail validation before
# the library touches HIP, so they are never dereferenced
A, Bp, Cp, D = 0x10000000, 0x20000000, 0x30000000, 0x40000000


def _win(q=A, k=Bp, v=Cp, out=D, B=1, heads=2, grid=(1, 16, 16), window=(1, 8, 8), shift=(0, 4, 4),
         head_dim=64, dtype=0):
    return _lib.load().basa_window_attn_fwd(q, k, v, out, B, heads, *grid, *window, *shift, head_dim, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(out=None), 1),
    (dict(B=0), 2), (dict(heads=-1), 2), (dict(grid=(1, 0, 16)), 2), (dict(window=(1, 8, 0)), 2),
    (dict(window=(1, 6, 8)), 2), (dict(grid=(3, 16, 16), window=(2, 8, 8)), 2),
    (dict(head_dim=96), 3), (dict(head_dim=256), 3), (dict(dtype=2), 3), (dict(dtype=-1), 3),
    (dict(out=A), 4), (dict(out=Bp + 64), 4), (dict(q=D + 128 * 64 * 4 - 16), 4),
    (dict(grid=(1, 65536, 65536), window=(1, 1, 1)), 5),
    (dict(grid=(1, 4096, 8192), window=(1, 1, 1), head_dim=128), 5),
    (dict(B=65536, heads=65536), 5),
    # bf16: one head may hold at most 0xffffff00 bytes (N*d = 0x7fffffc0 here: 0xffffff80 bytes)
    (dict(grid=(1, 1, 0x7fffffc0 // 64), window=(1, 1, 1), dtype=1), 5),
    (dict(q=A + 8), 7), (dict(out=D + 4), 7),
])
def test_argument_errors_return_codes(kw, code):
    assert _win(**kw) == code


ERROR_CASES = [(dict(q=None), 1), (dict(window=(1, 6, 8)), 2), (dict(head_dim=96), 3), (dict(out=A), 4),
               (dict(B=65536, heads=65536), 5), (dict(q=A + 8), 7)]


@pytest.mark.parametrize("kw,code", ERROR_CASES)
def test_noalloc_argument_errors_match(kw, code):
    """The no-allocation entry point validates exactly like basa_window_attn_fwd."""
    args = dict(q=A, k=Bp, v=Cp, out=D, B=1, heads=2, grid=(1, 16, 16), window=(1, 8, 8), shift=(0, 4, 4),
                head_dim=64, dtype=0)
    args.update(kw)
    rc = _lib.load().basa_window_attn_fwd_noalloc(args["q"], args["k"], args["v"], args["out"], args["B"],
                                                  args["heads"], *args["grid"], *args["window"], *args["shift"],
                                                  args["head_dim"], args["dtype"], None)
    assert rc == code == _win(**kw)


def test_full_and_perm_argument_errors():
    lib = _lib.load()
    assert lib.basa_full_attn_fwd(None, Bp, Cp, D, 1, 1, 64, 64, 1, None) == 1
    assert lib.basa_full_attn_fwd(A, Bp, Cp, D, 1, 1, 0, 64, 1, None) == 2
    assert lib.basa_full_attn_fwd(A, Bp, Cp, D, 1, 1, 64, 80, 1, None) == 3
    assert lib.basa_full_attn_fwd(A, Bp, Cp, A, 1, 1, 64, 64, 1, None) == 4
    assert lib.basa_window_perm(1, 16, 16, 1, 8, 8, 0, 0, 0, None, None) == 1
    assert lib.basa_window_perm(1, 16, 16, 1, 5, 8, 0, 0, 0, A, None) == 2
    assert lib.basa_window_perm(1, 16, 16, 1, 8, 8, 0, 0, 0, A + 2, None) == 7


def test_memory_and_pool_argument_errors():
    lib = _lib.load()
    E, F = 0x50000000, 0x60000000  # fake memory buffers, far from A..D

    def mem(q=A, k=Bp, v=Cp, km=E, vm=F, n_mem=16, out=D, lse=None, dtype=1, d=128):
        return lib.basa_window_attn_mem_fwd(q, k, v, km, vm, n_mem, out, lse, 1, 2, 1, 16, 16, 1, 8, 8, 0, 4, 4, d,
                                            dtype, None)
    assert mem(n_mem=-1) == 2
    assert mem(km=None) == 1 and mem(vm=None) == 1
    assert mem(km=E + 8) == 7
    assert mem(lse=D + 2) == 7
    assert mem(lse=A) == 4            # lse over q
    assert mem(out=E) == 4            # out over the memory
    assert mem(d=96) == 3
    assert mem(n_mem=(0xffffff00 // 256) + 1) == 5   # bf16 memory beyond the 32-bit byte range

    def pool(k=A, v=Bp, km=E, vm=F, ph=4, pw=4, dtype=1, d=128):
        return lib.basa_pool_kv(k, v, km, vm, 1, 2, 1, 16, 16, ph, pw, d, dtype, None)
    assert pool(k=None) == 1 and pool(vm=None) == 1
    assert pool(ph=0) == 2 and pool(pw=-1) == 2
    assert pool(dtype=5) == 3 and pool(d=32) == 3
    assert pool(km=E + 4) == 7
    assert pool(km=A) == 4 and pool(vm=E) == 4


def test_routing_argument_errors():
    """The routing entry points through the Python binding's own argument lists (so a
    binding/signature mismatch fails here too) and the raw ABI."""
    lib = _lib.load()
    E, F, G = 0x50000000, 0x60000000, 0x70000000

    def means(q=A, k=Bp, qb=E, kb=F, d=128, dtype=1, window=(1, 8, 8)):
        return lib.basa_window_means(q, k, qb, kb, 1, 2, 1, 16, 16, *window, 0, 4, 4, d, dtype, None)
    assert means(q=None) == 1 and means(kb=None) == 1
    assert means(window=(1, 5, 8)) == 2
    assert means(d=80) == 3 and means(dtype=7) == 3
    assert means(qb=E + 4) == 7
    assert means(qb=A) == 4 and means(kb=E) == 4

    def route(qb=E, kb=F, r=G, radius=1, d=128):
        return lib.basa_route_top1(qb, kb, r, 1, 2, 1, 16, 16, 1, 8, 8, radius, d, None)
    assert route(r=None) == 1
    assert route(radius=-1) == 2
    assert route(d=32) == 3
    assert route(r=G + 2) == 7
    assert route(r=E) == 4

    def routed(rt=G, km=None, vm=None, n_mem=0, lse=None):
        return lib.basa_window_attn_routed_fwd(A, Bp, Cp, rt, km, vm, n_mem, D, lse, 1, 2, 1, 16, 16, 1, 8, 8, 0, 4, 4,
                                               128, 1, None)
    assert routed(rt=G + 2) == 7
    assert routed(n_mem=4) == 1
    assert routed(lse=D) == 4
    # the route table is an input: it must not overlap out or lse
    assert routed(rt=D) == 4
    assert routed(rt=D + 128 * 256 * 2 * 2 - 4) == 4      # last int32 of out
    assert routed(rt=G, lse=G - 4 * 2 * 256 + 4) == 4      # lse's last row over route's first


@pytest.fixture(scope="module")
def index_tool(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("idx") / "index_map_check")
    subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", "-I", CSRC,
                    os.path.join(ROOT, "tests", "host", "index_map_check.cpp"), "-o", exe], check=True)
    return exe


def test_fastdiv_matches_division(index_tool):
    res = subprocess.run([index_tool, "fastdiv"], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr


CASES = [(w.grid, w.window, s) for w in WORKLOADS for s in w.shifts] + [
    ((21, 30, 52), (21, 15, 26), (5, -7, 40)),
    ((6, 6, 6), (3, 2, 3), (-1, -5, 8)),
    ((1, 1, 4096), (1, 1, 4096), (0, 0, 0)),       # the dense baseline's degenerate map
    ((2, 3, 5), (1, 1, 1), (1, 1, 1)),
]


@pytest.mark.parametrize("grid,window,shift", CASES)
def test_index_map_header_matches_oracle_table(index_tool, tmp_path, grid, window, shift):
    out = str(tmp_path / "t.bin")
    subprocess.run([index_tool, "table", *map(str, grid), *map(str, window), *map(str, shift), out], check=True)
    got = np.fromfile(out, dtype=np.int32)
    ref = O.window_members(grid, window, shift).ravel()
    assert np.array_equal(got, ref)


def test_binding_rejects_host_tensors_before_any_library_call():
    """The Python binding checks its tensors before it calls an entry point: host tensors
    are refused with BASA_ERR_NULL's code."""
    import torch
    from sparse_attention_dit_amd import _lib
    q = torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16)
    with pytest.raises(_lib.BasaError) as e:
        _lib.window_attn_fwd(q, q, q, torch.empty_like(q), (1, 8, 8), (1, 8, 8), (0, 0, 0))
    assert e.value.status == 1 and "device tensor" in str(e.value)


def test_binding_loads_only_the_in_tree_library():
    """The binding always loads the library built in the package directory: an environment
    variable naming another build is not consulted (checked in a fresh interpreter)."""
    import sys
    assert _lib.LIB_PATH == os.path.join(ROOT, "sparse_attention_dit_amd", "libbasa.so")
    info = _lib.library_info()
    assert info["path"] == os.path.join("sparse_attention_dit_amd", "libbasa.so")
    assert len(info["sha256_16"]) == 16
    env = dict(os.environ, BASA_LIB="/nonexistent/libother.so")
    res = subprocess.run([sys.executable, "-c", "from sparse_attention_dit_amd import _lib; print(_lib.LIB_PATH)"],
                         cwd=ROOT, env=env, capture_output=True, text=True, check=True)
    assert res.stdout.strip() == _lib.LIB_PATH
