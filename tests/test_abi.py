"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, answers the workspace queries, and rejects invalid arguments
on the host before touching a device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "xmoe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(xmoe_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def xm():
    import padding_free_expert_amd as m
    return m


def test_header_declares_the_layer_calls():
    names = _declared()
    for n in ["xmoe_route", "xmoe_build_pft", "xmoe_dispatch", "xmoe_expert_ffn", "xmoe_combine",
              "xmoe_combine_bwd", "xmoe_expert_ffn_bwd", "xmoe_dispatch_bwd", "xmoe_route_bwd"]:
        assert n in names


def test_library_exports_every_declared_symbol(xm):
    lib = ctypes.CDLL(xm.lib_path())
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_c_caller_links_the_library():
    """The C program that drives the layer through the C ABI (built with the
    library) loads libxmoe.so through its run path; without arguments it
    prints its usage before any HIP call."""
    import subprocess
    exe = os.path.join(ROOT, "tests", "c_abi", "layer_c")
    assert os.path.exists(exe), "tests/c_abi/layer_c is not built"
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "usage" in r.stderr, (r.returncode, r.stderr)


def test_workspace_queries(xm):
    import torch
    assert xm.xmoe_build_pft_workspace_size(32768, 160, 8) >= 2 * 128 * 160 * 4
    assert xm.xmoe_build_pft_workspace_size(0, 8, 2) > 0
    assert xm.xmoe_build_pft_workspace_size(10, 8, 9) == 0          # k > E
    assert xm.xmoe_build_pft_workspace_size(10, 2000, 2) == 0       # E > 1024
    assert xm.xmoe_route_bwd_workspace_size(4096, 2048, 64, torch.bfloat16) >= 4096 * 64 * 2
    # bf16 routing: up to 64 experts one fused launch (no workspace), beyond
    # that fp32 partial sums over a split of d
    assert xm.xmoe_route_workspace_size(4096, 2048, 64, torch.bfloat16) == 0
    assert xm.xmoe_route_workspace_size(4096, 2048, 128, torch.bfloat16) >= 4096 * 128 * 4
    assert xm.xmoe_route_workspace_size(4096, 2048, 160, torch.bfloat16) >= 4096 * 160 * 4
    assert xm.xmoe_route_workspace_size(4096, 2048, 64, torch.float32) == 0
    assert xm.xmoe_route_bwd_workspace_size(4096, 2048, 0, torch.bfloat16) == 0


def test_invalid_arguments_rejected_on_host(xm):
    lib = xm._lib
    # xmoe_route with NULL pointers
    assert xm._lib_route(None, None, 1, 10, 8, 8, 2, 1.0, None, None, None, None, None, None, 0, None) == 1
    assert b"NULL" in xm._lib_last_error()
    p = ctypes.c_void_p(16)  # never dereferenced: validation fails before any use
    # k > E
    assert xm._lib_route(p, p, 1, 10, 8, 8, 9, 1.0, None, None, p, p, p, None, 0, None) == 1
    # unknown dtype
    assert xm._lib_route(p, p, 7, 10, 8, 8, 2, 1.0, None, None, p, p, p, None, 0, None) == 2
    # bf16 with d not a multiple of 8
    assert xm._lib_route(p, p, 1, 10, 12, 8, 2, 1.0, None, None, p, p, p, None, 0, None) == 2
    # bf16 routing over more than 64 experts without its workspace
    assert xm._lib_route(p, p, 1, 10, 64, 256, 2, 1.0, None, None, p, p, p, None, 0, None) == 3
    # expert FFN: h not a multiple of 8, E out of range, NULL offsets
    assert xm._lib_up(p, p, p, 1, p, 4, 100, 64, 12, p, None, None) == 2
    assert xm._lib_up(p, p, p, 1, p, 0, 100, 64, 64, p, None, None) == 1
    assert xm._lib_up(p, p, p, 1, None, 4, 100, 64, 64, p, None, None) == 1
    # neither act nor h13 to write
    assert xm._lib_up(p, p, p, 1, p, 4, 100, 64, 64, None, None, None) == 1
    # build_pft: workspace too small
    pft = xm._CPft(16, 16, 16, 16, 16, 16)
    assert xm._lib_pft(p, p, 1000, 16, 4, ctypes.byref(pft), p, 8, None) == 3
    # dispatch: T*k overflow
    assert lib.xmoe_dispatch(p, 1, ctypes.c_int64(1 << 30), 64, 8, ctypes.byref(pft), p, None) == 1
    assert xm._lib_last_error() != b""


def test_pilot_and_ep_entry_points_reject_on_host(xm):
    p = ctypes.c_void_p(16)  # never dereferenced
    assert xm.xmoe_build_pilots_workspace_size(4096, 64, 6, 8) >= 16 * 8 * 4
    assert xm.xmoe_build_pilots_workspace_size(4096, 64, 6, 5) == 0      # 5 does not divide 64
    assert xm.xmoe_ep_recv_plan_workspace_size(8, 8) >= 2 * 64 * 4
    assert xm.xmoe_ep_recv_plan_workspace_size(64, 32) == 0              # more than 1024 cells
    # pilots: experts_per_node not dividing E; workspace too small
    assert xm._lib_pilots(p, 100, 64, 6, 5, p, p, p, p, p, p, 1 << 20, None) == 1
    assert xm._lib_pilots(p, 100000, 64, 6, 8, p, p, p, p, p, p, 16, None) == 3
    # send plan: G not dividing E
    assert xm._lib_ep_send(p, 64, 6, p, p, None) == 1
    # recv plan: too many cells, missing maps
    assert xm._lib_ep_recv(p, 64, 32, 10, p, p, p, p, p, 1 << 20, None) == 1
    assert xm._lib_ep_recv(p, 8, 8, 10, p, p, None, p, p, 1 << 20, None) == 1
    # row scatter: d not a multiple of 8, unknown dtype
    assert xm._lib_scatter_rows(p, 1, 10, 12, p, 10, p, None) == 2
    assert xm._lib_scatter_rows(p, 9, 10, 16, p, 10, p, None) == 2


def test_shared_buffer_and_route_bwd_reject_on_host(xm):
    p = ctypes.c_void_p(16)  # never dereferenced
    pft = xm._CPft(16, 16, 16, 16, 16, 16)
    assert xm._lib_pft_sh(p, p, 100, 64, 6, -1, ctypes.byref(pft), p, 1 << 20, None) == 1      # n_shared < 0
    assert xm._lib_pft_sh(p, p, 100, 1020, 6, 8, ctypes.byref(pft), p, 1 << 20, None) == 1     # > 1024 experts
    assert xm._lib_pft_sh(p, p, 100000, 64, 6, 2, ctypes.byref(pft), p, 16, None) == 3         # workspace
    # route_bwd: ldw < k
    assert xm._lib_rbwd(p, p, p, p, p, 3, 1, 100, 64, 64, 6, 1.0, 1, p, p, p, 1 << 24, None) == 1


def test_gathered_dact_rejects_on_host(xm):
    p = ctypes.c_void_p(16)  # never dereferenced
    f = xm._lib_bwd_dact_g
    # dy [T, d] of 2^31 bytes or more cannot be gathered through one buffer
    assert f(p, p, p, p, p, 1, p, 4, 1 << 17, 100, 8192, 64, p, None) == 2
    # NULL dy or token_ids with rows to gather; NULL row weights
    assert f(None, p, p, p, p, 1, p, 4, 100, 100, 64, 64, p, None) == 1
    assert f(p, None, p, p, p, 1, p, 4, 100, 100, 64, 64, p, None) == 1
    assert f(p, p, None, p, p, 1, p, 4, 100, 100, 64, 64, p, None) == 1
    # h not a multiple of 8, misaligned dy
    assert f(p, p, p, p, p, 1, p, 4, 100, 100, 64, 12, p, None) == 2
    assert f(ctypes.c_void_p(18), p, p, p, p, 1, p, 4, 100, 100, 64, 64, p, None) == 2
    assert xm._lib_last_error() != b""


def test_gathered_wgrad_rejects_on_host(xm):
    p = ctypes.c_void_p(16)  # never dereferenced
    f = xm._lib_bwd_dw13_g
    # x [T, d] of 2^31 bytes or more cannot be gathered through one buffer
    assert f(p, p, p, 1, p, 4, 1 << 17, 100, 8192, 64, p, p, 1, 0, None) == 2
    # NULL x or token_ids with rows to gather; NULL dh13
    assert f(None, p, p, 1, p, 4, 100, 100, 64, 64, p, p, 1, 0, None) == 1
    assert f(p, None, p, 1, p, 4, 100, 100, 64, 64, p, p, 1, 0, None) == 1
    assert f(p, p, None, 1, p, 4, 100, 100, 64, 64, p, p, 1, 0, None) == 1
    # no tokens but rows to gather, h not a multiple of 8, misaligned x
    assert f(p, p, p, 1, p, 4, 0, 100, 64, 64, p, p, 1, 0, None) == 1
    assert f(p, p, p, 1, p, 4, 100, 100, 64, 12, p, p, 1, 0, None) == 2
    assert f(ctypes.c_void_p(18), p, p, 1, p, 4, 100, 100, 64, 64, p, p, 1, 0, None) == 2
    assert xm._lib_last_error() != b""
    # an empty batch (no tokens, no rows) passes validation in every gathered
    # product: what follows is the device check, or nothing to launch
    assert f(None, None, None, 1, p, 4, 0, 0, 64, 64, p, p, 1, 0, None) not in (1, 2, 3)
    assert xm._lib_up_g(None, None, p, p, 1, p, 4, 0, 0, 64, 64, None, None, None) not in (1, 2, 3)
    assert xm._lib_bwd_dact_g(None, None, None, p, None, 1, p, 4, 0, 0, 64, 64, None, None) not in (1, 2, 3)


def test_weight_gradient_dtype_and_accumulate_rejected_on_host(xm):
    """grad_dt: the input dtype, or fp32 with bf16 inputs; accumulating into the
    weight gradients needs fp32 gradients."""
    p = ctypes.c_void_p(16)  # never dereferenced
    BF16, F32 = 1, 0
    dw2 = xm._lib_bwd_dw2
    assert dw2(p, p, BF16, p, 4, 100, 64, 64, p, 7, 0, None) == 2           # unknown grad_dt
    assert dw2(p, p, F32, p, 4, 100, 64, 64, p, BF16, 0, None) == 2        # fp32 inputs, bf16 gradients
    assert dw2(p, p, BF16, p, 4, 100, 64, 64, p, BF16, 1, None) == 2       # accumulate into bf16
    assert b"grad_dt" in xm._lib_last_error()
    dw13 = xm._lib_bwd_dw13
    assert dw13(p, p, BF16, p, 4, 100, 64, 64, p, p, BF16, 1, None) == 2
    assert xm._lib_bwd_dw13_g(p, p, p, BF16, p, 4, 100, 100, 64, 64, p, p, BF16, 1, None) == 2
    bwd = xm._lib_ffn_bwd
    assert bwd(p, p, p, p, p, p, p, BF16, p, 4, 100, 64, 64, p, p, 0, p, p, p, BF16, 1, None) == 2
    assert bwd(p, p, p, p, p, p, p, F32, p, 4, 100, 64, 64, p, p, 0, p, p, p, BF16, 0, None) == 2
    assert xm.xmoe_version() == 200


def test_noalloc_pft_build_limit_on_host(xm):
    """The allocation-free PFT build takes at most its static scratch
    (4 MiB: 511 blocks of 256 tokens at 1024 experts) and rejects larger sizes
    before any launch."""
    p = ctypes.c_void_p(16)  # never dereferenced
    pft = xm._CPft(16, 16, 16, 16, 16, 16)
    mx = xm.xmoe_build_pft_noalloc_max_bytes()
    assert mx == 4 << 20
    assert xm.xmoe_build_pft_workspace_size(130816, 1024, 8) <= mx
    assert xm.xmoe_build_pft_workspace_size(130817, 1024, 8) > mx
    assert xm._lib_pft_na(p, p, 130817, 1024, 8, ctypes.byref(pft), None) == 2
    assert b"scratch" in xm._lib_last_error()
    assert xm._lib_pft_na(p, p, 100, 64, 65, ctypes.byref(pft), None) == 1      # k > E
    assert xm._lib_pft_na(None, p, 100, 64, 6, ctypes.byref(pft), None) == 1


def test_binding_checks_tensor_shapes_before_calling(xm):
    """The binding passes pointers and sizes; it takes the sizes from the
    inputs and requires every other tensor of the call to hold exactly them,
    in the call's dtype, so a mismatched output raises instead of being written
    past.  (CPU tensors of the right shapes pass these checks and are then
    refused as host memory, also before any call.)"""
    import torch
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    E, d, h, rows = 4, 64, 32, 10
    xs = torch.zeros(rows, d, dtype=bf)
    w1, w3 = torch.zeros(E, d, h, dtype=bf), torch.zeros(E, d, h, dtype=bf)
    w2 = torch.zeros(E, h, d, dtype=bf)
    off = torch.zeros(E + 1, dtype=i32)
    act, ye = torch.zeros(rows, h, dtype=bf), torch.zeros(rows, d, dtype=bf)
    with pytest.raises(ValueError, match="act"):
        xm.xmoe_expert_ffn_up(xs, w1, w3, off, torch.zeros(rows - 1, h, dtype=bf))
    with pytest.raises(ValueError, match="h13"):
        xm.xmoe_expert_ffn_up(xs, w1, w3, off, act, torch.zeros(rows, h, dtype=bf))
    with pytest.raises(TypeError, match="act"):
        xm.xmoe_expert_ffn_up(xs, w1, w3, off, torch.zeros(rows, h, dtype=f32))
    with pytest.raises(ValueError, match="w3"):
        xm.xmoe_expert_ffn_up(xs, w1, torch.zeros(E, d, h + 8, dtype=bf), off, act)
    with pytest.raises(ValueError, match="expert_offsets"):
        xm.xmoe_expert_ffn(xs, w1, w3, w2, torch.zeros(E, dtype=i32), act, ye)
    with pytest.raises(ValueError, match="ye"):
        xm.xmoe_expert_ffn_down(act, w2, off, torch.zeros(rows, d + 8, dtype=bf))
    with pytest.raises(ValueError, match="dw2"):
        xm.xmoe_expert_ffn_bwd_dw2(act, ye, off, torch.zeros(E, d, h, dtype=f32))
    T, k = 5, 2
    pft = xm.PFT(T, E, k, device="cpu")
    ids, w = torch.zeros(T, k, dtype=i32), torch.zeros(T, k, dtype=f32)
    with pytest.raises(ValueError, match="pft.tokens_per_expert"):
        xm.xmoe_build_pft(ids, w, E + 1, pft, torch.zeros(16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="y"):
        xm.xmoe_combine(torch.zeros(T * k, d, dtype=bf), pft, T, torch.zeros(T + 1, d, dtype=bf))
    with pytest.raises(ValueError, match="dtopk_w"):
        xm.xmoe_combine_bwd(torch.zeros(T, d, dtype=bf), torch.zeros(T * k, d, dtype=bf), pft,
                            torch.zeros(T * k, d, dtype=bf), torch.zeros(T, k + 1, dtype=f32))
    with pytest.raises(TypeError, match="topk_ids"):
        xm.xmoe_route(torch.zeros(T, d, dtype=bf), torch.zeros(d, E, dtype=bf), k, w, w,
                      torch.zeros(T, E, dtype=f32))
    # the right shapes pass the checks and reach the device-memory check
    with pytest.raises(ValueError, match="device tensors"):
        xm.xmoe_expert_ffn(xs, w1, w3, w2, off, act, ye)


def test_every_binding_call_checks_its_tensors():
    """Every binding function that calls into the library (through _check)
    first checks the tensors it passes (_shape, _atleast, _ffn_shapes,
    _pft_sized or an explicit shape test), so no future entry point can pass
    an unchecked buffer size."""
    import ast
    src = open(os.path.join(ROOT, "padding_free_expert_amd", "__init__.py")).read()
    tree = ast.parse(src)
    checks = {"_shape", "_atleast", "_ffn_shapes", "_pft_sized"}
    missing = []
    for fn in tree.body:
        if not isinstance(fn, ast.FunctionDef) or not fn.name.startswith("xmoe_"):
            continue
        called = {n.func.id for n in ast.walk(fn) if isinstance(n, ast.Call) and isinstance(n.func, ast.Name)}
        takes_tensors = any(a.arg not in ("stream",) for a in fn.args.args) and "_ptr" in called
        if "_check" in called and takes_tensors and not (called & checks):
            missing.append(fn.name)
    assert not missing, f"binding calls without tensor checks: {missing}"


def test_package_fails_loudly_without_the_library(tmp_path):
    """A copy of the package without libxmoe.so refuses to import (no CPU or
    PyTorch fallback), and no product source imports or loads the oracle."""
    import shutil
    import subprocess
    import sys
    pkg = os.path.join(ROOT, "padding_free_expert_amd")
    dst = tmp_path / "padding_free_expert_amd"
    dst.mkdir()
    for f in ("__init__.py", "layer.py"):
        shutil.copy(os.path.join(pkg, f), dst / f)
    r = subprocess.run([sys.executable, "-c", "import padding_free_expert_amd"], cwd=tmp_path,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "ImportError" in r.stderr and "not built" in r.stderr, r.stderr[-2000:]
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".hpp")):
                src = open(os.path.join(dirpath, f), errors="replace").read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b|liboracle", src, re.M), f
