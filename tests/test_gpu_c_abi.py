"""The layer driven from C.

tests/c_abi/layer_c runs the forward and backward of a bf16 padding-free layer
through libxmoe's C ABI and the HIP runtime's C API alone, as a caller without
Python would.  On the same inputs its outputs must be bitwise those of the
Python layer (whose binding only marshals arguments to the same calls): the
routing, the PFT-driven forward, every gradient.
"""
import os
import subprocess

import numpy as np
import pytest
import torch

import workloads
from _helpers import need_gpu

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_abi", "layer_c")


def _bits(t: torch.Tensor) -> bytes:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().tobytes()


@pytest.mark.parametrize("T,d,E,h,k", [(300, 256, 16, 136, 4), (1000, 512, 128, 128, 8), (1031, 40, 56, 344, 7)])
def test_c_driver_matches_python_layer(tmp_path, T, d, E, h, k):
    need_gpu()
    assert os.path.exists(EXE), "tests/c_abi/layer_c is not built (__graft_entry__.build() builds it)"
    wl = workloads.Workload("c_abi", "bf16", T=T, d=d, E=E, h=h, k=k, backward=True)
    inp = workloads.generate(wl, backward=True)
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        for key in ("x", "wg", "w1", "w3", "w2", "dy"):
            f.write(_bits(inp[key]))
    print(f"\n[c driver] T={T} d={d} E={E} h={h} k={k}", flush=True)
    r = subprocess.run([EXE, str(src), str(dst), str(T), str(d), str(E), str(h), str(k)], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    raw = open(dst, "rb").read()
    R = T * k
    layout = [("topk_ids", np.int32, R), ("topk_w", np.float32, R), ("y", np.uint16, T * d),
              ("dx", np.uint16, T * d), ("dw1", np.uint16, E * d * h), ("dw3", np.uint16, E * d * h),
              ("dw2", np.uint16, E * h * d), ("dwg", np.float32, d * E)]
    out, pos = {}, 0
    for name, dt, n in layout:
        nb = n * np.dtype(dt).itemsize
        out[name] = np.frombuffer(raw, dtype=dt, count=n, offset=pos)
        pos += nb
    assert pos == len(raw)

    from padding_free_expert_amd.layer import PaddingFreeMoE
    g = {key: v.cuda() for key, v in inp.items() if v is not None}
    layer = PaddingFreeMoE({key: g[key] for key in ("wg", "w1", "w3", "w2")}, T, k, 1.0, backward=True)
    layer.forward(g["x"])
    layer.backward(g["dy"])
    torch.cuda.synchronize()
    u16 = lambda t: t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16).ravel()
    py = {"topk_ids": layer.topk_ids.cpu().numpy().ravel(), "topk_w": layer.topk_w.cpu().numpy().ravel(),
          "y": u16(layer.y), "dx": u16(layer.dx), "dw1": u16(layer.dW1), "dw3": u16(layer.dW3),
          "dw2": u16(layer.dW2), "dwg": layer.dwg.cpu().numpy().ravel()}
    for name, _, _ in layout:
        a, b = out[name], py[name]
        assert a.shape == b.shape, name
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"{name}: C and Python layers differ"
