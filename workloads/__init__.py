"""Seeded synthetic inputs for the padding-free MoE layer.

This module is shared by the tests, the benchmark and the smoke check. It holds
the workload table and the random-number recipes only: none of the layer's
arithmetic (routing, token buffers, expert FFN, combine, gradients) lives here,
so the CPU oracle and the GPU path can both consume its tensors without sharing
any of the method.

Shapes follow DeepSeek-MoE / DeepSeek-V3-style fine-grained layers (many small
experts, large top-k), the class of model the X-MoE notes ("略读笔记90",
section 需求) and the X-MoE article (section 1) describe. No public dataset or
trained checkpoint is needed or used: every tensor is Gaussian noise.

Recipe (one line per tensor kind):
  * X ~ N(0, 1); dY ~ N(0, 1).
  * Router Wg [d, E] and expert weights ~ N(0, 1/fan_in): fan_in = d for Wg,
    W1, W3 and the shared up-projections; fan_in = h for W2 and the shared
    down-projection.
  * bf16 workloads round every input to bf16 once (round to nearest even);
    both sides read the identical bits.
  * Each tensor (and each expert's slice of the expert weights) draws from its
    own torch.Generator seeded from (workload seed, tensor id, expert index), so
    tensors can be regenerated independently and in chunks.
  * Values depend on the device the generator runs on (torch's CPU and GPU
    generators differ); a test always hands the same arrays to both sides.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Tuple

import numpy as np
import torch

__all__ = [
    "Workload", "WORKLOADS", "get", "small", "generate", "random_topk",
    "random_segments", "exact_router_inputs", "to_numpy_f32", "bf16_bits",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32" or "bf16"
    T: int                # tokens
    d: int                # model width
    E: int                # routed experts
    h: int                # expert hidden width
    k: int                # experts per token
    n_shared: int = 0     # always-on shared experts (hidden width h_shared each)
    h_shared: int = 0
    inv_tau: float = 1.0  # router logit scale 1/temperature
    select_bias_var: float = 0.0   # variance of the selection-only expert bias
    zipf_s: float = 0.0   # > 0: per-expert logit offset 2*ln(Zipf(s) weight of rank e+1)
    backward: bool = False
    seed: int = 0

    @property
    def R(self) -> int:
        return self.T * self.k

    def useful_flops(self) -> Dict[str, float]:
        """Useful GEMM FLOPs on unpadded rows (router, routed and shared experts).

        Backward GEMMs count twice their forward term; elementwise work is not
        counted."""
        T, d, E, h, k = self.T, self.d, self.E, self.h, self.k
        fwd = 2.0 * T * d * E + 6.0 * T * k * d * h + 6.0 * T * self.n_shared * d * self.h_shared
        bwd = 2.0 * fwd if self.backward else 0.0
        return {"fwd": fwd, "bwd": bwd, "total": fwd + bwd}


# The five workloads: a tiny fp32 parity case, then four DeepSeek-style bf16 layers.
WORKLOADS: Dict[str, Workload] = {
    "tiny_f32": Workload("tiny_f32", "f32", T=256, d=128, E=8, h=64, k=2),
    "dsmoe16b": Workload("dsmoe16b", "bf16", T=4096, d=2048, E=64, h=1408, k=6,
                         n_shared=2, h_shared=1408, backward=True),
    "dsv3": Workload("dsv3", "bf16", T=8192, d=7168, E=256, h=2048, k=8,
                     select_bias_var=0.1),
    "zipf_skew": Workload("zipf_skew", "bf16", T=16384, d=2048, E=128, h=768, k=8,
                          zipf_s=1.2, backward=True),
    "long_batch": Workload("long_batch", "bf16", T=32768, d=4096, E=160, h=1024, k=8,
                           inv_tau=2.0, backward=True),
}

# Reduced-size cousins: same structure, sizes the oracle finishes in seconds while
# still spanning several GEMM tiles and ragged tails.
_SMALL: Dict[str, Workload] = {
    "tiny_f32": WORKLOADS["tiny_f32"],
    "dsmoe16b": Workload("dsmoe16b_small", "bf16", T=300, d=256, E=16, h=200, k=6,
                         n_shared=2, h_shared=200, backward=True),
    "dsv3": Workload("dsv3_small", "bf16", T=260, d=448, E=32, h=136, k=8,
                     select_bias_var=0.1),
    "zipf_skew": Workload("zipf_skew_small", "bf16", T=520, d=256, E=32, h=96, k=8,
                          zipf_s=1.2, backward=True),
    "long_batch": Workload("long_batch_small", "bf16", T=384, d=320, E=40, h=128, k=8,
                           inv_tau=2.0, backward=True),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def small(name: str) -> Workload:
    return _SMALL[name]


_TENSOR_ID = {"x": 1, "wg": 2, "w1": 3, "w3": 4, "w2": 5, "s1": 6, "s3": 7, "s2": 8,
              "dy": 9, "select_bias": 10, "topk": 11, "topk_w": 12, "seg": 13, "rows": 14}


def _gen(device: str, seed: int, tensor: str, part: int = 0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + _TENSOR_ID[tensor]) * 65_537 + part)
    return g


def _gauss(shape, std: float, dtype: str, device: str, seed: int, tensor: str, part: int = 0):
    g = _gen(device, seed, tensor, part)
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        v.mul_(std)
    return v.to(torch.bfloat16) if dtype == "bf16" else v


def _expert_weights(E: int, rows: int, cols: int, std: float, dtype: str, device: str,
                    seed: int, tensor: str) -> torch.Tensor:
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = torch.empty((E, rows, cols), dtype=tdt, device=device)
    for e in range(E):
        out[e].copy_(_gauss((rows, cols), std, dtype, device, seed, tensor, part=e + 1))
    return out


def zipf_logit_offset(E: int, s: float) -> torch.Tensor:
    """2*ln(w_{e+1}) with w_r = r^-s / sum_{r'=1..E} r'^-s, expert e <-> rank e+1."""
    r = np.arange(1, E + 1, dtype=np.float64)
    w = r ** (-s)
    w /= w.sum()
    return torch.from_numpy((2.0 * np.log(w)).astype(np.float32))


def generate(wl: Workload, device: str = "cpu", backward: Optional[bool] = None,
             experts: bool = True) -> Dict[str, torch.Tensor]:
    """All inputs of one layer invocation on `device`.

    Keys: x [T,d], wg [d,E], w1/w3 [E,d,h], w2 [E,h,d], logit_bias [E] or None,
    select_bias [E] or None, s1/s3 [d, n_shared*h_shared] and s2
    [n_shared*h_shared, d] (the shared experts side by side along the hidden
    axis), dy [T,d] when the backward runs."""
    T, d, E, h = wl.T, wl.d, wl.E, wl.h
    dt = wl.dtype
    out: Dict[str, Optional[torch.Tensor]] = {}
    out["x"] = _gauss((T, d), 1.0, dt, device, wl.seed, "x")
    out["wg"] = _gauss((d, E), 1.0 / math.sqrt(d), dt, device, wl.seed, "wg")
    if experts:
        out["w1"] = _expert_weights(E, d, h, 1.0 / math.sqrt(d), dt, device, wl.seed, "w1")
        out["w3"] = _expert_weights(E, d, h, 1.0 / math.sqrt(d), dt, device, wl.seed, "w3")
        out["w2"] = _expert_weights(E, h, d, 1.0 / math.sqrt(h), dt, device, wl.seed, "w2")
    out["logit_bias"] = zipf_logit_offset(E, wl.zipf_s).to(device) if wl.zipf_s > 0 else None
    if wl.select_bias_var > 0:
        g = _gen(device, wl.seed, "select_bias")
        out["select_bias"] = (torch.randn(E, generator=g, device=device, dtype=torch.float32)
                              * math.sqrt(wl.select_bias_var))
    else:
        out["select_bias"] = None
    if wl.n_shared and experts:
        hs = wl.h_shared
        tdt = torch.bfloat16 if dt == "bf16" else torch.float32
        s1 = torch.empty((d, wl.n_shared * hs), dtype=tdt, device=device)
        s3 = torch.empty((d, wl.n_shared * hs), dtype=tdt, device=device)
        s2 = torch.empty((wl.n_shared * hs, d), dtype=tdt, device=device)
        for s in range(wl.n_shared):
            s1[:, s * hs:(s + 1) * hs] = _gauss((d, hs), 1.0 / math.sqrt(d), dt, device, wl.seed, "s1", s + 1)
            s3[:, s * hs:(s + 1) * hs] = _gauss((d, hs), 1.0 / math.sqrt(d), dt, device, wl.seed, "s3", s + 1)
            s2[s * hs:(s + 1) * hs, :] = _gauss((hs, d), 1.0 / math.sqrt(hs), dt, device, wl.seed, "s2", s + 1)
        out["s1"], out["s3"], out["s2"] = s1, s3, s2
    bwd = wl.backward if backward is None else backward
    if bwd:
        out["dy"] = _gauss((T, d), 1.0, dt, device, wl.seed, "dy")
    return out


def random_topk(T: int, E: int, k: int, seed: int = 0, skew: float = 0.0,
                device: str = "cpu") -> Tuple[torch.Tensor, torch.Tensor]:
    """A random valid routing result: k distinct experts per token (in random slot
    order) and positive fp32 weights. skew > 0 draws experts with Gumbel-top-k
    over log-weights -skew*ln(rank), which leaves some experts empty."""
    g = _gen(device, seed, "topk")
    u = torch.rand((T, E), generator=g, device=device, dtype=torch.float64).clamp_(1e-300, 1.0)
    key = -torch.log(-torch.log(u))
    if skew > 0:
        key = key - skew * torch.log(torch.arange(1, E + 1, device=device, dtype=torch.float64))
    ids = torch.topk(key, k, dim=1).indices
    perm = torch.rand((T, k), generator=g, device=device).argsort(dim=1)
    ids = torch.gather(ids, 1, perm).to(torch.int32).contiguous()
    gw = _gen(device, seed, "topk_w")
    w = torch.rand((T, k), generator=gw, device=device, dtype=torch.float32) * 0.9 + 0.05
    return ids, w.contiguous()


def random_segments(rows_total: int, E: int, seed: int = 0, empty_frac: float = 0.25,
                    device: str = "cpu") -> torch.Tensor:
    """Random non-decreasing offsets [E+1] with offsets[0]=0, offsets[E]=rows_total,
    some segments empty and the rest of random, ragged length."""
    g = _gen("cpu", seed, "seg")
    w = torch.rand(E, generator=g, dtype=torch.float64) ** 3
    w[torch.rand(E, generator=g) < empty_frac] = 0.0
    if w.sum() == 0:
        w[0] = 1.0
    cuts = torch.floor(torch.cumsum(w, 0) / w.sum() * rows_total).to(torch.int64)
    cuts[-1] = rows_total
    off = torch.zeros(E + 1, dtype=torch.int32)
    off[1:] = cuts.to(torch.int32)
    return off.to(device)


def random_rows(rows: int, cols: int, dtype: str, seed: int = 0, device: str = "cpu",
                std: float = 1.0) -> torch.Tensor:
    """Gaussian [rows, cols] block (activations, upstream gradients, ...)."""
    return _gauss((rows, cols), std, dtype, device, seed, "rows", part=cols)


def exact_router_inputs(T: int, d: int, E: int, seed: int = 0, device: str = "cpu"):
    """X and Wg whose entries are small multiples of powers of two, so that every
    partial sum of X[t]·Wg[:,e] is exact in fp32 whatever the summation order.
    Ties between experts are then frequent and exactly reproducible."""
    g = _gen(device, seed, "x", part=777)
    x = torch.randint(-3, 4, (T, d), generator=g, device=device).to(torch.float32) * 0.25
    wg = torch.randint(-2, 3, (d, E), generator=g, device=device).to(torch.float32) * 0.125
    # a few tokens get an all-zero row so every expert ties exactly
    x[::17] = 0.0
    return x, wg


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (host)."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def to_numpy_f32(t: torch.Tensor) -> np.ndarray:
    """Exact widening of an fp32/bf16 tensor to a host float32 array."""
    return t.detach().cpu().to(torch.float32).contiguous().numpy()
