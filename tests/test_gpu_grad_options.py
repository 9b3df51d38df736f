"""GPU parity of the expert FFN's output options: fp32 weight gradients of bf16
inputs (grad_dt), adding into the weight gradients (accumulate over
micro-batches), adding into dxs and into the expert output (two shared experts
as two calls, the second adding to the first).

The backward is the reverse path of "5.4 MoE模型在分布式训练中的应用", section
训练流程, per expert over its own rows (X-MoE article, section 2.1.2).

Exact checks come first where the arithmetic fixes them: an fp32 gradient
holds the very fp32 sum the bf16 gradient rounds once (round to nearest even),
and accumulation is one IEEE addition of that sum to the caller's value.  The
oracle then checks values within the stated tolerance.
"""
import numpy as np
import pytest
import torch

import oracle as orc
import workloads
from _helpers import RTOL, assert_close, assert_wgrad_close, host, need_gpu, orc_in, swiglu_wgrad_scales, wgrad_acc

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}

CASES = [
    # dtype, rows, d, h, E, empty_frac (ragged d/h, empty experts, one busy expert)
    ("bf16", 700, 256, 200, 16, 0.25),
    ("bf16", 517, 328, 264, 7, 0.3),
    ("bf16", 12000, 256, 192, 8, 1.0),
    ("f32", 301, 64, 40, 5, 0.4),
]


def _random_cases(n: int, seed: int):
    """Seeded shapes as the expert-FFN parity cases: widths down to 8, 1-64
    experts with empty and ragged segments."""
    rs = np.random.RandomState(seed)
    out = []
    while len(out) < n:
        dt = "f32" if len(out) % 3 == 2 else "bf16"
        rows, E = int(rs.choice([1, 64, 300, 1000, 2500])), int(rs.choice([1, 3, 8, 13, 64]))
        d, h = 8 * int(rs.randint(1, 97)), 8 * int(rs.randint(1, 97))
        if rows * d * h <= (3e8 if dt == "bf16" else 1e8):
            out.append((dt, rows, d, h, E, float(rs.choice([0.0, 0.3, 0.7]))))
    return out


CASES += _random_cases(6, 15)


@pytest.fixture(scope="module")
def xm():
    need_gpu()
    import padding_free_expert_amd as m
    assert m.xmoe_query_device(0)
    return m


def _inputs(dtype, rows, d, h, E, empty, seed):
    off = workloads.random_segments(rows, E, seed=seed, empty_frac=empty)
    xs = workloads.random_rows(rows, d, dtype, seed=seed + 1)
    g = torch.Generator().manual_seed(seed)
    tdt = DT[dtype]
    w1 = (torch.randn((E, d, h), generator=g) / d ** 0.5).to(tdt)
    w3 = (torch.randn((E, d, h), generator=g) / d ** 0.5).to(tdt)
    w2 = (torch.randn((E, h, d), generator=g) / h ** 0.5).to(tdt)
    dye = workloads.random_rows(rows, d, dtype, seed=seed + 2)
    re_ = np.repeat(np.arange(E, dtype=np.int32), np.diff(off.numpy()))
    return [t.cuda() for t in (off, xs, w1, w3, w2, dye)] + [re_]


def _forward(xm, xs, w1, w3, w2, off):
    rows, h = xs.shape[0], w1.shape[2]
    act = torch.empty((rows, h), dtype=xs.dtype, device="cuda")
    h13 = torch.empty((rows, 2 * h), dtype=xs.dtype, device="cuda")
    ye = torch.empty((rows, xs.shape[1]), dtype=xs.dtype, device="cuda")
    xm.xmoe_expert_ffn(xs, w1, w3, w2, off, act, ye, h13=h13)
    return act, h13


def _grads(E, d, h, dt, fill=None):
    mk = lambda *s: (torch.full(s, float("nan"), dtype=dt, device="cuda") if fill is None
                     else fill(s).to(dt).cuda())
    return mk(E, d, h), mk(E, d, h), mk(E, h, d)


@pytest.mark.parametrize("dtype,rows,d,h,E,empty", CASES)
def test_fp32_weight_gradients(xm, dtype, rows, d, h, E, empty):
    """grad_dt = fp32: the unrounded sums.  Rounded to bf16 they are bitwise the
    bf16 gradients; against the oracle they meet the bf16 tolerance with the
    same rounding floors (their inputs dH1, dH3, act are still bf16)."""
    off, xs, w1, w3, w2, dye, re_ = _inputs(dtype, rows, d, h, E, empty, seed=rows + h)
    act, h13 = _forward(xm, xs, w1, w3, w2, off)
    tdt = DT[dtype]
    dh13 = torch.empty((rows, 2 * h), dtype=tdt, device="cuda")
    dxs = torch.empty((rows, d), dtype=tdt, device="cuda")
    g32 = _grads(E, d, h, torch.float32)
    xm.xmoe_expert_ffn_bwd(xs, w1, w3, w2, act, h13, dye, off, dh13, dxs, *g32)
    if dtype == "bf16":
        g16 = _grads(E, d, h, torch.bfloat16)
        xm.xmoe_expert_ffn_bwd(xs, w1, w3, w2, act, h13, dye, off, dh13, dxs, *g16)
        torch.cuda.synchronize()
        for name, a, b in zip(("dw1", "dw3", "dw2"), g32, g16):
            assert torch.equal(a.to(torch.bfloat16), b), name
    ref = orc.ffn_bwd(orc_in(xs), re_, orc_in(w1), orc_in(w3), orc_in(w2), orc_in(dye), want_dh=True)
    fwd = orc.ffn(orc_in(xs), re_, orc_in(w1), orc_in(w3), orc_in(w2), want_hidden=True)
    o = off.cpu().numpy()
    X, G = host(xs), host(dye)
    rows_of = lambda e: o[e + 1] - o[e]
    scales = {}

    def floors(e):
        if e not in scales:
            sl = slice(o[e], o[e + 1])
            scales[e] = swiglu_wgrad_scales(X[sl], ref["da"][sl], fwd["h1"][sl], fwd["h3"][sl], fwd["act"][sl],
                                            G[sl], host(w2[e]), (host(w1[e]), host(w3[e])), wgrad_acc(dtype, d))
        return scales[e]

    rt = RTOL[dtype]
    for i, name in enumerate(("dw1", "dw3", "dw2")):
        assert_wgrad_close(host(g32[i]), ref[name], rows_of, lambda e, i=i: floors(e)[i], rt, name)


@pytest.mark.parametrize("dtype,rows,d,h,E,empty", CASES)
def test_accumulated_weight_gradients(xm, dtype, rows, d, h, E, empty):
    """accumulate: dW = D0 + (the sums), one fp32 addition per element, so the
    result is bitwise D0 + the fp32 gradients of a plain call.  Experts with no
    rows keep D0.  Through the composite call and the split calls (dW1/dW3 with
    and without the fused gather, dW2)."""
    off, xs, w1, w3, w2, dye, _ = _inputs(dtype, rows, d, h, E, empty, seed=rows + 3 * h)
    act, h13 = _forward(xm, xs, w1, w3, w2, off)
    tdt = DT[dtype]
    dh13 = torch.empty((rows, 2 * h), dtype=tdt, device="cuda")
    dxs = torch.empty((rows, d), dtype=tdt, device="cuda")
    plain = _grads(E, d, h, torch.float32)
    xm.xmoe_expert_ffn_bwd(xs, w1, w3, w2, act, h13, dye, off, dh13, dxs, *plain)
    gen = torch.Generator().manual_seed(rows)
    d0 = _grads(E, d, h, torch.float32, fill=lambda s: torch.randn(s, generator=gen))
    acc = [t.clone() for t in d0]
    xm.xmoe_expert_ffn_bwd(xs, w1, w3, w2, act, h13, dye, off, dh13, dxs, *acc, accumulate_dw=True)
    split = [t.clone() for t in d0]
    xm.xmoe_expert_ffn_bwd_dw13(xs, dh13, off, split[0], split[1], accumulate=True)
    xm.xmoe_expert_ffn_bwd_dw2(act, dye, off, split[2], accumulate=True)
    torch.cuda.synchronize()
    for name, p, z, a, s in zip(("dw1", "dw3", "dw2"), plain, d0, acc, split):
        want = z + p
        assert torch.equal(a, want), name
        assert torch.equal(s, want), name + " (split call)"
    if dtype == "bf16":
        # the gathered dW1/dW3: x itself with identity token ids
        ids = torch.arange(rows, dtype=torch.int32, device="cuda")
        gat = [t.clone() for t in d0[:2]]
        xm.xmoe_expert_ffn_bwd_dw13_gather(xs, ids, dh13, off, gat[0], gat[1], accumulate=True)
        torch.cuda.synchronize()
        assert torch.equal(gat[0], d0[0] + plain[0]) and torch.equal(gat[1], d0[1] + plain[1])
    # a second accumulation adds the same sums again
    xm.xmoe_expert_ffn_bwd(xs, w1, w3, w2, act, h13, dye, off, dh13, dxs, *acc, accumulate_dw=True)
    torch.cuda.synchronize()
    for name, p, z, a in zip(("dw1", "dw3", "dw2"), plain, d0, acc):
        assert torch.equal(a, (z + p) + p), name + " (second call)"


@pytest.mark.parametrize("dtype,rows,d,h,E,empty", CASES[:2] + CASES[3:])
def test_accumulated_dxs_and_expert_output(xm, dtype, rows, d, h, E, empty):
    """accumulate_dxs / accumulate: dxs += ..., ye += ... (the sum rounded once).
    Adding into zeros is bitwise the plain call; adding into a random start
    meets the tolerance against start + the oracle's values."""
    off, xs, w1, w3, w2, dye, re_ = _inputs(dtype, rows, d, h, E, empty, seed=rows + 5 * h)
    act, h13 = _forward(xm, xs, w1, w3, w2, off)
    tdt = DT[dtype]
    dh13 = torch.empty((rows, 2 * h), dtype=tdt, device="cuda")
    g = _grads(E, d, h, tdt if dtype == "f32" else torch.bfloat16)
    dxs = torch.empty((rows, d), dtype=tdt, device="cuda")
    xm.xmoe_expert_ffn_bwd(xs, w1, w3, w2, act, h13, dye, off, dh13, dxs, *g)
    z = torch.zeros_like(dxs)
    xm.xmoe_expert_ffn_bwd(xs, w1, w3, w2, act, h13, dye, off, dh13, z, *g, accumulate_dxs=True)
    start = workloads.random_rows(rows, d, dtype, seed=rows + 9).cuda()
    sx = start.clone()
    xm.xmoe_expert_ffn_bwd_dx(dh13, w1, w3, off, sx, accumulate=True)
    ye = torch.empty((rows, d), dtype=tdt, device="cuda")
    xm.xmoe_expert_ffn_down(act, w2, off, ye)
    yz = torch.zeros_like(ye)
    xm.xmoe_expert_ffn_down(act, w2, off, yz, accumulate=True)
    sy = start.clone()
    xm.xmoe_expert_ffn(xs, w1, w3, w2, off, torch.empty_like(act), sy, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(z, dxs) and torch.equal(yz, ye)
    ref = orc.ffn_bwd(orc_in(xs), re_, orc_in(w1), orc_in(w3), orc_in(w2), orc_in(dye), want_dh=True)
    fwd = orc.ffn(orc_in(xs), re_, orc_in(w1), orc_in(w3), orc_in(w2))
    rt = RTOL[dtype]
    s = host(start)
    assert_close(host(sx), s + ref["dxs"], rt, "dxs += ", floor=np.sqrt(np.mean(ref["dxs"] ** 2)) + np.abs(s))
    assert_close(host(sy), s + fwd["ye"], rt, "ye += ", floor=np.sqrt(np.mean(fwd["ye"] ** 2)) + np.abs(s))


def test_two_shared_experts_as_two_calls(xm):
    """Shared experts one call each, the second adding into the first's output
    (the shared experts' forward through the expert FFN with E = 1, offsets
    {0, T}): equals the oracle's sum of the two dense FFNs; and the backward
    the same way, the second call adding into dx."""
    T, d, hs = 300, 256, 136
    x = workloads.random_rows(T, d, "bf16", seed=1).cuda()
    g = torch.Generator().manual_seed(2)
    ws = [((torch.randn((1, d, hs), generator=g) / d ** 0.5).to(torch.bfloat16).cuda(),
           (torch.randn((1, d, hs), generator=g) / d ** 0.5).to(torch.bfloat16).cuda(),
           (torch.randn((1, hs, d), generator=g) / hs ** 0.5).to(torch.bfloat16).cuda()) for _ in range(2)]
    off = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    y = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    acts, h13s = [], []
    for i, (a, b, c) in enumerate(ws):
        acts.append(torch.empty((T, hs), dtype=torch.bfloat16, device="cuda"))
        h13s.append(torch.empty((T, 2 * hs), dtype=torch.bfloat16, device="cuda"))
        xm.xmoe_expert_ffn(x, a, b, c, off, acts[i], y, h13=h13s[i], accumulate=i > 0)
    dy = workloads.random_rows(T, d, "bf16", seed=3).cuda()
    dx = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    for i, (a, b, c) in enumerate(ws):
        gr = [torch.empty_like(a), torch.empty_like(b), torch.empty_like(c)]
        xm.xmoe_expert_ffn_bwd(x, a, b, c, acts[i], h13s[i], dy, off,
                               torch.empty((T, 2 * hs), dtype=torch.bfloat16, device="cuda"), dx, *gr,
                               accumulate_dxs=i > 0)
    torch.cuda.synchronize()
    z = np.zeros(T, np.int32)
    want_y = np.zeros((T, d))
    want_dx = np.zeros((T, d))
    for a, b, c in ws:
        want_y += orc.ffn(orc_in(x), z, orc_in(a), orc_in(b), orc_in(c))["ye"]
        want_dx += orc.ffn_bwd(orc_in(x), z, orc_in(a), orc_in(b), orc_in(c), orc_in(dy))["dxs"]
    assert_close(host(y), want_y, RTOL["bf16"], "y")
    assert_close(host(dx), want_dx, RTOL["bf16"], "dx")
