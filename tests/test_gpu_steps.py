"""Per-step GPU parity: each libxmoe entry point against the CPU oracle on the
same seeded generator inputs (never on another GPU step's output).

Integer work (routing indices, the Padding-Free Token buffer, the dispatch copy)
must match bit for bit; floating-point outputs must meet the tolerance of
_helpers.assert_close.
"""
import numpy as np
import pytest
import torch

import oracle as orc
import workloads
from _helpers import (RTOL, assert_close, assert_wgrad_close, host, need_gpu, orc_in, routing_check, rss_rows,
                      swiglu_wgrad_scales, wgrad_acc)

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def xm():
    need_gpu()
    import padding_free_expert_amd as m
    assert m.xmoe_query_device(0), "device 0 is not gfx950"
    return m


def _gpu_pft(xm, ids, w, E):
    T, k = ids.shape
    pft = xm.PFT(T, E, k)
    ws = torch.empty(max(xm.xmoe_build_pft_workspace_size(T, E, k), 16), dtype=torch.uint8, device="cuda")
    xm.xmoe_build_pft(ids.cuda(), w.cuda(), E, pft, ws)
    torch.cuda.synchronize()
    return pft


# ------------------------------------------------------------------ routing

def test_router_fp32_is_bit_exact(xm):
    """fp32 path: one fused multiply-add per feature in ascending order on both
    sides -> identical logits and identical selections, tie-break included."""
    wl = workloads.get("tiny_f32")
    inp = workloads.generate(wl, experts=False)
    x, wg = inp["x"], inp["wg"]
    T, E, k = wl.T, wl.E, wl.k
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    xm.xmoe_route(x.cuda(), wg.cuda(), k, ids, w, lg)
    r = orc.route(orc_in(x), orc_in(wg), k, 0)
    np.testing.assert_array_equal(host(lg), r["scores"])
    np.testing.assert_array_equal(host(ids), r["topk_ids"])
    assert_close(host(w), r["topk_w"], 1e-5, "topk_w")


@pytest.mark.parametrize("dtype,T,d,E,k", [("f32", 300, 64, 16, 4), ("bf16", 300, 64, 16, 4),
                                          ("bf16", 77, 264, 64, 8), ("bf16", 33, 2048, 56, 6),
                                          ("bf16", 129, 1032, 200, 8)])
def test_router_exact_grid_ties(xm, dtype, T, d, E, k):
    """Inputs on a coarse binary grid: every logit is exact in any summation
    order, so the matrix-core path must match bit for bit, ties included.  The
    bf16 shapes cover the fused kernel (up to 64 experts: a partial last
    token block, d ending 8 past a 32-deep k block, more waves than k blocks,
    fewer experts than its 64-wide column block) and the split-d path (200
    experts)."""
    x, wg = workloads.exact_router_inputs(T, d, E, seed=5)
    x, wg = x.to(DT[dtype]), wg.to(DT[dtype])
    sb = torch.zeros(E)
    sb[3] = 0.25
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    xm.xmoe_route(x.cuda(), wg.cuda(), k, ids, w, lg, 2.0, None, sb.cuda())
    r = orc.route(orc_in(x), orc_in(wg), k, 1, 2.0, None, sb.numpy())
    np.testing.assert_array_equal(host(lg), r["scores"])
    np.testing.assert_array_equal(host(ids), r["topk_ids"])
    assert_close(host(w), r["topk_w"], 1e-5, "topk_w")


@pytest.mark.parametrize("name", ["dsmoe16b", "dsv3", "zipf_skew", "long_batch"])
def test_router_bf16_small(xm, name):
    wl = workloads.small(name)
    inp = workloads.generate(wl, experts=False, backward=False)
    T, E, k = wl.T, wl.E, wl.k
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    lb, sb = inp["logit_bias"], inp["select_bias"]
    xm.xmoe_route(inp["x"].cuda(), inp["wg"].cuda(), k, ids, w, lg, wl.inv_tau,
                  None if lb is None else lb.cuda(), None if sb is None else sb.cuda())
    r = orc.route(orc_in(inp["x"]), orc_in(inp["wg"]), k, 1, wl.inv_tau,
                  None if lb is None else lb.numpy(), None if sb is None else sb.numpy())
    mism = routing_check(host(ids), host(lg), r, None if sb is None else sb.numpy(), k, 1e-5)
    keep = ~mism
    ok = (host(ids) == r["topk_ids"]).all(axis=1) & keep
    assert_close(host(w)[ok], r["topk_w"][ok], 1e-4, "topk_w")


def _random_routers(n: int, seed: int):
    """Seeded routing shapes: bf16 with d and E multiples of 8 (the fused
    kernel up to 64 experts, the split product above), fp32 with any d and E,
    up to 1024 experts and k up to 64 or k = E."""
    rs = np.random.RandomState(seed)
    out = []
    for i in range(n):
        dt = "f32" if i % 3 == 2 else "bf16"
        E = 8 * int(rs.randint(1, 129)) if dt == "bf16" else int(rs.randint(1, 1025))
        k = E if rs.rand() < 0.1 and E <= 128 else int(rs.randint(1, min(E, 64) + 1))
        T = int(rs.choice([1, 5, 64, 300, 1031, 4097]))
        d = 8 * int(rs.randint(1, 513)) if dt == "bf16" else int(rs.randint(1, 600))
        out.append((dt, T, d, E, k))
    return out


RANDOM_ROUTERS = _random_routers(12, 9)


@pytest.mark.parametrize("dtype,T,d,E,k", [("bf16", 300, 256, 384, 16), ("bf16", 130, 128, 1024, 8),
                                          ("f32", 257, 64, 10, 3), ("f32", 100, 32, 300, 5),
                                          ("f32", 64, 16, 1021, 4), ("f32", 33, 8, 1, 1),
                                          ("bf16", 1, 2048, 160, 8), ("bf16", 7, 7168, 256, 8),
                                          ("bf16", 1, 2048, 64, 6), ("bf16", 33, 264, 8, 2),
                                          ("bf16", 4097, 2048, 64, 6), ("bf16", 257, 7168, 128, 8),
                                          ("bf16", 100, 512, 72, 8), ("bf16", 65, 136, 120, 4),
                                          ("bf16", 300, 7168, 48, 6), ("bf16", 50, 8, 16, 4),
                                          ("bf16", 40, 24, 64, 64)] + RANDOM_ROUTERS)
def test_router_expert_counts(xm, dtype, T, d, E, k):
    """Expert counts beyond the workloads': more than 256 experts (16 and 32
    lanes per token in the top-k), fp32 counts that are not a multiple of 4
    (element loads instead of 16-byte vectors), a single expert; and a few
    tokens, where the logits' d reduction is split into the most parts.  bf16
    with up to 64 experts runs the fused kernel: expert counts below its
    64-wide column block, one token, ragged token blocks, a d tail of 8, d =
    7168, d = 8 (one k block, seven idle waves), k = E = 64; 72-128 experts
    the split-d path.  fp32 logits are
    bit-exact, so its selections must match outright; bf16 through routing_check."""
    x = workloads.random_rows(T, d, dtype, seed=E)
    wg = workloads.random_rows(d, E, dtype, seed=E + 1, std=d ** -0.5)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    xm.xmoe_route(x.cuda(), wg.cuda(), k, ids, w, lg)
    r = orc.route(orc_in(x), orc_in(wg), k, 0 if dtype == "f32" else 1)
    if dtype == "f32":
        np.testing.assert_array_equal(host(lg), r["scores"])
        np.testing.assert_array_equal(host(ids), r["topk_ids"])
        assert_close(host(w), r["topk_w"], 1e-5, "topk_w")
        return
    mism = routing_check(host(ids), host(lg), r, None, k, 1e-5)
    ok = (host(ids) == r["topk_ids"]).all(axis=1) & ~mism
    assert ok.sum() >= 0.9 * T
    assert_close(host(w)[ok], r["topk_w"][ok], 1e-4, "topk_w")


# ------------------------------------------------------------------ PFT

def _random_pfts(n: int, seed: int):
    """Seeded buffer shapes: up to 40000 tokens, 1-1024 experts, k up to 32."""
    rs = np.random.RandomState(seed)
    out = []
    for _ in range(n):
        E = int(rs.randint(1, 1025))
        out.append((int(rs.choice([1, 2, 63, 500, 4097, 40000])), E, int(rs.randint(1, min(E, 32) + 1)),
                    float(rs.choice([0.0, 1.0, 2.5]))))
    return out


RANDOM_PFTS = _random_pfts(10, 10)


@pytest.mark.parametrize("T,E,k,skew", [(1, 8, 2, 0.0), (255, 8, 2, 0.0), (256, 64, 6, 0.0), (257, 64, 6, 0.0),
                                        (1000, 128, 8, 2.5), (3000, 160, 8, 0.0), (700, 1024, 16, 1.0),
                                        (64, 8, 8, 0.0), (32768, 160, 8, 0.0), (16384, 128, 8, 3.0)]
                         + RANDOM_PFTS)
def test_build_pft_bit_exact(xm, T, E, k, skew):
    ids, w = workloads.random_topk(T, E, k, seed=T * 7 + E, skew=skew)
    pft = _gpu_pft(xm, ids, w, E)
    ref = orc.build_pft(ids.numpy(), w.numpy(), E)
    for key, t in pft.fields().items():
        got = t.cpu().numpy()
        if key == "combine_weights":
            np.testing.assert_array_equal(got.view(np.uint32), ref[key].view(np.uint32), err_msg=key)
        else:
            np.testing.assert_array_equal(got, ref[key], err_msg=key)


@pytest.mark.parametrize("T,E,k,ns,seed", [(300, 16, 6, 2, 0), (1, 8, 2, 1, 1), (4096, 64, 6, 2, 2), (777, 32, 4, 3, 3)])
def test_build_pft_shared_bit_exact(xm, T, E, k, ns, seed):
    """Shared experts as always-routed ones: the buffer equals the oracle's
    buffer of the routing with the n shared experts appended to every token."""
    ids, w = workloads.random_topk(T, E, k, seed=seed)
    pft = xm.PFT(T, E + ns, k + ns)
    ws = torch.empty(max(xm.xmoe_build_pft_workspace_size(T, E + ns, k + ns), 16), dtype=torch.uint8, device="cuda")
    xm.xmoe_build_pft_shared(ids.cuda(), w.cuda(), E, ns, pft, ws)
    torch.cuda.synchronize()
    ids_b = np.concatenate([ids.numpy(), np.tile(np.arange(E, E + ns, dtype=np.int32), (T, 1))], axis=1)
    w_b = np.concatenate([w.numpy(), np.ones((T, ns), np.float32)], axis=1)
    ref = orc.build_pft(ids_b, w_b, E + ns)
    for key, v in pft.fields().items():
        got = v.cpu().numpy()
        if key == "combine_weights":
            np.testing.assert_array_equal(got.view(np.uint32), ref[key].view(np.uint32), err_msg=key)
        else:
            np.testing.assert_array_equal(got, ref[key], err_msg=key)


def test_build_pft_zero_tokens(xm):
    E, k = 16, 4
    pft = xm.PFT(0, E, k)
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    ids = torch.empty((0, k), dtype=torch.int32, device="cuda")
    w = torch.empty((0, k), dtype=torch.float32, device="cuda")
    xm.xmoe_build_pft(ids, w, E, pft, ws)
    torch.cuda.synchronize()
    assert (pft.tokens_per_expert.cpu() == 0).all() and (pft.expert_offsets.cpu() == 0).all()


# ------------------------------------------------------------------ dispatch / combine

# Rows of fewer 16-byte vectors than slots per token (d / 8 < k in bf16,
# d / 4 < k in fp32), more than 64 slots, and a last pass over the row that
# leaves lanes idle while slots beyond them remain: each lane holds one slot's
# row index, which the others read by shuffle.
NARROW = [("bf16", 1031, 40, 56, 7), ("f32", 100, 16, 8, 6), ("bf16", 5, 16, 128, 100), ("bf16", 20, 2400, 64, 60)]


@pytest.mark.parametrize("dtype,T,d,E,k", [("bf16", 300, 256, 16, 6), ("f32", 256, 128, 8, 2),
                                           ("bf16", 1, 2048, 64, 6), ("bf16", 4096, 7168, 256, 8)] + NARROW)
def test_dispatch_exact(xm, dtype, T, d, E, k):
    ids, w = workloads.random_topk(T, E, k, seed=3)
    x = workloads.random_rows(T, d, dtype, seed=4)
    pft = _gpu_pft(xm, ids, w, E)
    xs = torch.empty((T * k, d), dtype=DT[dtype], device="cuda")
    xm.xmoe_dispatch(x.cuda(), k, pft, xs)
    ref = orc.build_pft(ids.numpy(), w.numpy(), E)
    got = xs.cpu()
    want = orc.gather(orc_in(x), ref["token_ids"])
    np.testing.assert_array_equal(got.to(torch.float64).numpy(), want)


@pytest.mark.parametrize("dtype,T,d,E,k,with_add", [("bf16", 300, 256, 16, 6, True), ("f32", 256, 128, 8, 2, False),
                                                    ("bf16", 777, 520, 40, 8, False), ("bf16", 2, 64, 8, 8, True)]
                         + [c + (i % 2 == 0,) for i, c in enumerate(NARROW)])
def test_combine(xm, dtype, T, d, E, k, with_add):
    ids, w = workloads.random_topk(T, E, k, seed=11)
    pft = _gpu_pft(xm, ids, w, E)
    ye = workloads.random_rows(T * k, d, dtype, seed=12)
    add = workloads.random_rows(T, d, dtype, seed=13) if with_add else None
    y = torch.empty((T, d), dtype=DT[dtype], device="cuda")
    xm.xmoe_combine(ye.cuda(), pft, T, y, y_add=None if add is None else add.cuda())
    ref = orc.build_pft(ids.numpy(), w.numpy(), E)
    want = orc.combine(host(ye), ref["token_ids"], ref["combine_weights"].astype(np.float64), T,
                       y_add=None if add is None else orc_in(add))
    assert_close(host(y), want, RTOL[dtype] if dtype == "bf16" else 1e-5, "y")


@pytest.mark.parametrize("dtype,T,d,E,k", [("bf16", 300, 256, 16, 6), ("f32", 256, 128, 8, 2), ("bf16", 513, 2048, 64, 6)]
                         + NARROW)
def test_combine_bwd(xm, dtype, T, d, E, k):
    ids, w = workloads.random_topk(T, E, k, seed=21)
    pft = _gpu_pft(xm, ids, w, E)
    ye = workloads.random_rows(T * k, d, dtype, seed=22)
    dy = workloads.random_rows(T, d, dtype, seed=23)
    dye = torch.empty((T * k, d), dtype=DT[dtype], device="cuda")
    dtw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    xm.xmoe_combine_bwd(dy.cuda(), ye.cuda(), pft, dye, dtw)
    ref = orc.build_pft(ids.numpy(), w.numpy(), E)
    g = orc.combine_bwd(orc_in(dy), host(ye), ref["token_ids"], ref["combine_weights"].astype(np.float64))
    assert_close(host(dye), g["dye"], RTOL[dtype] if dtype == "bf16" else 1e-6, "dye")
    dw_slot = g["dw"][ref["slot_to_row"]].reshape(T, k)
    assert_close(host(dtw), dw_slot, 1e-4, "dtopk_w")


@pytest.mark.parametrize("dtype,T,d,E,k,with_add", [("bf16", 300, 256, 16, 6, True), ("f32", 256, 128, 8, 2, True),
                                                    ("bf16", 1000, 1024, 128, 8, False)]
                         + [c + (i % 2 == 1,) for i, c in enumerate(NARROW)])
def test_dispatch_bwd(xm, dtype, T, d, E, k, with_add):
    ids, w = workloads.random_topk(T, E, k, seed=31)
    pft = _gpu_pft(xm, ids, w, E)
    dxs = workloads.random_rows(T * k, d, dtype, seed=32)
    add = workloads.random_rows(T, d, dtype, seed=33) if with_add else None
    dx = torch.empty((T, d), dtype=DT[dtype], device="cuda")
    xm.xmoe_dispatch_bwd(dxs.cuda(), pft, T, dx, dx_add=None if add is None else add.cuda())
    ref = orc.build_pft(ids.numpy(), w.numpy(), E)
    want = orc.scatter_add(orc_in(dxs), ref["token_ids"], T, dx_add=None if add is None else orc_in(add))
    assert_close(host(dx), want, RTOL[dtype] if dtype == "bf16" else 1e-6, "dx")


# ------------------------------------------------------------------ expert FFN

FFN_CASES = [
    # dtype, rows, d, h, E, empty_frac
    ("f32", 512, 128, 64, 8, 0.0),
    ("f32", 301, 64, 40, 5, 0.4),
    ("bf16", 700, 256, 200, 16, 0.25),
    ("bf16", 1030, 448, 136, 32, 0.5),
    ("bf16", 129, 128, 128, 1, 0.0),
    ("bf16", 3000, 512, 384, 4, 0.0),
    # d and h off every tile multiple: partial k blocks in all six products,
    # partial m/n tiles in the weight gradients
    ("bf16", 517, 328, 264, 7, 0.3),
    # every row on expert 0, seven empty experts; the mean of 1500 rows per
    # expert selects the 256-row tiles
    ("bf16", 12000, 256, 192, 8, 1.0),
]


def _random_ffn_cases(n: int, seed: int):
    """Seeded expert-FFN shapes: widths that are multiples of 8 down to 8 and
    rarely of a tile, 1-64 experts with empty and ragged segments, and up to
    5000 rows (the 256-row tiles from 1024 rows per expert).  A cap on
    rows*d*h keeps the fp64 oracle to seconds."""
    rs = np.random.RandomState(seed)
    out = []
    while len(out) < n:
        dt = "f32" if len(out) % 4 == 3 else "bf16"
        E = int(rs.choice([1, 2, 3, 5, 8, 13, 32, 64]))
        rows = int(rs.choice([1, 5, 64, 129, 300, 1000, 2500, 5000]))
        d, h = 8 * int(rs.randint(1, 129)), 8 * int(rs.randint(1, 129))
        empty = float(rs.choice([0.0, 0.3, 0.7]))
        if rows * d * h > (5e8 if dt == "bf16" else 1.5e8):
            continue
        out.append((dt, rows, d, h, E, empty))
    return out


FFN_CASES += _random_ffn_cases(16, 7)


def _ffn_inputs(dtype, rows, d, h, E, empty, seed):
    off = workloads.random_segments(rows, E, seed=seed, empty_frac=empty)
    xs = workloads.random_rows(rows, d, dtype, seed=seed + 1)
    g = torch.Generator().manual_seed(seed)
    tdt = DT[dtype]
    w1 = (torch.randn((E, d, h), generator=g) / d ** 0.5).to(tdt)
    w3 = (torch.randn((E, d, h), generator=g) / d ** 0.5).to(tdt)
    w2 = (torch.randn((E, h, d), generator=g) / h ** 0.5).to(tdt)
    re_ = np.repeat(np.arange(E, dtype=np.int32), np.diff(off.numpy()))
    return off, xs, w1, w3, w2, re_


@pytest.mark.parametrize("dtype,rows,d,h,E,empty", FFN_CASES)
def test_expert_ffn_forward(xm, dtype, rows, d, h, E, empty):
    off, xs, w1, w3, w2, re_ = _ffn_inputs(dtype, rows, d, h, E, empty, seed=rows + d)
    tdt = DT[dtype]
    act = torch.empty((rows, h), dtype=tdt, device="cuda")
    h13 = torch.empty((rows, 2 * h), dtype=tdt, device="cuda")
    ye = torch.empty((rows, d), dtype=tdt, device="cuda")
    xm.xmoe_expert_ffn(xs.cuda(), w1.cuda(), w3.cuda(), w2.cuda(), off.cuda(), act, ye, h13=h13)
    ref = orc.ffn(orc_in(xs), re_, orc_in(w1), orc_in(w3), orc_in(w2), want_hidden=True)
    rt = RTOL[dtype]
    hh = host(h13)
    assert_close(hh[:, :h], ref["h1"], rt, "h1")
    assert_close(hh[:, h:], ref["h3"], rt, "h3")
    assert_close(host(act), ref["act"], rt, "act")
    assert_close(host(ye), ref["ye"], rt, "ye")


def test_expert_ffn_bwd_split_calls_match_composite(xm):
    """The four backward products called one by one (as a caller running the
    weight gradients on another stream does) give bitwise the composite call's
    results."""
    dtype, rows, d, h, E, empty = "bf16", 517, 328, 264, 7, 0.3
    off, xs, w1, w3, w2, _ = _ffn_inputs(dtype, rows, d, h, E, empty, seed=11)
    c = lambda t: t.cuda()
    tdt = DT[dtype]
    act = torch.empty((rows, h), dtype=tdt, device="cuda")
    h13 = torch.empty((rows, 2 * h), dtype=tdt, device="cuda")
    ye = torch.empty((rows, d), dtype=tdt, device="cuda")
    xm.xmoe_expert_ffn(c(xs), c(w1), c(w3), c(w2), c(off), act, ye, h13=h13)
    dye = c(workloads.random_rows(rows, d, dtype, seed=12))
    bufs = lambda: (torch.empty((rows, 2 * h), dtype=tdt, device="cuda"), torch.empty((rows, d), dtype=tdt, device="cuda"),
                    torch.empty((E, d, h), dtype=tdt, device="cuda"), torch.empty((E, d, h), dtype=tdt, device="cuda"),
                    torch.empty((E, h, d), dtype=tdt, device="cuda"))
    a = bufs()
    xm.xmoe_expert_ffn_bwd(c(xs), c(w1), c(w3), c(w2), act, h13, dye, c(off), *a)
    b = bufs()
    xm.xmoe_expert_ffn_bwd_dw2(act, dye, c(off), b[4])
    xm.xmoe_expert_ffn_bwd_dact(dye, c(w2), h13, c(off), b[0])
    xm.xmoe_expert_ffn_bwd_dw13(c(xs), b[0], c(off), b[2], b[3])
    xm.xmoe_expert_ffn_bwd_dx(b[0], c(w1), c(w3), c(off), b[1])
    for name, u, v in zip(["dh13", "dxs", "dw1", "dw3", "dw2"], a, b):
        assert torch.equal(u, v), name


GATHER_CASES = [
    ("f32", 97, 64, 40, 5, 2, 0.0),
    ("bf16", 300, 256, 200, 16, 6, 1.5),   # skewed: some experts empty
    ("bf16", 517, 328, 264, 7, 3, 0.7),    # d and h off every tile multiple
    ("bf16", 129, 128, 128, 1, 1, 0.0),
    ("bf16", 400, 192, 512, 8, 4, 0.8),    # h a multiple of 256 below 1024 rows per expert
]


def _random_gather_cases(n: int, seed: int):
    """Seeded shapes for the products that read rows through the PFT: as the
    FFN cases above, with tokens, slots per token and a routing skew."""
    rs = np.random.RandomState(seed)
    out = []
    while len(out) < n:
        dt = "f32" if len(out) % 4 == 3 else "bf16"
        E = int(rs.choice([1, 4, 8, 16, 40, 64, 128]))
        k = int(rs.randint(1, min(E, 8) + 1))
        T = int(rs.choice([1, 3, 50, 300, 777, 1500]))
        d, h = 8 * int(rs.randint(1, 129)), 8 * int(rs.randint(1, 129))
        skew = float(rs.choice([0.0, 0.7, 1.5]))
        if T * k * d * h > (5e8 if dt == "bf16" else 1.5e8):
            continue
        out.append((dt, T, d, h, E, k, skew))
    return out


GATHER_CASES += _random_gather_cases(12, 8)


@pytest.mark.parametrize("dtype,T,d,h,E,k,skew", GATHER_CASES)
def test_expert_ffn_gather(xm, dtype, T, d, h, E, k, skew):
    """The FFN with the dispatch gather fused into the up-projection's loads,
    on expert-sorted rows built by the oracle's PFT, against the oracle's FFN
    over the same token-to-row map."""
    ids, w = workloads.random_topk(T, E, k, seed=T + d, skew=skew)
    ref_pft = orc.build_pft(ids.numpy(), w.numpy(), E)
    tok, off = ref_pft["token_ids"], ref_pft["expert_offsets"]
    R = T * k
    row_expert = np.repeat(np.arange(E, dtype=np.int32), np.diff(off))
    x = workloads.random_rows(T, d, dtype, seed=T + 7)
    g = torch.Generator().manual_seed(T + d)
    tdt = DT[dtype]
    w1 = (torch.randn((E, d, h), generator=g) / d ** 0.5).to(tdt)
    w3 = (torch.randn((E, d, h), generator=g) / d ** 0.5).to(tdt)
    w2 = (torch.randn((E, h, d), generator=g) / h ** 0.5).to(tdt)
    c = lambda t: t.cuda()
    tok_d, off_d = torch.from_numpy(tok).cuda(), torch.from_numpy(off).cuda()
    act = torch.empty((R, h), dtype=tdt, device="cuda")
    h13 = torch.empty((R, 2 * h), dtype=tdt, device="cuda")
    ye = torch.empty((R, d), dtype=tdt, device="cuda")
    xm.xmoe_expert_ffn_gather(c(x), tok_d, c(w1), c(w3), c(w2), off_d, act, ye, h13=h13)
    ref = orc.ffn(orc_in(x), row_expert, orc_in(w1), orc_in(w3), orc_in(w2), row_token=tok, want_hidden=True)
    rt = RTOL[dtype]
    hh = host(h13)
    assert_close(hh[:, :h], ref["h1"], rt, "h1")
    assert_close(hh[:, h:], ref["h3"], rt, "h3")
    assert_close(host(act), ref["act"], rt, "act")
    assert_close(host(ye), ref["ye"], rt, "ye")
    # consistency with the materialised path (same arithmetic, so bitwise)
    xs = c(x)[tok_d.long()].contiguous()
    act2, h132, ye2 = torch.empty_like(act), torch.empty_like(h13), torch.empty_like(ye)
    xm.xmoe_expert_ffn(xs, c(w1), c(w3), c(w2), off_d, act2, ye2, h13=h132)
    assert torch.equal(act, act2) and torch.equal(h13, h132) and torch.equal(ye, ye2)
    # up-projection alone, without the saved pre-activations
    act3 = torch.empty_like(act)
    xm.xmoe_expert_ffn_up_gather(c(x), tok_d, c(w1), c(w3), off_d, act3)
    assert torch.equal(act3, act)
    # and the pre-activations alone (no act), gathered and over xs
    h13b, h13c = torch.full_like(h13, float("nan")), torch.full_like(h13, float("nan"))
    xm.xmoe_expert_ffn_up_gather(c(x), tok_d, c(w1), c(w3), off_d, None, h13b)
    xm.xmoe_expert_ffn_up(xs, c(w1), c(w3), off_d, None, h13c)
    torch.cuda.synchronize()
    assert torch.equal(h13b, h13) and torch.equal(h13c, h13)


# the gathered weight gradient: ragged and empty experts, d and h off the
# 128-wide tiles, and more than 1024 rows per expert (the three-slot ring)
DW13_GATHER_CASES = GATHER_CASES + [
    ("bf16", 2600, 192, 136, 4, 2, 0.5),
    ("bf16", 1100, 256, 128, 1, 1, 0.0),
]


@pytest.mark.parametrize("dtype,T,d,h,E,k,skew", DW13_GATHER_CASES)
def test_expert_ffn_bwd_dw13_gather(xm, dtype, T, d, h, E, k, skew):
    """dW1/dW3 with the dispatch gather fused into the loads of x: against the
    oracle's expert backward over the same token-to-row map, and bitwise
    against the same product over the materialised rows x[token_ids]."""
    ids, w = workloads.random_topk(T, E, k, seed=T + 3 * d, skew=skew)
    ref_pft = orc.build_pft(ids.numpy(), w.numpy(), E)
    tok, off = ref_pft["token_ids"], ref_pft["expert_offsets"]
    R = T * k
    row_expert = np.repeat(np.arange(E, dtype=np.int32), np.diff(off))
    x = workloads.random_rows(T, d, dtype, seed=T + 11)
    dye = workloads.random_rows(R, d, dtype, seed=T + 12)
    g = torch.Generator().manual_seed(T + h)
    tdt = DT[dtype]
    w1 = (torch.randn((E, d, h), generator=g) / d ** 0.5).to(tdt)
    w3 = (torch.randn((E, d, h), generator=g) / d ** 0.5).to(tdt)
    w2 = (torch.randn((E, h, d), generator=g) / h ** 0.5).to(tdt)
    c = lambda t: t.cuda()
    tok_d, off_d = torch.from_numpy(tok).cuda(), torch.from_numpy(off).cuda()
    act = torch.empty((R, h), dtype=tdt, device="cuda")
    h13 = torch.empty((R, 2 * h), dtype=tdt, device="cuda")
    ye = torch.empty((R, d), dtype=tdt, device="cuda")
    xm.xmoe_expert_ffn_gather(c(x), tok_d, c(w1), c(w3), c(w2), off_d, act, ye, h13=h13)
    dh13 = torch.empty((R, 2 * h), dtype=tdt, device="cuda")
    xm.xmoe_expert_ffn_bwd_dact(c(dye), c(w2), h13, off_d, dh13)
    dw1 = torch.full((E, d, h), float("nan"), dtype=tdt, device="cuda")   # must be fully overwritten
    dw3 = torch.full((E, d, h), float("nan"), dtype=tdt, device="cuda")
    xm.xmoe_expert_ffn_bwd_dw13_gather(c(x), tok_d, dh13, off_d, dw1, dw3)
    # the materialised path: same products on the same values, so bitwise
    xs = c(x)[tok_d.long()].contiguous()
    dw1m, dw3m = torch.empty_like(dw1), torch.empty_like(dw3)
    xm.xmoe_expert_ffn_bwd_dw13(xs, dh13, off_d, dw1m, dw3m)
    torch.cuda.synchronize()
    assert torch.equal(dw1, dw1m) and torch.equal(dw3, dw3m)
    # the oracle over the token-to-row map
    X = host(x)
    ref = orc.ffn_bwd(orc_in(x), row_expert, orc_in(w1), orc_in(w3), orc_in(w2), orc_in(dye), row_token=tok,
                      want_dh=True)
    fwd = orc.ffn(orc_in(x), row_expert, orc_in(w1), orc_in(w3), orc_in(w2), row_token=tok, want_hidden=True)
    Xr, G = X[tok], host(dye)
    scales = {}

    def floors(e):
        if e not in scales:
            sl = slice(off[e], off[e + 1])
            scales[e] = swiglu_wgrad_scales(Xr[sl], ref["da"][sl], fwd["h1"][sl], fwd["h3"][sl], fwd["act"][sl],
                                            G[sl], host(w2[e]), (host(w1[e]), host(w3[e])), wgrad_acc(dtype, d))
        return scales[e]

    rows = lambda e: off[e + 1] - off[e]
    rt = RTOL[dtype]
    assert_wgrad_close(host(dw1), ref["dw1"], rows, lambda e: floors(e)[0], rt, "dw1")
    assert_wgrad_close(host(dw3), ref["dw3"], rows, lambda e: floors(e)[1], rt, "dw3")


# the gathered dA: the gather cases plus 1300 rows per expert
DACT_GATHER_CASES = GATHER_CASES + [("bf16", 2600, 192, 136, 4, 2, 0.5)]


@pytest.mark.parametrize("dtype,T,d,h,E,k,skew", DACT_GATHER_CASES)
def test_expert_ffn_bwd_dact_gather(xm, dtype, T, d, h, E, k, skew):
    """dA straight from the upstream gradient: row r reads dy[token_ids[r]] and
    its product is scaled by the row's combine weight before the SwiGLU
    backward.  Against the oracle's combine backward (dye = w * dy[token],
    unrounded) followed by its expert backward, and against the two-call GPU
    path, which rounds dye to the input dtype first."""
    ids, w = workloads.random_topk(T, E, k, seed=T + 5 * d, skew=skew)
    ref_pft = orc.build_pft(ids.numpy(), w.numpy(), E)
    tok, off, cw = ref_pft["token_ids"], ref_pft["expert_offsets"], ref_pft["combine_weights"]
    R = T * k
    row_expert = np.repeat(np.arange(E, dtype=np.int32), np.diff(off))
    x = workloads.random_rows(T, d, dtype, seed=T + 21)
    dy = workloads.random_rows(T, d, dtype, seed=T + 22)
    g = torch.Generator().manual_seed(T + 2 * h)
    tdt = DT[dtype]
    w1 = (torch.randn((E, d, h), generator=g) / d ** 0.5).to(tdt)
    w3 = (torch.randn((E, d, h), generator=g) / d ** 0.5).to(tdt)
    w2 = (torch.randn((E, h, d), generator=g) / h ** 0.5).to(tdt)
    c = lambda t: t.cuda()
    tok_d, off_d = torch.from_numpy(tok).cuda(), torch.from_numpy(off).cuda()
    cw_d = torch.from_numpy(cw.astype(np.float32)).cuda()
    act = torch.empty((R, h), dtype=tdt, device="cuda")
    h13 = torch.empty((R, 2 * h), dtype=tdt, device="cuda")
    xm.xmoe_expert_ffn_up_gather(c(x), tok_d, c(w1), c(w3), off_d, act, h13)
    dh13 = torch.full((R, 2 * h), float("nan"), dtype=tdt, device="cuda")   # must be fully overwritten
    xm.xmoe_expert_ffn_bwd_dact_gather(c(dy), tok_d, cw_d, c(w2), h13, off_d, dh13)
    # the oracle: the combine backward's dye (not rounded), then the expert backward
    fwd = orc.ffn(orc_in(x), row_expert, orc_in(w1), orc_in(w3), orc_in(w2), row_token=tok, want_hidden=True)
    dye = orc.combine_bwd(orc_in(dy), fwd["ye"], tok, cw)["dye"]
    ref = orc.ffn_bwd(orc_in(x), row_expert, orc_in(w1), orc_in(w3), orc_in(w2), dye, row_token=tok,
                      want_dh=True, want_dw=False)
    rt = RTOL[dtype]
    got = host(dh13)
    assert_close(got[:, :h], ref["dh1"], rt, "dh1")
    assert_close(got[:, h:], ref["dh3"], rt, "dh3")
    # the two-call path: dye = w * dy[token] rounded to the input dtype, then dA
    dye_d = torch.empty((R, d), dtype=tdt, device="cuda")
    dtw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    pft = xm.PFT(T, E, k)
    for name, t in pft.fields().items():
        t.copy_(torch.from_numpy(ref_pft[name]))
    ye = torch.empty((R, d), dtype=tdt, device="cuda")
    xm.xmoe_expert_ffn_down(act, c(w2), off_d, ye)
    xm.xmoe_combine_bwd(c(dy), ye, pft, dye_d, dtw)
    dh13b = torch.empty_like(dh13)
    xm.xmoe_expert_ffn_bwd_dact(dye_d, c(w2), h13, off_d, dh13b)
    torch.cuda.synchronize()
    # the two-call path rounds w * dy to the input dtype before the product,
    # which moves elements where the product cancels by several ulps; the
    # gathered path scales the fp32 product, so it is at least as close
    ref_dh = np.concatenate([ref["dh1"], ref["dh3"]], 1)
    rms = float(np.sqrt(np.mean(ref_dh * ref_dh))) if ref_dh.size else 0.0
    worst = lambda a: float(np.max(np.abs(a - ref_dh) / (np.abs(ref_dh) + rms))) if ref_dh.size else 0.0
    e_new, e_old = worst(got), worst(host(dh13b))
    assert e_new <= 1.05 * e_old + 1e-6, (e_new, e_old)


def test_gathered_reads_outside_x_are_zero(xm):
    """bf16 gathers read x through a bounds-checked buffer: a token id past T
    or negative reads a zero row, in the up-projection and in dW1/dW3 alike
    (bitwise the products over x[token_ids] with those rows zeroed)."""
    T, d, h, E, k = 200, 256, 128, 4, 2
    ids, w = workloads.random_topk(T, E, k, seed=5)
    ref_pft = orc.build_pft(ids.numpy(), w.numpy(), E)
    tok = ref_pft["token_ids"].copy()
    R = T * k
    bad = np.arange(0, R, 17)
    tok[bad] = np.resize(np.array([T, T + 1000, -1, -7], np.int32), bad.size)
    bf = torch.bfloat16
    g = torch.Generator().manual_seed(9)
    x = torch.randn((T, d), generator=g).to(bf).cuda()
    w1 = (torch.randn((E, d, h), generator=g) / d ** 0.5).to(bf).cuda()
    w3 = (torch.randn((E, d, h), generator=g) / d ** 0.5).to(bf).cuda()
    dh13 = torch.randn((R, 2 * h), generator=g).to(bf).cuda()
    tok_d, off_d = torch.from_numpy(tok).cuda(), torch.from_numpy(ref_pft["expert_offsets"]).cuda()
    act, h13 = torch.empty((R, h), dtype=bf, device="cuda"), torch.empty((R, 2 * h), dtype=bf, device="cuda")
    dw1, dw3 = torch.empty((E, d, h), dtype=bf, device="cuda"), torch.empty((E, d, h), dtype=bf, device="cuda")
    xm.xmoe_expert_ffn_up_gather(x, tok_d, w1, w3, off_d, act, h13)
    xm.xmoe_expert_ffn_bwd_dw13_gather(x, tok_d, dh13, off_d, dw1, dw3)
    ok = (tok_d >= 0) & (tok_d < T)
    xs = torch.where(ok[:, None], x[tok_d.clamp(0, T - 1).long()], torch.zeros((), dtype=bf, device="cuda"))
    act2, h132 = torch.empty_like(act), torch.empty_like(h13)
    dw1m, dw3m = torch.empty_like(dw1), torch.empty_like(dw3)
    xm.xmoe_expert_ffn_up(xs.contiguous(), w1, w3, off_d, act2, h132)
    xm.xmoe_expert_ffn_bwd_dw13(xs.contiguous(), dh13, off_d, dw1m, dw3m)
    torch.cuda.synchronize()
    assert torch.equal(act, act2) and torch.equal(h13, h132)
    assert torch.equal(dw1, dw1m) and torch.equal(dw3, dw3m)
    assert (h13[torch.from_numpy(bad).cuda()] == 0).all()


@pytest.mark.parametrize("dtype,rows,d,h,E,empty", FFN_CASES)
def test_expert_ffn_backward(xm, dtype, rows, d, h, E, empty):
    off, xs, w1, w3, w2, re_ = _ffn_inputs(dtype, rows, d, h, E, empty, seed=rows + 2 * d)
    tdt = DT[dtype]
    dye = workloads.random_rows(rows, d, dtype, seed=rows + 5)
    c = lambda t: t.cuda()
    act = torch.empty((rows, h), dtype=tdt, device="cuda")
    h13 = torch.empty((rows, 2 * h), dtype=tdt, device="cuda")
    ye = torch.empty((rows, d), dtype=tdt, device="cuda")
    xm.xmoe_expert_ffn(c(xs), c(w1), c(w3), c(w2), c(off), act, ye, h13=h13)
    dh13 = torch.empty((rows, 2 * h), dtype=tdt, device="cuda")
    dxs = torch.empty((rows, d), dtype=tdt, device="cuda")
    dw1 = torch.full((E, d, h), float("nan"), dtype=tdt, device="cuda")   # must be fully overwritten
    dw3 = torch.full((E, d, h), float("nan"), dtype=tdt, device="cuda")
    dw2 = torch.full((E, h, d), float("nan"), dtype=tdt, device="cuda")
    xm.xmoe_expert_ffn_bwd(c(xs), c(w1), c(w3), c(w2), act, h13, c(dye), c(off), dh13, dxs, dw1, dw3, dw2)
    ref = orc.ffn_bwd(orc_in(xs), re_, orc_in(w1), orc_in(w3), orc_in(w2), orc_in(dye), want_dh=True)
    fwd = orc.ffn(orc_in(xs), re_, orc_in(w1), orc_in(w3), orc_in(w2), want_hidden=True)
    rt = RTOL[dtype]
    g = host(dh13)
    assert_close(g[:, :h], ref["dh1"], rt, "dh1")
    assert_close(g[:, h:], ref["dh3"], rt, "dh3")
    assert_close(host(dxs), ref["dxs"], rt, "dxs")
    o = off.numpy()
    X, G = host(xs), host(dye)
    scales = {}

    def floors(e):
        if e not in scales:
            sl = slice(o[e], o[e + 1])
            scales[e] = swiglu_wgrad_scales(X[sl], ref["da"][sl], fwd["h1"][sl], fwd["h3"][sl], fwd["act"][sl], G[sl],
                                            host(w2[e]), (host(w1[e]), host(w3[e])), wgrad_acc(dtype, d))
        return scales[e]

    rows = lambda e: o[e + 1] - o[e]
    assert_wgrad_close(host(dw1), ref["dw1"], rows, lambda e: floors(e)[0], rt, "dw1")
    assert_wgrad_close(host(dw3), ref["dw3"], rows, lambda e: floors(e)[1], rt, "dw3")
    assert_wgrad_close(host(dw2), ref["dw2"], rows, lambda e: floors(e)[2], rt, "dw2")


def test_expert_ffn_zero_rows(xm):
    """No rows at all: nothing to compute, and every weight gradient is zero."""
    E, d, h = 4, 128, 64
    bf = torch.bfloat16
    off = torch.zeros(E + 1, dtype=torch.int32, device="cuda")
    w1 = torch.randn((E, d, h), device="cuda").to(bf)
    w3 = torch.randn((E, d, h), device="cuda").to(bf)
    w2 = torch.randn((E, h, d), device="cuda").to(bf)
    e = lambda *s: torch.empty(s, dtype=bf, device="cuda")
    act, h13, ye = e(0, h), e(0, 2 * h), e(0, d)
    xm.xmoe_expert_ffn(e(0, d), w1, w3, w2, off, act, ye, h13=h13)
    dw1 = torch.full((E, d, h), float("nan"), dtype=bf, device="cuda")
    dw3 = torch.full((E, d, h), float("nan"), dtype=bf, device="cuda")
    dw2 = torch.full((E, h, d), float("nan"), dtype=bf, device="cuda")
    xm.xmoe_expert_ffn_bwd(e(0, d), w1, w3, w2, act, h13, e(0, d), off, e(0, 2 * h), e(0, d), dw1, dw3, dw2)
    torch.cuda.synchronize()
    for t in (dw1, dw3, dw2):
        assert torch.equal(t, torch.zeros_like(t))


# ------------------------------------------------------------------ router backward

def _random_route_bwd(n: int, seed: int):
    """Seeded gate-backward shapes: as the routing ones, k up to 128."""
    rs = np.random.RandomState(seed)
    out = []
    for i in range(n):
        dt = "f32" if i % 3 == 2 else "bf16"
        E = 8 * int(rs.randint(1, 129)) if dt == "bf16" else int(rs.randint(1, 1025))
        k = int(rs.randint(1, min(E, 128) + 1))
        T = int(rs.choice([1, 5, 64, 300, 1031, 4097]))
        d = 8 * int(rs.randint(1, 257)) if dt == "bf16" else int(rs.randint(1, 400))
        out.append((dt, T, d, E, k, float(rs.choice([0.5, 1.0, 2.0]))))
    return out


RANDOM_ROUTE_BWD = _random_route_bwd(10, 14)


@pytest.mark.parametrize("dtype,T,d,E,k,inv_tau", [("f32", 256, 128, 8, 2, 1.0), ("bf16", 300, 256, 16, 6, 1.0),
                                                   ("bf16", 2500, 512, 160, 8, 2.0), ("bf16", 777, 448, 64, 6, 1.0),
                                                   ("bf16", 600, 256, 256, 8, 1.0), ("f32", 40, 32, 320, 70, 1.0),
                                                   ("bf16", 64, 64, 512, 100, 0.5)] + RANDOM_ROUTE_BWD)
def test_route_bwd(xm, dtype, T, d, E, k, inv_tau):
    """Includes 256 experts (the 2x2-wave 256-column tile of Wg's gradient), and
    k above 64 (a token's slots read in two chunks)."""
    tdt = DT[dtype]
    g = torch.Generator().manual_seed(T + E)
    x = workloads.random_rows(T, d, dtype, seed=41)
    wg = (torch.randn((d, E), generator=g) / d ** 0.5).to(tdt)
    logits = torch.randn((T, E), generator=g) * 2.0
    ids, _ = workloads.random_topk(T, E, k, seed=42)
    dtw = torch.randn((T, k), generator=g)
    dx0 = workloads.random_rows(T, d, dtype, seed=43)
    dx = dx0.cuda().clone()
    dwg = torch.empty((d, E), dtype=torch.float32, device="cuda")
    ws = torch.empty(xm.xmoe_route_bwd_workspace_size(T, d, E, tdt), dtype=torch.uint8, device="cuda")
    xm.xmoe_route_bwd(x.cuda(), wg.cuda(), logits.cuda(), ids.cuda(), dtw.cuda(), dx, dwg, ws, inv_tau)
    ref = orc.route_bwd(logits.numpy().astype(np.float64), ids.numpy(), dtw.numpy().astype(np.float64),
                        orc_in(x), orc_in(wg), inv_tau)
    rt = RTOL[dtype]
    assert_close(host(dx), host(dx0) + ref["dx"], rt, "dx")
    assert_close(host(dwg), ref["dwg"], rt, "dwg", floor=rss_rows(host(x), ref["dz"]))


# ------------------------------------------------------------------ error paths on the device

def test_rejects_bad_arguments_without_launching(xm):
    x = torch.zeros((8, 12), dtype=torch.bfloat16, device="cuda")   # d = 12: not a multiple of 8
    wg = torch.zeros((12, 8), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((8, 2), dtype=torch.int32, device="cuda")
    w = torch.empty((8, 2), dtype=torch.float32, device="cuda")
    lg = torch.empty((8, 8), dtype=torch.float32, device="cuda")
    with pytest.raises(xm.XmoeError) as e:
        xm.xmoe_route(x, wg, 2, ids, w, lg)
    assert e.value.status == 2
    ids9 = torch.empty((8, 9), dtype=torch.int32, device="cuda")
    w9 = torch.empty((8, 9), dtype=torch.float32, device="cuda")
    with pytest.raises(xm.XmoeError) as e:
        xm.xmoe_route(x[:, :8].contiguous(), wg[:8].contiguous(), 9, ids9, w9, lg)   # k > E
    assert e.value.status == 1
    pft = xm.PFT(8, 8, 2)
    small_ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(xm.XmoeError) as e:
        xm.xmoe_build_pft(ids, w, 8, pft, small_ws)
    assert e.value.status == 3


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_route_bwd_strided_dw_and_overwrite(xm, dt):
    """dtopk_w read as the first k columns of a wider slot buffer, and dx
    written instead of accumulated: bitwise the dense, accumulate-into-zeros
    result (and the same dWg)."""
    T, d, E, k = 333, 256, 16, 4
    g = torch.Generator().manual_seed(7)
    x = torch.randn(T, d, generator=g).to(dt).cuda()
    wg = (torch.randn(d, E, generator=g) / d ** 0.5).to(dt).cuda()
    logits = torch.randn(T, E, generator=g).cuda()
    ids, _ = workloads.random_topk(T, E, k, seed=8)
    ids = ids.cuda()
    wide = torch.randn(T, k + 3, generator=g).cuda()
    wide[:, k:] = float("nan")        # never read
    dense = wide[:, :k].contiguous()
    ws = torch.empty(xm.xmoe_route_bwd_workspace_size(T, d, E, dt), dtype=torch.uint8, device="cuda")
    dx1, dwg1 = torch.zeros(T, d, dtype=dt, device="cuda"), torch.empty(d, E, device="cuda")
    xm.xmoe_route_bwd(x, wg, logits, ids, dense, dx1, dwg1, ws, 1.5)
    dx2 = torch.full((T, d), float("nan"), dtype=dt, device="cuda")
    dwg2 = torch.empty(d, E, device="cuda")
    xm.xmoe_route_bwd(x, wg, logits, ids, wide[:, :k], dx2, dwg2, ws, 1.5, accumulate=False)
    torch.cuda.synchronize()
    assert torch.equal(dx1, dx2) and torch.equal(dwg1, dwg2)


@pytest.mark.parametrize("T,d,E,k,inv_tau", [(4096, 2048, 64, 6, 1.0), (32768, 4096, 160, 8, 2.0)])
def test_route_bwd_fullsize(xm, T, d, E, k, inv_tau):
    """Router backward at the full sizes of the DeepSeek-MoE-16B-like and the
    long-batch workloads (generator inputs on the GPU, oracle on the host)."""
    orc.set_threads(min(16, orc.get_threads()))
    g = torch.Generator(device="cuda").manual_seed(T + d)
    x = torch.randn((T, d), generator=g, device="cuda").to(torch.bfloat16)
    wg = (torch.randn((d, E), generator=g, device="cuda") / d ** 0.5).to(torch.bfloat16)
    logits = torch.randn((T, E), generator=g, device="cuda") * 2.0
    ids, _ = workloads.random_topk(T, E, k, seed=7)
    dtw = torch.randn((T, k), generator=g, device="cuda")
    dx0 = torch.randn((T, d), generator=g, device="cuda").to(torch.bfloat16)
    dx = dx0.clone()
    dwg = torch.empty((d, E), dtype=torch.float32, device="cuda")
    ws = torch.empty(xm.xmoe_route_bwd_workspace_size(T, d, E, torch.bfloat16), dtype=torch.uint8, device="cuda")
    xm.xmoe_route_bwd(x, wg, logits, ids.cuda(), dtw, dx, dwg, ws, inv_tau)
    torch.cuda.synchronize()
    ref = orc.route_bwd(host(logits), ids.numpy(), host(dtw), orc_in(x), orc_in(wg), inv_tau)
    assert_close(host(dx), host(dx0) + ref["dx"], RTOL["bf16"], "dx")
    assert_close(host(dwg), ref["dwg"], RTOL["bf16"], "dwg", floor=rss_rows(host(x), ref["dz"]))
