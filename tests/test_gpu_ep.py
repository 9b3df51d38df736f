"""GPU parity of the pilot-token build and the expert-parallel plans (integer
work: bit-exact against the oracle), and an emulated expert-parallel round
trip: G ranks on one GPU, the alltoallv replaced by slicing, which must give
every expert row and every expert's weight gradient bit for bit as the
single-GPU path does on all ranks' tokens at once."""
import numpy as np
import pytest
import torch

import oracle as orc
import workloads
from _helpers import host, need_gpu
from oracle import ep

pytestmark = pytest.mark.gpu

I32 = dict(dtype=torch.int32, device="cuda")


@pytest.fixture(scope="module")
def xm():
    need_gpu()
    import padding_free_expert_amd as m
    assert m.xmoe_query_device(0), "device 0 is not gfx950"
    return m


def _pilots(xm, ids, E, P):
    T, k = ids.shape
    N = E // P
    out = {"pilot_token_ids": torch.full((max(T * k, 1),), -7, **I32),
           "pilot_node_ids": torch.full((max(T * k, 1),), -7, **I32),
           "node_counts": torch.empty((N,), **I32), "node_offsets": torch.empty((N + 1,), **I32),
           "slot_to_pilot": torch.empty((max(T * k, 1),), **I32)}
    ws = torch.empty(max(xm.xmoe_build_pilots_workspace_size(T, E, k, P), 16), dtype=torch.uint8, device="cuda")
    xm.xmoe_build_pilots(ids.cuda(), E, P, out["pilot_token_ids"], out["pilot_node_ids"], out["node_counts"],
                         out["node_offsets"], out["slot_to_pilot"], ws)
    torch.cuda.synchronize()
    return {key: host(v) for key, v in out.items()}


def _divisors(n: int):
    return [q for q in range(1, n + 1) if n % q == 0]


def _random_ep(n: int, seed: int):
    """Seeded (T, E, k, divisor of E, seed) shapes: up to 1024 experts, k up to
    32, up to 3000 tokens; T*k at most 40000 keeps the pure-Python plans of
    the oracle to seconds."""
    rs = np.random.RandomState(seed)
    out = []
    while len(out) < n:
        E = int(rs.randint(1, 1025))
        T, k = int(rs.choice([1, 2, 77, 256, 257, 3000])), int(rs.randint(1, min(E, 32) + 1))
        if T * k <= 40000:
            out.append((T, E, k, int(rs.choice(_divisors(E))), 100 + len(out)))
    return out


@pytest.mark.parametrize("T,E,k,P,seed", [
    (300, 16, 6, 4, 0),       # small, several blocks of 256 tokens and a ragged tail
    (1, 8, 3, 2, 1),
    (513, 64, 6, 64, 2),      # one node: one pilot per token
    (257, 32, 4, 1, 3),       # one expert per node: the pilots are the buffer's rows
    (4096, 64, 6, 8, 4),      # DeepSeek-MoE-16B shape, 8 nodes of 8 experts
    (8192, 256, 8, 32, 5),    # DeepSeek-V3 shape, 8 nodes of 32 experts
] + _random_ep(10, 20))
def test_pilots_match_oracle(xm, T, E, k, P, seed):
    ids, _ = workloads.random_topk(T, E, k, seed=seed)
    got = _pilots(xm, ids, E, P)
    ref = ep.rbd_pilots(ids.numpy(), E, P)
    n = int(ref["node_offsets"][-1])
    for key in ("node_counts", "node_offsets", "slot_to_pilot"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
    np.testing.assert_array_equal(got["pilot_token_ids"][:n], ref["pilot_token_ids"])
    np.testing.assert_array_equal(got["pilot_node_ids"][:n], ref["pilot_node_ids"])
    assert (got["pilot_token_ids"][n:] == -7).all()  # nothing written past the pilots


def test_pilots_empty(xm):
    ids = torch.empty((0, 4), dtype=torch.int32)
    got = _pilots(xm, ids, 16, 4)
    np.testing.assert_array_equal(got["node_counts"], np.zeros(4, np.int32))
    np.testing.assert_array_equal(got["node_offsets"], np.zeros(5, np.int32))


@pytest.mark.parametrize("T,E,k,G,seed", [(300, 16, 6, 4, 0), (64, 8, 8, 8, 1), (4096, 64, 6, 8, 2),
                                          (10, 12, 3, 3, 3)] + _random_ep(8, 21))
def test_send_plan_matches_oracle(xm, T, E, k, G, seed):
    ids, w = workloads.random_topk(T, E, k, seed=seed)
    pft = xm.PFT(T, E, k)
    ws = torch.empty(max(xm.xmoe_build_pft_workspace_size(T, E, k), 16), dtype=torch.uint8, device="cuda")
    xm.xmoe_build_pft(ids.cuda(), w.cuda(), E, pft, ws)
    counts, displs = torch.empty((G,), **I32), torch.empty((G + 1,), **I32)
    xm.xmoe_ep_send_plan(pft.expert_offsets, G, counts, displs)
    torch.cuda.synchronize()
    ref = ep.ep_send_plan(orc.build_pft(ids.numpy(), w.numpy(), E)["tokens_per_expert"], G)
    np.testing.assert_array_equal(host(counts), ref["send_counts"])
    np.testing.assert_array_equal(host(displs), ref["send_displs"])


def _recv_plan(xm, C):
    G, el = C.shape
    n = int(C.sum())
    out = {"local_offsets": torch.empty((el + 1,), **I32), "recv_displs": torch.empty((G + 1,), **I32),
           "local_to_recv": torch.full((max(n, 1),), -7, **I32), "recv_to_local": torch.full((max(n, 1),), -7, **I32)}
    ws = torch.empty(max(xm.xmoe_ep_recv_plan_workspace_size(G, el), 16), dtype=torch.uint8, device="cuda")
    xm.xmoe_ep_recv_plan(torch.as_tensor(C, dtype=torch.int32).cuda(), n, out["local_offsets"], out["recv_displs"],
                         out["local_to_recv"], out["recv_to_local"], ws)
    torch.cuda.synchronize()
    return {key: host(v)[:n] if key in ("local_to_recv", "recv_to_local") else host(v) for key, v in out.items()}


def _random_recv(seed: int):
    """Seeded receive-count matrices: 1-200 ranks, up to 1024 cells, counts up
    to 100 per cell, some cells empty."""
    rs = np.random.RandomState(seed)
    return [(G, int(rs.randint(1, 1024 // G + 1)), int(rs.randint(1, 100)), float(rs.choice([0.0, 0.3, 0.9])), 100 + i)
            for i, G in enumerate([1, 2, 5, 7, 16, 31, 64, 200])]


RANDOM_RECV = _random_recv(30)


@pytest.mark.parametrize("G,el,hi,zero_frac,seed", [
    (4, 4, 40, 0.2, 0), (1, 16, 30, 0.1, 1), (8, 1, 50, 0.3, 2), (3, 5, 7, 0.5, 3),
    (8, 8, 900, 0.0, 4),       # DeepSeek-MoE-16B on 8 ranks: ~380 rows per (source, expert)
    (32, 32, 40, 0.1, 5),      # 1024 cells, the most the plan supports
    (2, 3, 1, 1.0, 6),         # nothing received
] + RANDOM_RECV)
def test_recv_plan_matches_oracle(xm, G, el, hi, zero_frac, seed):
    rng = np.random.default_rng(seed)
    C = rng.integers(0, hi + 1, size=(G, el)).astype(np.int32)
    C[rng.random((G, el)) < zero_frac] = 0
    got = _recv_plan(xm, C)
    ref = ep.ep_recv_plan(C)
    for key in ref:
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("n,d,rows", [(1000, 264, 1200), (1, 8, 3), (3000, 8, 3100), (257, 2056, 300)])
def test_scatter_rows_is_the_indexed_copy(xm, dt, n, d, rows):
    g = torch.Generator().manual_seed(0)
    src = torch.randn(n, d, generator=g).to(dt).cuda()
    perm = torch.randperm(rows, generator=g)[:n].to(torch.int32)
    perm[1::97] = -1           # skipped
    perm[5::211] = rows + 3    # skipped
    dst = torch.full((rows, d), 7.0, dtype=dt, device="cuda")
    xm.xmoe_scatter_rows(src, perm.cuda(), dst)
    torch.cuda.synchronize()
    ref = torch.full((rows, d), 7.0, dtype=dt)
    ok = (perm >= 0) & (perm < rows)
    ref[perm[ok].long()] = src.cpu()[ok]
    assert torch.equal(dst.cpu(), ref)


def _emulated_ep(xm, G, T, E, k, d, h, seed):
    """Forward and backward of the routed experts over G emulated ranks.
    Returns per-rank ye / dxs in each rank's buffer order and the weight
    gradients, next to the single-GPU results on all ranks' tokens at once."""
    el = E // G
    bf = torch.bfloat16
    g = torch.Generator(device="cuda").manual_seed(seed)
    rn = lambda *s, sc=1.0: (torch.randn(s, generator=g, device="cuda") * sc).to(bf)
    w1, w3, w2 = rn(E, d, h, sc=d ** -.5), rn(E, d, h, sc=d ** -.5), rn(E, h, d, sc=h ** -.5)
    routes = [workloads.random_topk(T, E, k, seed=seed + 31 * s) for s in range(G)]
    xs_in = [rn(T, d) for _ in range(G)]
    # source side: buffer, dispatch copy, send plan, and an upstream gradient per row
    src = []
    for s in range(G):
        ids, w = routes[s]
        pft = xm.PFT(T, E, k)
        ws = torch.empty(max(xm.xmoe_build_pft_workspace_size(T, E, k), 16), dtype=torch.uint8, device="cuda")
        xm.xmoe_build_pft(ids.cuda(), w.cuda(), E, pft, ws)
        xs = torch.empty(T * k, d, dtype=bf, device="cuda")
        xm.xmoe_dispatch(xs_in[s], k, pft, xs)
        counts, displs = torch.empty((G,), **I32), torch.empty((G + 1,), **I32)
        xm.xmoe_ep_send_plan(pft.expert_offsets, G, counts, displs)
        src.append(dict(pft=pft, xs=xs, dye=rn(T * k, d), displs=host(displs), tpe=host(pft.tokens_per_expert)))
    torch.cuda.synchronize()
    # receiver side
    ye_back = [[None] * G for _ in range(G)]
    dxs_back = [[None] * G for _ in range(G)]
    dw1 = torch.empty_like(w1)
    dw3 = torch.empty_like(w3)
    dw2 = torch.empty_like(w2)
    for q in range(G):
        C = np.stack([src[s]["tpe"][q * el:(q + 1) * el] for s in range(G)]).astype(np.int32)
        n = int(C.sum())
        plan = {"lo": torch.empty((el + 1,), **I32), "rd": torch.empty((G + 1,), **I32),
                "l2r": torch.empty((max(n, 1),), **I32), "r2l": torch.empty((max(n, 1),), **I32)}
        ws = torch.empty(max(xm.xmoe_ep_recv_plan_workspace_size(G, el), 16), dtype=torch.uint8, device="cuda")
        xm.xmoe_ep_recv_plan(torch.as_tensor(C).cuda(), n, plan["lo"], plan["rd"], plan["l2r"], plan["r2l"], ws)
        # the alltoallv: source s's run for rank q, sources in order
        cut = lambda t, s: t[src[s]["displs"][q]:src[s]["displs"][q + 1]]
        recv_x = torch.cat([cut(src[s]["xs"], s) for s in range(G)])
        recv_dy = torch.cat([cut(src[s]["dye"], s) for s in range(G)])
        loc_x, loc_dy = torch.empty_like(recv_x), torch.empty_like(recv_dy)
        xm.xmoe_scatter_rows(recv_x, plan["r2l"], loc_x, n=n)
        xm.xmoe_scatter_rows(recv_dy, plan["r2l"], loc_dy, n=n)
        sl = slice(q * el, (q + 1) * el)
        act = torch.empty(n, h, dtype=bf, device="cuda")
        h13 = torch.empty(n, 2 * h, dtype=bf, device="cuda")
        ye = torch.empty(n, d, dtype=bf, device="cuda")
        xm.xmoe_expert_ffn(loc_x, w1[sl], w3[sl], w2[sl], plan["lo"], act, ye, h13=h13)
        dh13 = torch.empty(n, 2 * h, dtype=bf, device="cuda")
        dxs = torch.empty(n, d, dtype=bf, device="cuda")
        xm.xmoe_expert_ffn_bwd(loc_x, w1[sl], w3[sl], w2[sl], act, h13, loc_dy, plan["lo"], dh13, dxs,
                               dw1[sl], dw3[sl], dw2[sl])
        # back to arrival order, then each source's part returns to it
        ye_r, dxs_r = torch.empty_like(ye), torch.empty_like(dxs)
        xm.xmoe_scatter_rows(ye, plan["l2r"], ye_r, n=n)
        xm.xmoe_scatter_rows(dxs, plan["l2r"], dxs_r, n=n)
        rd = host(plan["rd"])
        for s in range(G):
            ye_back[s][q] = ye_r[rd[s]:rd[s + 1]]
            dxs_back[s][q] = dxs_r[rd[s]:rd[s + 1]]
    torch.cuda.synchronize()
    ep_ye = [torch.cat(ye_back[s]) for s in range(G)]
    ep_dxs = [torch.cat(dxs_back[s]) for s in range(G)]
    # single GPU, all tokens at once (token s*T + t): each expert sees the same
    # rows in the same (source, token) order
    ids_all = torch.cat([routes[s][0] for s in range(G)])
    w_all = torch.cat([routes[s][1] for s in range(G)])
    TT = G * T
    pft = xm.PFT(TT, E, k)
    ws = torch.empty(max(xm.xmoe_build_pft_workspace_size(TT, E, k), 16), dtype=torch.uint8, device="cuda")
    xm.xmoe_build_pft(ids_all.cuda(), w_all.cuda(), E, pft, ws)
    xs = torch.empty(TT * k, d, dtype=bf, device="cuda")
    xm.xmoe_dispatch(torch.cat(xs_in), k, pft, xs)
    # the upstream gradient of each (token, expert) pair, placed by the big buffer
    s2r_all = host(pft.slot_to_row)
    dye = torch.empty(TT * k, d, dtype=bf, device="cuda")
    for s in range(G):
        s2r = host(src[s]["pft"].slot_to_row)
        rows_big = torch.as_tensor(s2r_all[s * T * k:(s + 1) * T * k], device="cuda").long()
        dye[rows_big] = src[s]["dye"][torch.as_tensor(s2r, device="cuda").long()]
    R = TT * k
    act = torch.empty(R, h, dtype=bf, device="cuda")
    h13 = torch.empty(R, 2 * h, dtype=bf, device="cuda")
    ye = torch.empty(R, d, dtype=bf, device="cuda")
    xm.xmoe_expert_ffn(xs, w1, w3, w2, pft.expert_offsets, act, ye, h13=h13)
    dh13 = torch.empty(R, 2 * h, dtype=bf, device="cuda")
    dxs = torch.empty(R, d, dtype=bf, device="cuda")
    rdw1, rdw3, rdw2 = torch.empty_like(w1), torch.empty_like(w3), torch.empty_like(w2)
    xm.xmoe_expert_ffn_bwd(xs, w1, w3, w2, act, h13, dye, pft.expert_offsets, dh13, dxs, rdw1, rdw3, rdw2)
    torch.cuda.synchronize()
    ref_ye, ref_dxs = [], []
    for s in range(G):
        s2r = torch.as_tensor(host(src[s]["pft"].slot_to_row), device="cuda").long()
        rows_big = torch.as_tensor(s2r_all[s * T * k:(s + 1) * T * k], device="cuda").long()
        # row r of rank s's buffer is slot j with s2r[j] == r
        order = torch.empty_like(s2r)
        order[s2r] = torch.arange(T * k, device="cuda")
        ref_ye.append(ye[rows_big[order]])
        ref_dxs.append(dxs[rows_big[order]])
    return ep_ye, ep_dxs, (dw1, dw3, dw2), ref_ye, ref_dxs, (rdw1, rdw3, rdw2)


@pytest.mark.parametrize("G,T,E,k,d,h,seed", [
    (4, 300, 16, 6, 256, 200, 0),      # small, ragged
    (2, 37, 8, 2, 64, 64, 1),
    (4, 2048, 64, 6, 2048, 1408, 2),   # DeepSeek-MoE-16B dimensions, 4 ranks of 16 experts
])
def test_emulated_expert_parallel_round_trip_is_bitwise(xm, G, T, E, k, d, h, seed):
    ep_ye, ep_dxs, ep_dw, ref_ye, ref_dxs, ref_dw = _emulated_ep(xm, G, T, E, k, d, h, seed)
    for s in range(G):
        assert torch.equal(ep_ye[s], ref_ye[s]), f"ye of rank {s}"
        assert torch.equal(ep_dxs[s], ref_dxs[s]), f"dxs of rank {s}"
    for a, b, name in zip(ep_dw, ref_dw, ("dw1", "dw3", "dw2")):
        assert torch.equal(a, b), name
