"""GPU parity at the five workloads' full sizes, in the launch configuration the
benchmark times (the whole layer through the C ABI).

The oracle cannot redo a full-size layer in seconds, so it checks:
  * routing of every token (exact where unambiguous, valid where near-tied);
  * the Padding-Free Token buffer bit for bit: always against the oracle's
    construction from the device's own routing, and against the oracle's
    routing when the two routings agree;
  * the dispatch copy of the layer's buffer on sampled rows;
  * forward output, input gradient and routing-weight gradient of sampled
    tokens, recomputed token by token;
  * weight gradients: sampled columns of the busiest expert, the whole gradient
    of a small expert, and exact zeros for every expert no token chose.
The router weight gradient at full size is checked per step in
test_gpu_steps.py::test_route_bwd_fullsize.
"""
import numpy as np
import pytest
import torch

import oracle as orc
import workloads
from _helpers import (buffer_routing, RTOL, assert_close, by_expert, dx_floor, host, near_tie_bound, need_gpu, orc_in,
                      pft_contract, report, routing_check, swiglu_wgrad_scales, used_str, wgrad_acc)

pytestmark = pytest.mark.gpu

SAMPLE = {"tiny_f32": 64, "dsmoe16b": 32, "dsv3": 8, "zipf_skew": 32, "long_batch": 12}


@pytest.fixture(scope="module")
def xm():
    need_gpu()
    import padding_free_expert_amd as m
    assert m.xmoe_query_device(0)
    orc.set_threads(min(16, orc.get_threads()))
    return m


def _sub(t: torch.Tensor, idx) -> np.ndarray:
    return orc_in(t[torch.as_tensor(idx, device=t.device, dtype=torch.long)])


CASES = [(n, False, False) for n in ["tiny_f32", "dsmoe16b", "dsv3", "zipf_skew", "long_batch"]] + \
        [("dsmoe16b", True, True)]


@pytest.mark.parametrize("name,lean,merge", CASES,
                         ids=[n + ("-lean-shared-merged" if lean else "") for n, lean, _ in CASES])
def test_full_size_layer(xm, name, lean, merge):
    """lean: H1/H3 recomputed in the backward instead of kept; merge: the shared
    experts carried as always-routed experts in the routed buffer."""
    from padding_free_expert_amd.layer import PaddingFreeMoE
    wl = workloads.get(name)
    print(f"\n[{name}] T={wl.T} d={wl.d} E={wl.E} h={wl.h} k={wl.k} lean={lean} merge={merge}", flush=True)
    inp = workloads.generate(wl, device="cuda", backward=True)
    weights = {k: inp[k] for k in ("wg", "w1", "w3", "w2", "s1", "s3", "s2", "logit_bias", "select_bias")
               if k in inp}
    bwd_on = True
    layer = PaddingFreeMoE(weights, wl.T, wl.k, wl.inv_tau, backward=bwd_on, lean=lean, merge_shared=merge)
    layer.forward(inp["x"])
    layer.backward(inp["dy"])
    torch.cuda.synchronize()
    rt = RTOL[wl.dtype]
    mode = 0 if wl.dtype == "f32" else 1
    lb = None if inp["logit_bias"] is None else inp["logit_bias"].cpu().numpy()
    sb = None if inp["select_bias"] is None else inp["select_bias"].cpu().numpy()
    ox, owg = orc_in(inp["x"]), orc_in(inp["wg"])

    # routing of every token
    r = orc.route(ox, owg, wl.k, mode, wl.inv_tau, lb, sb)
    gids = host(layer.topk_ids)
    stats = {}
    mism = routing_check(gids, host(layer.logits), r, sb, wl.k, 1e-5, stats=stats)
    tag = f"full {name}" + ("-lean-merged" if lean else "")
    print(f"[{name}] near-tie tokens routed differently: {int(mism.sum())}", flush=True)
    near_tie_bound(tag, stats, wl.T)

    # PFT given the device's own routing: the oracle's construction, all six
    # fields bit for bit, whatever the near-ties
    pft = {k: v.cpu().numpy() for k, v in layer.pft.fields().items()}
    bids, bw, bE = buffer_routing(layer, gids, layer.topk_w.cpu().numpy())
    kb = bids.shape[1]
    pft_contract(pft, bids, bw, bE, orc)
    # and against the oracle's own routing where it agrees
    if not mism.any():
        rids, rw, _ = buffer_routing(layer, r["topk_ids"], r["topk_w"].astype(np.float32))
        ref = orc.build_pft(rids, rw, bE)
        for key in ("token_ids", "expert_ids", "tokens_per_expert", "expert_offsets"):
            np.testing.assert_array_equal(pft[key], ref[key], err_msg=key)
        # slots of near-tied experts may be ordered differently: compare where the order agrees
        same = (gids == r["topk_ids"]).all(axis=1)
        print(f"[{name}] tokens with near-tied slot order: {int((~same).sum())}", flush=True)
        np.testing.assert_array_equal(pft["slot_to_row"].reshape(wl.T, kb)[same],
                                      ref["slot_to_row"].reshape(wl.T, kb)[same])
    if wl.zipf_s > 0:
        tpe = pft["tokens_per_expert"]
        assert (tpe == 0).any() and tpe.max() > 10 * tpe.mean()

    # the dispatch copy over the layer's buffer (the layer itself gathers inside
    # its products), on sampled rows
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(layer.R, size=min(4096, layer.R), replace=False))
    xs = torch.empty((layer.R, wl.d), dtype=layer.x.dtype, device="cuda")
    xm.xmoe_dispatch(layer.x, layer.kc, layer.pft, xs)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_sub(xs, rows), _sub(inp["x"], pft["token_ids"][rows]))
    del xs

    # sampled tokens, recomputed by the oracle
    ok = np.nonzero(~mism)[0]
    tokens = np.sort(rng.choice(ok, size=min(SAMPLE[name], ok.size), replace=False))
    needed = np.unique(r["topk_ids"][tokens])
    o = {"x": ox, "wg": owg, "w1": _sub(inp["w1"], needed), "w3": _sub(inp["w3"], needed),
         "w2": _sub(inp["w2"], needed)}
    if lb is not None:
        o["logit_bias"] = lb
    if sb is not None:
        o["select_bias"] = sb
    for kk in ("s1", "s3", "s2"):
        if kk in inp:
            o[kk] = orc_in(inp[kk])
    fwd = orc.layer_forward(o, wl.k, mode, wl.inv_tau, n_shared=wl.n_shared, tokens=tokens, expert_subset=needed)
    u = {"y": assert_close(_as64(layer.y, tokens), fwd["y"], rt, "y")}
    dy_s = _sub(inp["dy"], tokens)
    bwd = orc.layer_backward(o, fwd, dy_s, wl.inv_tau, n_shared=wl.n_shared, want_dw=False)
    u["dx"] = assert_close(_as64(layer.dx, tokens), bwd["dx"], rt, "dx",
                           floor=dx_floor(o, fwd, bwd, dy_s, wl.n_shared))
    u["dtopk_w"] = assert_close(by_expert(gids[tokens], host(layer.dtopk_w)[tokens]),
                                by_expert(r["topk_ids"][tokens], bwd["dtopk_w"]), rt, "dtopk_w")

    # weight gradients
    tpe = pft["tokens_per_expert"]
    for e in np.nonzero(tpe == 0)[0]:
        assert not layer.dw1[e].any() and not layer.dw3[e].any() and not layer.dw2[e].any()
    bad_e = set()
    for t in np.nonzero(mism)[0]:
        bad_e |= set(gids[t].tolist()) | set(r["topk_ids"][t].tolist())
    cand = [e for e in range(wl.E) if e not in bad_e and tpe[e] > 0]
    busiest = max(cand, key=lambda e: tpe[e])
    u.update(_check_expert_columns(layer, inp, r, busiest, rt, rng))
    small = min(cand, key=lambda e: tpe[e])
    if tpe[small] <= 64:
        u.update(_check_expert_whole(layer, inp, r, small, rt))
    report(f"{tag}: " + ", ".join(f"{k} {used_str(v)}" for k, v in u.items()))


def _as64(t, idx):
    return t[torch.as_tensor(idx, device=t.device, dtype=torch.long)].detach().to(torch.float64).cpu().numpy()


def _expert_rows(r, e):
    t, j = np.nonzero(r["topk_ids"] == e)           # ascending token order
    return t.astype(np.int32), r["topk_w"][t, j]


def _check_expert_columns(layer, inp, r, e, rt, rng):
    """dW1[e][:, cols], dW3[e][:, cols], dW2[e][cols, :] of a busy expert."""
    tok, w = _expert_rows(r, e)
    h = inp["w1"].shape[2]
    cols = np.sort(rng.choice(h, size=4, replace=False))
    dye = w[:, None] * host(inp["dy"][torch.as_tensor(tok, device="cuda", dtype=torch.long)])
    x = orc_in(inp["x"])
    c = orc.ffn_wgrad_cols(x, np.zeros(tok.size, np.int32), _sub(inp["w1"], [e]), _sub(inp["w3"], [e]),
                           _sub(inp["w2"], [e]), dye, 0, cols, row_token=tok)
    g1 = host(layer.dw1[e])[:, cols]
    g3 = host(layer.dw3[e])[:, cols]
    g2 = host(layer.dw2[e])[cols, :]
    print(f"  expert {e}: {tok.size} rows, columns {cols.tolist()}", flush=True)
    return {"dw1 cols": assert_close(g1, c["dw1"], rt, f"dw1[{e}][:, cols]"),
            "dw3 cols": assert_close(g3, c["dw3"], rt, f"dw3[{e}][:, cols]"),
            "dw2 rows": assert_close(g2, c["dw2"], rt, f"dw2[{e}][cols, :]")}


def _check_expert_whole(layer, inp, r, e, rt):
    """The whole weight gradient of an expert with few rows, with the derived
    rounding floors."""
    tok, w = _expert_rows(r, e)
    dy = host(inp["dy"][torch.as_tensor(tok, device="cuda", dtype=torch.long)])
    dye = w[:, None] * dy
    x = orc_in(inp["x"])
    w1, w3, w2 = _sub(inp["w1"], [e]), _sub(inp["w3"], [e]), _sub(inp["w2"], [e])
    z = np.zeros(tok.size, np.int32)
    f = orc.ffn(x, z, w1, w3, w2, row_token=tok, want_hidden=True)
    b = orc.ffn_bwd(x, z, w1, w3, w2, dye, row_token=tok, want_dh=True)
    X = host(inp["x"][torch.as_tensor(tok, device="cuda", dtype=torch.long)])
    f1, f3, f2 = swiglu_wgrad_scales(X, b["da"], f["h1"], f["h3"], f["act"], dye, host(inp["w2"][e]),
                                     (host(inp["w1"][e]), host(inp["w3"][e])),
                                     wgrad_acc("f32" if layer.dtype == torch.float32 else "bf16", layer.d))
    print(f"  expert {e}: {tok.size} rows, whole gradient", flush=True)
    return {"dw1 small": assert_close(host(layer.dw1[e]), b["dw1"][0], rt, f"dw1[{e}]", floor=f1),
            "dw3 small": assert_close(host(layer.dw3[e]), b["dw3"][0], rt, f"dw3[{e}]", floor=f3),
            "dw2 small": assert_close(host(layer.dw2[e]), b["dw2"][0], rt, f"dw2[{e}]", floor=f2)}
