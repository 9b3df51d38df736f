"""End-to-end GPU parity of the whole padding-free MoE layer (forward and
backward through the C ABI) against the oracle's layer, on reduced sizes of the
five workloads that still span several tiles and ragged tails.

The GPU chain (route -> PFT -> gathered experts -> combine, and back) runs
on its own intermediate results; the oracle runs its own slot-order chain on
the same generator inputs and never sees a GPU value.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as orc
import workloads
from _helpers import (buffer_routing, RTOL, assert_close, assert_wgrad_close, by_expert, dx_floor, host, near_tie_bound,
                      need_gpu, orc_in, pft_contract, report, router_wgrad_floor, routing_check, swiglu_wgrad_scales,
                      used_str, wgrad_acc)

pytestmark = pytest.mark.gpu

NAMES = ["tiny_f32", "dsmoe16b", "dsv3", "zipf_skew", "long_batch"]


@pytest.fixture(scope="module")
def xm():
    need_gpu()
    import padding_free_expert_amd as m
    assert m.xmoe_query_device(0)
    return m


def _oracle_inputs(inp):
    out = {}
    for key, v in inp.items():
        if v is None:
            continue
        out[key] = v.numpy() if key in ("logit_bias", "select_bias") else orc_in(v)
    return out


def run_layer(xm, wl, inp, lean=False, overlap=True, merge=False):
    from padding_free_expert_amd.layer import PaddingFreeMoE
    g = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    weights = {k: g[k] for k in ("wg", "w1", "w3", "w2", "s1", "s3", "s2", "logit_bias", "select_bias") if k in g}
    layer = PaddingFreeMoE(weights, wl.T, wl.k, wl.inv_tau, backward=True, lean=lean, overlap=overlap,
                           merge_shared=merge)
    layer.forward(g["x"])
    layer.backward(g["dy"])
    torch.cuda.synchronize()
    return layer


@pytest.mark.parametrize("lean", [False, True], ids=["saved-h13", "lean"])
@pytest.mark.parametrize("name,merge", [(n, False) for n in NAMES] + [("dsmoe16b", True)],
                         ids=[n for n in NAMES] + ["dsmoe16b-shared-merged"])
def test_layer_forward_backward(xm, name, merge, lean):
    """lean=True recomputes H1/H3 in the backward instead of keeping them;
    merge=True carries the shared experts as always-routed experts in the
    routed buffer instead of as their own FFN on a second stream."""
    wl = workloads.small(name)
    inp = workloads.generate(wl, backward=True)
    tag = f"layer {name}" + ("-merged" if merge else "") + ("-lean" if lean else "")
    check_layer(xm, wl, inp, tag, lean=lean, merge=merge)


# Degenerate layers: one token (64 experts, 58 of them empty, through the
# fused router), top-1, every token to every expert, a single fp32 expert, and
# widths that are no tile multiple.
DEGENERATE = [
    workloads.Workload("one_token", "bf16", T=1, d=256, E=64, h=96, k=6, backward=True),
    workloads.Workload("top1", "bf16", T=37, d=128, E=8, h=64, k=1, backward=True),
    workloads.Workload("k_equals_E", "bf16", T=96, d=128, E=8, h=64, k=8, backward=True),
    workloads.Workload("one_expert_f32", "f32", T=50, d=64, E=1, h=32, k=1, backward=True),
    workloads.Workload("ragged_widths", "bf16", T=70, d=72, E=16, h=40, k=3, n_shared=1, h_shared=24,
                       backward=True),
    # the most experts the boundary takes, with many slots per token (split router)
    workloads.Workload("max_experts", "bf16", T=64, d=64, E=1024, h=32, k=32, backward=True),
    # every token to all 64 experts through the fused router
    workloads.Workload("k_equals_E_64", "bf16", T=40, d=64, E=64, h=16, k=64, n_shared=1, h_shared=16,
                       backward=True),
    # more than 64 slots per token (the row kernels and the gate read them in two chunks), rows of 16
    workloads.Workload("k_100", "bf16", T=20, d=16, E=128, h=16, k=100, n_shared=1, h_shared=16, backward=True),
    # a very peaked router: most selected experts' weights underflow towards zero
    workloads.Workload("peaked", "bf16", T=64, d=64, E=16, h=32, k=4, inv_tau=50.0, backward=True),
]


@pytest.mark.parametrize("wl", DEGENERATE, ids=[w.name for w in DEGENERATE])
def test_layer_degenerate(xm, wl):
    inp = workloads.generate(wl, backward=True)
    check_layer(xm, wl, inp, f"layer {wl.name}")


def _random_layers(n: int, seed: int):
    """Seeded layer shapes drawn across the limits the boundary states:
    widths that are multiples of 8 but rarely of a tile (down to 8), experts
    per token up to 16 (and up to E), bf16 expert counts that are multiples of
    8 up to 256 (any count in fp32), shared experts, Zipf-skewed or
    select-biased routing, a logit scale, and the lean and merged layer
    variants.  A cap on T*k*d*h keeps the fp64 oracle to seconds per case."""
    rs = np.random.RandomState(seed)
    out = []
    while len(out) < n:
        i = len(out)
        dt = "f32" if i % 4 == 3 else "bf16"
        E = int(rs.randint(1, 33)) * 8 if dt == "bf16" else int(rs.randint(1, 41))
        k = int(rs.randint(1, min(E, 16) + 1))
        T = int(rs.choice([1, 2, 3, 7, 33, 100, 257, 511, 700, 1031, 1500, 2049]))
        d = 8 * int(rs.randint(1, 129))
        h = 8 * int(rs.randint(1, 97))
        ns = int(rs.randint(0, 3))
        hs = h * int(rs.randint(1, 3)) if ns and rs.rand() < 0.5 else (8 * int(rs.randint(1, 65)) if ns else 0)
        zipf = float(rs.choice([0.0, 0.0, 1.1]))
        sbv = float(rs.choice([0.0, 0.0, 0.1]))
        inv_tau = float(rs.choice([1.0, 1.0, 0.5, 2.0]))
        lean, merge = bool(rs.rand() < 0.3), bool(ns and hs % h == 0 and rs.rand() < 0.5)
        if T * (k * h + ns * hs) * d > 3e9:
            continue
        wl = workloads.Workload(f"rand{i}", dt, T=T, d=d, E=E, h=h, k=k, n_shared=ns, h_shared=hs, inv_tau=inv_tau,
                                select_bias_var=sbv, zipf_s=zipf, backward=True, seed=1000 + i)
        out.append((wl, lean, merge))
    return out


RANDOM_LAYERS = _random_layers(48, 2026)


@pytest.mark.parametrize("wl,lean,merge", RANDOM_LAYERS,
                         ids=[f"{w.name}-{w.dtype}-T{w.T}-d{w.d}-E{w.E}-h{w.h}-k{w.k}-s{w.n_shared}x{w.h_shared}"
                              + ("-lean" if ln else "") + ("-merged" if mg else "") for w, ln, mg in RANDOM_LAYERS])
def test_layer_random_shapes(xm, wl, lean, merge):
    """Whole-layer parity on seeded random shapes (the same checks as the
    named workloads)."""
    inp = workloads.generate(wl, backward=True)
    check_layer(xm, wl, inp, f"layer {wl.name}", lean=lean, merge=merge)


def check_layer(xm, wl, inp, tag, lean=False, merge=False):
    """The GPU layer against the oracle's layer on the same inputs: routing,
    the PFT, y, dX, the routing weights' gradient, the shared and routed weight
    gradients and dWg."""
    layer = run_layer(xm, wl, inp, lean=lean, merge=merge)
    assert layer.merged == (merge and wl.n_shared > 0)
    o = _oracle_inputs(inp)
    mode = 0 if wl.dtype == "f32" else 1
    fwd = orc.layer_forward(o, wl.k, mode, wl.inv_tau, n_shared=wl.n_shared)
    bwd = orc.layer_backward(o, fwd, o["dy"], wl.inv_tau, n_shared=wl.n_shared)
    rt = RTOL[wl.dtype]
    sb = None if inp["select_bias"] is None else inp["select_bias"].numpy()

    # routing: exact where unambiguous, valid where near-tied (none expected in fp32)
    gids = host(layer.topk_ids)
    stats = {}
    mism = routing_check(gids, host(layer.logits), fwd["route"], sb, wl.k, 1e-5, stats=stats)
    near_tie_bound(tag, stats, wl.T)
    if wl.dtype == "f32":
        np.testing.assert_array_equal(host(layer.logits), fwd["route"]["scores"])
        assert not mism.any()

    # PFT given the device's own routing: all six fields bit for bit, always
    pft = {k: v.cpu().numpy() for k, v in layer.pft.fields().items()}
    bids, bw, bE = buffer_routing(layer, gids, layer.topk_w.cpu().numpy())
    kb = bids.shape[1]
    pft_contract(pft, bids, bw, bE, orc)
    # and against the oracle's own routing when the two agree
    if not mism.any():
        rids, rw, _ = buffer_routing(layer, fwd["route"]["topk_ids"], fwd["route"]["topk_w"].astype(np.float32))
        ref = orc.build_pft(rids, rw, bE)
        for key in ("token_ids", "expert_ids", "tokens_per_expert", "expert_offsets"):
            np.testing.assert_array_equal(pft[key], ref[key], err_msg=key)
        # slots of near-tied experts may be ordered differently: compare where the order agrees
        same = (gids == fwd["route"]["topk_ids"]).all(axis=1)
        np.testing.assert_array_equal(pft["slot_to_row"].reshape(wl.T, kb)[same],
                                      ref["slot_to_row"].reshape(wl.T, kb)[same])
        assert_close(pft["combine_weights"], ref["combine_weights"], 1e-5, "combine_weights")
    else:
        # a near-tie has more than one correct selection (checked valid above):
        # evaluate the oracle's layer on the device's choice for those tokens,
        # so that every token, every expert and the gate's gradient compare
        sel = {int(t): gids[t] for t in np.nonzero(mism)[0]}
        fwd = orc.layer_forward(o, wl.k, mode, wl.inv_tau, n_shared=wl.n_shared, select=sel)
        bwd = orc.layer_backward(o, fwd, o["dy"], wl.inv_tau, n_shared=wl.n_shared)
        mism = np.zeros_like(mism)

    # forward output and input gradient on every token
    u = {"y": assert_close(host(layer.y), fwd["y"], rt, "y"),
         "dx": assert_close(host(layer.dx), bwd["dx"], rt, "dx", floor=dx_floor(o, fwd, bwd, o["dy"], wl.n_shared))}
    # the routing weights' gradient, per slot
    u["dtopk_w"] = assert_close(by_expert(gids, host(layer.dtopk_w)),
                                by_expert(fwd["route"]["topk_ids"], bwd["dtopk_w"]), rt, "dtopk_w")
    X = host(inp["x"])
    if wl.n_shared:
        hs = wl.h_shared
        for s_ in range(wl.n_shared):
            f, b = fwd["shared"][s_], bwd["shared"][s_]
            cs = slice(s_ * hs, (s_ + 1) * hs)
            f1, f3, f2 = swiglu_wgrad_scales(X, b["da"], f["h1"], f["h3"], f["act"], host(inp["dy"]),
                                             host(inp["s2"])[cs, :], (host(inp["s1"])[:, cs], host(inp["s3"])[:, cs]),
                                             wgrad_acc(wl.dtype, wl.d))
            cs = slice(s_ * hs, (s_ + 1) * hs)
            u[f"ds1[{s_}]"] = assert_close(host(layer.ds1[0])[:, cs], bwd["ds1"][:, cs], rt, f"ds1[{s_}]", floor=f1)
            u[f"ds3[{s_}]"] = assert_close(host(layer.ds3[0])[:, cs], bwd["ds3"][:, cs], rt, f"ds3[{s_}]", floor=f3)
            u[f"ds2[{s_}]"] = assert_close(host(layer.ds2[0])[cs, :], bwd["ds2"][cs, :], rt, f"ds2[{s_}]", floor=f2)
    # weight gradients: every expert, with the rounding scales of its own rows
    # (oracle values, slot order)
    Xr = X[fwd["row_token"]]
    scales = {}

    def floors(e):
        if e not in scales:
            r = fwd["row_expert"] == e
            scales[e] = swiglu_wgrad_scales(Xr[r], bwd["da"][r], fwd["h1"][r], fwd["h3"][r], fwd["act"][r],
                                            bwd["dye"][r], host(inp["w2"][e]), (host(inp["w1"][e]), host(inp["w3"][e])),
                                            wgrad_acc(wl.dtype, wl.d))
        return scales[e]

    def rows(e):
        return int((fwd["row_expert"] == e).sum())

    fl = lambda i: (lambda e: floors(e)[i])
    u["dw1"] = assert_wgrad_close(host(layer.dw1), bwd["dw1"], rows, fl(0), rt, "dw1")
    u["dw3"] = assert_wgrad_close(host(layer.dw3), bwd["dw3"], rows, fl(1), rt, "dw3")
    u["dw2"] = assert_wgrad_close(host(layer.dw2), bwd["dw2"], rows, fl(2), rt, "dw2")
    fl = router_wgrad_floor(X, fwd["route"]["probs"], fwd["route"]["topk_ids"], fwd["ye"], host(inp["dy"]),
                            bwd["dz"], wl.inv_tau)
    u["dwg"] = assert_close(host(layer.dwg), bwd["dwg"], rt, "dwg", floor=fl)
    report(f"{tag}: " + ", ".join(f"{k} {used_str(v)}" for k, v in u.items()))
    # experts no token chose get an explicit zero gradient
    for e in np.nonzero(pft["tokens_per_expert"] == 0)[0]:
        assert (layer.dw1[e] == 0).all() and (layer.dw3[e] == 0).all() and (layer.dw2[e] == 0).all()


def test_lean_layer_matches_saved_layer_bitwise(xm):
    """Recomputing H1/H3 runs the same kernel on the same inputs, so the lean
    layer's outputs and gradients are bitwise those of the layer that keeps
    them; it also keeps fewer bytes from the forward."""
    wl = workloads.small("dsmoe16b")
    inp = workloads.generate(wl, backward=True)
    a = run_layer(xm, wl, inp, lean=False)
    b = run_layer(xm, wl, inp, lean=True)
    for key, ga in a.grads().items():
        assert torch.equal(ga, b.grads()[key]), key
    assert torch.equal(a.y, b.y)
    assert b.saved_bytes() < a.saved_bytes()


@pytest.mark.parametrize("merge", [True, False], ids=["shared-merged", "shared-apart"])
def test_side_stream_matches_serial_bitwise(xm, merge):
    """The gate backward, the weight gradients and (unmerged) the shared experts
    on their own streams give bitwise the results of the serial call order
    (the stream waits carry every dependency)."""
    wl = workloads.small("dsmoe16b")
    inp = workloads.generate(wl, backward=True)
    a = run_layer(xm, wl, inp, overlap=False, merge=merge)
    b = run_layer(xm, wl, inp, overlap=True, merge=merge)
    assert torch.equal(a.y, b.y)
    for key, ga in a.grads().items():
        assert torch.equal(ga, b.grads()[key]), key


@pytest.mark.parametrize("wl", [w for w, _, _ in RANDOM_LAYERS[:12]], ids=[w.name for w, _, _ in RANDOM_LAYERS[:12]])
def test_layer_variants_bitwise_random(xm, wl):
    """On seeded random shapes: the overlapped streams give the serial call
    order's results and the lean layer the saved layer's, bit for bit."""
    inp = workloads.generate(wl, backward=True)
    a = run_layer(xm, wl, inp, overlap=False)
    ya, ga = a.y.clone(), {key: v.clone() for key, v in a.grads().items()}
    for kw in (dict(overlap=True), dict(lean=True)):
        b = run_layer(xm, wl, inp, **kw)
        assert torch.equal(ya, b.y), kw
        for key, g in ga.items():
            assert torch.equal(g, b.grads()[key]), (key, kw)


@pytest.mark.parametrize("name,lean,merge", [("dsmoe16b", False, False), ("zipf_skew", True, False),
                                             ("dsmoe16b", False, True)])
def test_second_step_matches_a_fresh_layer(xm, name, lean, merge):
    """A layer object reused for a second step with other inputs (other
    routing, other expert loads) gives bitwise what a fresh layer gives on
    those inputs: nothing of the first step survives in its buffers."""
    from padding_free_expert_amd.layer import PaddingFreeMoE
    wl = workloads.small(name)
    wl2 = dataclasses.replace(wl, seed=wl.seed + 77)
    inp1 = workloads.generate(wl, backward=True)
    inp2 = workloads.generate(wl2, backward=True)
    g1 = {k: (None if v is None else v.cuda()) for k, v in inp1.items()}
    g2 = {k: (None if v is None else v.cuda()) for k, v in inp2.items()}
    weights = {k: g1[k] for k in ("wg", "w1", "w3", "w2", "s1", "s3", "s2", "logit_bias", "select_bias") if k in g1}
    layer = PaddingFreeMoE(weights, wl.T, wl.k, wl.inv_tau, backward=True, lean=lean, merge_shared=merge)
    layer.forward(g1["x"])
    layer.backward(g1["dy"])
    ids1 = layer.topk_ids.clone()
    layer.forward(g2["x"])
    layer.backward(g2["dy"])
    torch.cuda.synchronize()
    fresh = PaddingFreeMoE(weights, wl.T, wl.k, wl.inv_tau, backward=True, lean=lean, merge_shared=merge)
    fresh.forward(g2["x"])
    fresh.backward(g2["dy"])
    torch.cuda.synchronize()
    assert not torch.equal(ids1, layer.topk_ids)   # the second step routes differently
    assert torch.equal(layer.y, fresh.y)
    for key, g in fresh.grads().items():
        assert torch.equal(layer.grads()[key], g), key
    for key, t in fresh.pft.fields().items():
        assert torch.equal(layer.pft.fields()[key], t), key


@pytest.mark.parametrize("dtype,merge,lean", [("bf16", False, False), ("bf16", True, True), ("f32", False, False)])
def test_layer_with_no_tokens(xm, dtype, merge, lean):
    """T = 0: every call is a no-op that still leaves the layer consistent: y
    and dX are empty, and every weight gradient (routed, shared, gate) is an
    exact zero, since no token contributes to it."""
    from padding_free_expert_amd.layer import PaddingFreeMoE
    wl = workloads.Workload("no_tokens", dtype, T=0, d=64, E=8, h=32, k=2, n_shared=2, h_shared=32, backward=True)
    inp = workloads.generate(wl, backward=True)
    g = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    weights = {k: g[k] for k in ("wg", "w1", "w3", "w2", "s1", "s3", "s2") if k in g}
    layer = PaddingFreeMoE(weights, 0, wl.k, wl.inv_tau, backward=True, lean=lean, merge_shared=merge)
    grads = [layer.dW1, layer.dW3, layer.dW2, layer.dwg] + ([] if layer.merged else [layer._ds1, layer._ds3,
                                                                                       layer._ds2])
    for t in grads:
        t.fill_(float("nan"))
    y = layer.forward(g["x"])
    dx = layer.backward(g["dy"])
    torch.cuda.synchronize()
    assert y.shape == (0, wl.d) and dx.shape == (0, wl.d)
    for key, t in layer.grads().items():
        if key in ("dw1", "dw3", "dw2", "ds1", "ds3", "ds2", "dwg"):
            assert (t == 0).all(), key
    assert (layer.pft.tokens_per_expert == 0).all() and (layer.pft.expert_offsets == 0).all()


def _layer_outputs(layer):
    out = {"y": layer.y.clone()}
    out.update({key: g.clone() for key, g in layer.grads().items()})
    return out


@pytest.mark.parametrize("name,merge,lean", [("dsmoe16b", False, False), ("dsmoe16b", True, False),
                                             ("zipf_skew", False, True)])
def test_layer_on_a_caller_stream(xm, name, merge, lean):
    """The layer on a stream the caller passes (its side streams forked from
    and joined into that stream) gives bitwise the results on the current
    stream."""
    from padding_free_expert_amd.layer import PaddingFreeMoE
    wl = workloads.small(name)
    inp = workloads.generate(wl, backward=True)
    g = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    weights = {k: g[k] for k in ("wg", "w1", "w3", "w2", "s1", "s3", "s2", "logit_bias", "select_bias") if k in g}
    layer = PaddingFreeMoE(weights, wl.T, wl.k, wl.inv_tau, backward=True, merge_shared=merge, lean=lean)
    layer.forward(g["x"])
    layer.backward(g["dy"])
    torch.cuda.synchronize()
    ref = _layer_outputs(layer)
    for t in [layer.y] + list(layer.grads().values()):
        t.fill_(float("nan"))
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    layer.forward(g["x"], stream=cs)
    layer.backward(g["dy"], stream=cs)
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()
    for key, v in _layer_outputs(layer).items():
        assert torch.equal(v, ref[key]), key


def test_layer_is_deterministic(xm):
    """No floating-point atomics: two runs give bitwise identical results."""
    wl = workloads.small("long_batch")
    inp = workloads.generate(wl, backward=True)
    a = run_layer(xm, wl, inp)
    ya, dxa, dwga, dw1a = a.y.clone(), a.dx.clone(), a.dwg.clone(), a.dw1.clone()
    b = run_layer(xm, wl, inp)
    assert torch.equal(ya, b.y) and torch.equal(dxa, b.dx) and torch.equal(dwga, b.dwg)
    assert torch.equal(dw1a, b.dw1)


def test_full_size_steps_repeat_bitwise(xm):
    """Many full-size steps of one layer (the DeepSeek-MoE-16B shape, all its
    streams overlapped) reproduce the first step's outputs and gradients bit
    for bit: no race between the streams or inside the kernels shows."""
    from padding_free_expert_amd.layer import PaddingFreeMoE
    wl = workloads.get("dsmoe16b")
    inp = workloads.generate(wl, device="cuda", backward=True)
    w = {k: inp[k] for k in ("wg", "w1", "w3", "w2", "s1", "s3", "s2") if k in inp}
    layer = PaddingFreeMoE(w, wl.T, wl.k, wl.inv_tau, backward=True)
    layer.forward(inp["x"])
    layer.backward(inp["dy"])
    torch.cuda.synchronize()
    ref = _layer_outputs(layer)
    for i in range(60):
        layer.forward(inp["x"])
        layer.backward(inp["dy"])
        if i % 10 == 9:
            torch.cuda.synchronize()
            for key, v in _layer_outputs(layer).items():
                assert torch.equal(v, ref[key]), (i, key)


def test_two_layers_at_once_from_two_threads(xm):
    """Two independent layers, each driven by its own host thread on its own
    stream at the same time, give bitwise the results each gives alone: the
    library keeps no state between calls that two users could share."""
    import threading
    from padding_free_expert_amd.layer import PaddingFreeMoE
    made = []
    for name, seed in (("dsmoe16b", 3), ("zipf_skew", 4)):
        wl = dataclasses.replace(workloads.small(name), seed=seed)
        inp = workloads.generate(wl, backward=True)
        g = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
        w = {k: g[k] for k in ("wg", "w1", "w3", "w2", "s1", "s3", "s2", "logit_bias", "select_bias") if k in g}
        made.append((PaddingFreeMoE(w, wl.T, wl.k, wl.inv_tau, backward=True), g))
    refs = []
    for layer, g in made:
        layer.forward(g["x"])
        layer.backward(g["dy"])
        torch.cuda.synchronize()
        refs.append(_layer_outputs(layer))
        for t in [layer.y] + list(layer.grads().values()):
            t.fill_(float("nan"))
    torch.cuda.synchronize()
    errors = []

    def run(layer, g):
        try:
            st = torch.cuda.Stream()
            for _ in range(5):
                layer.forward(g["x"], stream=st)
                layer.backward(g["dy"], stream=st)
            st.synchronize()
        except Exception as e:  # reported below, in the test's thread
            errors.append(repr(e))

    threads = [threading.Thread(target=run, args=lg) for lg in made]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=60)
    torch.cuda.synchronize()
    assert not errors, errors
    for (layer, _), ref in zip(made, refs):
        for key, v in _layer_outputs(layer).items():
            assert torch.equal(v, ref[key]), key


def test_identity_like_combine_k_equals_E(xm):
    """k = E: every token goes to every expert; the PFT is [T]*E rows and the
    layer still matches the oracle."""
    wl = workloads.Workload("all_experts", "bf16", T=96, d=128, E=8, h=64, k=8, backward=True)
    inp = workloads.generate(wl, backward=True)
    layer = run_layer(xm, wl, inp)
    o = _oracle_inputs(inp)
    fwd = orc.layer_forward(o, wl.k, 1)
    assert (layer.pft.tokens_per_expert.cpu().numpy() == wl.T).all()
    assert_close(host(layer.y), fwd["y"], RTOL["bf16"], "y")


@pytest.mark.parametrize("merge", [False, True], ids=["shared-apart", "shared-merged"])
def test_layer_step_replays_as_graph(xm, merge):
    """The library allocates, clears and synchronises nothing, so one layer step
    (forward and backward, all three streams) can be captured as a HIP graph.
    Every replay, with eager steps run between replays, gives bitwise the
    outputs and gradients of an eager step."""
    wl = workloads.small("dsmoe16b")
    inp = workloads.generate(wl, backward=True)
    layer = run_layer(xm, wl, inp, merge=merge)
    g = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    ref = {"y": layer.y.clone(), **{k: v.clone() for k, v in layer.grads().items()}}

    def outs():
        return {"y": layer.y, **layer.grads()}

    graph = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=cs):
        layer.forward(g["x"])
        layer.backward(g["dy"])
    torch.cuda.synchronize()
    for _ in range(3):
        for t in outs().values():
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for key, t in outs().items():
            assert torch.equal(t, ref[key]), key
        layer.forward(g["x"])   # eager work between replays
        layer.backward(g["dy"])
        torch.cuda.synchronize()


@pytest.mark.parametrize("merge", [True, False], ids=["shared-merged", "shared-apart"])
def test_weight_update_between_steps(xm, merge):
    """Weights changed in place between two steps (as an optimizer step does):
    after refresh_weights() the next step gives bitwise the results of a layer
    built on the new weights, merged or not."""
    wl = workloads.small("dsmoe16b")
    inp = workloads.generate(wl, backward=True)
    layer = run_layer(xm, wl, inp, merge=merge)
    g = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    gen = torch.Generator(device="cuda").manual_seed(5)
    for key in ("w1", "w3", "w2", "s1", "s3", "s2"):
        w = layer.w[key]
        w.add_((torch.randn(w.shape, generator=gen, device="cuda") * 0.01).to(w.dtype))
    layer.refresh_weights()
    layer.forward(g["x"])
    layer.backward(g["dy"])
    torch.cuda.synchronize()
    new = dict(inp)
    for key in ("w1", "w3", "w2", "s1", "s3", "s2"):
        new[key] = layer.w[key].cpu()
    fresh = run_layer(xm, wl, new, merge=merge)
    assert torch.equal(layer.y, fresh.y)
    for key, t in fresh.grads().items():
        assert torch.equal(layer.grads()[key], t), key
