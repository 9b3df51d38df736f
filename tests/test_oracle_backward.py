"""Pins of the oracle's backward against central finite differences in fp64.

"5.4 MoE模型在分布式训练中的应用", section 训练流程: the backward propagates
gradients along the reverse path of the forward.  The reading is the exact
gradient of the forward with the top-k selection held fixed, so only tokens
whose selection cannot flip under the perturbation are probed.
"""
import numpy as np
import pytest

T, D, H, E, K, NSH, HSH = 12, 10, 6, 8, 2, 2, 4
EPS = 1e-6


def _inputs(seed=0):
    rng = np.random.default_rng(seed)
    inp = {
        "x": rng.standard_normal((T, D)),
        "wg": rng.standard_normal((D, E)) * 0.6,
        "w1": rng.standard_normal((E, D, H)) / np.sqrt(D),
        "w3": rng.standard_normal((E, D, H)) / np.sqrt(D),
        "w2": rng.standard_normal((E, H, D)) / np.sqrt(H),
        "s1": rng.standard_normal((D, NSH * HSH)) / np.sqrt(D),
        "s3": rng.standard_normal((D, NSH * HSH)) / np.sqrt(D),
        "s2": rng.standard_normal((NSH * HSH, D)) / np.sqrt(HSH),
        "logit_bias": (rng.standard_normal(E) * 0.3).astype(np.float32),
        "select_bias": (rng.standard_normal(E) * 0.3).astype(np.float32),
    }
    dy = rng.standard_normal((T, D))
    return inp, dy


def _loss(orc, inp, dy, inv_tau):
    f = orc.layer_forward(inp, K, 2, inv_tau, n_shared=NSH)
    return float(np.sum(f["y"] * dy)), f


@pytest.fixture(scope="module", params=[1.0, 2.0])
def case(request):
    import oracle as orc
    inv_tau = request.param
    inp, dy = _inputs(1 if inv_tau == 1.0 else 2)
    L, f = _loss(orc, inp, dy, inv_tau)
    g = orc.layer_backward(inp, f, dy, inv_tau, n_shared=NSH)
    return orc, inp, dy, inv_tau, f, g


def _fd(orc, inp, dy, inv_tau, key, idx):
    plus = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
    minus = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
    plus[key][idx] += EPS
    minus[key][idx] -= EPS
    lp, fp = _loss(orc, plus, dy, inv_tau)
    lm, fm = _loss(orc, minus, dy, inv_tau)
    same = (fp["route"]["topk_ids"] == fm["route"]["topk_ids"]).all()
    return (lp - lm) / (2 * EPS), same


def test_selection_margins_are_safe(case):
    orc, inp, dy, inv_tau, f, g = case
    assert f["route"]["margin"].min() > 1e3 * EPS


@pytest.mark.parametrize("key", ["x", "wg", "w1", "w3", "w2", "s1", "s3", "s2"])
def test_gradient_matches_central_differences(case, key):
    orc, inp, dy, inv_tau, f, g = case
    grad = {"x": g["dx"], "wg": g["dwg"], "w1": g["dw1"], "w3": g["dw3"], "w2": g["dw2"],
            "s1": g["ds1"], "s3": g["ds3"], "s2": g["ds2"]}[key]
    rng = np.random.default_rng(hash(key) % 1000)
    shape = inp[key].shape
    if key in ("w1", "w3", "w2"):
        # probe experts that have rows as well as ones that may not
        used = np.unique(f["route"]["topk_ids"])
        experts = list(used[:3]) + [e for e in range(E) if e not in used][:1]
    probes = []
    for n in range(6):
        idx = tuple(int(rng.integers(0, s)) for s in shape)
        if key in ("w1", "w3", "w2"):
            idx = (int(experts[n % len(experts)]),) + idx[1:]
        probes.append(idx)
    for idx in probes:
        fd, same = _fd(orc, inp, dy, inv_tau, key, idx)
        assert same
        assert abs(fd - grad[idx]) <= 1e-7 * (1 + abs(fd)), (key, idx, fd, grad[idx])


def test_router_gradient_sums_to_zero(case):
    """Softmax Jacobian: sum_e dz[t, e] = 0 for every token."""
    orc, inp, dy, inv_tau, f, g = case
    np.testing.assert_allclose(g["dz"].sum(1), 0.0, atol=1e-14)


def test_empty_expert_gets_zero_weight_gradient(case):
    orc, inp, dy, inv_tau, f, g = case
    used = set(np.unique(f["route"]["topk_ids"]).tolist())
    empty = [e for e in range(E) if e not in used]
    for e in empty:
        assert (g["dw1"][e] == 0).all() and (g["dw3"][e] == 0).all() and (g["dw2"][e] == 0).all()
    # the same holds when an expert is explicitly never routed to
    x = inp["x"]
    re_ = np.array([0, 1] * (T // 2), np.int32)
    out = orc.ffn_bwd(x, re_, inp["w1"], inp["w3"], inp["w2"], dy)
    assert (out["dw1"][2:] == 0).all() and (out["dw2"][2:] == 0).all()


def test_column_wgrad_equals_full_wgrad(case):
    orc, inp, dy, inv_tau, f, g = case
    e = int(f["route"]["topk_ids"][0, 0])
    cols = [0, 3, 5]
    c = orc.ffn_wgrad_cols(f["x"], f["row_expert"], inp["w1"], inp["w3"], inp["w2"], g["dye"], e,
                           cols, row_token=f["row_token"])
    np.testing.assert_allclose(c["dw1"], g["dw1"][e][:, cols], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(c["dw3"], g["dw3"][e][:, cols], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(c["dw2"], g["dw2"][e][cols, :], rtol=1e-12, atol=1e-14)
