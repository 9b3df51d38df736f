"""Pins of the oracle's gate (routing) against values fixed outside the oracle.

Reading under test (X-MoE notes "略读笔记90", section 需求: fine-grained experts
with large top-k; "5.4 MoE模型在分布式训练中的应用", section 训练流程: gate
scores computed per token): p = softmax over E of s = z*inv_tau + logit_bias,
z = x.Wg; the k experts with the largest sel = s + select_bias, ties to the
lower index; weight = p of the chosen expert, not renormalised.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import softmax

HERE = os.path.dirname(os.path.abspath(__file__))


def _rand(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


def test_hand_worked_example(orc):
    g = json.load(open(os.path.join(HERE, "golden", "route_tiny.json")))
    x = np.array(g["x"], np.float32)
    wg = np.array(g["wg"], np.float32)
    for mode in (0, 1, 2):
        r = orc.route(x, wg, g["k"], mode)
        assert r["topk_ids"].tolist() == g["expected_topk_ids"]
        np.testing.assert_allclose(r["topk_w"], np.array(g["expected_topk_w"]), rtol=1e-7)
    assert math.isclose(g["expected_topk_w"][0][0], math.e / (1 + 2 * math.e + 1 / math.e))


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_brute_force_full_sort(orc, mode):
    """Selection equals a full sort by (score desc, index asc) of logits computed
    by numpy's fp64 matmul (rounded to fp32 where the mode decides in fp32)."""
    T, d, E, k = 40, 24, 11, 4
    x, wg = _rand((T, d), 1), _rand((d, E), 2, 0.3)
    lb = _rand((E,), 3, 0.5)
    sb = _rand((E,), 4, 0.5)
    r = orc.route(x, wg, k, mode, 1.0, lb, sb)
    z = x.astype(np.float64) @ wg.astype(np.float64)
    if mode == 2:
        s = z + lb
        sel = s + sb
    else:
        s = (z.astype(np.float32) + lb).astype(np.float32)
        sel = (s + sb).astype(np.float32)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(sel[t, e]), e))[:k]
        if mode == 0:
            # fp32 sequential accumulation may differ from the rounded exact sum in
            # the last bits; only tokens whose order is unambiguous are compared
            srt = np.sort(sel[t])[::-1][:k + 1]
            if np.min(-np.diff(srt)) < 1e-5:
                continue
        assert r["topk_ids"][t].tolist() == order
    if mode == 1:   # one fp32 rounding of sums taken in different orders: <= 1 ulp apart
        np.testing.assert_allclose(r["scores"], s.astype(np.float64), rtol=2.0 ** -23, atol=1e-30)
    if mode == 2:
        np.testing.assert_allclose(r["scores"], s, rtol=1e-13, atol=1e-14)
    # weights: library softmax of the oracle's scores
    p = softmax(r["scores"], axis=1)
    np.testing.assert_allclose(r["probs"], p, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(r["topk_w"], np.take_along_axis(p, r["topk_ids"], 1), rtol=1e-12)


def test_fp32_sequential_logits_within_rounding_bound(orc):
    """Mode 0 logits lie within the classic bound d*u*sum|x w| of the exact sum."""
    T, d, E, k = 16, 300, 6, 2
    x, wg = _rand((T, d), 5), _rand((d, E), 6, 0.1)
    r = orc.route(x, wg, k, 0)
    exact = x.astype(np.float64) @ wg.astype(np.float64)
    bound = d * 2.0 ** -24 * (np.abs(x).astype(np.float64) @ np.abs(wg).astype(np.float64))
    assert np.all(np.abs(r["scores"] - exact) <= bound + 1e-30)


@pytest.mark.parametrize("E,k", [(8, 2), (16, 5), (64, 6)])
def test_zero_gate_closed_form(orc, E, k):
    """Wg = 0: every logit is 0, every expert ties, so S_t = {0..k-1} and p = 1/E
    exactly for a power-of-two E."""
    T, d = 33, 16
    x = _rand((T, d), 7)
    wg = np.zeros((d, E), np.float32)
    for mode in (0, 1, 2):
        r = orc.route(x, wg, k, mode)
        assert (r["topk_ids"] == np.arange(k)[None, :]).all()
        assert (r["topk_w"] == 1.0 / E).all()


def test_k_equals_E_selects_all_in_score_order(orc):
    T, d, E = 25, 12, 7
    x, wg = _rand((T, d), 8), _rand((d, E), 9)
    r = orc.route(x, wg, E, 1)
    assert (np.sort(r["topk_ids"], axis=1) == np.arange(E)).all()
    s = r["scores"]
    ordered = np.take_along_axis(s, r["topk_ids"], 1)
    assert (np.diff(ordered, axis=1) <= 0).all()
    np.testing.assert_allclose(r["topk_w"].sum(1), 1.0, rtol=1e-12)


def test_single_expert_weight_one(orc):
    x, wg = _rand((9, 5), 10), _rand((5, 1), 11)
    r = orc.route(x, wg, 1, 1)
    assert (r["topk_ids"] == 0).all() and (r["topk_w"] == 1.0).all()


def test_temperature_leaves_selection_unchanged(orc):
    """Doubling the scores is exact in fp32 and monotone: same experts, sharper weights."""
    T, d, E, k = 64, 32, 20, 4
    x, wg = _rand((T, d), 12), _rand((d, E), 13, 0.2)
    a = orc.route(x, wg, k, 1, 1.0)
    b = orc.route(x, wg, k, 1, 2.0)
    assert (a["topk_ids"] == b["topk_ids"]).all()
    assert (b["scores"] == 2.0 * a["scores"]).all()
    assert (b["topk_w"][:, 0] >= a["topk_w"][:, 0]).all()


def test_exact_inputs_ties_go_to_lower_index(orc):
    """Inputs on a coarse binary grid make every logit exact; integer brute force
    (exact arithmetic) then fixes the selection including all ties."""
    import workloads
    T, d, E, k = 70, 40, 12, 3
    xt, wt = workloads.exact_router_inputs(T, d, E, seed=3)
    x, wg = xt.numpy(), wt.numpy()
    zi = (x * 4).astype(np.int64) @ (wg * 8).astype(np.int64)     # exact integers
    for mode in (0, 1, 2):
        r = orc.route(x, wg, k, mode)
        assert (r["scores"] * 32 == zi).all()
        for t in range(T):
            assert r["topk_ids"][t].tolist() == sorted(range(E), key=lambda e: (-zi[t, e], e))[:k]
    assert (r["topk_ids"][0] == np.arange(k)).all()       # an all-zero token row


def test_selection_bias_changes_selection_only(orc):
    T, d, E, k = 50, 16, 10, 3
    x, wg = _rand((T, d), 14), _rand((d, E), 15, 0.1)
    sb = np.zeros(E, np.float32)
    sb[7] = 100.0
    r = orc.route(x, wg, k, 1, 1.0, None, sb)
    r0 = orc.route(x, wg, k, 1)
    assert (r["topk_ids"][:, 0] == 7).all()
    np.testing.assert_array_equal(r["probs"], r0["probs"])
    np.testing.assert_array_equal(r["topk_w"][:, 0], r0["probs"][:, 7])


def test_logit_bias_shifts_weights(orc):
    """A logit offset is part of the softmax input: p follows softmax(z + b)."""
    T, d, E, k = 20, 8, 6, 2
    x, wg = _rand((T, d), 16), _rand((d, E), 17)
    lb = np.log(np.arange(1, E + 1, dtype=np.float64) ** -1.2).astype(np.float32)
    r = orc.route(x, wg, k, 2, 1.0, lb)
    p = softmax(x.astype(np.float64) @ wg.astype(np.float64) + lb, axis=1)
    np.testing.assert_allclose(r["probs"], p, rtol=1e-12)


def test_probabilities_sum_to_one(orc):
    x, wg = _rand((100, 30), 18), _rand((30, 40), 19, 2.0)
    r = orc.route(x, wg, 8, 1)
    np.testing.assert_allclose(r["probs"].sum(1), 1.0, rtol=1e-13)
    assert (r["probs"] > 0).all() and (r["probs"] <= 1).all()
    assert (r["margin"] >= 0).all()
