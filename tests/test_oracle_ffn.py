"""Pins of the oracle's expert FFN, gather, combine and their adjoints.

X-MoE article (adg.csdn.net), section 2.1.2: each expert multiplies only its
own rows by its weights ("dynamic slice without padding"); the gather copies
row token_ids[r] of the input into row r.  "5.4 MoE模型在分布式训练中的应用",
section 专家并行: results return to the owning token (combine).  The SwiGLU form
of the expert is a reading (the pages give no FFN formula).
"""
import numpy as np
import pytest
from scipy.special import expit

import workloads


def _rand(shape, seed, scale=1.0, dtype=np.float32):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(dtype)


def _swiglu_numpy(x, w1, w3, w2):
    """Textbook dense SwiGLU with numpy's fp64 matmul."""
    h1 = x @ w1
    return ((h1 * expit(h1)) * (x @ w3)) @ w2


def test_single_expert_is_dense_swiglu(orc):
    T, d, h = 21, 30, 17
    x = _rand((T, d), 1)
    w1, w3, w2 = _rand((1, d, h), 2, 0.2), _rand((1, d, h), 3, 0.2), _rand((1, h, d), 4, 0.2)
    got = orc.ffn(x, np.zeros(T, np.int32), w1, w3, w2, want_hidden=True)
    ref = _swiglu_numpy(x.astype(np.float64), w1[0].astype(np.float64), w3[0].astype(np.float64),
                        w2[0].astype(np.float64))
    np.testing.assert_allclose(got["ye"], ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(got["h1"], x.astype(np.float64) @ w1[0], rtol=1e-12, atol=1e-13)


def test_per_expert_rows_match_numpy(orc):
    """Tiny fp32 workload shapes: every row equals numpy's SwiGLU of its own expert."""
    wl = workloads.get("tiny_f32")
    inp = workloads.generate(wl)
    x = inp["x"].numpy()
    ids, _ = workloads.random_topk(wl.T, wl.E, wl.k, seed=5)
    rt = np.repeat(np.arange(wl.T, dtype=np.int32), wl.k)
    re_ = ids.numpy().reshape(-1)
    w1, w3, w2 = inp["w1"].numpy(), inp["w3"].numpy(), inp["w2"].numpy()
    got = orc.ffn(x, re_, w1, w3, w2, row_token=rt)["ye"]
    for e in range(wl.E):
        rows = np.nonzero(re_ == e)[0]
        ref = _swiglu_numpy(x[rt[rows]].astype(np.float64), w1[e].astype(np.float64),
                            w3[e].astype(np.float64), w2[e].astype(np.float64))
        np.testing.assert_allclose(got[rows], ref, rtol=1e-11, atol=1e-12)


def test_bf16_inputs_are_read_exactly(orc):
    """bf16 bit patterns and their exact fp64 widening give identical results."""
    import torch
    T, d, h, E = 9, 16, 8, 3
    xt = torch.randn(T, d).to(torch.bfloat16)
    wt = [torch.randn(E, d, h).to(torch.bfloat16), torch.randn(E, d, h).to(torch.bfloat16),
          torch.randn(E, h, d).to(torch.bfloat16)]
    re_ = np.array([0, 2, 1, 1, 0, 2, 2, 0, 1], np.int32)
    a = orc.ffn(workloads.bf16_bits(xt), re_, *[workloads.bf16_bits(w) for w in wt])["ye"]
    b = orc.ffn(xt.double().numpy(), re_, *[w.double().numpy() for w in wt])["ye"]
    np.testing.assert_array_equal(a, b)


def test_two_shared_experts_equal_one_twice_as_wide(orc):
    """sum_s FFN_s(x) == FFN with [W1_0|W1_1], [W3_0|W3_1], [W2_0; W2_1]."""
    T, d, h = 13, 12, 7
    x = _rand((T, d), 6)
    a = [(_rand((1, d, h), 10 + s, 0.3), _rand((1, d, h), 20 + s, 0.3), _rand((1, h, d), 30 + s, 0.3))
         for s in range(2)]
    z = np.zeros(T, np.int32)
    two = orc.ffn(x, z, *a[0])["ye"] + orc.ffn(x, z, *a[1])["ye"]
    wide = orc.ffn(x, z, np.concatenate([a[0][0], a[1][0]], 2), np.concatenate([a[0][1], a[1][1]], 2),
                   np.concatenate([a[0][2], a[1][2]], 1))["ye"]
    np.testing.assert_allclose(two, wide, rtol=1e-12, atol=1e-13)


def test_zero_input_gives_zero_output(orc):
    """silu(0) = 0: a zero row stays zero through the expert."""
    d, h = 10, 6
    w = [_rand((2, d, h), 1), _rand((2, d, h), 2), _rand((2, h, d), 3)]
    out = orc.ffn(np.zeros((3, d), np.float32), np.array([0, 1, 1], np.int32), *w)["ye"]
    assert (out == 0).all()


def test_gather_is_exact_and_adjoint_of_scatter_add(orc):
    T, d, R = 40, 9, 120
    rng = np.random.default_rng(7)
    x = _rand((T, d), 8)
    rt = rng.integers(0, T, R).astype(np.int32)
    xs = orc.gather(x, rt)
    np.testing.assert_array_equal(xs, x[rt].astype(np.float64))
    g = _rand((R, d), 9, dtype=np.float64)
    lhs = np.sum(xs * g)
    rhs = np.sum(x.astype(np.float64) * orc.scatter_add(g, rt, T))
    assert abs(lhs - rhs) <= 1e-12 * (np.abs(xs * g).sum())


def test_combine_identity_experts(orc):
    """Identity experts (Ye = Xs) give Y[t] = X[t] * sum_j w[t, j]."""
    wl = workloads.get("tiny_f32")
    x = workloads.generate(wl, experts=False)["x"].numpy()
    ids, w = workloads.random_topk(wl.T, wl.E, wl.k, seed=1)
    pft = orc.build_pft(ids.numpy(), w.numpy(), wl.E)
    xs = orc.gather(x, pft["token_ids"])
    y = orc.combine(xs, pft["token_ids"], pft["combine_weights"], wl.T)
    ref = x.astype(np.float64) * w.numpy().astype(np.float64).sum(1, keepdims=True)
    np.testing.assert_allclose(y, ref, rtol=1e-14, atol=1e-15)


def test_combine_all_experts_recovers_input(orc):
    """k = E with identity experts: the weights are the full softmax, so Y = X."""
    T, d, E = 30, 11, 6
    x, wg = _rand((T, d), 11), _rand((d, E), 12)
    r = orc.route(x, wg, E, 2)
    rt = np.repeat(np.arange(T, dtype=np.int32), E)
    y = orc.combine(orc.gather(x, rt), rt, r["topk_w"].reshape(-1), T)
    np.testing.assert_allclose(y, x.astype(np.float64), rtol=1e-13, atol=1e-14)


def test_combine_backward_adjoint_and_weight_gradient(orc):
    T, d, R = 25, 13, 75
    rng = np.random.default_rng(3)
    rt = rng.integers(0, T, R).astype(np.int32)
    rw = rng.random(R)
    ye = rng.standard_normal((R, d))
    dy = rng.standard_normal((T, d))
    y = orc.combine(ye, rt, rw, T)
    g = orc.combine_bwd(dy, ye, rt, rw)
    # adjoint in the expert output: <combine(ye), dy> = <ye, dye>
    assert abs(np.sum(y * dy) - np.sum(ye * g["dye"])) < 1e-11
    # the combine is linear in each weight: dY/dw[r] is the row ye[r] at token rt[r]
    for r in (0, 17, 74):
        bump = rw.copy()
        bump[r] += 1.0
        dl = np.sum(orc.combine(ye, rt, bump, T) * dy) - np.sum(y * dy)
        assert abs(dl - g["dw"][r]) < 1e-11


def test_y_add_is_added(orc):
    T, d = 6, 4
    ya = _rand((T, d), 13)
    y = orc.combine(np.zeros((0, d)), np.zeros(0, np.int32), np.zeros(0), T, y_add=ya)
    np.testing.assert_array_equal(y, ya.astype(np.float64))


def _tiny_layer_inputs():
    wl = workloads.get("tiny_f32")
    inp = workloads.generate(wl, backward=True)
    return wl, {k: v.numpy() for k, v in inp.items() if v is not None}


def test_layer_select_own_choice_changes_nothing(orc):
    """select= hands a token's selection to the oracle's layer (the GPU tests
    use it where a near-tie admits more than one correct selection).  Handing
    back the oracle's own selection must change nothing, bit for bit."""
    wl, o = _tiny_layer_inputs()
    ref = orc.layer_forward(o, wl.k, 0)
    own = {t: ref["route"]["topk_ids"][t].copy() for t in (0, 7, wl.T - 1)}
    got = orc.layer_forward(o, wl.k, 0, select=own)
    for key in ("y", "ye", "row_w"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
    np.testing.assert_array_equal(got["route"]["topk_ids"], ref["route"]["topk_ids"])


def test_layer_select_other_choice_is_the_textbook_mixture(orc):
    """Another selection for one token: every other token's output is bitwise
    unchanged, and the token's output is sum_j p[t, e_j] * SwiGLU_{e_j}(x_t)
    with the oracle's softmax probabilities, computed here with numpy."""
    wl, o = _tiny_layer_inputs()
    ref = orc.layer_forward(o, wl.k, 0)
    t0 = 5
    own = ref["route"]["topk_ids"][t0]
    other = np.array([e for e in range(wl.E) if e not in own.tolist()][:wl.k], np.int32)
    got = orc.layer_forward(o, wl.k, 0, select={t0: other})
    keep = np.arange(wl.T) != t0
    np.testing.assert_array_equal(got["y"][keep], ref["y"][keep])
    p = ref["route"]["probs"][t0]
    x = o["x"][t0:t0 + 1].astype(np.float64)
    want = sum(p[e] * _swiglu_numpy(x, o["w1"][e].astype(np.float64), o["w3"][e].astype(np.float64),
                                    o["w2"][e].astype(np.float64))[0] for e in other)
    np.testing.assert_allclose(got["y"][t0], want, rtol=1e-9, atol=1e-12)
    np.testing.assert_array_equal(got["route"]["topk_w"][t0], p[other].astype(got["route"]["topk_w"].dtype))


@pytest.mark.parametrize("bad", [[0, 0], [0], [0, 99], [-1, 2]])
def test_layer_select_rejects_invalid_choices(orc, bad):
    wl, o = _tiny_layer_inputs()
    with pytest.raises(orc.OracleError):
        orc.layer_forward(o, wl.k, 0, select={3: np.array(bad, np.int32)})
