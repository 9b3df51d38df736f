"""Pins of the oracle's Padding-Free Token buffer construction.

X-MoE article (adg.csdn.net), section 2.1.1 "PFT数据结构创新": token_ids are
positions in the input, expert_ids the target experts, tokens_per_expert the
per-expert counts, combine_weights the combine coefficients; section 2.1.2:
experts are visited in ascending id and each expert's rows keep the input
order, with no padding and (section 2.1.1) no dropped tokens.
"""
import json
import os

import numpy as np
import pytest

import workloads

HERE = os.path.dirname(os.path.abspath(__file__))


def test_hand_worked_example(orc):
    g = json.load(open(os.path.join(HERE, "golden", "pft_tiny.json")))
    ids = np.array(g["topk_ids"], np.int32)
    w = np.array(g["topk_w"], np.float32)
    out = orc.build_pft(ids, w, g["E"])
    for key, val in g["expected"].items():
        if key == "combine_weights":
            np.testing.assert_array_equal(out[key], np.array(val, np.float32))
        else:
            assert out[key].tolist() == val, key


def _check_invariants(ids, w, E, out):
    T, k = ids.shape
    R = T * k
    tpe, off = out["tokens_per_expert"], out["expert_offsets"]
    assert tpe.sum() == R                                     # nothing dropped, nothing padded
    assert off[0] == 0 and off[-1] == R and (np.diff(off) == tpe).all()
    assert (np.bincount(out["token_ids"], minlength=T) == k).all()   # each token k times
    pairs = out["token_ids"].astype(np.int64) * E + out["expert_ids"]
    assert np.unique(pairs).size == R                        # (t, e) at most once
    for e in range(E):
        seg = slice(off[e], off[e + 1])
        assert (out["expert_ids"][seg] == e).all()
        assert (np.diff(out["token_ids"][seg]) > 0).all()     # input order kept
    s2r = out["slot_to_row"].reshape(T, k)
    assert (out["token_ids"][s2r] == np.arange(T)[:, None]).all()
    assert (out["expert_ids"][s2r] == ids).all()
    np.testing.assert_array_equal(out["combine_weights"][s2r], w)   # bit-for-bit


@pytest.mark.parametrize("T,E,k,skew", [(1000, 37, 5, 0.0), (513, 64, 6, 0.0), (700, 128, 8, 2.5),
                                        (64, 8, 8, 0.0), (1, 4, 1, 0.0), (0, 5, 2, 0.0)])
def test_invariants_and_counting_sort(orc, T, E, k, skew):
    if T:
        ids_t, w_t = workloads.random_topk(T, E, k, seed=T + E, skew=skew)
        ids, w = ids_t.numpy(), w_t.numpy()
    else:
        ids, w = np.zeros((0, k), np.int32), np.zeros((0, k), np.float32)
    out = orc.build_pft(ids, w, E)
    _check_invariants(ids, w, E, out)
    # a library stable sort of the (expert, token) keys gives the same rows
    flat_e = ids.reshape(-1).astype(np.int64)
    flat_t = np.repeat(np.arange(T, dtype=np.int64), k)
    order = np.argsort(flat_e * max(T, 1) + flat_t, kind="stable")
    np.testing.assert_array_equal(out["token_ids"], flat_t[order])
    np.testing.assert_array_equal(out["expert_ids"], flat_e[order])
    np.testing.assert_array_equal(out["tokens_per_expert"], np.bincount(flat_e, minlength=E))
    if skew > 0:
        assert (out["tokens_per_expert"] == 0).any()


def test_zero_gate_closed_form(orc):
    """Wg = 0 routes every token to experts 0..k-1: counts [T]*k + [0]*(E-k) and
    token_ids = 0..T-1 repeated k times."""
    T, d, E, k = 97, 8, 12, 4
    x = np.random.default_rng(0).standard_normal((T, d)).astype(np.float32)
    r = orc.route(x, np.zeros((d, E), np.float32), k, 1)
    out = orc.build_pft(r["topk_ids"], r["topk_w"].astype(np.float32), E)
    assert out["tokens_per_expert"].tolist() == [T] * k + [0] * (E - k)
    assert out["token_ids"].tolist() == list(range(T)) * k
    assert out["expert_ids"].tolist() == sum([[e] * T for e in range(k)], [])


def test_rejects_invalid_routing(orc):
    with pytest.raises(orc.OracleError):
        orc.build_pft(np.array([[0, 0]], np.int32), np.ones((1, 2), np.float32), 4)
    with pytest.raises(orc.OracleError):
        orc.build_pft(np.array([[0, 4]], np.int32), np.ones((1, 2), np.float32), 4)


def test_zipf_workload_load_shape(orc):
    """The skewed workload at full size (16384 tokens, 2048 wide, 128 experts,
    top-8, Zipf(1.2) logit offset): some experts get no token, the busiest gets
    more than 10x the mean, and no token is dropped."""
    wl = workloads.get("zipf_skew")
    inp = workloads.generate(wl, experts=False, backward=False)
    r = orc.route(workloads.bf16_bits(inp["x"]), workloads.bf16_bits(inp["wg"]), wl.k, 1,
                  wl.inv_tau, inp["logit_bias"].numpy())
    out = orc.build_pft(r["topk_ids"], r["topk_w"].astype(np.float32), wl.E)
    tpe = out["tokens_per_expert"]
    assert tpe.sum() == wl.T * wl.k
    assert (tpe == 0).sum() > 0
    assert tpe.max() > 10 * tpe.mean()


def _corruptions(out):
    """Buffers that break one property each, built from a valid one."""
    bad = []

    def mod(key, f):
        o = {k: v.copy() for k, v in out.items()}
        f(o[key])
        bad.append((key, o))

    # counts and offsets that no longer match the rows' experts (totals kept)
    def shift_count(a):
        a[0] += 1
        a[1] -= 1
    mod("tokens_per_expert", shift_count)
    o = {k: v.copy() for k, v in out.items()}
    shift_count(o["tokens_per_expert"])
    o["expert_offsets"][1:] = np.cumsum(o["tokens_per_expert"])
    bad.append(("tokens_per_expert+offsets", o))
    mod("expert_ids", lambda a: a.__setitem__(0, a[-1]))      # a row in the wrong expert
    mod("token_ids", lambda a: a.__setitem__(slice(0, 2), a[1::-1].copy()))  # order inside a segment
    mod("slot_to_row", lambda a: a.__setitem__(slice(0, 2), a[1::-1].copy()))
    mod("combine_weights", lambda a: a.__setitem__(0, np.nextafter(a[0], np.float32(2))))
    return bad


def test_gpu_side_invariant_check_catches_corruptions(orc):
    """The validity check the GPU tests apply to the device's buffer (tests/
    _helpers.pft_invariants) accepts the oracle's buffer and rejects each
    planted corruption, including counts that disagree with the expert
    segments while their sum and scan stay consistent."""
    from _helpers import pft_invariants
    ids_t, w_t = workloads.random_topk(40, 6, 2, seed=3)
    ids, w = ids_t.numpy(), w_t.numpy()
    out = orc.build_pft(ids, w, 6)
    pft_invariants(ids, w, 6, out)
    for what, o in _corruptions(out):
        with pytest.raises(AssertionError):
            pft_invariants(ids, w, 6, o)
            print("not caught:", what)
    # the counterexample of four rows: expert_ids [0,0,1,1] with counts [3,1]
    four = {"token_ids": np.arange(4, dtype=np.int32), "expert_ids": np.array([0, 0, 1, 1], np.int32),
            "tokens_per_expert": np.array([3, 1], np.int32), "expert_offsets": np.array([0, 3, 4], np.int32),
            "combine_weights": np.ones(4, np.float32), "slot_to_row": np.arange(4, dtype=np.int32)}
    with pytest.raises(AssertionError):
        pft_invariants(np.array([[0], [0], [1], [1]], np.int32), np.ones((4, 1), np.float32), 2, four)
