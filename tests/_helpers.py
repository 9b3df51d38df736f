"""Shared test helpers: comparison to the oracle under the stated tolerances.

Tolerance (one reading for every floating-point output): normwise
||g - r||_2 <= rtol * ||r||_2 and elementwise |g - r| <= rtol * (|r| + floor),
with rtol = 1e-4 for fp32 workloads and 2e-2 for bf16 workloads (an fp64 oracle
on the identical bf16 inputs).  The floor is rms(r) for outputs computed
element by element.  For outputs that are sums over rows (weight gradients
c_ij = sum_r a_ri b_rj) it is the root-sum-square of the summed terms,
sqrt(sum_r (a_ri b_rj)^2), taken from the oracle's fp64 factors: each term
carries the rounding of its bf16 factors, so that is the scale of the sum's
error, and a sum whose terms cancel has no meaningful relative error of its
own.  The floor keeps entries near zero from producing meaningless relative
errors.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

RTOL = {"f32": 1e-4, "bf16": 2e-2}

# Bound on the tokens whose GPU selection differs from the oracle's inside a
# near-tie (both correct; see routing_check), per workload.  Measured: 0-1.
NEAR_TIE_MAX = 8

# Lines printed at the end of the pytest run (tests/conftest.py), so that a
# quiet run still shows the near-tie counts and how much of each tolerance the
# outputs use.
REPORT: list = []


def report(line: str) -> None:
    REPORT.append(line)


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def host(t: torch.Tensor) -> np.ndarray:
    """GPU/CPU tensor -> float64 (floats) or int array on the host."""
    t = t.detach().cpu()
    if t.dtype in (torch.int32, torch.int64):
        return t.numpy()
    return t.to(torch.float64).numpy()


def orc_in(t: torch.Tensor) -> np.ndarray:
    """Tensor -> oracle input: bf16 as uint16 bit patterns, fp32 as float32."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype == torch.int32:
        return t.numpy()
    raise TypeError(t.dtype)


def rss_rows(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """sqrt(sum_r (a[r,i] * b[r,j])^2): the scale of c = a^T b's rounding error."""
    return np.sqrt(np.maximum((a * a).T @ (b * b), 0.0))


def assert_close(got, ref, rtol: float, name: str = "", floor=None):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{name}: non-finite output"
    if ref.size == 0:
        return {"elem": 0.0, "norm": 0.0}
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = np.abs(got - ref)
    lim = rtol * (np.abs(ref) + (rms if floor is None else np.asarray(floor, np.float64)))
    bad = err > lim
    if bad.any():
        i = np.unravel_index(np.argmax(err - lim), err.shape)
        fl = rms if floor is None else float(np.broadcast_to(floor, err.shape)[i])
        raise AssertionError(f"{name}: {int(bad.sum())}/{err.size} elements beyond tolerance; worst at {i}: "
                             f"got {got[i]!r} ref {ref[i]!r} (floor {fl:.3e}, rms {rms:.3e}, rtol {rtol})")
    nrm = float(np.linalg.norm(ref))
    rel = 0.0
    if nrm > 0:
        rel = float(np.linalg.norm(got - ref)) / nrm
        assert rel <= rtol, f"{name}: normwise relative error {rel:.3e} > {rtol}"
    # the largest err / limit over the elements (1.0 = at the tolerance) and
    # the normwise error as a fraction of rtol
    used = float(np.max(np.where(lim > 0, err / np.where(lim > 0, lim, 1.0), 0.0)))
    return {"elem": used, "norm": rel / rtol}


def routing_check(gpu_ids: np.ndarray, gpu_logits: np.ndarray, orc, select_bias, k: int, score_tol: float,
                  stats: dict = None):
    """Compare the GPU's top-k with the oracle's.

    Both sides decide in fp32 on their own logits; the GPU's logits may differ
    from the oracle's by rounding.  With delta = 2 * max |s_gpu - s_oracle|
    (checked against score_tol), a token whose top-(k+1) fp32 selection keys
    are all more than delta apart has one correct answer and must match
    exactly; for the others any choice consistent within delta is correct and
    is checked for validity.  Returns the boolean mask of tokens whose GPU
    expert set differs from the oracle's."""
    s_orc = orc["scores"]
    T, E = s_orc.shape
    diff = float(np.max(np.abs(gpu_logits - s_orc))) if s_orc.size else 0.0
    scale = float(np.max(np.abs(s_orc))) if s_orc.size else 1.0
    assert diff <= score_tol * max(scale, 1.0), f"router scores differ by {diff:.3e}"
    sel = s_orc.astype(np.float32)
    if select_bias is not None:
        sel = (sel + np.asarray(select_bias, np.float32)).astype(np.float32)
    sel = sel.astype(np.float64)
    # two fp32 roundings of the bias add may also differ by an ulp
    delta = 2.0 * diff + 4.0 * np.finfo(np.float32).eps * max(float(np.max(np.abs(sel))), 1.0)
    order = np.argsort(-sel, axis=1, kind="stable")
    top = np.take_along_axis(sel, order[:, :min(k + 1, E)], 1)
    gaps = -np.diff(top, axis=1)
    ambiguous = (gaps.min(axis=1) <= delta) if gaps.shape[1] else np.zeros(T, bool)
    oid = orc["topk_ids"]
    clear = ~ambiguous
    if stats is not None:
        stats.update(delta=delta, ambiguous=int(ambiguous.sum()))
    np.testing.assert_array_equal(gpu_ids[clear], oid[clear])
    mismatch = np.zeros(T, bool)
    for t in np.nonzero(ambiguous)[0]:
        g = gpu_ids[t]
        assert len(set(g.tolist())) == k and g.min() >= 0 and g.max() < E
        kth = sel[t, order[t, k - 1]]
        nxt = sel[t, order[t, k]] if k < E else -np.inf
        gs = sel[t, g]
        assert (gs >= kth - delta).all(), (t, g, gs, kth, delta)
        must = np.nonzero(sel[t] > nxt + delta)[0]
        assert set(must.tolist()) <= set(g.tolist()), (t, must, g)
        assert (np.diff(gs) <= delta).all(), (t, gs)
        mismatch[t] = set(g.tolist()) != set(oid[t].tolist())
    if stats is not None:
        stats["mismatch"] = int(mismatch.sum())
    return mismatch


def near_tie_bound(name: str, stats: dict, T: int) -> None:
    """Report the near-tie counts and hold the differently routed ones to
    NEAR_TIE_MAX."""
    report(f"{name}: near-tied tokens {stats['ambiguous']}, routed differently {stats['mismatch']} of {T} "
           f"(bound {NEAR_TIE_MAX}; delta {stats['delta']:.2e})")
    assert stats["mismatch"] <= NEAR_TIE_MAX, \
        f"{name}: {stats['mismatch']} tokens routed differently inside near-ties (bound {NEAR_TIE_MAX})"


def pft_contract(pft: dict, ids: np.ndarray, w: np.ndarray, E: int, orc_mod) -> None:
    """The buffer given its routing: the oracle's construction from the same
    (ids, w) must equal the device's buffer in all six fields, bit for bit,
    whatever the near-ties (the buffer is a function of the routing alone),
    and the buffer must have every property of a valid one."""
    ref = orc_mod.build_pft(ids, np.asarray(w, np.float32), E)
    for key in ("token_ids", "expert_ids", "tokens_per_expert", "expert_offsets", "slot_to_row"):
        np.testing.assert_array_equal(pft[key], ref[key], err_msg=key)
    np.testing.assert_array_equal(pft["combine_weights"].view(np.uint32), ref["combine_weights"].view(np.uint32),
                                  err_msg="combine_weights")
    pft_invariants(ids, w, E, pft)


def wgrad_acc(dtype: str, K: int) -> float:
    """Weight of H1/H3's summation error in the weight-gradient floors, in
    units of the stored values' rounding (see swiglu_wgrad_scales): fp32 keeps
    H unrounded, so its error is the fp32 sum's, 1 in units of 2^-24 per
    root-sum-square of the products; bf16 rounds H to 2^-9 relative, and the
    fp32 sum over K products adds about 2^-24 sqrt(K) of their rss, which is
    2^-15 sqrt(K) in bf16 units (taken 4x: 2^-13 sqrt(K))."""
    return 1.0 if dtype == "f32" else 2.0 ** -13 * float(np.sqrt(K))


def swiglu_wgrad_scales(x, da, h1, h3, act, dye, w2, w13=None, acc=1.0):
    """Root-sum-square error scales of one expert's weight gradients.

    dW1 = x^T dH1 with dH1 = dA*H3*g(H1), g(a) = sig(a)(1 + a(1 - sig(a))):
    rounding H1 and H3 to bf16 moves dH1 by up to ~2.3 * 2^-9 * |dA*H3|
    (|g| <= 1.1 and |a g'(a)| <= 0.13), whatever the size of dH1 itself --
    g has a zero near a = -1.28, where dH1 vanishes but its error does not.
    Likewise dH3 = dA*silu(H1) moves by ~|dA*H1| * 2^-9.  dA = dYe.W2^T itself
    carries the rounding of dYe, whose scale is the root-sum-square of the
    terms dYe*W2 (not |dA|, which may cancel), so the magnitude used for dA is
    |dA| + sqrt(dYe^2 . (W2^2)^T).  dW2 = act^T dYe carries the rounding of act
    and dYe.  The scales are the root-sum-square over rows of those
    magnitudes; every input is an oracle (fp64) value or a generator input.

    H1 and H3 are sums of d products, whose summation error scales with the
    root-sum-square of the products, s = sqrt(x^2 . W^2), not with |H|: where
    H cancels to near zero that error dominates.  With w13 = (W1, W3) given,
    the magnitudes become |H1| + acc*s1 and |H3| + acc*s3 (acc from
    wgrad_acc), dH1 also carries H1's error through g (|g'| <= 0.5), and act =
    silu(H1) H3 carries both."""
    w2 = np.asarray(w2, np.float64)
    dam = np.abs(da) + np.sqrt(np.maximum((dye * dye) @ (w2 * w2).T, 0.0))
    a1, a3 = np.abs(h1), np.abs(h3)
    if w13 is None:
        return (rss_rows(x, dam * a3), rss_rows(x, dam * a1), rss_rows(act, dye))
    x2 = np.asarray(x, np.float64) ** 2
    s1 = acc * np.sqrt(np.maximum(x2 @ (np.asarray(w13[0], np.float64) ** 2), 0.0))
    s3 = acc * np.sqrt(np.maximum(x2 @ (np.asarray(w13[1], np.float64) ** 2), 0.0))
    return (rss_rows(x, dam * (a3 + s3 + a3 * s1)), rss_rows(x, dam * (a1 + s1)),
            rss_rows(np.abs(act) + s1 * a3 + a1 * s3, dye))


def assert_wgrad_close(got, ref, rows_of, floors_of, rtol: float, name: str):
    """Per-expert weight gradient: normwise per expert that has rows,
    elementwise with the given per-expert floor, exact zeros for experts
    without rows.  rows_of(e) -> number of rows; floors_of(e) -> floor array."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    worst = {"elem": 0.0, "norm": 0.0}
    for e in range(ref.shape[0]):
        if rows_of(e) == 0:
            assert (got[e] == 0).all(), f"{name}[{e}]: expert without rows must get a zero gradient"
            continue
        u = assert_close(got[e], ref[e], rtol, f"{name}[{e}]", floor=floors_of(e))
        worst = {key: max(worst[key], u[key]) for key in worst}
    return worst


def used_str(used: dict) -> str:
    return f"{used['elem']:.2f}/{used['norm']:.2f}"


def by_expert(ids: np.ndarray, vals: np.ndarray) -> np.ndarray:
    """Per-slot values reordered by expert id within each token, so that two
    routings that chose the same experts in a different slot order compare."""
    order = np.argsort(ids, axis=1, kind="stable")
    return np.take_along_axis(np.asarray(vals), order, 1)


def buffer_routing(layer, ids: np.ndarray, w: np.ndarray):
    """(ids, w, E) of the routing a layer's buffer holds: the routed slots, then,
    when the layer carries its shared experts as always-routed ones, one slot
    per shared expert (experts E .. E+n-1) with weight 1."""
    if not getattr(layer, "merged", False):
        return ids, w, layer.E
    T, ns, E = ids.shape[0], layer.ns, layer.E
    ids_b = np.concatenate([ids, np.tile(np.arange(E, E + ns, dtype=ids.dtype), (T, 1))], axis=1)
    w_b = np.concatenate([np.asarray(w, np.float32), np.ones((T, ns), np.float32)], axis=1)
    return ids_b, w_b, E + ns


def pft_invariants(ids: np.ndarray, w: np.ndarray, E: int, pft: dict):
    """Properties every valid Padding-Free Token buffer of routing (ids, w) has:
    T*k rows, each token k times, each (token, expert) once, rows grouped by
    ascending expert with tokens ascending inside a group, offsets = scan of
    the counts, slot_to_row consistent with the routing, weights copied bit
    for bit.  Checks a buffer against its own routing, without any oracle."""
    T, k = ids.shape
    R = T * k
    tpe, off = pft["tokens_per_expert"], pft["expert_offsets"]
    eid = pft["expert_ids"]
    assert tpe.shape == (E,) and off.shape == (E + 1,) and eid.shape == (R,)
    assert tpe.sum() == R and off[0] == 0 and off[-1] == R and (np.diff(off) == tpe).all()
    # the counts are those of the rows' experts, and each expert's segment
    # [off[e], off[e+1]) holds exactly its rows
    assert eid.min(initial=0) >= 0 and eid.max(initial=0) < E
    np.testing.assert_array_equal(tpe, np.bincount(eid, minlength=E), err_msg="tokens_per_expert")
    np.testing.assert_array_equal(eid, np.repeat(np.arange(E, dtype=eid.dtype), tpe), err_msg="expert segments")
    np.testing.assert_array_equal(tpe, np.bincount(np.asarray(ids).reshape(-1), minlength=E),
                                  err_msg="tokens_per_expert against the routing")
    assert (np.bincount(pft["token_ids"], minlength=T) == k).all()
    assert np.unique(pft["token_ids"].astype(np.int64) * E + pft["expert_ids"]).size == R
    assert (np.diff(pft["expert_ids"]) >= 0).all()
    same = np.diff(pft["expert_ids"]) == 0
    assert (np.diff(pft["token_ids"])[same] > 0).all()
    assert (pft["expert_ids"][off[:-1][tpe > 0]] == np.nonzero(tpe > 0)[0]).all()
    s2r = pft["slot_to_row"].reshape(T, k)
    assert (pft["token_ids"][s2r] == np.arange(T)[:, None]).all()
    assert (pft["expert_ids"][s2r] == ids).all()
    np.testing.assert_array_equal(pft["combine_weights"][s2r].view(np.uint32), np.asarray(w, np.float32).view(np.uint32))


def _f64(a) -> np.ndarray:
    """Oracle input (bf16 bit patterns as uint16, or fp32) -> float64."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def dx_floor(o, fwd, bwd, dy, n_shared: int = 0) -> np.ndarray:
    """Error scale of the layer's input gradient dX, per element.

    dX[t] = sum_j dXs[row(t,j)] + sum_s dXsh_s[t] + dz[t].Wg^T.  Each expert
    term is dXs[r] = dH1[r].W1^T + dH3[r].W3^T over the expert width, whose
    factors dH1 and dH3 carry the rounding of H1, H3 and dA: it moves them by
    amounts that scale with |dA*H3| and |dA*H1| (swiglu_wgrad_scales), not with
    |dH1|, |dH3|, and the magnitude used for dA again includes the root-sum-
    square of its own terms dYe*W2.  Where one heavily weighted expert's
    products cancel inside dXs, neither |dX| nor its rms shows that error.  The
    scale is therefore the root-sum-square, over every term of dX[t], of the
    magnitudes of the products inside it (expert terms as above, shared
    experts alike with dY in place of dYe, and the gate's dz*Wg), together with
    the terms themselves (each is rounded before the sum).  o: the oracle's
    inputs (routed weights in the order of fwd's row experts); dy: the
    upstream gradient of fwd's tokens; every value is an oracle (fp64) value
    or a generator input."""
    dx = bwd["dx"]
    F2 = np.zeros(dx.shape)

    def add(tok, da, dye, h1, h3, w1, w3, w2, dxs):
        # w1, w3 [d, h]; w2 [h, d]; rows of da, h1, h3 [., h] and dye, dxs [., d]
        dam = np.abs(da) + np.sqrt(np.maximum((dye * dye) @ (w2 * w2).T, 0.0))
        m1, m3 = dam * np.abs(h3), dam * np.abs(h1)
        np.add.at(F2, tok, (m1 * m1) @ (w1 * w1).T + (m3 * m3) @ (w3 * w3).T + dxs * dxs)

    W1, W3, W2 = _f64(o["w1"]), _f64(o["w3"]), _f64(o["w2"])
    re_, rt = fwd["row_expert"], fwd["row_token"]
    for e in np.unique(re_):
        r = np.nonzero(re_ == e)[0]
        add(rt[r], bwd["da"][r], bwd["dye"][r], fwd["h1"][r], fwd["h3"][r], W1[e], W3[e], W2[e], bwd["dxs"][r])
    if n_shared:
        S1, S3, S2 = _f64(o["s1"]), _f64(o["s3"]), _f64(o["s2"])
        hs = S1.shape[1] // n_shared
        dyf = _f64(dy)
        tok = np.arange(dx.shape[0])
        for s_ in range(n_shared):
            cs = slice(s_ * hs, (s_ + 1) * hs)
            f, b = fwd["shared"][s_], bwd["shared"][s_]
            add(tok, b["da"], dyf, f["h1"], f["h3"], S1[:, cs], S3[:, cs], S2[cs, :], b["dxs"])
    Wg = _f64(o["wg"])
    F2 += (bwd["dz"] ** 2) @ (Wg * Wg).T
    return np.sqrt(F2)


def router_wgrad_floor(x, probs, ids, ye_slot, dy, dz, inv_tau):
    """Error scale of dWg = x^T dz when dz comes out of the layer's own chain.

    dz[t,e] = p[t,e] * (g[t,e] - c_t) * inv_tau with g the routing-weight
    gradient <dy[t], Ye[t,j]> at the chosen experts.  Those dot products carry
    the bf16 rounding of Ye; their error scale is G[t,j] = sqrt(sum_c
    (dy[t,c] Ye[t,j,c])^2), which g - c may cancel but its error does not.
    The magnitude per term is |dz| + inv_tau * p * (G + sum_j p_j G_j), and the
    floor is its root-sum-square over tokens (oracle values throughout)."""
    T, k = ids.shape
    G = np.sqrt(((ye_slot.reshape(T, k, -1) * dy[:, None, :]) ** 2).sum(-1))
    Gfull = np.zeros_like(probs)
    np.put_along_axis(Gfull, ids, G, 1)
    pc = (np.take_along_axis(probs, ids, 1) * G).sum(1, keepdims=True)
    mag = np.abs(dz) + inv_tau * probs * (Gfull + pc)
    return rss_rows(x, mag)
