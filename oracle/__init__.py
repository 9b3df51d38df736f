"""CPU oracle of the padding-free MoE layer (ctypes wrapper over liboracle.so).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product library never imports,
links or runs anything in this directory, and this directory imports nothing
from the product package.

Arrays are numpy: float32, uint16 (bf16 bit patterns) or float64 inputs;
float64 outputs (int32 for indices).  Each function is one step of the layer as
the X-MoE pages describe it (see oracle.c for the step-by-step citations); the
composites `layer_forward` / `layer_backward` chain them in slot order
(row r = t*k + j) without building the Padding-Free Token buffer, so the
oracle's layer result does not depend on its own buffer construction.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# XMOE_ORACLE_LIB names another build of oracle.c: the mutation check of the
# pins (tests/test_oracle_mutants.py) loads copies with planted mistakes this way
_LIB_PATH = os.environ.get("XMOE_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16, F64 = 0, 1, 2
_ERR = {1: "invalid argument", 2: "invalid routing (id out of range or repeated in a token)",
        3: "out of memory"}


class OracleError(RuntimeError):
    pass


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        _lib = ctypes.CDLL(_LIB_PATH)
    return _lib


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


def get_threads() -> int:
    return int(lib().orc_get_threads())


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"unsupported oracle input dtype {a.dtype}")


def _c(a: Optional[np.ndarray], dtype=None):
    if a is None:
        return None
    if dtype is not None and a.dtype != dtype:
        a = a.astype(dtype)
    return np.ascontiguousarray(a)


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError(f"{what}: {_ERR.get(rc, rc)}")


I64 = ctypes.c_int64
I32 = ctypes.c_int
DBL = ctypes.c_double


def route(x, wg, k: int, mode: int, inv_tau: float = 1.0, logit_bias=None, select_bias=None):
    """Gate: returns dict(topk_ids [T,k] i32, topk_w [T,k], scores [T,E], probs [T,E], margin [T]).

    mode 0: fp32 logits by sequential fused multiply-add (the fp32 path);
    mode 1: exact logits rounded once to fp32 (bf16 inputs);
    mode 2: all double."""
    x, wg = _c(x), _c(wg)
    T, d = x.shape
    E = wg.shape[1]
    lb, sb = _c(logit_bias, np.float32), _c(select_bias, np.float32)
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    s = np.empty((T, E), np.float64)
    p = np.empty((T, E), np.float64)
    m = np.empty((T,), np.float64)
    rc = lib().orc_route(_p(x), I32(_dt(x)), _p(wg), I32(_dt(wg)), I64(T), I32(d), I32(E), I32(k),
                         I32(mode), DBL(inv_tau), _p(lb), _p(sb), _p(ids), _p(w), _p(s), _p(p), _p(m))
    _check(rc, "route")
    return {"topk_ids": ids, "topk_w": w, "scores": s, "probs": p, "margin": m}


def build_pft(topk_ids, topk_w, E: int):
    """Padding-Free Token buffer from a routing result (bit-exact integer work)."""
    ids = _c(topk_ids, np.int32)
    w = _c(topk_w, np.float32)
    T, k = ids.shape
    R = T * k
    out = {"token_ids": np.empty(R, np.int32), "expert_ids": np.empty(R, np.int32),
           "tokens_per_expert": np.empty(E, np.int32), "expert_offsets": np.empty(E + 1, np.int32),
           "combine_weights": np.empty(R, np.float32), "slot_to_row": np.empty(R, np.int32)}
    rc = lib().orc_build_pft(_p(ids), _p(w), I64(T), I32(E), I32(k), _p(out["token_ids"]),
                             _p(out["expert_ids"]), _p(out["tokens_per_expert"]),
                             _p(out["expert_offsets"]), _p(out["combine_weights"]),
                             _p(out["slot_to_row"]))
    _check(rc, "build_pft")
    return out


def gather(x, row_token):
    x = _c(x)
    rt = _c(row_token, np.int32)
    T, d = x.shape
    xs = np.empty((rt.shape[0], d), np.float64)
    _check(lib().orc_gather(_p(x), I32(_dt(x)), _p(rt), I64(rt.shape[0]), I64(T), I32(d), _p(xs)),
           "gather")
    return xs


def ffn(xs, row_expert, w1, w3, w2, row_token=None, want_hidden: bool = False):
    """SwiGLU experts per row.  xs [rows or T, d]; w1/w3 [E,d,h]; w2 [E,h,d].
    With row_token, row r reads xs[row_token[r]].  Returns dict(ye, [h1, h3, act])."""
    xs = _c(xs)
    re_ = _c(row_expert, np.int32)
    rt = _c(row_token, np.int32)
    w1, w3, w2 = _c(w1), _c(w3), _c(w2)
    assert w1.dtype == w3.dtype == w2.dtype
    E, d, h = w1.shape
    rows = re_.shape[0]
    ye = np.empty((rows, d), np.float64)
    h1 = np.empty((rows, h), np.float64) if want_hidden else None
    h3 = np.empty((rows, h), np.float64) if want_hidden else None
    act = np.empty((rows, h), np.float64) if want_hidden else None
    rc = lib().orc_ffn(_p(xs), I32(_dt(xs)), _p(rt), _p(re_), I64(rows), I32(d), I32(h), I32(E),
                       _p(w1), _p(w3), _p(w2), I32(_dt(w1)), _p(h1), _p(h3), _p(act), _p(ye))
    _check(rc, "ffn")
    out = {"ye": ye}
    if want_hidden:
        out.update(h1=h1, h3=h3, act=act)
    return out


def ffn_bwd(xs, row_expert, w1, w3, w2, dye, row_token=None, want_dh: bool = False,
            want_dw: bool = True):
    """Backward of the SwiGLU experts.  Returns dict(dxs, dw1, dw3, dw2, [dh1, dh3, da])."""
    xs = _c(xs)
    re_ = _c(row_expert, np.int32)
    rt = _c(row_token, np.int32)
    w1, w3, w2 = _c(w1), _c(w3), _c(w2)
    dye = _c(dye)
    E, d, h = w1.shape
    rows = re_.shape[0]
    dxs = np.empty((rows, d), np.float64)
    dh1 = np.empty((rows, h), np.float64) if want_dh else None
    dh3 = np.empty((rows, h), np.float64) if want_dh else None
    da = np.empty((rows, h), np.float64) if want_dh else None
    dw1 = np.empty((E, d, h), np.float64) if want_dw else None
    dw3 = np.empty((E, d, h), np.float64) if want_dw else None
    dw2 = np.empty((E, h, d), np.float64) if want_dw else None
    rc = lib().orc_ffn_bwd(_p(xs), I32(_dt(xs)), _p(rt), _p(re_), I64(rows), I32(d), I32(h), I32(E),
                           _p(w1), _p(w3), _p(w2), I32(_dt(w1)), _p(dye), I32(_dt(dye)), _p(dxs),
                           _p(dh1), _p(dh3), _p(da), _p(dw1), _p(dw3), _p(dw2))
    _check(rc, "ffn_bwd")
    out = {"dxs": dxs}
    if want_dw:
        out.update(dw1=dw1, dw3=dw3, dw2=dw2)
    if want_dh:
        out.update(dh1=dh1, dh3=dh3, da=da)
    return out


def ffn_wgrad_cols(xs, row_expert, w1, w3, w2, dye, expert: int, cols, row_token=None):
    """dW1[e][:, cols], dW3[e][:, cols] ([d, n]) and dW2[e][cols, :] ([n, d])."""
    xs = _c(xs)
    re_ = _c(row_expert, np.int32)
    rt = _c(row_token, np.int32)
    w1, w3, w2 = _c(w1), _c(w3), _c(w2)
    dye = _c(dye)
    cols = _c(np.asarray(cols), np.int32)
    E, d, h = w1.shape
    n = cols.shape[0]
    dw1c = np.empty((d, n), np.float64)
    dw3c = np.empty((d, n), np.float64)
    dw2c = np.empty((n, d), np.float64)
    rc = lib().orc_ffn_wgrad_cols(_p(xs), I32(_dt(xs)), _p(rt), _p(re_), I64(re_.shape[0]), I32(d),
                                  I32(h), I32(E), _p(w1), _p(w3), _p(w2), I32(_dt(w1)), _p(dye),
                                  I32(_dt(dye)), I32(expert), _p(cols), I32(n), _p(dw1c), _p(dw3c),
                                  _p(dw2c))
    _check(rc, "ffn_wgrad_cols")
    return {"dw1": dw1c, "dw3": dw3c, "dw2": dw2c}


def combine(ye, row_token, row_w, T: int, y_add=None):
    ye = _c(ye, np.float64)
    rt = _c(row_token, np.int32)
    rw = _c(row_w, np.float64)
    ya = _c(y_add)
    rows, d = ye.shape
    y = np.empty((T, d), np.float64)
    rc = lib().orc_combine(_p(ye), _p(rt), _p(rw), I64(rows), I64(T), I32(d), _p(ya),
                           I32(_dt(ya) if ya is not None else 0), _p(y))
    _check(rc, "combine")
    return y


def combine_bwd(dy, ye, row_token, row_w):
    dy = _c(dy)
    ye = _c(ye, np.float64)
    rt = _c(row_token, np.int32)
    rw = _c(row_w, np.float64)
    T, d = dy.shape
    rows = rt.shape[0]
    dye = np.empty((rows, d), np.float64)
    dw = np.empty((rows,), np.float64)
    rc = lib().orc_combine_bwd(_p(dy), I32(_dt(dy)), _p(ye), _p(rt), _p(rw), I64(rows), I64(T),
                               I32(d), _p(dye), _p(dw))
    _check(rc, "combine_bwd")
    return {"dye": dye, "dw": dw}


def scatter_add(dxs, row_token, T: int, dx_add=None):
    dxs = _c(dxs)
    rt = _c(row_token, np.int32)
    da = _c(dx_add)
    d = dxs.shape[1]
    dx = np.empty((T, d), np.float64)
    rc = lib().orc_scatter_add(_p(dxs), I32(_dt(dxs)), _p(rt), I64(rt.shape[0]), I64(T), I32(d),
                               _p(da), I32(_dt(da) if da is not None else 0), _p(dx))
    _check(rc, "scatter_add")
    return dx


def route_bwd(scores, topk_ids, dtopk_w, x, wg, inv_tau: float = 1.0, want_dx=True, want_dwg=True):
    s = _c(scores, np.float64)
    ids = _c(topk_ids, np.int32)
    dw = _c(dtopk_w, np.float64)
    x, wg = _c(x), _c(wg)
    T, d = x.shape
    E = wg.shape[1]
    k = ids.shape[1]
    dz = np.empty((T, E), np.float64)
    dx = np.empty((T, d), np.float64) if want_dx else None
    dwg = np.empty((d, E), np.float64) if want_dwg else None
    rc = lib().orc_route_bwd(_p(s), _p(ids), _p(dw), _p(x), I32(_dt(x)), _p(wg), I32(_dt(wg)),
                             I64(T), I32(d), I32(E), I32(k), DBL(inv_tau), _p(dz), _p(dx), _p(dwg))
    _check(rc, "route_bwd")
    return {"dz": dz, "dx": dx, "dwg": dwg}


# ------------------------------------------------------------------ composites

def _shared_slices(s1, s3, s2, n_shared: int):
    """Shared experts stored side by side along the hidden axis -> one [1,d,h_s]
    slice per shared expert."""
    hs = s1.shape[1] // n_shared
    out = []
    for s in range(n_shared):
        out.append((np.ascontiguousarray(s1[None, :, s * hs:(s + 1) * hs]),
                    np.ascontiguousarray(s3[None, :, s * hs:(s + 1) * hs]),
                    np.ascontiguousarray(s2[None, s * hs:(s + 1) * hs, :])))
    return out


def layer_forward(inp: Dict[str, np.ndarray], k: int, mode: int, inv_tau: float = 1.0,
                  n_shared: int = 0, tokens: Optional[np.ndarray] = None,
                  expert_subset: Optional[np.ndarray] = None, select: Optional[Dict[int, np.ndarray]] = None):
    """Forward of the whole layer for every token (or only `tokens`).

    Y[t] = sum_{j} p[t, S_t(j)] * FFN_{S_t(j)}(X[t]) + sum_s FFN^shared_s(X[t]).
    With expert_subset (sorted expert ids), inp's w1/w3/w2 hold only those
    experts, in that order; every routed expert must be in the subset.
    select {t: ids[k]}: token t's selection is taken as given instead of the
    oracle's own (for a near-tie, where more than one selection is correct);
    its weights are still the oracle's probabilities of those experts.
    Returns a dict with the routing, the per-slot expert outputs and y."""
    x = inp["x"]
    if tokens is not None:
        x = np.ascontiguousarray(x[tokens])
    T = x.shape[0]
    r = route(x, inp["wg"], k, mode, inv_tau, inp.get("logit_bias"), inp.get("select_bias"))
    for t, ids in (select or {}).items():
        ids = np.asarray(ids, np.int32)
        if ids.shape != (k,) or len(set(ids.tolist())) != k or ids.min() < 0 or ids.max() >= r["probs"].shape[1]:
            raise OracleError(f"select: token {t} needs {k} distinct experts")
        r["topk_ids"][t] = ids
        r["topk_w"][t] = r["probs"][t, ids]
    row_token = np.repeat(np.arange(T, dtype=np.int32), k)
    row_expert = r["topk_ids"].reshape(-1)
    if expert_subset is not None:
        sub = np.asarray(expert_subset)
        pos = np.searchsorted(sub, row_expert)
        if (pos >= sub.size).any() or (sub[np.minimum(pos, sub.size - 1)] != row_expert).any():
            raise OracleError("a token routes to an expert outside expert_subset")
        row_expert = pos.astype(np.int32)
    row_w = r["topk_w"].reshape(-1)
    f = ffn(x, row_expert, inp["w1"], inp["w3"], inp["w2"], row_token=row_token, want_hidden=True)
    ysh = None
    sh = []
    if n_shared:
        ysh = np.zeros((T, x.shape[1]), np.float64)
        zeros = np.zeros(T, np.int32)
        for (a, b, c) in _shared_slices(inp["s1"], inp["s3"], inp["s2"], n_shared):
            g = ffn(x, zeros, a, b, c, want_hidden=True)
            ysh += g["ye"]
            sh.append(g)
    y = combine(f["ye"], row_token, row_w, T, y_add=ysh)
    return {"x": x, "route": r, "row_token": row_token, "row_expert": row_expert, "row_w": row_w,
            "ye": f["ye"], "h1": f["h1"], "h3": f["h3"], "act": f["act"], "ysh": ysh, "shared": sh, "y": y}


def layer_backward(inp: Dict[str, np.ndarray], fwd: Dict, dy: np.ndarray, inv_tau: float = 1.0,
                   n_shared: int = 0, want_dw: bool = True):
    """Exact gradient of the layer with the selection held fixed.

    dX = scatter_add(dXs) + dX_shared + dz.Wg^T;  dW* per expert; dWg = X^T dz."""
    x = fwd["x"]
    T = x.shape[0]
    cb = combine_bwd(dy, fwd["ye"], fwd["row_token"], fwd["row_w"])
    fb = ffn_bwd(x, fwd["row_expert"], inp["w1"], inp["w3"], inp["w2"], cb["dye"],
                 row_token=fwd["row_token"], want_dw=want_dw, want_dh=True)
    dx_sh = None
    sh_grads = []
    if n_shared:
        dx_sh = np.zeros_like(x, dtype=np.float64)
        zeros = np.zeros(T, np.int32)
        for (a, b, c) in _shared_slices(inp["s1"], inp["s3"], inp["s2"], n_shared):
            g = ffn_bwd(x, zeros, a, b, c, dy, want_dw=want_dw, want_dh=True)
            dx_sh += g["dxs"]
            sh_grads.append(g)
    dx_moe = scatter_add(fb["dxs"], fwd["row_token"], T, dx_add=dx_sh)
    k = fwd["route"]["topk_ids"].shape[1]
    rb = route_bwd(fwd["route"]["scores"], fwd["route"]["topk_ids"], cb["dw"].reshape(T, k), x,
                   inp["wg"], inv_tau)
    out = {"dye": cb["dye"], "dtopk_w": cb["dw"].reshape(T, k), "dxs": fb["dxs"], "da": fb["da"],
           "dh1": fb["dh1"], "dh3": fb["dh3"], "dx_moe": dx_moe, "dx": dx_moe + rb["dx"], "dz": rb["dz"],
           "dwg": rb["dwg"], "shared": sh_grads}
    if want_dw:
        out.update(dw1=fb["dw1"], dw3=fb["dw3"], dw2=fb["dw2"])
        if n_shared:
            out["ds1"] = np.concatenate([g["dw1"][0] for g in sh_grads], axis=1)
            out["ds3"] = np.concatenate([g["dw3"][0] for g in sh_grads], axis=1)
            out["ds2"] = np.concatenate([g["dw2"][0] for g in sh_grads], axis=0)
    return out
