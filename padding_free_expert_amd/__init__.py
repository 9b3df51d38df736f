"""Padding-free MoE layer for AMD Instinct MI355X (gfx950).

Thin ctypes binding of libxmoe.so (the C ABI in include/xmoe.h): the same entry
points under the same names, taking torch tensors that already live on the GPU.
The binding only marshals arguments -- pointers, sizes, the current HIP stream
-- and every step of the layer runs in the library's HIP kernels.  There is no
CPU or PyTorch fallback: if the library is missing the import fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "XmoeError", "PFT", "lib_path", "xmoe_version", "xmoe_query_device", "xmoe_route",
    "xmoe_route_workspace_size",
    "xmoe_build_pft_workspace_size", "xmoe_build_pft", "xmoe_build_pft_noalloc", "xmoe_build_pft_noalloc_max_bytes",
    "xmoe_build_pft_shared", "xmoe_dispatch", "xmoe_expert_ffn_up",
    "xmoe_expert_ffn_down", "xmoe_expert_ffn", "xmoe_expert_ffn_up_gather", "xmoe_expert_ffn_gather",
    "xmoe_combine", "xmoe_combine_bwd",
    "xmoe_expert_ffn_bwd", "xmoe_expert_ffn_bwd_dact", "xmoe_expert_ffn_bwd_dact_gather", "xmoe_expert_ffn_bwd_dx", "xmoe_expert_ffn_bwd_dw13", "xmoe_expert_ffn_bwd_dw13_gather",
    "xmoe_expert_ffn_bwd_dw2", "xmoe_dispatch_bwd", "xmoe_route_bwd_workspace_size", "xmoe_route_bwd",
    "xmoe_build_pilots_workspace_size", "xmoe_build_pilots", "xmoe_ep_send_plan", "xmoe_ep_recv_plan_workspace_size",
    "xmoe_ep_recv_plan", "xmoe_scatter_rows",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_FILE = os.path.join(_HERE, "libxmoe.so")

if not os.path.exists(_LIB_FILE):
    raise ImportError(f"{_LIB_FILE} is not built; run __graft_entry__.build() (or "
                      f"python padding_free_expert_amd/build.py) first")

_lib = ctypes.CDLL(_LIB_FILE)

XMOE_F32, XMOE_BF16 = 0, 1
_STATUS = {0: "ok", 1: "invalid value", 2: "unsupported", 3: "workspace", 4: "hip error"}

_vp, _i64, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t


class _CPft(ctypes.Structure):
    _fields_ = [("token_ids", _vp), ("expert_ids", _vp), ("tokens_per_expert", _vp),
                ("expert_offsets", _vp), ("combine_weights", _vp), ("slot_to_row", _vp)]


def _sig(name, args, res=ctypes.c_int):
    f = getattr(_lib, name)
    f.argtypes = args
    f.restype = res
    return f


_lib_last_error = _sig("xmoe_last_error", [], ctypes.c_char_p)
_lib_version = _sig("xmoe_version", [])
_lib_query = _sig("xmoe_query_device", [ctypes.c_int, ctypes.POINTER(ctypes.c_int)])
_lib_route = _sig("xmoe_route", [_vp, _vp, ctypes.c_int, _i64, _i32, _i32, _i32, _f32, _vp, _vp, _vp, _vp,
                                 _vp, _vp, _sz, _vp])
_lib_route_ws = _sig("xmoe_route_workspace_size", [_i64, _i32, _i32, ctypes.c_int], _sz)
_lib_pft_ws = _sig("xmoe_build_pft_workspace_size", [_i64, _i32, _i32], _sz)
_lib_pft = _sig("xmoe_build_pft", [_vp, _vp, _i64, _i32, _i32, ctypes.POINTER(_CPft), _vp, _sz, _vp])
_lib_dispatch = _sig("xmoe_dispatch", [_vp, ctypes.c_int, _i64, _i32, _i32, ctypes.POINTER(_CPft), _vp, _vp])
_lib_up = _sig("xmoe_expert_ffn_up", [_vp, _vp, _vp, ctypes.c_int, _vp, _i32, _i64, _i32, _i32, _vp, _vp, _vp])
_lib_down = _sig("xmoe_expert_ffn_down", [_vp, _vp, ctypes.c_int, _vp, _i32, _i64, _i32, _i32, _vp, _i32, _vp])
_lib_ffn = _sig("xmoe_expert_ffn", [_vp, _vp, _vp, _vp, ctypes.c_int, _vp, _i32, _i64, _i32, _i32, _vp, _vp,
                                    _vp, _i32, _vp])
_lib_up_g = _sig("xmoe_expert_ffn_up_gather", [_vp, _vp, _vp, _vp, ctypes.c_int, _vp, _i32, _i64, _i64, _i32, _i32,
                                                _vp, _vp, _vp])
_lib_ffn_g = _sig("xmoe_expert_ffn_gather", [_vp, _vp, _vp, _vp, _vp, ctypes.c_int, _vp, _i32, _i64, _i64, _i32,
                                             _i32, _vp, _vp, _vp, _i32, _vp])
_lib_combine = _sig("xmoe_combine", [_vp, ctypes.POINTER(_CPft), _i64, _i32, _i32, ctypes.c_int, _vp, _vp, _vp])
_lib_combine_bwd = _sig("xmoe_combine_bwd", [_vp, _vp, ctypes.POINTER(_CPft), _i64, _i32, _i32, ctypes.c_int,
                                             _vp, _vp, _vp])
_lib_ffn_bwd = _sig("xmoe_expert_ffn_bwd", [_vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _vp, _i32, _i64,
                                            _i32, _i32, _vp, _vp, _i32, _vp, _vp, _vp, ctypes.c_int, _i32, _vp])
_lib_bwd_dact = _sig("xmoe_expert_ffn_bwd_dact", [_vp, _vp, _vp, ctypes.c_int, _vp, _i32, _i64, _i32, _i32, _vp, _vp])
_lib_bwd_dact_g = _sig("xmoe_expert_ffn_bwd_dact_gather",
                       [_vp, _vp, _vp, _vp, _vp, ctypes.c_int, _vp, _i32, _i64, _i64, _i32, _i32, _vp, _vp])
_lib_bwd_dx = _sig("xmoe_expert_ffn_bwd_dx", [_vp, _vp, _vp, ctypes.c_int, _vp, _i32, _i64, _i32, _i32, _vp, _i32,
                                              _vp])
_lib_bwd_dw13 = _sig("xmoe_expert_ffn_bwd_dw13", [_vp, _vp, ctypes.c_int, _vp, _i32, _i64, _i32, _i32, _vp, _vp,
                                                  ctypes.c_int, _i32, _vp])
_lib_bwd_dw13_g = _sig("xmoe_expert_ffn_bwd_dw13_gather",
                       [_vp, _vp, _vp, ctypes.c_int, _vp, _i32, _i64, _i64, _i32, _i32, _vp, _vp, ctypes.c_int, _i32,
                        _vp])
_lib_bwd_dw2 = _sig("xmoe_expert_ffn_bwd_dw2", [_vp, _vp, ctypes.c_int, _vp, _i32, _i64, _i32, _i32, _vp,
                                                ctypes.c_int, _i32, _vp])
_lib_dispatch_bwd = _sig("xmoe_dispatch_bwd", [_vp, ctypes.POINTER(_CPft), _i64, _i32, _i32, ctypes.c_int, _vp,
                                               _vp, _vp])
_lib_rbwd_ws = _sig("xmoe_route_bwd_workspace_size", [_i64, _i32, _i32, ctypes.c_int], _sz)
_lib_rbwd = _sig("xmoe_route_bwd", [_vp, _vp, _vp, _vp, _vp, _i32, ctypes.c_int, _i64, _i32, _i32, _i32, _f32,
                                    _i32, _vp, _vp, _vp, _sz, _vp])
_lib_pft_na = _sig("xmoe_build_pft_noalloc", [_vp, _vp, _i64, _i32, _i32, ctypes.POINTER(_CPft), _vp])
_lib_pft_na_max = _sig("xmoe_build_pft_noalloc_max_bytes", [], _sz)
_lib_pft_sh = _sig("xmoe_build_pft_shared", [_vp, _vp, _i64, _i32, _i32, _i32, ctypes.POINTER(_CPft), _vp, _sz, _vp])
_lib_pilots_ws = _sig("xmoe_build_pilots_workspace_size", [_i64, _i32, _i32, _i32], _sz)
_lib_pilots = _sig("xmoe_build_pilots", [_vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp])
_lib_ep_send = _sig("xmoe_ep_send_plan", [_vp, _i32, _i32, _vp, _vp, _vp])
_lib_ep_recv_ws = _sig("xmoe_ep_recv_plan_workspace_size", [_i32, _i32], _sz)
_lib_ep_recv = _sig("xmoe_ep_recv_plan", [_vp, _i32, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _sz, _vp])
_lib_scatter_rows = _sig("xmoe_scatter_rows", [_vp, ctypes.c_int, _i64, _i32, _vp, _i64, _vp, _vp])


class XmoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = _lib_last_error().decode(errors="replace")
        super().__init__(f"{where}: {_STATUS.get(status, status)}: {msg}")
        self.status = status


def _check(st: int, where: str):
    if st != 0:
        raise XmoeError(st, where)


def lib_path() -> str:
    return _LIB_FILE


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libxmoe takes device tensors only")
    if not t.is_contiguous():
        raise ValueError("libxmoe takes contiguous tensors only")
    return t.data_ptr()


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return XMOE_BF16
    if t.dtype == torch.float32:
        return XMOE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _grad_dt(*grads: torch.Tensor) -> int:
    """Weight-gradient dtype of the call: that of the gradient tensors (fp32
    gradients of bf16 inputs are the unrounded sums)."""
    if any(g.dtype != grads[0].dtype for g in grads):
        raise ValueError("the weight gradients must share one dtype")
    return _dt(grads[0])


# The library sees pointers and the sizes it is given, nothing else: each
# tensor must hold exactly those sizes, in the call's dtype, or a kernel would
# read or write past it.  These checks turn such a mismatch into an exception.
_I32, _F32 = torch.int32, torch.float32


def _shape(t: Optional[torch.Tensor], shape, name: str, dtype=None) -> None:
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, the call needs {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, the call needs {dtype}")


def _atleast(t: Optional[torch.Tensor], n: int, name: str, dtype=None) -> None:
    if t is None:
        return
    if t.numel() < n:
        raise ValueError(f"{name}: {t.numel()} elements, the call needs at least {n}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, the call needs {dtype}")


def _ffn_shapes(dt, E: int, d: int, h: int, w1=None, w3=None, w2=None, offsets=None,
                names=("w1", "w3", "w2")) -> None:
    """Expert weights (or their gradients, dt None: any one dtype) of E experts
    [E, d, h] / [E, h, d] and the offsets [E + 1]."""
    _shape(w1, (E, d, h), names[0], dt)
    _shape(w3, (E, d, h), names[1], dt)
    _shape(w2, (E, h, d), names[2], dt)
    _shape(offsets, (E + 1,), "expert_offsets", _I32)


def _pft_sized(pft: "PFT", T: int, E: int, k: int) -> None:
    R = T * k
    for name, n in (("token_ids", R), ("expert_ids", R), ("combine_weights", R), ("slot_to_row", R),
                    ("tokens_per_expert", E), ("expert_offsets", E + 1)):
        _shape(getattr(pft, name), (n,), f"pft.{name}")


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


class PFT:
    """Device tensors of the Padding-Free Token buffer for T tokens, E experts, top-k."""

    def __init__(self, T: int, E: int, k: int, device="cuda"):
        R = T * k
        i32 = dict(dtype=torch.int32, device=device)
        self.T, self.E, self.k = T, E, k
        self.token_ids = torch.empty(R, **i32)
        self.expert_ids = torch.empty(R, **i32)
        self.tokens_per_expert = torch.empty(E, **i32)
        self.expert_offsets = torch.empty(E + 1, **i32)
        self.combine_weights = torch.empty(R, dtype=torch.float32, device=device)
        self.slot_to_row = torch.empty(R, **i32)

    def c(self) -> _CPft:
        return _CPft(_ptr(self.token_ids), _ptr(self.expert_ids), _ptr(self.tokens_per_expert),
                     _ptr(self.expert_offsets), _ptr(self.combine_weights), _ptr(self.slot_to_row))

    def fields(self):
        return {"token_ids": self.token_ids, "expert_ids": self.expert_ids,
                "tokens_per_expert": self.tokens_per_expert, "expert_offsets": self.expert_offsets,
                "combine_weights": self.combine_weights, "slot_to_row": self.slot_to_row}


def xmoe_version() -> int:
    return int(_lib_version())


def xmoe_query_device(ordinal: int = 0) -> bool:
    v = ctypes.c_int(0)
    _check(_lib_query(ordinal, ctypes.byref(v)), "xmoe_query_device")
    return bool(v.value)


def xmoe_route_workspace_size(T: int, d: int, E: int, dtype) -> int:
    return int(_lib_route_ws(T, d, E, XMOE_BF16 if dtype == torch.bfloat16 else XMOE_F32))


def xmoe_route(x, wg, k: int, topk_ids, topk_w, logits, inv_temperature: float = 1.0,
               logit_bias=None, select_bias=None, workspace=None, stream=None):
    """workspace: device tensor of at least xmoe_route_workspace_size bytes; allocated
    here (torch) when None."""
    T, d = x.shape
    E = wg.shape[1]
    _shape(wg, (d, E), "wg", x.dtype)
    _shape(topk_ids, (T, k), "topk_ids", _I32)
    _shape(topk_w, (T, k), "topk_w", _F32)
    _shape(logits, (T, E), "logits", _F32)
    _shape(logit_bias, (E,), "logit_bias", _F32)
    _shape(select_bias, (E,), "select_bias", _F32)
    need = xmoe_route_workspace_size(T, d, E, x.dtype)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib_route(_ptr(x), _ptr(wg), _dt(x), T, d, E, k, inv_temperature, _ptr(logit_bias),
                      _ptr(select_bias), _ptr(topk_ids), _ptr(topk_w), _ptr(logits), _ptr(workspace), nbytes,
                      _stream(stream)),
           "xmoe_route")


def xmoe_build_pft_workspace_size(T: int, E: int, k: int) -> int:
    return int(_lib_pft_ws(T, E, k))


def xmoe_build_pft(topk_ids, topk_w, E: int, pft: PFT, workspace, stream=None):
    T, k = topk_ids.shape
    _shape(topk_ids, (T, k), "topk_ids", _I32)
    _shape(topk_w, (T, k), "topk_w", _F32)
    _pft_sized(pft, T, E, k)
    c = pft.c()
    _check(_lib_pft(_ptr(topk_ids), _ptr(topk_w), T, E, k, ctypes.byref(c), _ptr(workspace),
                    workspace.numel() * workspace.element_size(), _stream(stream)), "xmoe_build_pft")


def xmoe_build_pft_noalloc(topk_ids, topk_w, E: int, pft: PFT, stream=None):
    """xmoe_build_pft on the library's static scratch: no workspace, nothing
    allocated (calls overlapping on one device race)."""
    T, k = topk_ids.shape
    _shape(topk_ids, (T, k), "topk_ids", _I32)
    _shape(topk_w, (T, k), "topk_w", _F32)
    _pft_sized(pft, T, E, k)
    c = pft.c()
    _check(_lib_pft_na(_ptr(topk_ids), _ptr(topk_w), T, E, k, ctypes.byref(c), _stream(stream)),
           "xmoe_build_pft_noalloc")


def xmoe_build_pft_noalloc_max_bytes() -> int:
    return int(_lib_pft_na_max())


def xmoe_build_pft_shared(topk_ids, topk_w, E_routed: int, n_shared: int, pft: PFT, workspace, stream=None):
    """The buffer with n_shared always-routed experts after the E_routed routed
    ones (weight 1); pft must be PFT(T, E_routed + n_shared, k + n_shared)."""
    T, k = topk_ids.shape
    if pft.k != k + n_shared or pft.E != E_routed + n_shared:
        raise ValueError("pft must be sized for E_routed + n_shared experts and k + n_shared slots")
    _shape(topk_ids, (T, k), "topk_ids", _I32)
    _shape(topk_w, (T, k), "topk_w", _F32)
    _pft_sized(pft, T, E_routed + n_shared, k + n_shared)
    c = pft.c()
    _check(_lib_pft_sh(_ptr(topk_ids), _ptr(topk_w), T, E_routed, k, n_shared, ctypes.byref(c), _ptr(workspace),
                       workspace.numel() * workspace.element_size(), _stream(stream)), "xmoe_build_pft_shared")


def xmoe_dispatch(x, k: int, pft: PFT, xs, stream=None):
    T, d = x.shape
    _pft_sized(pft, T, pft.E, k)
    _shape(xs, (T * k, d), "xs", x.dtype)
    c = pft.c()
    _check(_lib_dispatch(_ptr(x), _dt(x), T, d, k, ctypes.byref(c), _ptr(xs), _stream(stream)),
           "xmoe_dispatch")


def xmoe_expert_ffn_up(xs, w1, w3, expert_offsets, act, h13=None, stream=None):
    rows, d = xs.shape
    E, _, h = w1.shape
    _ffn_shapes(xs.dtype, E, d, h, w1=w1, w3=w3, offsets=expert_offsets)
    _shape(act, (rows, h), "act", xs.dtype)
    _shape(h13, (rows, 2 * h), "h13", xs.dtype)
    _check(_lib_up(_ptr(xs), _ptr(w1), _ptr(w3), _dt(xs), _ptr(expert_offsets), E, rows, d, h, _ptr(act),
                   _ptr(h13), _stream(stream)), "xmoe_expert_ffn_up")


def xmoe_expert_ffn_up_gather(x, token_ids, w1, w3, expert_offsets, act, h13=None, stream=None):
    T, d = x.shape
    E, _, h = w1.shape
    rows = token_ids.shape[0]
    _ffn_shapes(x.dtype, E, d, h, w1=w1, w3=w3, offsets=expert_offsets)
    _shape(token_ids, (rows,), "token_ids", _I32)
    _shape(act, (rows, h), "act", x.dtype)
    _shape(h13, (rows, 2 * h), "h13", x.dtype)
    _check(_lib_up_g(_ptr(x), _ptr(token_ids), _ptr(w1), _ptr(w3), _dt(x), _ptr(expert_offsets), E, T, rows, d, h,
                     _ptr(act), _ptr(h13), _stream(stream)), "xmoe_expert_ffn_up_gather")


def xmoe_expert_ffn_gather(x, token_ids, w1, w3, w2, expert_offsets, act, ye, h13=None, accumulate=False,
                           stream=None):
    T, d = x.shape
    E, _, h = w1.shape
    rows = token_ids.shape[0]
    _ffn_shapes(x.dtype, E, d, h, w1=w1, w3=w3, w2=w2, offsets=expert_offsets)
    _shape(token_ids, (rows,), "token_ids", _I32)
    _shape(act, (rows, h), "act", x.dtype)
    _shape(h13, (rows, 2 * h), "h13", x.dtype)
    _shape(ye, (rows, d), "ye", x.dtype)
    _check(_lib_ffn_g(_ptr(x), _ptr(token_ids), _ptr(w1), _ptr(w3), _ptr(w2), _dt(x), _ptr(expert_offsets), E, T,
                      rows, d, h, _ptr(act), _ptr(h13), _ptr(ye), int(bool(accumulate)), _stream(stream)),
           "xmoe_expert_ffn_gather")


def xmoe_expert_ffn_down(act, w2, expert_offsets, ye, accumulate=False, stream=None):
    """accumulate=True: ye += act . W2."""
    rows, h = act.shape
    E, _, d = w2.shape
    _ffn_shapes(act.dtype, E, d, h, w2=w2, offsets=expert_offsets)
    _shape(ye, (rows, d), "ye", act.dtype)
    _check(_lib_down(_ptr(act), _ptr(w2), _dt(act), _ptr(expert_offsets), E, rows, d, h, _ptr(ye),
                     int(bool(accumulate)), _stream(stream)), "xmoe_expert_ffn_down")


def xmoe_expert_ffn(xs, w1, w3, w2, expert_offsets, act, ye, h13=None, accumulate=False, stream=None):
    """accumulate=True: ye += the experts' outputs."""
    rows, d = xs.shape
    E, _, h = w1.shape
    _ffn_shapes(xs.dtype, E, d, h, w1=w1, w3=w3, w2=w2, offsets=expert_offsets)
    _shape(act, (rows, h), "act", xs.dtype)
    _shape(h13, (rows, 2 * h), "h13", xs.dtype)
    _shape(ye, (rows, d), "ye", xs.dtype)
    _check(_lib_ffn(_ptr(xs), _ptr(w1), _ptr(w3), _ptr(w2), _dt(xs), _ptr(expert_offsets), E, rows, d, h,
                    _ptr(act), _ptr(h13), _ptr(ye), int(bool(accumulate)), _stream(stream)), "xmoe_expert_ffn")


def xmoe_combine(ye, pft: PFT, T: int, y, y_add=None, stream=None):
    d = ye.shape[1]
    _pft_sized(pft, T, pft.E, pft.k)
    _shape(ye, (T * pft.k, d), "ye")
    _shape(y, (T, d), "y", ye.dtype)
    _shape(y_add, (T, d), "y_add", ye.dtype)
    c = pft.c()
    _check(_lib_combine(_ptr(ye), ctypes.byref(c), T, d, pft.k, _dt(ye), _ptr(y_add), _ptr(y), _stream(stream)),
           "xmoe_combine")


def xmoe_combine_bwd(dy, ye, pft: PFT, dye, dtopk_w, stream=None):
    T, d = dy.shape
    _pft_sized(pft, T, pft.E, pft.k)
    _shape(ye, (T * pft.k, d), "ye", dy.dtype)
    _shape(dye, (T * pft.k, d), "dye", dy.dtype)
    _shape(dtopk_w, (T, pft.k), "dtopk_w", _F32)
    c = pft.c()
    _check(_lib_combine_bwd(_ptr(dy), _ptr(ye), ctypes.byref(c), T, d, pft.k, _dt(dy), _ptr(dye), _ptr(dtopk_w),
                            _stream(stream)), "xmoe_combine_bwd")


def xmoe_expert_ffn_bwd(xs, w1, w3, w2, act, h13, dye, expert_offsets, dh13, dxs, dw1, dw3, dw2,
                        accumulate_dxs=False, accumulate_dw=False, stream=None):
    """The weight gradients' dtype (dw1/dw3/dw2, one dtype) is grad_dt: fp32
    tensors with bf16 inputs receive the unrounded sums; accumulate_dw adds to
    them (fp32 only), accumulate_dxs adds to dxs."""
    rows, d = xs.shape
    E, _, h = w1.shape
    _ffn_shapes(xs.dtype, E, d, h, w1=w1, w3=w3, w2=w2, offsets=expert_offsets)
    for t, shp, name in ((act, (rows, h), "act"), (h13, (rows, 2 * h), "h13"), (dye, (rows, d), "dye"),
                         (dh13, (rows, 2 * h), "dh13"), (dxs, (rows, d), "dxs")):
        _shape(t, shp, name, xs.dtype)
    _ffn_shapes(None, E, d, h, w1=dw1, w3=dw3, w2=dw2, names=("dw1", "dw3", "dw2"))
    _check(_lib_ffn_bwd(_ptr(xs), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(act), _ptr(h13), _ptr(dye), _dt(xs),
                        _ptr(expert_offsets), E, rows, d, h, _ptr(dh13), _ptr(dxs), int(bool(accumulate_dxs)),
                        _ptr(dw1), _ptr(dw3), _ptr(dw2), _grad_dt(dw1, dw3, dw2), int(bool(accumulate_dw)),
                        _stream(stream)), "xmoe_expert_ffn_bwd")


def xmoe_expert_ffn_bwd_dact(dye, w2, h13, expert_offsets, dh13, stream=None):
    rows, d = dye.shape
    E, h, _ = w2.shape
    _ffn_shapes(dye.dtype, E, d, h, w2=w2, offsets=expert_offsets)
    _shape(h13, (rows, 2 * h), "h13", dye.dtype)
    _shape(dh13, (rows, 2 * h), "dh13", dye.dtype)
    _check(_lib_bwd_dact(_ptr(dye), _ptr(w2), _ptr(h13), _dt(dye), _ptr(expert_offsets), E, rows, d, h, _ptr(dh13),
                         _stream(stream)), "xmoe_expert_ffn_bwd_dact")


def xmoe_expert_ffn_bwd_dact_gather(dy, token_ids, row_weights, w2, h13, expert_offsets, dh13, stream=None):
    T, d = dy.shape
    E, h, _ = w2.shape
    rows = token_ids.shape[0]
    _ffn_shapes(dy.dtype, E, d, h, w2=w2, offsets=expert_offsets)
    _shape(token_ids, (rows,), "token_ids", _I32)
    _shape(row_weights, (rows,), "row_weights", _F32)
    _shape(h13, (rows, 2 * h), "h13", dy.dtype)
    _shape(dh13, (rows, 2 * h), "dh13", dy.dtype)
    _check(_lib_bwd_dact_g(_ptr(dy), _ptr(token_ids), _ptr(row_weights), _ptr(w2), _ptr(h13), _dt(dy),
                           _ptr(expert_offsets), E, T, rows, d, h, _ptr(dh13), _stream(stream)),
           "xmoe_expert_ffn_bwd_dact_gather")


def xmoe_expert_ffn_bwd_dx(dh13, w1, w3, expert_offsets, dxs, accumulate=False, stream=None):
    rows, d = dxs.shape
    E, _, h = w1.shape
    _ffn_shapes(dxs.dtype, E, d, h, w1=w1, w3=w3, offsets=expert_offsets)
    _shape(dh13, (rows, 2 * h), "dh13", dxs.dtype)
    _check(_lib_bwd_dx(_ptr(dh13), _ptr(w1), _ptr(w3), _dt(dh13), _ptr(expert_offsets), E, rows, d, h, _ptr(dxs),
                       int(bool(accumulate)), _stream(stream)), "xmoe_expert_ffn_bwd_dx")


def xmoe_expert_ffn_bwd_dw13(xs, dh13, expert_offsets, dw1, dw3, accumulate=False, stream=None):
    """grad_dt = dw1/dw3's dtype; accumulate adds to them (fp32 only)."""
    rows, d = xs.shape
    E, _, h = dw1.shape
    _ffn_shapes(None, E, d, h, w1=dw1, w3=dw3, offsets=expert_offsets, names=("dw1", "dw3", "dw2"))
    _shape(dh13, (rows, 2 * h), "dh13", xs.dtype)
    _check(_lib_bwd_dw13(_ptr(xs), _ptr(dh13), _dt(xs), _ptr(expert_offsets), E, rows, d, h, _ptr(dw1), _ptr(dw3),
                         _grad_dt(dw1, dw3), int(bool(accumulate)), _stream(stream)), "xmoe_expert_ffn_bwd_dw13")


def xmoe_expert_ffn_bwd_dw13_gather(x, token_ids, dh13, expert_offsets, dw1, dw3, accumulate=False, stream=None):
    T, d = x.shape
    E, _, h = dw1.shape
    rows = dh13.shape[0]
    _ffn_shapes(None, E, d, h, w1=dw1, w3=dw3, offsets=expert_offsets, names=("dw1", "dw3", "dw2"))
    _shape(token_ids, (rows,), "token_ids", _I32)
    _shape(dh13, (rows, 2 * h), "dh13", x.dtype)
    _check(_lib_bwd_dw13_g(_ptr(x), _ptr(token_ids), _ptr(dh13), _dt(x), _ptr(expert_offsets), E, T, rows, d, h,
                           _ptr(dw1), _ptr(dw3), _grad_dt(dw1, dw3), int(bool(accumulate)), _stream(stream)),
           "xmoe_expert_ffn_bwd_dw13_gather")


def xmoe_expert_ffn_bwd_dw2(act, dye, expert_offsets, dw2, accumulate=False, stream=None):
    """grad_dt = dw2's dtype; accumulate adds to it (fp32 only)."""
    rows, h = act.shape
    E, _, d = dw2.shape
    _ffn_shapes(None, E, d, h, w2=dw2, offsets=expert_offsets, names=("dw1", "dw3", "dw2"))
    _shape(dye, (rows, d), "dye", act.dtype)
    _check(_lib_bwd_dw2(_ptr(act), _ptr(dye), _dt(act), _ptr(expert_offsets), E, rows, d, h, _ptr(dw2),
                        _grad_dt(dw2), int(bool(accumulate)), _stream(stream)), "xmoe_expert_ffn_bwd_dw2")


def xmoe_dispatch_bwd(dxs, pft: PFT, T: int, dx, dx_add=None, stream=None):
    d = dxs.shape[1]
    _pft_sized(pft, T, pft.E, pft.k)
    _shape(dxs, (T * pft.k, d), "dxs")
    _shape(dx, (T, d), "dx", dxs.dtype)
    _shape(dx_add, (T, d), "dx_add", dxs.dtype)
    c = pft.c()
    _check(_lib_dispatch_bwd(_ptr(dxs), ctypes.byref(c), T, d, pft.k, _dt(dxs), _ptr(dx_add), _ptr(dx),
                             _stream(stream)), "xmoe_dispatch_bwd")


def xmoe_route_bwd_workspace_size(T: int, d: int, E: int, dtype: torch.dtype) -> int:
    return int(_lib_rbwd_ws(T, d, E, XMOE_BF16 if dtype == torch.bfloat16 else XMOE_F32))


def xmoe_route_bwd(x, wg, logits, topk_ids, dtopk_w, dx, dwg, workspace, inv_temperature: float = 1.0,
                   accumulate: bool = True, stream=None):
    """dtopk_w [T, k] may be the first k columns of a wider [T, k'] buffer
    (rows of unit stride); accumulate=False writes dx instead of adding to it."""
    T, d = x.shape
    E = wg.shape[1]
    k = topk_ids.shape[1]
    if not dtopk_w.is_cuda or dtopk_w.dim() != 2 or dtopk_w.stride(1) != 1 or dtopk_w.shape != (T, k):
        raise ValueError("dtopk_w must be a [T, k] device tensor with unit column stride")
    if dtopk_w.dtype != _F32:
        raise TypeError("dtopk_w must be fp32")
    _shape(wg, (d, E), "wg", x.dtype)
    _shape(logits, (T, E), "logits", _F32)
    _shape(topk_ids, (T, k), "topk_ids", _I32)
    _shape(dx, (T, d), "dx", x.dtype)
    _shape(dwg, (d, E), "dwg", _F32)
    _check(_lib_rbwd(_ptr(x), _ptr(wg), _ptr(logits), _ptr(topk_ids), dtopk_w.data_ptr(), dtopk_w.stride(0), _dt(x),
                     T, d, E, k, inv_temperature, 1 if accumulate else 0, _ptr(dx), _ptr(dwg), _ptr(workspace),
                     workspace.numel() * workspace.element_size(), _stream(stream)), "xmoe_route_bwd")


def xmoe_build_pilots_workspace_size(T: int, E: int, k: int, experts_per_node: int) -> int:
    return int(_lib_pilots_ws(T, E, k, experts_per_node))


def xmoe_build_pilots(topk_ids, E: int, experts_per_node: int, pilot_token_ids, pilot_node_ids, node_counts,
                      node_offsets, slot_to_pilot, workspace, stream=None):
    """Pilot tokens of Redundancy-Bypassing Dispatch (see xmoe.h); all int32 device tensors."""
    T, k = topk_ids.shape
    _shape(topk_ids, (T, k), "topk_ids", _I32)
    N = E // experts_per_node if experts_per_node > 0 else 0
    for t, n, name in ((pilot_token_ids, T * min(k, N), "pilot_token_ids"),
                       (pilot_node_ids, T * min(k, N), "pilot_node_ids"), (slot_to_pilot, T * k, "slot_to_pilot")):
        _atleast(t, n, name, _I32)
    _shape(node_counts, (N,), "node_counts", _I32)
    _shape(node_offsets, (N + 1,), "node_offsets", _I32)
    _check(_lib_pilots(_ptr(topk_ids), T, E, k, experts_per_node, _ptr(pilot_token_ids), _ptr(pilot_node_ids),
                       _ptr(node_counts), _ptr(node_offsets), _ptr(slot_to_pilot), _ptr(workspace),
                       workspace.numel() * workspace.element_size(), _stream(stream)), "xmoe_build_pilots")


def xmoe_ep_send_plan(expert_offsets, G: int, send_counts, send_displs, stream=None):
    E = expert_offsets.numel() - 1
    _shape(expert_offsets, (E + 1,), "expert_offsets", _I32)
    _shape(send_counts, (G,), "send_counts", _I32)
    _shape(send_displs, (G + 1,), "send_displs", _I32)
    _check(_lib_ep_send(_ptr(expert_offsets), E, G, _ptr(send_counts), _ptr(send_displs), _stream(stream)),
           "xmoe_ep_send_plan")


def xmoe_ep_recv_plan_workspace_size(G: int, E_local: int) -> int:
    return int(_lib_ep_recv_ws(G, E_local))


def xmoe_ep_recv_plan(recv_counts, n_recv: int, local_offsets, recv_displs, local_to_recv, recv_to_local,
                      workspace, stream=None):
    """recv_counts: int32 device [G, E_local]; n_recv: its sum (host int)."""
    G, el = recv_counts.shape
    _shape(recv_counts, (G, el), "recv_counts", _I32)
    _shape(local_offsets, (el + 1,), "local_offsets", _I32)
    _shape(recv_displs, (G + 1,), "recv_displs", _I32)
    _atleast(local_to_recv, n_recv, "local_to_recv", _I32)
    _atleast(recv_to_local, n_recv, "recv_to_local", _I32)
    _check(_lib_ep_recv(_ptr(recv_counts), G, el, n_recv, _ptr(local_offsets), _ptr(recv_displs),
                        _ptr(local_to_recv), _ptr(recv_to_local), _ptr(workspace),
                        workspace.numel() * workspace.element_size(), _stream(stream)), "xmoe_ep_recv_plan")


def xmoe_scatter_rows(src, index, dst, n: Optional[int] = None, stream=None):
    """dst[index[i]] = src[i] for i < n (default: all rows of src)."""
    rows, d = src.shape
    n = rows if n is None else n
    if n > rows:
        raise ValueError(f"n = {n} exceeds the {rows} rows of src")
    _atleast(index, n, "index", _I32)
    if dst.dim() != 2 or dst.shape[1] != d or dst.dtype != src.dtype:
        raise ValueError("dst must be [rows, d] in src's dtype")
    _check(_lib_scatter_rows(_ptr(src), _dt(src), n, d, _ptr(index), dst.shape[0], _ptr(dst), _stream(stream)),
           "xmoe_scatter_rows")
