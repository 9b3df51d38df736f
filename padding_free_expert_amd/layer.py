"""A padding-free MoE layer driven through libxmoe.

Owns every buffer of one layer invocation (allocated once, with torch, on the
GPU) and runs the forward and backward as the sequence of C-ABI calls the
X-MoE pages describe ("5.4 MoE模型在分布式训练中的应用", section 训练流程: gate,
dispatch, experts, combine, then the reverse path).  No arithmetic happens in
Python: every step is a libxmoe kernel.
"""
from __future__ import annotations

from typing import Dict, Optional

import torch

from . import (PFT, xmoe_build_pft, xmoe_build_pft_workspace_size, xmoe_combine, xmoe_combine_bwd,
               xmoe_dispatch, xmoe_dispatch_bwd, xmoe_expert_ffn, xmoe_expert_ffn_bwd, xmoe_expert_ffn_bwd_dact,
               xmoe_expert_ffn_bwd_dw13, xmoe_expert_ffn_bwd_dw2, xmoe_expert_ffn_bwd_dx, xmoe_expert_ffn_gather,
               xmoe_expert_ffn_up, xmoe_expert_ffn_up_gather, xmoe_route, xmoe_route_bwd,
               xmoe_route_bwd_workspace_size, xmoe_route_workspace_size)


class PaddingFreeMoE:
    """Buffers and call sequence for one layer of T tokens.

    weights: dict with wg [d,E], w1/w3 [E,d,h], w2 [E,h,d]; optional shared-expert
    weights s1/s3 [d, n*h_s], s2 [n*h_s, d] (the shared experts side by side),
    logit_bias / select_bias fp32 [E].

    The forward never materialises the expert-sorted copy of x: the gather is
    fused into the up-projection's operand loads (X-MoE article, section 2.1.2).
    The backward re-gathers it once, as scratch, for the weight gradient of
    W1/W3.  lean=True also drops the saved pre-activations H1/H3 and recomputes
    them in the backward (the same kernel, so bitwise the same values): what
    the backward needs from the forward shrinks to act, ye and the routing."""

    def __init__(self, weights: Dict[str, torch.Tensor], T: int, k: int, inv_tau: float = 1.0,
                 backward: bool = True, lean: bool = False, overlap: bool = True):
        self.w = weights
        wg, w1 = weights["wg"], weights["w1"]
        self.dtype = wg.dtype
        self.device = wg.device
        self.T, self.k, self.inv_tau = T, k, inv_tau
        self.d, self.E = wg.shape
        self.h = w1.shape[2]
        self.shared = weights.get("s1") is not None
        self.backward_enabled = backward
        self.lean = lean
        # the shared experts depend only on x (forward) and dy (backward): with
        # overlap they run on a second stream (default priority) beside the
        # routed path and fill the tail of its GEMMs; the routed weight
        # gradients run on a third one beside the data gradients
        self.overlap = overlap
        self.wside = torch.cuda.Stream(device=self.device) if backward else None
        dev, dt = self.device, self.dtype
        T, d, E, h, R = T, self.d, self.E, self.h, T * k
        f32 = dict(dtype=torch.float32, device=dev)
        self.topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.topk_w = torch.empty((T, k), **f32)
        self.logits = torch.empty((T, E), **f32)
        self.pft = PFT(T, E, k, dev)
        self.pft_ws = torch.empty(max(xmoe_build_pft_workspace_size(T, E, k), 16), dtype=torch.uint8, device=dev)
        self.route_ws = torch.empty(max(xmoe_route_workspace_size(T, d, E, dt), 16), dtype=torch.uint8, device=dev)
        # scratch of the backward (re-gathered rows), not kept from the forward
        self.xs = torch.empty((R, d), dtype=dt, device=dev) if backward else None
        self.act = torch.empty((R, h), dtype=dt, device=dev)
        self.h13 = torch.empty((R, 2 * h), dtype=dt, device=dev) if backward else None
        self.ye = torch.empty((R, d), dtype=dt, device=dev)
        self.y = torch.empty((T, d), dtype=dt, device=dev)
        if self.shared:
            hs = weights["s1"].shape[1]
            self.hs = hs
            self.sh_off = torch.tensor([0, T], dtype=torch.int32, device=dev)
            self.sh_act = torch.empty((T, hs), dtype=dt, device=dev)
            self.sh_h13 = torch.empty((T, 2 * hs), dtype=dt, device=dev) if backward else None
            self.sh_y = torch.empty((T, d), dtype=dt, device=dev)
            self.side = torch.cuda.Stream(device=dev)
        if backward:
            self.dtopk_w = torch.empty((T, k), **f32)
            self.dye = torch.empty((R, d), dtype=dt, device=dev)
            self.dh13 = torch.empty((R, 2 * h), dtype=dt, device=dev)
            self.dxs = torch.empty((R, d), dtype=dt, device=dev)
            self.dw1 = torch.empty((E, d, h), dtype=dt, device=dev)
            self.dw3 = torch.empty((E, d, h), dtype=dt, device=dev)
            self.dw2 = torch.empty((E, h, d), dtype=dt, device=dev)
            self.dx = torch.empty((T, d), dtype=dt, device=dev)
            self.dwg = torch.empty((d, E), **f32)
            self.rbwd_ws = torch.empty(max(xmoe_route_bwd_workspace_size(T, d, E, dt), 16), dtype=torch.uint8,
                                       device=dev)
            if self.shared:
                hs = self.hs
                self.sh_dh13 = torch.empty((T, 2 * hs), dtype=dt, device=dev)
                self.sh_dx = torch.empty((T, d), dtype=dt, device=dev)
                self.ds1 = torch.empty((1, d, hs), dtype=dt, device=dev)
                self.ds3 = torch.empty((1, d, hs), dtype=dt, device=dev)
                self.ds2 = torch.empty((1, hs, d), dtype=dt, device=dev)

    # views of the shared-expert weights as a single expert of width n*h_s
    def _shared_w(self):
        w = self.w
        return w["s1"].unsqueeze(0), w["s3"].unsqueeze(0), w["s2"].unsqueeze(0)

    def _streams(self, stream):
        main = stream if stream is not None else torch.cuda.current_stream(self.device)
        side = self.side if (self.shared and self.overlap) else main
        return main, side

    def forward(self, x: torch.Tensor, stream=None, hook=None) -> torch.Tensor:
        """hook(name), if given, is called after each library call is enqueued."""
        w = self.w
        mark = hook or (lambda name: None)
        main, side = self._streams(stream)
        keep = self.backward_enabled and not self.lean
        if self.shared:
            side.wait_stream(main)
            s1, s3, s2 = self._shared_w()
            xmoe_expert_ffn(x, s1, s3, s2, self.sh_off, self.sh_act, self.sh_y,
                            h13=self.sh_h13 if keep else None, stream=side)
            if side is main:
                mark("shared_ffn")
        xmoe_route(x, w["wg"], self.k, self.topk_ids, self.topk_w, self.logits, self.inv_tau,
                   w.get("logit_bias"), w.get("select_bias"), workspace=self.route_ws, stream=main)
        mark("route")
        xmoe_build_pft(self.topk_ids, self.topk_w, self.E, self.pft, self.pft_ws, stream=main)
        mark("build_pft")
        xmoe_expert_ffn_gather(x, self.pft.token_ids, w["w1"], w["w3"], w["w2"], self.pft.expert_offsets,
                               self.act, self.ye, h13=self.h13 if keep else None, stream=main)
        mark("expert_ffn")
        y_add = None
        if self.shared:
            main.wait_stream(side)
            y_add = self.sh_y
        xmoe_combine(self.ye, self.pft, self.T, self.y, y_add=y_add, stream=main)
        mark("combine")
        self.x = x
        return self.y

    def backward(self, dy: torch.Tensor, stream=None, hook=None) -> torch.Tensor:
        w = self.w
        mark = hook or (lambda name: None)
        main, side = self._streams(stream)
        dx_add = None
        if self.shared:
            side.wait_stream(main)
            s1, s3, s2 = self._shared_w()
            if self.lean:
                xmoe_expert_ffn_up(self.x, s1, s3, self.sh_off, self.sh_act, self.sh_h13, stream=side)
                if side is main:
                    mark("recompute_shared_h13")
            xmoe_expert_ffn_bwd(self.x, s1, s3, s2, self.sh_act, self.sh_h13, dy, self.sh_off, self.sh_dh13,
                                self.sh_dx, self.ds1, self.ds3, self.ds2, stream=side)
            if side is main:
                mark("shared_ffn_bwd")
            dx_add = self.sh_dx
        xmoe_combine_bwd(dy, self.ye, self.pft, self.dye, self.dtopk_w, stream=main)
        mark("combine_bwd")
        if self.shared:
            # the gate's backward needs only dtopk_w, the logits and x: it runs
            # beside the expert backward and adds dz . wg^T into the shared
            # experts' dx, which the dispatch backward folds into dx
            side.wait_stream(main)
            xmoe_route_bwd(self.x, w["wg"], self.logits, self.topk_ids, self.dtopk_w, self.sh_dx, self.dwg,
                           self.rbwd_ws, self.inv_tau, stream=side)
            if side is main:
                mark("route_bwd")
        if self.lean:
            # recompute the pre-activations (act is rewritten with the same values)
            xmoe_expert_ffn_up_gather(self.x, self.pft.token_ids, w["w1"], w["w3"], self.pft.expert_offsets,
                                      self.act, self.h13, stream=main)
            mark("recompute_h13")
        off = self.pft.expert_offsets
        ws = self.wside if self.overlap else main
        # weight gradients: dW2 needs act and dye only; dW1/dW3 need the rows
        # (re-gathered as scratch) and dH1/dH3
        ws.wait_stream(main)
        xmoe_expert_ffn_bwd_dw2(self.act, self.dye, off, self.dw2, stream=ws)
        if ws is main:
            mark("bwd_dw2")
        xmoe_dispatch(self.x, self.k, self.pft, self.xs, stream=ws)
        if ws is main:
            mark("dispatch")
        xmoe_expert_ffn_bwd_dact(self.dye, w["w2"], self.h13, off, self.dh13, stream=main)
        mark("bwd_dact")
        ws.wait_stream(main)
        xmoe_expert_ffn_bwd_dw13(self.xs, self.dh13, off, self.dw1, self.dw3, stream=ws)
        if ws is main:
            mark("bwd_dw13")
        xmoe_expert_ffn_bwd_dx(self.dh13, w["w1"], w["w3"], off, self.dxs, stream=main)
        mark("bwd_dx")
        if self.shared:
            main.wait_stream(side)
        xmoe_dispatch_bwd(self.dxs, self.pft, self.T, self.dx, dx_add=dx_add, stream=main)
        mark("dispatch_bwd")
        if not self.shared:
            xmoe_route_bwd(self.x, w["wg"], self.logits, self.topk_ids, self.dtopk_w, self.dx, self.dwg,
                           self.rbwd_ws, self.inv_tau, stream=main)
            mark("route_bwd")
        main.wait_stream(self.wside)  # every gradient is complete in the caller's stream order
        return self.dx

    def saved_bytes(self) -> int:
        """Bytes the backward needs from the forward (beyond x and the weights):
        routing results, the PFT, act and ye, plus H1/H3 unless lean."""
        def nb(t):
            return 0 if t is None else t.numel() * t.element_size()
        n = nb(self.topk_ids) + nb(self.topk_w) + nb(self.logits) + nb(self.act) + nb(self.ye)
        n += sum(nb(t) for t in self.pft.fields().values())
        if not self.lean:
            n += nb(self.h13)
        if self.shared:
            n += nb(self.sh_act) + (0 if self.lean else nb(self.sh_h13))
        return n

    def grads(self) -> Dict[str, torch.Tensor]:
        g = {"dx": self.dx, "dwg": self.dwg, "dw1": self.dw1, "dw3": self.dw3, "dw2": self.dw2,
             "dtopk_w": self.dtopk_w, "dye": self.dye, "dxs": self.dxs, "dh13": self.dh13}
        if self.shared:
            g.update(ds1=self.ds1[0], ds3=self.ds3[0], ds2=self.ds2[0])
        return g
