"""A padding-free MoE layer driven through libxmoe.

Owns every buffer of one layer invocation (allocated once, with torch, on the
GPU) and runs the forward and backward as the sequence of C-ABI calls the
X-MoE pages describe ("5.4 MoE模型在分布式训练中的应用", section 训练流程: gate,
dispatch, experts, combine, then the reverse path).  No arithmetic happens in
Python: every step is a libxmoe kernel.
"""
from __future__ import annotations

from typing import Dict

import torch

from . import (PFT, xmoe_build_pft, xmoe_build_pft_shared, xmoe_build_pft_workspace_size, xmoe_combine,
               xmoe_combine_bwd, xmoe_dispatch_bwd, xmoe_expert_ffn_bwd,
               xmoe_expert_ffn_bwd_dact_gather, xmoe_expert_ffn_bwd_dw13_gather, xmoe_expert_ffn_bwd_dw2, xmoe_expert_ffn_bwd_dx,
               xmoe_expert_ffn_down, xmoe_expert_ffn_up, xmoe_expert_ffn_up_gather, xmoe_route, xmoe_route_bwd,
               xmoe_route_bwd_workspace_size, xmoe_route_workspace_size)


class PaddingFreeMoE:
    """Buffers and call sequence for one layer of T tokens.

    weights: dict with wg [d,E], w1/w3 [E,d,h], w2 [E,h,d]; optional shared-expert
    weights s1/s3 [d, n*h_s], s2 [n*h_s, d] (the shared experts side by side),
    logit_bias / select_bias fp32 [E].

    Neither pass materialises the expert-sorted copy of x: the gather is fused
    into the operand loads of the up-projection and of the weight gradient of
    W1/W3 (X-MoE article, section 2.1.2).  lean=True also drops the saved
    pre-activations H1/H3 and recomputes
    them in the backward (the same kernel, so bitwise the same values): what
    the backward needs from the forward shrinks to act, ye and the routing.

    Shared experts: a SwiGLU FFN of width n*h is the sum of n FFNs of width h
    over its column blocks.  When the shared width is a multiple of the routed
    h (and merge_shared), the shared experts become that many more experts that
    every token is routed to with weight 1: one buffer, one call per product
    for routed and shared experts together.  The layer then keeps the routed
    and shared weights in one [E + n, d, h] / [E + n, h, d] buffer, copied at
    construction and again by refresh_weights() (call it after changing the
    weights).  Otherwise (the default) the shared FFN runs as a separate
    FFN of its own width on a second stream beside the routed path.  Measured
    on the DeepSeek-MoE-16B shape the separate stream is ~2.7% faster: it fills
    the routed products' tails, and the merged buffer's mean rows per expert
    (routed and shared together) moves the down-projection and dA products to
    the smaller tile."""

    def __init__(self, weights: Dict[str, torch.Tensor], T: int, k: int, inv_tau: float = 1.0,
                 backward: bool = True, lean: bool = False, overlap: bool = True, merge_shared: bool = False):
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
        # overlap: the gate's backward and the routed weight gradients run on
        # streams of their own (default priority) beside the data gradients;
        # unmerged shared experts run on a second stream beside the routed path
        self.overlap = overlap
        dev, dt = self.device, self.dtype
        T, d, E, h = T, self.d, self.E, self.h
        self.hs = weights["s1"].shape[1] if self.shared else 0
        self.merged = self.shared and merge_shared and self.hs % h == 0
        self.ns = self.hs // h if self.merged else 0       # shared experts carried as routed ones
        Ec, kc = E + self.ns, k + self.ns                   # experts and slots per token in the buffer
        self.Ec, self.kc = Ec, kc
        R = T * kc
        self.R = R
        # dW1/dW3 beside dA and dX on the caller's stream when experts are
        # small (mean rows per expert <= 1024), else on the weight-gradient
        # stream after dW2.  Whole steps: DeepSeek-MoE-16B shape -1.0%,
        # Zipf-skewed -4%, long batch (1638 rows per expert) +0.4%.
        self.dw13_main = R <= 1024 * Ec
        if self.merged:
            self.W1 = torch.empty((Ec, d, h), dtype=dt, device=dev)
            self.W3 = torch.empty((Ec, d, h), dtype=dt, device=dev)
            self.W2 = torch.empty((Ec, h, d), dtype=dt, device=dev)
            self.refresh_weights()
        else:
            self.W1, self.W3, self.W2 = w1, weights["w3"], weights["w2"]
        self.wside = torch.cuda.Stream(device=dev) if backward else None
        self.gside = torch.cuda.Stream(device=dev) if backward else None
        f32 = dict(dtype=torch.float32, device=dev)
        self.topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.topk_w = torch.empty((T, k), **f32)
        self.logits = torch.empty((T, E), **f32)
        self.pft = PFT(T, Ec, kc, dev)
        self.pft_ws = torch.empty(max(xmoe_build_pft_workspace_size(T, Ec, kc), 16), dtype=torch.uint8, device=dev)
        self.route_ws = torch.empty(max(xmoe_route_workspace_size(T, d, E, dt), 16), dtype=torch.uint8, device=dev)
        self.act = torch.empty((R, h), dtype=dt, device=dev)
        self.h13 = torch.empty((R, 2 * h), dtype=dt, device=dev) if backward else None
        self.ye = torch.empty((R, d), dtype=dt, device=dev)
        self.y = torch.empty((T, d), dtype=dt, device=dev)
        self.side_shared = self.shared and not self.merged
        if self.side_shared:
            hs = self.hs
            self.sh_off = torch.tensor([0, T], dtype=torch.int32, device=dev)
            self.sh_act = torch.empty((T, hs), dtype=dt, device=dev)
            self.sh_h13 = torch.empty((T, 2 * hs), dtype=dt, device=dev) if backward else None
            self.sh_y = torch.empty((T, d), dtype=dt, device=dev)
            self.side = torch.cuda.Stream(device=dev)
        if backward:
            self.dtopk_w_all = torch.empty((T, kc), **f32)  # every slot; the routed ones first
            self.dye = torch.empty((R, d), dtype=dt, device=dev)
            self.dh13 = torch.empty((R, 2 * h), dtype=dt, device=dev)
            self.dxs = torch.empty((R, d), dtype=dt, device=dev)
            self.dW1 = torch.empty((Ec, d, h), dtype=dt, device=dev)
            self.dW3 = torch.empty((Ec, d, h), dtype=dt, device=dev)
            self.dW2 = torch.empty((Ec, h, d), dtype=dt, device=dev)
            self.dx = torch.empty((T, d), dtype=dt, device=dev)
            self.dwg = torch.empty((d, E), **f32)
            self.rdx = torch.empty((T, d), dtype=dt, device=dev)  # the gate's term of dx
            self.rbwd_ws = torch.empty(max(xmoe_route_bwd_workspace_size(T, d, E, dt), 16), dtype=torch.uint8,
                                       device=dev)
            if self.side_shared:
                hs = self.hs
                self.sh_dh13 = torch.empty((T, 2 * hs), dtype=dt, device=dev)
                self.sh_dx = torch.empty((T, d), dtype=dt, device=dev)
                self._ds1 = torch.empty((1, d, hs), dtype=dt, device=dev)
                self._ds3 = torch.empty((1, d, hs), dtype=dt, device=dev)
                self._ds2 = torch.empty((1, hs, d), dtype=dt, device=dev)

    def refresh_weights(self, stream=None) -> None:
        """Merged layout only: copy the routed and shared weights (the tensors in
        the weights dict, in their own layouts) into the layer's [E + n, ...]
        buffers, in place on `stream`.  The merged buffers are copies, so a
        caller that updates the weights (an optimizer step) calls this before
        the next forward; without merging the layer reads the caller's tensors
        directly and this does nothing.  It allocates nothing, so it can sit
        inside a captured graph."""
        if not self.merged:
            return
        w, E, ns, d, h = self.w, self.E, self.ns, self.d, self.h
        main = stream if stream is not None else torch.cuda.current_stream(self.device)
        with torch.cuda.stream(main):
            self.W1[:E].copy_(w["w1"])
            self.W3[:E].copy_(w["w3"])
            self.W2[:E].copy_(w["w2"])
            self.W1[E:].copy_(w["s1"].view(d, ns, h).permute(1, 0, 2))
            self.W3[E:].copy_(w["s3"].view(d, ns, h).permute(1, 0, 2))
            self.W2[E:].copy_(w["s2"].view(ns, h, d))

    # views of the unmerged shared-expert weights as a single expert of width n*h_s
    def _shared_w(self):
        w = self.w
        return w["s1"].unsqueeze(0), w["s3"].unsqueeze(0), w["s2"].unsqueeze(0)

    def _streams(self, stream):
        main = stream if stream is not None else torch.cuda.current_stream(self.device)
        side = self.side if (self.side_shared and self.overlap) else main
        return main, side

    def forward(self, x: torch.Tensor, stream=None, hook=None, probe=None) -> torch.Tensor:
        """hook(name), if given, is called after each library call is enqueued.
        probe(name, stream), if given, is called right before and right after
        each up-projection launch ("up" / "up_end" for the routed experts,
        "shared_up" / "shared_up_end" for the shared ones) with the stream the
        launch goes to, e.g. to record events around it."""
        w = self.w
        mark = hook or (lambda name: None)
        around = probe or (lambda name, s: None)
        main, side = self._streams(stream)
        keep = self.backward_enabled and not self.lean
        if self.side_shared:
            side.wait_stream(main)
            s1, s3, s2 = self._shared_w()
            around("shared_up", side)
            xmoe_expert_ffn_up(x, s1, s3, self.sh_off, self.sh_act, h13=self.sh_h13 if keep else None, stream=side)
            around("shared_up_end", side)
            xmoe_expert_ffn_down(self.sh_act, s2, self.sh_off, self.sh_y, stream=side)
            if side is main:
                mark("shared_ffn")
        xmoe_route(x, w["wg"], self.k, self.topk_ids, self.topk_w, self.logits, self.inv_tau,
                   w.get("logit_bias"), w.get("select_bias"), workspace=self.route_ws, stream=main)
        mark("route")
        if self.merged:
            xmoe_build_pft_shared(self.topk_ids, self.topk_w, self.E, self.ns, self.pft, self.pft_ws, stream=main)
        else:
            xmoe_build_pft(self.topk_ids, self.topk_w, self.E, self.pft, self.pft_ws, stream=main)
        mark("build_pft")
        around("up", main)
        xmoe_expert_ffn_up_gather(x, self.pft.token_ids, self.W1, self.W3, self.pft.expert_offsets, self.act,
                                  h13=self.h13 if keep else None, stream=main)
        around("up_end", main)
        xmoe_expert_ffn_down(self.act, self.W2, self.pft.expert_offsets, self.ye, stream=main)
        mark("expert_ffn")
        y_add = None
        if self.side_shared:
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
        gs = self.gside if self.overlap else main
        dx_add = None
        if self.side_shared:
            side.wait_stream(main)
            s1, s3, s2 = self._shared_w()
            if self.lean:
                xmoe_expert_ffn_up(self.x, s1, s3, self.sh_off, None, self.sh_h13, stream=side)
                if side is main:
                    mark("recompute_shared_h13")
            xmoe_expert_ffn_bwd(self.x, s1, s3, s2, self.sh_act, self.sh_h13, dy, self.sh_off, self.sh_dh13,
                                self.sh_dx, self._ds1, self._ds3, self._ds2, stream=side)
            if side is main:
                mark("shared_ffn_bwd")
        off = self.pft.expert_offsets
        ws = self.wside if self.overlap else main
        # dA reads dy through the PFT and applies each row's combine weight
        # itself, so it does not wait for the combine backward, which runs
        # beside it on the weight-gradient stream: its dye feeds dW2 there and
        # its dtopk_w the gate's backward
        if ws is not main:
            ws.wait_stream(main)
        xmoe_combine_bwd(dy, self.ye, self.pft, self.dye, self.dtopk_w_all, stream=ws)
        if ws is main:
            mark("combine_bwd")
        # the gate's backward needs only the routed slots' dtopk_w, the logits
        # and x: it runs beside the expert backward.  With unmerged shared
        # experts it adds dz . wg^T into their dx; otherwise it writes its own
        # term, which the dispatch backward adds.
        rdst = self.sh_dx if self.side_shared else self.rdx
        if self.side_shared:
            gs = side
        if gs is not ws:
            gs.wait_stream(ws)
        xmoe_route_bwd(self.x, w["wg"], self.logits, self.topk_ids, self.dtopk_w, rdst, self.dwg,
                       self.rbwd_ws, self.inv_tau, accumulate=self.side_shared, stream=gs)
        if gs is main:
            mark("route_bwd")
        dx_add = rdst
        if self.lean:
            # recompute the pre-activations only (act is kept from the forward)
            xmoe_expert_ffn_up_gather(self.x, self.pft.token_ids, self.W1, self.W3, self.pft.expert_offsets,
                                      None, self.h13, stream=main)
            mark("recompute_h13")
        xmoe_expert_ffn_bwd_dact_gather(dy, self.pft.token_ids, self.pft.combine_weights, self.W2, self.h13, off,
                                        self.dh13, stream=main)
        mark("bwd_dact")
        # weight gradients: dW2 needs act and dye only; dW1/dW3 need dH1/dH3 and
        # the token rows, gathered through the PFT inside their loads
        xmoe_expert_ffn_bwd_dw2(self.act, self.dye, off, self.dW2, stream=ws)
        if ws is main:
            mark("bwd_dw2")
        w13 = main if self.dw13_main else ws
        if w13 is not main:
            w13.wait_stream(main)
        xmoe_expert_ffn_bwd_dw13_gather(self.x, self.pft.token_ids, self.dh13, off, self.dW1, self.dW3, stream=w13)
        if w13 is main:
            mark("bwd_dw13")
        xmoe_expert_ffn_bwd_dx(self.dh13, self.W1, self.W3, off, self.dxs, stream=main)
        mark("bwd_dx")
        main.wait_stream(gs)
        xmoe_dispatch_bwd(self.dxs, self.pft, self.T, self.dx, dx_add=dx_add, stream=main)
        mark("dispatch_bwd")
        # every gradient is complete in the caller's stream order (the gate's
        # stream joined before the dispatch backward); only streams this call
        # used are joined, so that the step can also be captured as a graph
        if ws is not main:
            main.wait_stream(ws)
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
        if self.side_shared:
            n += nb(self.sh_act) + (0 if self.lean else nb(self.sh_h13))
        return n

    # gradients in the layer's argument layout
    @property
    def dtopk_w(self) -> torch.Tensor:
        """[T, k] gradient of the routing weights (the routed slots)."""
        return self.dtopk_w_all[:, :self.k]

    @property
    def dw1(self) -> torch.Tensor:
        return self.dW1[:self.E]

    @property
    def dw3(self) -> torch.Tensor:
        return self.dW3[:self.E]

    @property
    def dw2(self) -> torch.Tensor:
        return self.dW2[:self.E]

    def _shared_grad(self, which: int) -> torch.Tensor:
        """[1, d, n*h_s] (ds1, ds3) or [1, n*h_s, d] (ds2)."""
        if not self.merged:
            return (self._ds1, self._ds3, self._ds2)[which]
        E, ns, d, h = self.E, self.ns, self.d, self.h
        if which == 2:
            return self.dW2[E:].reshape(1, ns * h, d)
        src = self.dW1 if which == 0 else self.dW3
        return src[E:].permute(1, 0, 2).reshape(1, d, ns * h)

    @property
    def ds1(self) -> torch.Tensor:
        return self._shared_grad(0)

    @property
    def ds3(self) -> torch.Tensor:
        return self._shared_grad(1)

    @property
    def ds2(self) -> torch.Tensor:
        return self._shared_grad(2)

    def grads(self) -> Dict[str, torch.Tensor]:
        g = {"dx": self.dx, "dwg": self.dwg, "dw1": self.dw1, "dw3": self.dw3, "dw2": self.dw2,
             "dtopk_w": self.dtopk_w, "dye": self.dye, "dxs": self.dxs, "dh13": self.dh13}
        if self.shared:
            g.update(ds1=self.ds1[0], ds3=self.ds3[0], ds2=self.ds2[0])
        return g
