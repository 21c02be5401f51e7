"""A stack of MoE feed-forward layers joined by RMSNorm + residual.

The decoder of "Mixtral > Architecture Overview" (mbrenndoerfer.com,
layer-components list) stacks 32 blocks; this driver keeps only their MoE
feed-forward halves, joined pre-norm style:

    u_0 = RMSNorm(x_0);  for l in 0..L-1:  y_l = MoE_l(u_l);  x_{l+1} = x_l + y_l;  u_{l+1} = RMSNorm(x_{l+1})

with an fp32 residual stream and bf16 layer inputs.  Every step runs in
libmoe; this module only sequences the calls and owns the buffers.  Each layer writes its per-expert
token counts into one row of ``hist`` [L, 8].
"""

from __future__ import annotations

import torch

from . import inputs, moe

MODES = ("combine", "router", "none")


class MoEStack:
    """``mode`` says how much of the glue between layers is fused (all three
    compute the same function):

    * ``"combine"`` (default): each layer's combine adds its output straight
      into the residual, and the same launch normalises and computes the
      next layer's routing (``moe_ffn_forward_routed_residual``); y is never
      written;
    * ``"router"``: the layer writes y (``moe_ffn_forward_routed``), then the
      glue adds it, normalises and routes the next layer
      (``moe_rmsnorm_residual_route``);
    * ``"none"``: every layer routes its own input (``moe_ffn_forward``) and
      the glue only adds and normalises (``moe_rmsnorm_residual``).
    """

    def __init__(self, T, d, f, layers, seed=5, device="cuda", eps=1e-5, mode="combine"):
        assert mode in MODES
        self.T, self.d, self.f, self.L, self.eps, self.mode = T, d, f, layers, eps, mode
        self.weights = [inputs.make_layer_weights(d, f, 8, "bf16", seed, layer, device) for layer in range(layers)]
        self.resid = torch.empty((T, d), dtype=torch.float32, device=device)
        self.u = torch.empty((T, d), dtype=torch.bfloat16, device=device)
        self.hist = torch.zeros((layers, 8), dtype=torch.int32, device=device)
        self.y = torch.empty((T, d), dtype=torch.bfloat16, device=device)
        # routing of the current and the next layer (the fused glue writes the next while the layer reads its own)
        self.idx = [torch.empty((T, 2), dtype=torch.int32, device=device) for _ in range(2)]
        self.w = [torch.empty((T, 2), dtype=torch.float32, device=device) for _ in range(2)]
        ws = moe.alloc_workspace(T, d, f, torch.bfloat16, device=device)  # shared by all layers
        self.layers = [moe.FFN(self.u, lw["w_gate"], lw["w1"], lw["w3"], lw["w2"], lw["logit_bias"], y=self.y,
                               workspace=ws, counts=self.hist[layer])
                       for layer, lw in enumerate(self.weights)]
        self.routed = [moe.RoutedFFN(self.u, lw["w1"], lw["w3"], lw["w2"], y=self.y, workspace=ws,
                                     counts=self.hist[layer])
                       for layer, lw in enumerate(self.weights)]
        self.residual = [moe.RoutedResidualFFN(self.u, lw["w1"], lw["w3"], lw["w2"], workspace=ws,
                                               counts=self.hist[layer], eps=eps)
                         for layer, lw in enumerate(self.weights)]

    def _glue(self, y_add, next_layer):
        """resid += y_add; u = RMSNorm(resid); with a fused mode also the
        routing of layer ``next_layer`` (if any) into routing slot
        next_layer % 2."""
        if self.mode != "none" and next_layer is not None:
            lw = self.weights[next_layer]
            b = next_layer % 2
            moe.rmsnorm_residual_route(self.resid, y_add, self.u, lw["w_gate"], lw["logit_bias"], self.idx[b],
                                       self.w[b], self.eps)
            return
        lib = moe.load_library()
        moe._check("moe_rmsnorm_residual", lib.moe_rmsnorm_residual(
            self.T, self.d, moe.ptr(self.resid), moe.ptr(y_add), moe.ptr(self.u), self.eps, moe.MOE_BF16,
            moe.stream_handle()))

    def load_input(self, x0):
        """x_0 (fp32 [T, d]) into the residual stream; u_0 = RMSNorm(x_0)."""
        self.resid.copy_(x0)
        self._glue(None, 0)

    def forward(self, capture=(), rows=None):
        """Run all layers on the loaded input.  ``capture``: layer indices whose
        input u_l, output y_l and expert ids are copied and returned as
        {l: (u_l, y_l, topk_idx_l)}; ``rows`` (a device index tensor or None)
        keeps only those token rows of each.  In the "combine" mode y_l is
        never written; it is returned as the change of the fp32 residual
        (float64), which differs from the bf16 y_l that was added by at most
        the rounding of that addition."""
        out = {}

        def keep(t):
            return t.clone() if rows is None else t.index_select(0, rows)

        for layer_idx in range(self.L):
            cap = layer_idx in capture
            u_in = keep(self.u) if cap else None
            nxt = layer_idx + 1 if layer_idx + 1 < self.L else None
            b = layer_idx % 2
            if self.mode == "combine":
                idx_in = keep(self.idx[b]) if cap else None
                r_in = keep(self.resid).double() if cap else None
                lw = self.weights[nxt] if nxt is not None else None
                self.residual[layer_idx](self.idx[b], self.w[b], self.resid, self.u,
                                         lw["w_gate"] if lw else None, lw["logit_bias"] if lw else None,
                                         self.idx[1 - b] if lw else None, self.w[1 - b] if lw else None)
                if cap:
                    out[layer_idx] = (u_in, keep(self.resid).double() - r_in, idx_in)
                continue
            if self.mode == "router":
                idx_in = keep(self.idx[b]) if cap else None
                y = self.routed[layer_idx](self.idx[b], self.w[b])
            else:
                y = self.layers[layer_idx]()
                idx_in = keep(self.layers[layer_idx].idx) if cap else None
            if cap:
                out[layer_idx] = (u_in, keep(y), idx_in)
            self._glue(y, nxt)
        return out
