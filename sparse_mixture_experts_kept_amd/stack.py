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


class MoEStack:
    """``fused`` (default): the glue after layer l also computes layer l+1's
    routing (``moe_rmsnorm_residual_route``) and the layers run from it
    (``moe_ffn_forward_routed``); otherwise every layer routes its own input
    (``moe_rmsnorm_residual`` + ``moe_ffn_forward``).  Both compute the same
    function."""

    def __init__(self, T, d, f, layers, seed=5, device="cuda", eps=1e-5, fused=True):
        self.T, self.d, self.f, self.L, self.eps, self.fused = T, d, f, layers, eps, fused
        self.weights = [inputs.make_layer_weights(d, f, 8, "bf16", seed, layer, device) for layer in range(layers)]
        self.resid = torch.empty((T, d), dtype=torch.float32, device=device)
        self.u = torch.empty((T, d), dtype=torch.bfloat16, device=device)
        self.hist = torch.zeros((layers, 8), dtype=torch.int32, device=device)
        self.y = torch.empty((T, d), dtype=torch.bfloat16, device=device)
        self.idx = torch.empty((T, 2), dtype=torch.int32, device=device)  # next layer's routing (fused)
        self.w = torch.empty((T, 2), dtype=torch.float32, device=device)
        ws = moe.alloc_workspace(T, d, f, torch.bfloat16, device=device)  # shared by all layers
        self.layers = [moe.FFN(self.u, lw["w_gate"], lw["w1"], lw["w3"], lw["w2"], lw["logit_bias"], y=self.y,
                               workspace=ws, counts=self.hist[layer])
                       for layer, lw in enumerate(self.weights)]
        self.routed = [moe.RoutedFFN(self.u, lw["w1"], lw["w3"], lw["w2"], y=self.y, workspace=ws,
                                     counts=self.hist[layer])
                       for layer, lw in enumerate(self.weights)]

    def _glue(self, y_add, next_layer):
        """resid += y_add; u = RMSNorm(resid); with the fused form also the
        routing of layer ``next_layer`` (if any)."""
        if self.fused and next_layer is not None:
            lw = self.weights[next_layer]
            moe.rmsnorm_residual_route(self.resid, y_add, self.u, lw["w_gate"], lw["logit_bias"], self.idx, self.w,
                                       self.eps)
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
        keeps only those token rows of each."""
        out = {}

        def keep(t):
            return t.clone() if rows is None else t.index_select(0, rows)

        for layer_idx in range(self.L):
            u_in = keep(self.u) if layer_idx in capture else None
            if self.fused:
                idx_in = keep(self.idx) if layer_idx in capture else None
                y = self.routed[layer_idx](self.idx, self.w)
            else:
                y = self.layers[layer_idx]()
                idx_in = keep(self.layers[layer_idx].idx) if layer_idx in capture else None
            if layer_idx in capture:
                out[layer_idx] = (u_in, keep(y), idx_in)
            self._glue(y, layer_idx + 1 if layer_idx + 1 < self.L else None)
        return out
