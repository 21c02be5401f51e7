"""A stack of MoE feed-forward layers joined by RMSNorm + residual.

The decoder of "Mixtral > Architecture Overview" (mbrenndoerfer.com,
layer-components list) stacks 32 blocks; this driver keeps only their MoE
feed-forward halves, joined pre-norm style:

    u_0 = RMSNorm(x_0);  for l in 0..L-1:  y_l = MoE_l(u_l);  x_{l+1} = x_l + y_l;  u_{l+1} = RMSNorm(x_{l+1})

with an fp32 residual stream and bf16 layer inputs.  Every step runs in
libmoe (``moe_ffn_forward`` and ``moe_rmsnorm_residual``); this module only
sequences the calls and owns the buffers.  Each layer writes its per-expert
token counts into one row of ``hist`` [L, 8].
"""

from __future__ import annotations

import torch

from . import inputs, moe


class MoEStack:
    def __init__(self, T, d, f, layers, seed=5, device="cuda", eps=1e-5):
        self.T, self.d, self.f, self.L, self.eps = T, d, f, layers, eps
        self.weights = [inputs.make_layer_weights(d, f, 8, "bf16", seed, layer, device) for layer in range(layers)]
        self.resid = torch.empty((T, d), dtype=torch.float32, device=device)
        self.u = torch.empty((T, d), dtype=torch.bfloat16, device=device)
        self.hist = torch.zeros((layers, 8), dtype=torch.int32, device=device)
        self.y = torch.empty((T, d), dtype=torch.bfloat16, device=device)
        ws = moe.alloc_workspace(T, d, f, torch.bfloat16, device=device)  # shared by all layers
        self.layers = [moe.FFN(self.u, lw["w_gate"], lw["w1"], lw["w3"], lw["w2"], lw["logit_bias"], y=self.y,
                               workspace=ws, counts=self.hist[layer])
                       for layer, lw in enumerate(self.weights)]

    def load_input(self, x0):
        """x_0 (fp32 [T, d]) into the residual stream; u_0 = RMSNorm(x_0)."""
        self.resid.copy_(x0)
        lib = moe.load_library()
        moe._check("moe_rmsnorm_residual", lib.moe_rmsnorm_residual(
            self.T, self.d, moe.ptr(self.resid), None, moe.ptr(self.u), self.eps, moe.MOE_BF16, moe.stream_handle()))

    def forward(self, capture=()):
        """Run all layers on the loaded input.  ``capture``: layer indices whose
        input u_l, output y_l and expert ids are cloned and returned as
        {l: (u_l, y_l, topk_idx_l)}."""
        lib = moe.load_library()
        out = {}
        for layer_idx, layer in enumerate(self.layers):
            u_in = self.u.clone() if layer_idx in capture else None
            y = layer()
            if layer_idx in capture:
                out[layer_idx] = (u_in, y.clone(), layer.idx.clone())
            moe._check("moe_rmsnorm_residual", lib.moe_rmsnorm_residual(
                self.T, self.d, moe.ptr(self.resid), moe.ptr(y), moe.ptr(self.u), self.eps, moe.MOE_BF16,
                moe.stream_handle()))
        return out
