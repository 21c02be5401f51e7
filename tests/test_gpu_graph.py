"""The layer captured into a HIP graph (torch.cuda.CUDAGraph) and replayed.

moe_ffn_forward allocates nothing, synchronises nothing and records no
memory fills, so one call captures into a graph whose replays run the same
kernels on whatever the captured buffers hold.  Each replay here follows new
input data written into the captured x, eager work of the program itself
(the same layer called directly on another set of buffers) and a device
synchronisation; every replay must equal the eager call on the same input
bit for bit, and one replay is checked against the oracle.
"""

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from sparse_mixture_experts_kept_amd import inputs, moe

pytestmark = pytest.mark.gpu


def _oracle_check(x, layer, y, idx):
    """Every token's output under the pair the GPU chose (near-tie tokens
    included), and the pairs valid top-2 choices of the oracle's scores."""
    xs = x.cpu()
    w1, w3, w2 = (layer[n].cpu() for n in ("w1", "w3", "w2"))
    widen = lambda e: (w1[e].double().numpy(), w3[e].double().numpy(), w2[e].double().numpy())  # noqa: E731
    gi = idx.cpu().numpy().astype(np.int64)
    ref = O.moe_ffn(xs, layer["w_gate"].cpu(), None, None, None, idx=gi, widen_expert=widen)
    assert O.is_valid_top2(ref["logits"], gi, 1e-4).all()
    yr = ref["y"]
    err = np.abs(y.float().cpu().numpy().astype(np.float64) - yr).max()
    assert err <= 2e-2 * np.abs(yr).max() + 2e-3, err


@pytest.mark.parametrize("T,d,f", [(32, 512, 1024), (1100, 512, 1024)])
def test_layer_replays_from_a_hip_graph(T, d, f):
    # T=32: routing fused with the permutation, the streaming kernels, the
    # combine.  T=1100: router, group permutation, the prefill GEMMs with
    # their remainder split and fixups, the up projection's streamed tails
    # (about 275 rows per expert), the split down projection and its
    # two-partial combine.
    layer = inputs.make_custom(T, d, f, seed=T, device="cuda")
    x = layer["x"].clone()
    graphed = moe.FFN(x, layer["w_gate"], layer["w1"], layer["w3"], layer["w2"])
    x_eager = torch.empty_like(x)
    eager = moe.FFN(x_eager, layer["w_gate"], layer["w1"], layer["w3"], layer["w2"])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        graphed()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graphed()
    torch.cuda.synchronize()

    for r in range(4):
        xr = inputs.make_x(T, d, "bf16", 100 + r, 0, "cuda")
        x.copy_(xr)
        x_eager.copy_(xr)
        y_eager = eager().clone()
        idx_eager = eager.idx.clone()
        counts_eager = eager.counts.clone()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(graphed.y, y_eager), f"replay {r}"
        assert torch.equal(graphed.idx, idx_eager), f"replay {r}"
        assert torch.equal(graphed.counts, counts_eager), f"replay {r}"
        if r == 3:
            _oracle_check(x, layer, graphed.y, graphed.idx)
