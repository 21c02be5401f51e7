"""Seeded synthetic inputs for the sparse MoE feed-forward layer.

This module only draws random numbers in the layouts the library consumes; it
holds none of the layer's arithmetic.  Both the GPU tests and the CPU oracle
consume the tensors it returns (the oracle widens the very same bf16/fp32
values to float64), so generator details cannot confound parity.

Layouts (row-major, last index contiguous): x [T, d]; w_gate [E, d];
w1 (gate) and w3 (up) [E, f, d]; w2 (down) [E, d, f]; logit_bias [E] or None.

Workloads (shapes from "Mixtral > Architecture Overview", mbrenndoerfer.com,
hyperparameter list: hidden 4096, FFN width 14336, 8 experts, 2 active, 32
layers):

* ``tiny_fp32``: T=64, d=128, f=256, fp32; x ~ N(0, 1); w_gate, w1, w3 ~
  N(0, 1/d) and w2 ~ N(0, 1/f), the second argument read as a variance.
* ``decode``: T=32, bf16.  ``prefill``: T=4096, bf16.  ``prefill_skewed``:
  T=4096 plus a per-expert logit bias giving Zipf(1.2) slot shares.
  ``stack``: T=8192 and 32 layers with independent weights.  For all bf16
  workloads x is z / rms(z) with z ~ N(0, 1) (rms with eps 1e-5) rounded to
  bf16, and every weight is N(0, 0.02^2) rounded to bf16 (round to nearest
  even), which makes the router scores spread about 1.28 and routing close
  to uniform.

Smaller bf16 shapes used by the tests keep those spreads by scaling the
standard deviation of the matrices that read d (w_gate, w1, w3) by
sqrt(4096 / d) and of w2 by sqrt(14336 / f).
"""

from __future__ import annotations

import json
import os

import torch

WORKLOADS = {
    "tiny_fp32": dict(T=64, d=128, f=256, E=8, k=2, dtype="f32", layers=1, skew=False),
    "decode": dict(T=32, d=4096, f=14336, E=8, k=2, dtype="bf16", layers=1, skew=False),
    "prefill": dict(T=4096, d=4096, f=14336, E=8, k=2, dtype="bf16", layers=1, skew=False),
    "prefill_skewed": dict(T=4096, d=4096, f=14336, E=8, k=2, dtype="bf16", layers=1, skew=True),
    "stack": dict(T=8192, d=4096, f=14336, E=8, k=2, dtype="bf16", layers=32, skew=False),
}

_TENSOR_IDS = {"x": 0, "w_gate": 1, "w1": 2, "w3": 3, "w2": 4, "perm": 5}
_DATA = os.path.join(os.path.dirname(os.path.abspath(__file__)), "data")


def tensor_seed(base_seed: int, layer: int, name: str) -> int:
    """One independent seed per (base seed, layer, tensor)."""
    return (int(base_seed) * 1_000_003 + int(layer) * 1_009 + _TENSOR_IDS[name] * 7919 + 17) % (2 ** 63 - 1)


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, std, device, seed):
    return torch.randn(shape, generator=_gen(device, seed), device=device, dtype=torch.float32) * std


def zipf_bias_by_rank():
    with open(os.path.join(_DATA, "zipf_bias.json")) as fh:
        return json.load(fh)["bias_by_rank"]


def make_layer_weights(d, f, E=8, dtype="bf16", seed=0, layer=0, device="cpu", skew=False, wstd=None):
    """w_gate [E,d], w1/w3 [E,f,d], w2 [E,d,f] (and logit_bias [E] fp32 or None)."""
    if dtype == "f32":
        s_in, s_down = (d ** -0.5, f ** -0.5)
    else:
        s_in = 0.02 * (4096.0 / d) ** 0.5 if wstd is None else wstd
        s_down = 0.02 * (14336.0 / f) ** 0.5 if wstd is None else wstd
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    out = {}
    out["w_gate"] = _normal((E, d), s_in, device, tensor_seed(seed, layer, "w_gate")).to(tdt)
    out["w1"] = _normal((E, f, d), s_in, device, tensor_seed(seed, layer, "w1")).to(tdt)
    out["w3"] = _normal((E, f, d), s_in, device, tensor_seed(seed, layer, "w3")).to(tdt)
    out["w2"] = _normal((E, d, f), s_down, device, tensor_seed(seed, layer, "w2")).to(tdt)
    out["logit_bias"] = None
    if skew:
        ranks = torch.randperm(E, generator=_gen("cpu", tensor_seed(seed, layer, "perm")))
        by_rank = torch.tensor(zipf_bias_by_rank(), dtype=torch.float32)
        bias = torch.empty(E, dtype=torch.float32)
        bias[ranks] = by_rank  # expert ranks[r] gets the bias of rank r
        out["logit_bias"] = bias.to(device)
    return out


def make_x(T, d, dtype="bf16", seed=0, layer=0, device="cpu"):
    """Token activations [T, d]: N(0,1) for fp32, RMS-normalised N(0,1) in bf16."""
    z = _normal((T, d), 1.0, device, tensor_seed(seed, layer, "x"))
    if dtype == "f32":
        return z
    z = z / torch.sqrt(torch.mean(z * z, dim=1, keepdim=True) + 1e-5)
    return z.to(torch.bfloat16)


def make_workload(name, seed=None, device="cpu", layer=0, T=None):
    """Inputs of one named workload layer (weights of layer ``layer``)."""
    w = dict(WORKLOADS[name])
    if T is not None:
        w["T"] = T
    base = {"tiny_fp32": 1, "decode": 2, "prefill": 3, "prefill_skewed": 4, "stack": 5}[name] if seed is None else seed
    out = make_layer_weights(w["d"], w["f"], w["E"], w["dtype"], base, layer, device, w["skew"])
    out["x"] = make_x(w["T"], w["d"], w["dtype"], base, layer, device)
    out["dims"] = dict(T=w["T"], d=w["d"], f=w["f"], E=w["E"], k=w["k"], dtype=w["dtype"])
    return out


def make_custom(T, d, f, dtype="bf16", seed=0, device="cpu", skew=False, wstd=None):
    """A layer of arbitrary (test) shape with the workload recipes above."""
    out = make_layer_weights(d, f, 8, dtype, seed, 0, device, skew, wstd)
    out["x"] = make_x(T, d, dtype, seed, 0, device)
    out["dims"] = dict(T=T, d=d, f=f, E=8, k=2, dtype=dtype)
    return out
