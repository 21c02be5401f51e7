"""The flop/byte accounting reproduces the parameter counts the pages print
(tests/golden/param_counts.json cites them)."""

import json
import os

from sparse_mixture_experts_kept_amd import accounting as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rel(a, b):
    return abs(a - b) / abs(b)


def test_parameter_counts_match_the_pages():
    with open(os.path.join(GOLDEN, "param_counts.json")) as fh:
        g = json.load(fh)
    d, f, E, k, L = g["hidden"], g["ffn"], g["experts"], g["active"], g["layers"]
    assert _rel(A.projection_params(d, f), g["per_projection_params_approx"]) < g["per_projection_rel_tol"]
    assert _rel(A.expert_params(d, f, L), g["per_expert_all_layers_approx"]) < g["per_expert_rel_tol"]
    ffn = A.ffn_params(d, f, E, L)
    assert _rel(ffn, g["ffn_total_approx"]) < g["ffn_total_rel_tol"]
    total = ffn + g["non_ffn_params"]
    assert _rel(total, g["total_approx"]) < g["total_rel_tol"]
    assert _rel(total, g["total_headline"]) < g["headline_rel_tol"]
    active = A.active_ffn_params(d, f, k, L) + g["non_ffn_params"]
    assert _rel(active, g["active_approx"]) < g["active_rel_tol"]
    assert abs(k / E - g["active_expert_fraction"]) < 1e-12


def test_layer_flops_and_bytes():
    m = A.MIXTRAL
    d, f, E, k = m["d"], m["f"], m["E"], m["k"]
    assert A.layer_flops(1, d, f, E, k) == 704_708_608
    assert A.expert_weight_bytes(d, f, E) == 2_818_572_288
    assert A.layer_flops(4096, d, f, E, k) == 4096 * 704_708_608
    # up + down per slot equals the per-token expert flops divided by k
    assert k * (A.up_flops_per_slot(d, f) + A.down_flops_per_slot(d, f)) == A.expert_flops_per_token(d, f, k)
    assert A.decode_layer_bytes(32, d, f, E, k, 8) == 2_818_572_288 + 8 * 4096 * 2 + 2 * 32 * 4096 * 2


def test_prefill_rows_issued():
    # one expert per case: a full tile, ragged last tiles of each height, a
    # streamed tail, and experts with a single short tile
    assert A.prefill_rows_issued([256]) == (256, 256, 0)
    assert A.prefill_rows_issued([300]) == (300, 256 + 64, 0)
    assert A.prefill_rows_issued([256 + 100]) == (356, 256 + 128, 0)
    assert A.prefill_rows_issued([256 + 129]) == (385, 256 + 160, 0)
    assert A.prefill_rows_issued([256 + 161]) == (417, 512, 0)
    assert A.prefill_rows_issued([1025]) == (1025, 1024, 16)
    assert A.prefill_rows_issued([256 + 32]) == (288, 256, 32)
    assert A.prefill_rows_issued([256 + 33]) == (289, 256 + 64, 0)
    assert A.prefill_rows_issued([20]) == (20, 32, 0)
    assert A.prefill_rows_issued([160]) == (160, 160, 0)
    assert A.prefill_rows_issued([0, 0]) == (0, 0, 0)
    counts = [1024, 300, 1025, 20]
    n, g, t = A.prefill_rows_issued(counts)
    assert n == sum(counts) and g == 1024 + 320 + 1024 + 32 and t == 16
