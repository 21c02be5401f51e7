"""Pins for the fp64 oracle (CPU only).

Each test checks the oracle against something other than itself: hand-worked
fixtures under tests/golden/, brute force over all expert pairs, closed forms,
special cases that reduce to a textbook routine (scipy / torch), and
invariants that follow from the definition of the layer.  Together they are
chosen so that a dropped term, a wrong sign or index, swapped gate/up
projections, a transposed operand or a wrong tie-break fails at least one.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


def _rand_layer(seed, T=12, d=16, f=24, E=8, scale=0.5):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    wg = rng.standard_normal((E, d)) * scale
    w1 = rng.standard_normal((E, f, d)) / math.sqrt(d)
    w3 = rng.standard_normal((E, f, d)) / math.sqrt(d)
    w2 = rng.standard_normal((E, d, f)) / math.sqrt(f)
    return x, wg, w1, w3, w2


# --------------------------------------------------------------------------- router


def test_router_handworked_fixture():
    g = _load("router_handworked.json")
    logits = O.router_logits(g["x"], g["w_gate"])
    np.testing.assert_array_equal(logits, np.array(g["logits"], dtype=np.float64))
    idx = O.select_top_k(logits, 2)
    np.testing.assert_array_equal(idx, np.array(g["top2"]))
    gates = O.masked_softmax_gates(logits, idx)
    np.testing.assert_allclose(gates, np.array(g["gates"]), rtol=0, atol=1e-15)


def test_router_onehot_picks_a_column_of_the_expert_rows():
    # x = e_i must give logits[e] = W_g[e, i]: catches a transposed W_g.
    rng = np.random.default_rng(0)
    d, E = 5, 8
    wg = rng.standard_normal((E, d))
    for i in range(d):
        x = np.zeros((1, d))
        x[0, i] = 1.0
        np.testing.assert_array_equal(O.router_logits(x, wg)[0], wg[:, i])


def test_router_bias_is_added_per_expert():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 6))
    wg = rng.standard_normal((8, 6))
    b = np.arange(8, dtype=np.float64)
    np.testing.assert_allclose(O.router_logits(x, wg, b) - O.router_logits(x, wg), np.tile(b, (3, 1)),
                               atol=1e-14)


def test_top2_bruteforce_over_all_pairs():
    rng = np.random.default_rng(2)
    l = rng.standard_normal((500, 8))
    idx = O.select_top_k(l, 2)
    for t in range(l.shape[0]):
        best = max(itertools.combinations(range(8), 2), key=lambda p: l[t, p[0]] + l[t, p[1]])
        assert set(best) == set(idx[t].tolist())
        assert l[t, idx[t, 0]] > l[t, idx[t, 1]]  # slot 0 holds the larger score
        others = [l[t, e] for e in range(8) if e not in best]
        assert min(l[t, best[0]], l[t, best[1]]) > max(others)


def test_top2_ties_go_to_lower_index():
    l = np.array([[1.0, 2.0, 2.0, 2.0, 0, 0, 0, 0],
                  [0.0] * 8,
                  [5.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0]])
    np.testing.assert_array_equal(O.select_top_k(l, 2), [[1, 2], [0, 1], [0, 1]])


def test_gates_closed_form():
    rng = np.random.default_rng(3)
    l = rng.standard_normal((200, 8)) * 2
    idx = O.select_top_k(l, 2)
    g = O.masked_softmax_gates(l, idx)
    for t in range(l.shape[0]):
        la, lb = l[t, idx[t, 0]], l[t, idx[t, 1]]
        ga = 1.0 / (1.0 + math.exp(lb - la))
        assert abs(g[t, 0] - ga) < 1e-15
        assert abs(g[t, 1] - (1.0 - ga)) < 1e-15
        assert 0.5 <= g[t, 0] < 1.0
    assert np.all(g >= 0)
    np.testing.assert_allclose(g.sum(axis=1), 1.0, atol=1e-15)


def test_gates_with_k_equal_E_are_the_textbook_softmax():
    rng = np.random.default_rng(4)
    l = rng.standard_normal((50, 8)) * 3
    idx = O.select_top_k(l, 8)
    g = O.masked_softmax_gates(l, idx)
    ref = scipy.special.softmax(l, axis=1)
    np.testing.assert_allclose(g, np.take_along_axis(ref, idx, axis=1), rtol=1e-14, atol=1e-16)


def test_gates_shift_invariant():
    rng = np.random.default_rng(5)
    l = rng.standard_normal((64, 8))
    idx = O.select_top_k(l, 2)
    for c in (-7.5, 0.25, 40.0):
        np.testing.assert_array_equal(O.select_top_k(l + c, 2), idx)
        np.testing.assert_allclose(O.masked_softmax_gates(l + c, idx), O.masked_softmax_gates(l, idx), atol=1e-13)


def test_full_gating_closed_form_and_bruteforce():
    # Scores (2, 1, 0, ..., 0): softmax over all eight gives e^2 / (e^2 + e + 6)
    # and e / (e^2 + e + 6) to the two kept experts.
    l = np.array([[2.0, 1.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0], [0.0, 0.0, 0.0, -1.0, 0.0, 0.0, 3.0, 0.0]])
    idx = O.select_top_k(l, 2)
    np.testing.assert_array_equal(idx, [[0, 1], [6, 0]])
    g = O.softmax_top_k_gates(l, idx)
    den = math.e ** 2 + math.e + 6.0
    np.testing.assert_allclose(g[0], [math.e ** 2 / den, math.e / den], rtol=1e-15)
    den = math.e ** 3 + 6.0 + math.exp(-1.0)
    np.testing.assert_allclose(g[1], [math.e ** 3 / den, 1.0 / den], rtol=1e-15)
    # brute force with math.exp on random scores
    rng = np.random.default_rng(21)
    l = rng.standard_normal((40, 8)) * 2
    idx = O.select_top_k(l, 2)
    g = O.softmax_top_k_gates(l, idx)
    for t in range(l.shape[0]):
        z = sum(math.exp(v) for v in l[t])
        for j in range(2):
            assert abs(g[t, j] - math.exp(l[t, idx[t, j]]) / z) < 1e-14
        assert g[t].sum() < 1.0 and g[t, 0] >= 1.0 / 8


def test_full_gating_renormalises_to_the_pair_softmax():
    # The two readings select the same pair and their weights differ by the
    # common factor p_a + p_b; when the other six scores are far below, the
    # full softmax leaves them no probability and both readings coincide.
    rng = np.random.default_rng(22)
    l = rng.standard_normal((300, 8)) * 1.5
    idx = O.select_top_k(l, 2)
    full = O.softmax_top_k_gates(l, idx)
    pair = O.masked_softmax_gates(l, idx)
    np.testing.assert_allclose(full / full.sum(axis=1, keepdims=True), pair, rtol=1e-14)
    np.testing.assert_allclose(full[:, 0] / full[:, 1], pair[:, 0] / pair[:, 1], rtol=1e-13)
    far = l.copy()
    rows = np.arange(l.shape[0])[:, None]
    keep = np.zeros_like(l, dtype=bool)
    keep[rows, idx] = True
    far[~keep] = -1e4
    np.testing.assert_array_equal(O.softmax_top_k_gates(far, idx), O.masked_softmax_gates(far, idx))
    for c in (-3.0, 11.0):
        np.testing.assert_allclose(O.softmax_top_k_gates(l + c, idx), full, rtol=1e-13)


def test_full_gating_layer_scales_the_dense_output():
    # Shared expert weights: y = (p_a + p_b) * SwiGLU(x) for every token.
    rng = np.random.default_rng(23)
    T, d, f = 30, 16, 24
    x = rng.standard_normal((T, d))
    wg = rng.standard_normal((8, d)) * 0.5
    a1, a3, a2 = (rng.standard_normal((f, d)), rng.standard_normal((f, d)), rng.standard_normal((d, f)))
    out = O.moe_ffn(x, wg, np.stack([a1] * 8), np.stack([a3] * 8), np.stack([a2] * 8), gating="full")
    dense = O.swiglu_expert(x, a1, a3, a2)
    l = x @ wg.T
    p = np.exp(l - l.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    top2 = np.sort(p, axis=1)[:, -2:].sum(axis=1)
    np.testing.assert_allclose(out["y"], top2[:, None] * dense, rtol=1e-12, atol=1e-12)
    assert np.all(out["gates"].sum(axis=1) < 1.0)


def test_full_gating_scalar_and_vectorised_forms_agree():
    x, wg, w1, w3, w2 = _rand_layer(24, T=12, d=16, f=32)
    yv = O.moe_ffn(x, wg, w1, w3, w2, gating="full")["y"]
    ys = O.moe_ffn_scalar(x, wg, w1, w3, w2, gating="full")
    np.testing.assert_allclose(yv, ys, rtol=1e-12, atol=1e-12)
    with pytest.raises(ValueError):
        O.moe_ffn(x, wg, w1, w3, w2, gating="softmax")


# --------------------------------------------------------------------------- capacity limit, load-balance loss


def test_capacity_keep_matches_ranks_in_the_stable_permutation():
    # A slot is admitted iff its position among its expert's slots (the stable
    # expert-major order of expert_permutation) is below the capacity.
    rng = np.random.default_rng(31)
    l = rng.standard_normal((200, 8)) + np.array([1.5, 0.8, 0, 0, 0, 0, 0, -1.0])
    idx = O.select_top_k(l, 2)
    offsets, sorted_slots, slot_rows = O.expert_permutation(idx)
    flat = idx.reshape(-1)
    rank = slot_rows - offsets[flat]
    for cap in (1, 7, 40, 100, 400):
        keep = O.capacity_keep(idx, cap).reshape(-1)
        np.testing.assert_array_equal(keep, rank < cap)
        counts = np.bincount(flat, minlength=8)
        assert keep.sum() == np.minimum(counts, cap).sum()
    assert O.capacity_keep(idx, 0).all()


def test_capacity_handworked_and_no_renormalisation():
    # Four tokens routed (0, 1), (1, 0), (0, 2), (1, 2); capacity 2 admits
    # slots 0, 1, 2, 3 and 5 (expert 2 keeps both its slots) and drops slot 4
    # (expert 0's third) and slot 6 (expert 1's third).
    idx = np.array([[0, 1], [1, 0], [0, 2], [1, 2]])
    keep = O.capacity_keep(idx, 2)
    np.testing.assert_array_equal(keep, [[True, True], [True, True], [False, True], [False, True]])
    x, wg, w1, w3, w2 = _rand_layer(32, T=4)
    full = O.moe_ffn(x, wg, w1, w3, w2, idx=idx)
    capped = O.moe_ffn(x, wg, w1, w3, w2, idx=idx, capacity=2)
    np.testing.assert_allclose(capped["y"][:2], full["y"][:2], rtol=1e-15, atol=0)
    for t in (2, 3):  # only the second expert, weighted by its own (unrenormalised) gate
        o2 = O.swiglu_expert(x[t:t + 1], w1[2], w3[2], w2[2])[0]
        np.testing.assert_allclose(capped["y"][t], full["gates"][t, 1] * o2, rtol=1e-13, atol=1e-15)
    # a token with both slots dropped outputs zero
    idx2 = np.array([[3, 4], [3, 4]])
    y2 = O.moe_ffn(x[:2], wg, w1, w3, w2, idx=idx2, capacity=1)["y"]
    assert np.array_equal(y2[1], np.zeros(x.shape[1])) and np.abs(y2[0]).max() > 0


def test_capacity_at_least_the_largest_count_changes_nothing():
    x, wg, w1, w3, w2 = _rand_layer(33, T=40)
    ref = O.moe_ffn(x, wg, w1, w3, w2)
    big = int(np.bincount(ref["idx"].reshape(-1), minlength=8).max())
    out = O.moe_ffn(x, wg, w1, w3, w2, capacity=big)
    np.testing.assert_array_equal(out["y"], ref["y"])
    assert out["keep"].all()
    out = O.moe_ffn(x, wg, w1, w3, w2, capacity=big - 1)
    assert not out["keep"].all() and not np.array_equal(out["y"], ref["y"])


def test_load_balance_loss_closed_forms():
    # Even router, even routing: f_e = P_e = 1/8, loss 1.
    l = np.zeros((8, 8))
    idx = np.array([[e, (e + 1) % 8] for e in range(8)])
    assert abs(O.load_balance_loss(l, idx) - 1.0) < 1e-15
    # One token, scores (a, b, 0, ..., 0), routed to (0, 1): f = (1/2, 1/2, 0...)
    # and the loss is 8 * (p_0 + p_1) / 2.
    a, b = 2.0, 0.5
    z = math.exp(a) + math.exp(b) + 6.0
    loss = O.load_balance_loss(np.array([[a, b, 0, 0, 0, 0, 0, 0]]), np.array([[0, 1]]))
    assert abs(loss - 4.0 * (math.exp(a) + math.exp(b)) / z) < 1e-14
    # Collapse onto two experts with scores far above the rest: loss -> 4.
    l = np.full((50, 8), -40.0)
    l[:, :2] = 10.0
    assert abs(O.load_balance_loss(l, np.tile([0, 1], (50, 1))) - 4.0) < 1e-12
    assert O.load_balance_loss(np.zeros((0, 8)), np.zeros((0, 2), dtype=np.int64)) == 0.0


# --------------------------------------------------------------------------- experts


def test_silu_pointwise():
    z = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(O.silu(z), z * scipy.special.expit(z), rtol=1e-15, atol=1e-300)
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert O.silu(np.array([-800.0]))[0] == 0.0  # exp overflow gives the correct limit
    assert O.silu(np.array([800.0]))[0] == 800.0
    for v in (-3.0, -0.5, 0.1, 2.0):
        assert abs(O.silu(np.array([v]))[0] - v / (1.0 + math.exp(-v))) < 1e-15


def test_expert_handworked_fixture():
    g = _load("expert_handworked.json")
    for case in g["cases"]:
        h = O.swiglu_hidden(case["x"], case["w1"], case["w3"])
        np.testing.assert_allclose(h, case["h"], rtol=1e-15, atol=1e-15)
        y = O.swiglu_expert(case["x"], case["w1"], case["w3"], case["w2"])
        np.testing.assert_allclose(y, case["y"], rtol=1e-15, atol=1e-15)


def test_expert_matches_torch_functional_in_fp64():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((7, 16))
    w1 = rng.standard_normal((24, 16))
    w3 = rng.standard_normal((24, 16))
    w2 = rng.standard_normal((16, 24))
    tx = torch.from_numpy(x)
    ref = torch.nn.functional.linear(
        torch.nn.functional.silu(torch.nn.functional.linear(tx, torch.from_numpy(w1)))
        * torch.nn.functional.linear(tx, torch.from_numpy(w3)),
        torch.from_numpy(w2)).numpy()
    np.testing.assert_allclose(O.swiglu_expert(x, w1, w3, w2), ref, rtol=1e-12, atol=1e-12)


def test_expert_w3_zero_gives_zero_and_w2_is_linear():
    x, wg, w1, w3, w2 = _rand_layer(7)
    y0 = O.moe_ffn(x, wg, w1, np.zeros_like(w3), w2)["y"]
    assert np.all(y0 == 0.0)
    y = O.moe_ffn(x, wg, w1, w3, w2)["y"]
    y3 = O.moe_ffn(x, wg, w1, w3, 3.0 * w2)["y"]
    np.testing.assert_allclose(y3, 3.0 * y, rtol=1e-13, atol=1e-14)


# --------------------------------------------------------------------------- whole layer


def test_layer_handworked_fixture():
    g = _load("layer_handworked.json")
    E = 8
    w1 = np.tile(np.array([[[1.0, 0.0]]]), (E, 1, 1))
    w3 = np.tile(np.array([[[0.0, 1.0]]]), (E, 1, 1))
    w2 = np.stack([np.array([[e + 1.0], [-(e + 1.0)]]) for e in range(E)])
    out = O.moe_ffn(g["x"], g["w_gate"], w1, w3, w2)
    np.testing.assert_array_equal(out["idx"], g["top2"])
    np.testing.assert_allclose(out["gates"], g["gates"], atol=1e-15)
    np.testing.assert_allclose(out["y"], g["y"], rtol=1e-14, atol=1e-14)
    ys = O.moe_ffn_scalar(g["x"], g["w_gate"], w1, w3, w2)
    np.testing.assert_allclose(ys, g["y"], rtol=1e-14, atol=1e-14)


def test_dense_equivalence_when_experts_share_weights():
    # If every expert has the same weights the layer is one dense SwiGLU FFN,
    # whatever the routing, because the two gates sum to 1.
    rng = np.random.default_rng(8)
    T, d, f = 40, 16, 32
    x = rng.standard_normal((T, d))
    wg = rng.standard_normal((8, d))
    a1, a3, a2 = (rng.standard_normal((f, d)), rng.standard_normal((f, d)), rng.standard_normal((d, f)))
    out = O.moe_ffn(x, wg, np.stack([a1] * 8), np.stack([a3] * 8), np.stack([a2] * 8))
    tx = torch.from_numpy(x)
    dense = torch.nn.functional.linear(
        torch.nn.functional.silu(torch.nn.functional.linear(tx, torch.from_numpy(a1)))
        * torch.nn.functional.linear(tx, torch.from_numpy(a3)), torch.from_numpy(a2)).numpy()
    np.testing.assert_allclose(out["y"], dense, rtol=1e-12, atol=1e-12)


def test_output_equals_bruteforce_best_pair():
    # For each token, evaluate the layer under every one of the 28 expert pairs
    # with that pair's 2-way softmax; the oracle must return the pair with the
    # largest summed score.
    x, wg, w1, w3, w2 = _rand_layer(9, T=10)
    out = O.moe_ffn(x, wg, w1, w3, w2)
    l = x @ wg.T
    for t in range(x.shape[0]):
        best = None
        for a, b in itertools.combinations(range(8), 2):
            if best is None or l[t, a] + l[t, b] > best[0]:
                ea, eb = math.exp(l[t, a]), math.exp(l[t, b])
                ya = np.zeros(x.shape[1])
                for e, wgt in ((a, ea / (ea + eb)), (b, eb / (ea + eb))):
                    hid = np.array([
                        (x[t] @ w1[e, n]) / (1.0 + math.exp(-(x[t] @ w1[e, n]))) * (x[t] @ w3[e, n])
                        for n in range(w1.shape[1])])
                    ya += wgt * (w2[e] @ hid)
                best = (l[t, a] + l[t, b], ya)
        np.testing.assert_allclose(out["y"][t], best[1], rtol=1e-12, atol=1e-12)


def test_scalar_and_vectorised_forms_agree():
    x, wg, w1, w3, w2 = _rand_layer(10, T=16, d=32, f=48)
    b = np.linspace(-1, 1, 8)
    yv = O.moe_ffn(x, wg, w1, w3, w2, logit_bias=b)["y"]
    ys = O.moe_ffn_scalar(x, wg, w1, w3, w2, logit_bias=b)
    np.testing.assert_allclose(yv, ys, rtol=1e-12, atol=1e-12)


def test_token_permutation_equivariance_and_batch_split():
    x, wg, w1, w3, w2 = _rand_layer(11, T=30)
    y = O.moe_ffn(x, wg, w1, w3, w2)["y"]
    perm = np.random.default_rng(12).permutation(x.shape[0])
    np.testing.assert_allclose(O.moe_ffn(x[perm], wg, w1, w3, w2)["y"], y[perm], rtol=1e-13, atol=1e-14)
    ya = O.moe_ffn(x[:13], wg, w1, w3, w2)["y"]
    yb = O.moe_ffn(x[13:], wg, w1, w3, w2)["y"]
    np.testing.assert_allclose(np.concatenate([ya, yb]), y, rtol=1e-13, atol=1e-14)


def test_forced_assignment_matches_selected_one():
    x, wg, w1, w3, w2 = _rand_layer(13, T=20)
    out = O.moe_ffn(x, wg, w1, w3, w2)
    forced = O.moe_ffn(x, wg, w1, w3, w2, idx=out["idx"])
    np.testing.assert_array_equal(forced["y"], out["y"])


def test_exactly_two_distinct_experts_and_counts():
    rng = np.random.default_rng(14)
    l = rng.standard_normal((300, 8))
    idx = O.select_top_k(l, 2)
    assert np.all(idx[:, 0] != idx[:, 1])
    counts = np.bincount(idx.reshape(-1), minlength=8)
    assert counts.sum() == 2 * 300 and counts.max() <= 300


# --------------------------------------------------------------------------- permutation


def test_expert_permutation_matches_bucket_loops():
    rng = np.random.default_rng(15)
    l = rng.standard_normal((37, 8)) + np.array([2, 0, 0, 0, 0, 0, 0, -3.0])
    idx = O.select_top_k(l, 2)
    offsets, sorted_slots, slot_rows = O.expert_permutation(idx, 8)
    flat = idx.reshape(-1).tolist()
    buckets = [[s for s in range(len(flat)) if flat[s] == e] for e in range(8)]
    expect = [s for b in buckets for s in b]
    np.testing.assert_array_equal(sorted_slots, expect)
    assert offsets[0] == 0 and offsets[-1] == len(flat)
    for e in range(8):
        assert offsets[e + 1] - offsets[e] == len(buckets[e])
        assert all(flat[s] == e for s in sorted_slots[offsets[e]:offsets[e + 1]])
    for s in range(len(flat)):
        assert sorted_slots[slot_rows[s]] == s


def test_expert_permutation_empty_experts_and_empty_input():
    idx = np.array([[0, 1]] * 5)
    offsets, sorted_slots, slot_rows = O.expert_permutation(idx, 8)
    np.testing.assert_array_equal(offsets, [0, 5, 10, 10, 10, 10, 10, 10, 10])
    np.testing.assert_array_equal(sorted_slots, [0, 2, 4, 6, 8, 1, 3, 5, 7, 9])
    offsets, sorted_slots, slot_rows = O.expert_permutation(np.zeros((0, 2), dtype=np.int64), 8)
    np.testing.assert_array_equal(offsets, np.zeros(9))
    assert sorted_slots.size == 0 and slot_rows.size == 0


# --------------------------------------------------------------------------- helpers


def test_near_tie_helpers():
    l = np.array([[3.0, 2.0, 2.0 - 5e-5, 0, 0, 0, 0, 0],
                  [3.0, 2.0, 1.0, 0, 0, 0, 0, 0]])
    gap = O.second_third_gap(l)
    np.testing.assert_allclose(gap, [5e-5, 1.0])
    # (0, 2) is an acceptable answer for the near tie, not for the clear case
    ok = O.is_valid_top2(l, np.array([[0, 2], [0, 2]]), 1e-4)
    np.testing.assert_array_equal(ok, [True, False])
    assert not O.is_valid_top2(l, np.array([[0, 0], [0, 0]]), 1e-4).any()
    assert O.is_valid_top2(l, np.array([[0, 1], [0, 1]]), 0.0).all()


def test_rmsnorm_closed_form():
    z = np.array([[3.0, 4.0], [1.0, 1.0]])
    r = O.rmsnorm(z, eps=0.0)
    np.testing.assert_allclose(r[0], [3.0 / math.sqrt(12.5), 4.0 / math.sqrt(12.5)], rtol=1e-15)
    np.testing.assert_allclose(r[1], [1.0, 1.0], rtol=1e-15)
    r = O.rmsnorm(np.random.default_rng(16).standard_normal((4, 64)) * 7, eps=0.0)
    np.testing.assert_allclose(np.mean(r * r, axis=1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(O.rmsnorm(z, eps=1e-5)[0], z[0] / math.sqrt(12.5 + 1e-5), rtol=1e-15)


def test_empty_batch():
    _, wg, w1, w3, w2 = _rand_layer(17)
    out = O.moe_ffn(np.zeros((0, 16)), wg, w1, w3, w2)
    assert out["y"].shape == (0, 16) and out["idx"].shape == (0, 2)


@pytest.mark.parametrize("mistake", ["swap_gate_up", "no_renormalise", "ties_to_higher", "drop_second"])
def test_planted_mistakes_fail_a_pin(mistake, monkeypatch):
    """A plausible mistake planted in the oracle (on the CPU) must make one of
    the hand-worked pins fail."""
    g = _load("layer_handworked.json")
    E = 8
    w1 = np.tile(np.array([[[1.0, 0.0]]]), (E, 1, 1))
    w3 = np.tile(np.array([[[0.0, 1.0]]]), (E, 1, 1))
    w2 = np.stack([np.array([[e + 1.0], [-(e + 1.0)]]) for e in range(E)])
    if mistake == "swap_gate_up":
        orig = O.swiglu_expert
        monkeypatch.setattr(O, "swiglu_expert", lambda x, a, b, c: orig(x, b, a, c))
    elif mistake == "no_renormalise":  # softmax over all 8, then keep two
        monkeypatch.setattr(O, "masked_softmax_gates", lambda l, idx: np.take_along_axis(
            scipy.special.softmax(O._f64(l), axis=1), np.asarray(idx), axis=1))
    elif mistake == "ties_to_higher":
        monkeypatch.setattr(O, "select_top_k", lambda l, k=2: np.argsort(-O._f64(l)[:, ::-1], axis=1,
                                                                          kind="stable")[:, :k] * -1 + 7)
    elif mistake == "drop_second":
        orig_g = O.masked_softmax_gates
        monkeypatch.setattr(O, "masked_softmax_gates",
                            lambda l, idx: orig_g(l, idx) * np.array([[1.0, 0.0]]))
    out = O.moe_ffn(g["x"], g["w_gate"], w1, w3, w2)
    same = (np.array_equal(out["idx"], g["top2"]) and np.allclose(out["gates"], g["gates"], atol=1e-15)
            and np.allclose(out["y"], g["y"], rtol=1e-14, atol=1e-14))
    assert not same
