"""fp64 CPU oracle for the Mixtral sparse mixture-of-experts feed-forward layer.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously-correct statement
of what the GPU path computes.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import it; the product path never does, and
this module imports nothing from the product package.

Every function evaluates the definition in float64 with NumPy and no blocking,
fusion or reordering beyond what the definition states.  Inputs are whatever
tensors the GPU consumed (bf16 or fp32), widened exactly to float64.

Sources (page title, then the passage):

* "Mixtral of Experts" (azimuth.plus), paragraph on the router (gating network):
  the hidden state x times a weight matrix W_g gives 8 scores, one per expert;
  the top 2 scores are kept and every other score becomes -inf; a softmax over
  the survivors gives the gating weights, which both pick the experts and scale
  their outputs.  The next paragraph: the router has no state and no extra
  terms, only the matrix product and the selection.
* Same page, architecture paragraph: each expert is a SwiGLU feed-forward
  network with its own weights.
* "Mixtral > Architecture Overview" (mbrenndoerfer.com), parameter-count
  paragraph: each expert has three projections, gate, up and down, mapping the
  hidden size 4096 to 14336 and back.  Same page, the opening paragraphs: the
  FFN transforms each token in isolation.
* "Mixtral & Sparse MoE (2024) > The Solution" (mbrenndoerfer.com), routing
  paragraph: the selected experts' outputs are combined, weighted by the
  routing scores.

Readings taken where the pages are silent or disagree (each is listed with its
reason in the design notes of the repository):

* top-2 first, then the softmax over the surviving pair (the router paragraph
  of the azimuth.plus page; the mbrenndoerfer "The Solution" page states the
  opposite order, which gives the same weights once its pair is renormalised);
  that page's literal form, without the renormalisation, is available as the
  "full" gating (softmax_top_k_gates);
* ties in the selection go to the lower expert index, and slot 0 of a token is
  its larger score;
* SwiGLU(x) = (SiLU(x W_gate^T) * (x W_up^T)) W_down^T with SiLU(z) = z/(1+e^-z);
  w1 is the gate projection, w3 the up projection, w2 the down projection;
* no bias in the router or the experts; dropless (every selected pair runs);
* an optional per-expert logit bias exists only to build a skewed-routing
  workload and is added to the scores before selection.

Parity pins: every function here is pinned by tests that do not re-type its
formula (hand-worked golden fixtures, brute force over expert pairs, closed
forms, special cases that reduce to library routines, invariants).  The only
quantity left unpinned is the absolute output value of a full-size random
layer, for which the pages print no example.
"""

from __future__ import annotations

import numpy as np

N_EXPERTS = 8
TOP_K = 2


def _f64(a) -> np.ndarray:
    """Widen an array-like (NumPy array or CPU torch tensor of any float dtype)
    to a float64 NumPy array.  Widening bf16/fp32 to fp64 is exact."""
    if hasattr(a, "detach"):  # torch tensor without importing torch here
        a = a.detach().to("cpu")
        if str(a.dtype) in ("torch.bfloat16", "torch.float16"):
            a = a.float()
        a = a.numpy()
    return np.asarray(a, dtype=np.float64)


def router_logits(x, w_gate, logit_bias=None) -> np.ndarray:
    """Router scores l[t, e] = sum_i x[t, i] * W_g[e, i] (+ b[e]).

    "Mixtral of Experts" (azimuth.plus), router paragraph: a single linear map
    from the token's hidden state to one score per expert, with no other term.
    ``w_gate`` is stored as [E, d] (one row per expert), the transpose of the
    d x E map the page multiplies by.  ``logit_bias`` ([E] or None) is the
    skewed-workload device, not part of the published router.
    """
    x = _f64(x)
    wg = _f64(w_gate)
    assert x.ndim == 2 and wg.ndim == 2 and x.shape[1] == wg.shape[1]
    logits = x @ wg.T
    if logit_bias is not None:
        logits = logits + _f64(logit_bias)[None, :]
    return logits


def select_top_k(logits, k: int = TOP_K) -> np.ndarray:
    """Indices of the k largest scores per token, largest first.

    Router paragraph of "Mixtral of Experts" (azimuth.plus): the top-2 scores
    are kept.  Exact ties are broken toward the lower expert index (the pages
    are silent): a stable sort on the negated score keeps equal scores in index
    order.
    """
    l = _f64(logits)
    order = np.argsort(-l, axis=1, kind="stable")
    return order[:, :k].astype(np.int64)


def masked_softmax_gates(logits, idx) -> np.ndarray:
    """Gating weights per selected slot, shape [T, k].

    Router paragraph of "Mixtral of Experts" (azimuth.plus): every score that
    was not kept is set to -inf and a softmax is taken over all E entries, so
    the discarded experts get weight exactly 0 and the survivors share 1.
    """
    l = _f64(logits)
    idx = np.asarray(idx, dtype=np.int64)
    T, E = l.shape
    masked = np.full((T, E), -np.inf)
    rows = np.arange(T)[:, None]
    masked[rows, idx] = l[rows, idx]
    shifted = masked - masked.max(axis=1, keepdims=True)
    p = np.exp(shifted)  # exp(-inf) == 0 for the discarded experts
    p = p / p.sum(axis=1, keepdims=True)
    return p[rows, idx]


def softmax_top_k_gates(logits, idx) -> np.ndarray:
    """Gates of the other reading of the router, shape [T, k]: a softmax over
    all E scores first, then the probabilities of the selected experts as they
    stand, not renormalised (they sum to less than 1 whenever the unselected
    experts keep some probability).

    "Mixtral & Sparse MoE (2024) > The Solution" (mbrenndoerfer.com), routing
    paragraph: the scores are normalised by a softmax into a distribution over
    the experts, the top two are selected, and their outputs are combined by
    their routing scores.  The same two experts are selected as by the default
    reading (the softmax keeps the order of the scores); only the weights
    differ, by the common factor p_a + p_b.
    """
    l = _f64(logits)
    idx = np.asarray(idx, dtype=np.int64)
    rows = np.arange(l.shape[0])[:, None]
    p = np.exp(l - l.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    return p[rows, idx]


GATINGS = ("pair", "full")


def silu(z) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z)) (Swish with beta = 1, the
    activation inside the SwiGLU expert of "Mixtral of Experts", azimuth.plus,
    architecture paragraph)."""
    z = _f64(z)
    # exp(-z) overflows to inf for very negative z, which gives the correct 0.
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_expert(x_rows, w1_e, w3_e, w2_e) -> np.ndarray:
    """One expert: (SiLU(x w1^T) * (x w3^T)) w2^T.

    "Mixtral > Architecture Overview" (mbrenndoerfer.com), parameter-count
    paragraph: gate (w1, [f, d]), up (w3, [f, d]) and down (w2, [d, f])
    projections with the SwiGLU activation; "Mixtral of Experts"
    (azimuth.plus), architecture paragraph: SwiGLU expert with its own weights.
    """
    x_rows = _f64(x_rows)
    gate = x_rows @ _f64(w1_e).T
    up = x_rows @ _f64(w3_e).T
    h = silu(gate) * up
    return h @ _f64(w2_e).T


def swiglu_hidden(x_rows, w1_e, w3_e) -> np.ndarray:
    """The expert's hidden activation SiLU(x w1^T) * (x w3^T), shape [rows, f]
    (the intermediate between the up and down projections)."""
    x_rows = _f64(x_rows)
    return silu(x_rows @ _f64(w1_e).T) * (x_rows @ _f64(w3_e).T)


def moe_ffn(x, w_gate, w1, w3, w2, logit_bias=None, k: int = TOP_K, idx=None,
            widen_expert=None, gating: str = "pair", capacity: int = 0) -> dict:
    """The whole layer, vectorised over tokens (per expert, not per token).

    Returns a dict with ``y`` [T, d], ``idx`` [T, k], ``gates`` [T, k] and
    ``logits`` [T, E], all float64 / int64.

    Steps (pages as in the module docstring): scores -> keep top k -> softmax
    over the kept pair -> each token through each of its experts -> sum of the
    expert outputs weighted by the gates.  No capacity limit (dropless).

    ``idx`` (optional [T, k]) forces the expert assignment instead of selecting
    it; the gates are still the masked softmax of the scores over that
    assignment.  ``widen_expert`` (optional callable e -> (w1_e, w3_e, w2_e))
    lets the caller hand in one expert's weights at a time, so that a
    full-size layer never holds all experts in float64 at once.  ``gating``
    "pair" (default) takes the softmax over the kept pair; "full" the
    softmax over all scores without renormalising (softmax_top_k_gates).
    ``capacity`` > 0 drops the slots past each expert's capacity
    (capacity_keep); a dropped slot adds nothing and the token's other gate
    is left as it is.  The result then also holds ``keep`` [T, k].
    """
    if gating not in GATINGS:
        raise ValueError(f"unknown gating {gating!r}")
    x64 = _f64(x)
    logits = router_logits(x64, w_gate, logit_bias)
    T, E = logits.shape
    if idx is None:
        idx = select_top_k(logits, k)
    else:
        idx = np.asarray(idx, dtype=np.int64)
    gates = masked_softmax_gates(logits, idx) if gating == "pair" else softmax_top_k_gates(logits, idx)
    keep = capacity_keep(idx, capacity, E)
    y = None
    for e in range(E):
        tok, slot = np.nonzero((idx == e) & keep)
        if tok.size == 0:
            continue
        if widen_expert is not None:
            w1e, w3e, w2e = widen_expert(e)
        else:
            w1e, w3e, w2e = w1[e], w3[e], w2[e]
        out = swiglu_expert(x64[tok], w1e, w3e, w2e)
        if y is None:
            y = np.zeros((T, out.shape[1]))
        y[tok] += gates[tok, slot][:, None] * out
    if y is None:  # T == 0
        d = _f64(w2[0]).shape[0] if widen_expert is None else 0
        y = np.zeros((T, d))
    return {"y": y, "idx": idx, "gates": gates, "logits": logits, "keep": keep}


def moe_ffn_scalar(x, w_gate, w1, w3, w2, logit_bias=None, k: int = TOP_K, gating: str = "pair") -> np.ndarray:
    """The same layer written token by token with Python loops, for tiny inputs.

    For each token: score every expert, keep the k best (stable, lower index on
    ties), softmax over the kept scores ("full": over all scores), run each
    kept expert, add the weighted outputs.  Used to cross-check the vectorised
    form.
    """
    if gating not in GATINGS:
        raise ValueError(f"unknown gating {gating!r}")
    x64 = _f64(x)
    wg = _f64(w_gate)
    b = None if logit_bias is None else _f64(logit_bias)
    T = x64.shape[0]
    E = wg.shape[0]
    d_out = _f64(w2[0]).shape[0]
    y = np.zeros((T, d_out))
    for t in range(T):
        scores = []
        for e in range(E):
            s = 0.0
            for i in range(x64.shape[1]):
                s += x64[t, i] * wg[e, i]
            if b is not None:
                s += b[e]
            scores.append(s)
        kept = sorted(range(E), key=lambda e: (-scores[e], e))[:k]
        top = max(scores[e] for e in kept)
        num = [np.exp(scores[e] - top) for e in kept]
        den = sum(num) if gating == "pair" else sum(np.exp(scores[e] - top) for e in range(E))
        for j, e in enumerate(kept):
            y[t] += (num[j] / den) * swiglu_expert(x64[t:t + 1], w1[e], w3[e], w2[e])[0]
    return y


def expert_permutation(idx, n_experts: int = N_EXPERTS):
    """Expert-major order of the token slots.

    Slot s = t*k + j is token t's j-th selected expert.  Returns
    ``offsets`` [E+1] (offsets[e] = number of slots routed to experts < e),
    ``sorted_slots`` [T*k] (slots of expert 0 in increasing slot id, then
    expert 1, ...) and ``slot_rows`` [T*k] (the inverse: the position of slot s
    in that order).  This is the grouping step that lets each expert process
    its tokens together; it realises the per-token routing of "Mixtral & Sparse
    MoE (2024) > The Solution" (routing paragraph) and changes no value.
    """
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=n_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    sorted_slots = np.argsort(flat, kind="stable").astype(np.int64)
    slot_rows = np.empty_like(sorted_slots)
    slot_rows[sorted_slots] = np.arange(flat.size)
    return offsets, sorted_slots, slot_rows


def capacity_keep(idx, capacity: int, n_experts: int = N_EXPERTS) -> np.ndarray:
    """Which slots an expert capacity admits, shape [T, k] bool.

    "Mixtral & Sparse MoE (2024) > The Solution" (mbrenndoerfer.com),
    load-balancing paragraph: a capacity constraint limits how many tokens
    each expert receives.  The page gives no rule for which ones; the reading
    here: each expert admits its first ``capacity`` slots in slot order (slot
    s = t*k + j, so earlier tokens first and, within a token, its larger score
    first) and drops the rest.  ``capacity`` 0 means no limit (dropless).
    Written as a walk over the slots with one counter per expert.
    """
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    keep = np.ones(flat.size, dtype=bool)
    if capacity > 0:
        taken = np.zeros(n_experts, dtype=np.int64)
        for s, e in enumerate(flat):
            keep[s] = taken[e] < capacity
            taken[e] += 1
    return keep.reshape(np.asarray(idx).shape)


def load_balance_loss(logits, idx, n_experts: int = N_EXPERTS) -> float:
    """Auxiliary load-balancing loss E * sum_e f_e * P_e.

    "Mixtral & Sparse MoE (2024) > The Solution", load-balancing paragraph:
    auxiliary losses pushed the router towards an even spread of work over
    the experts; the page gives no formula.  The reading here is the usual
    product form: f_e = the fraction of the T*k routed slots that chose expert
    e (before any capacity limit), P_e = the mean over tokens of the softmax
    over all E scores at e.  It is 1 for a perfectly even router and grows
    towards E as the work collapses onto fewer experts.
    """
    l = _f64(logits)
    T, E = l.shape
    if T == 0:
        return 0.0
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    f = np.bincount(flat, minlength=n_experts) / flat.size
    p = np.exp(l - l.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    P = p.mean(axis=0)
    return float(n_experts * np.sum(f * P))


def second_third_gap(logits) -> np.ndarray:
    """Per token, the gap between the 2nd and 3rd largest scores (the margin
    by which the top-2 set is decided)."""
    s = -np.sort(-_f64(logits), axis=1)
    return s[:, 1] - s[:, 2]


def is_valid_top2(logits, pair, tol: float) -> np.ndarray:
    """True per token where ``pair`` ([T, 2]) is an acceptable top-2 set for
    these scores up to ``tol``: two distinct experts, pair[:, 0] scores at
    least pair[:, 1] - tol, and no unselected expert beats either selected one
    by more than ``tol``."""
    l = _f64(logits)
    pair = np.asarray(pair, dtype=np.int64)
    T, E = l.shape
    rows = np.arange(T)
    la = l[rows, pair[:, 0]]
    lb = l[rows, pair[:, 1]]
    other = l.copy()
    other[rows, pair[:, 0]] = -np.inf
    other[rows, pair[:, 1]] = -np.inf
    best_other = other.max(axis=1)
    return (pair[:, 0] != pair[:, 1]) & (la >= lb - tol) & (best_other <= np.minimum(la, lb) + tol)


def rmsnorm(z, eps: float = 1e-5) -> np.ndarray:
    """RMSNorm with unit gain: z / sqrt(mean(z^2) + eps).  Not on the pages;
    it is the normalisation between the stacked layers of the 32-layer
    workload (pre-norm decoder pattern of "Mixtral > Architecture Overview")."""
    z = _f64(z)
    return z / np.sqrt(np.mean(z * z, axis=1, keepdims=True) + eps)
