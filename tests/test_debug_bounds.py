"""Host-side bounds checks of the permutation arrays (the binding's
MOE_DEBUG_BOUNDS mode), on the CPU: valid permutations from the oracle pass,
every kind of corruption a kernel would index memory through is caught."""

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from sparse_mixture_experts_kept_amd import moe


def _perm(T, seed, capacity=0):
    rng = np.random.default_rng(seed)
    idx = O.select_top_k(rng.standard_normal((T, 8)) + np.linspace(1, -1, 8), 2)
    offs, ss, rows = O.expert_permutation(idx)
    if capacity:
        keep = O.capacity_keep(idx, capacity).reshape(-1)
        flat = idx.reshape(-1)
        kept = np.minimum(np.bincount(flat, minlength=8), capacity)
        offs = np.concatenate([[0], np.cumsum(kept)])
        rank = rows - O.expert_permutation(idx)[0][flat]
        rows = np.where(keep, offs[flat] + rank, -1)
        ss_kept = ss[keep[ss]]
        ss = np.concatenate([ss_kept, np.full(ss.size - ss_kept.size, 12345)])
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.int32))  # noqa: E731
    return idx, t(offs), t(ss), t(rows)


@pytest.mark.parametrize("T,capacity", [(1, 0), (300, 0), (3000, 0), (3000, 250)])
def test_valid_permutations_pass(T, capacity):
    idx, offs, ss, rows = _perm(T, T, capacity)
    moe.check_permutation(offs, ss, rows, T, capacity)
    moe.check_routing(torch.from_numpy(idx.astype(np.int32)), T)


def test_corruptions_are_caught():
    T = 200
    idx, offs, ss, rows = _perm(T, 7)
    bad = []
    o = offs.clone(); o[3] = o[2] - 1; bad.append((o, ss, rows))          # decreasing offsets
    o = offs.clone(); o[-1] = 2 * T + 1; bad.append((o, ss, rows))        # past the slots
    o = offs.clone(); o[0] = 1; bad.append((o, ss, rows))                 # not starting at 0
    s2 = ss.clone(); s2[5] = 2 * T; bad.append((offs, s2, rows))          # slot id out of range
    s2 = ss.clone(); s2[5] = -1; bad.append((offs, s2, rows))
    s2 = ss.clone(); s2[6] = s2[5]; bad.append((offs, s2, rows))          # a slot placed twice
    s2 = ss.clone(); s2[[0, 1]] = s2[[1, 0]]; bad.append((offs, s2, rows))  # order within an expert
    r2 = rows.clone(); r2[4] = 2 * T; bad.append((offs, ss, r2))          # row out of range
    r2 = rows.clone(); r2[[4, 9]] = r2[[9, 4]]; bad.append((offs, ss, r2))  # not the inverse
    r2 = rows.clone(); r2[4] = -1; bad.append((offs, ss, r2))             # placed slot without a row
    for o, s_, r in bad:
        with pytest.raises(moe.MoeIndexError):
            moe.check_permutation(o, s_, r, T)
    with pytest.raises(moe.MoeIndexError):
        moe.check_permutation(offs, ss, rows, T, capacity=int(torch.diff(offs).max()) - 1)
    bad_idx = torch.from_numpy(idx.astype(np.int32))
    bad_idx[3, 1] = bad_idx[3, 0]
    with pytest.raises(moe.MoeIndexError):
        moe.check_routing(bad_idx, T)
    bad_idx[3, 1] = 8
    with pytest.raises(moe.MoeIndexError):
        moe.check_routing(bad_idx, T)
