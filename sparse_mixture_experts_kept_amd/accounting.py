"""Algorithmic work of the sparse MoE feed-forward layer: flops and bytes.

These are the counts the roofline fractions are computed from.  They follow
the shapes of "Mixtral > Architecture Overview" (mbrenndoerfer.com),
hyperparameter list and parameter-count paragraph: per layer, E experts, each
with gate [f, d], up [f, d] and down [d, f] matrices; each token runs k of
them.  The router is one [E, d] matrix ("Mixtral of Experts", azimuth.plus,
router paragraph).

Nothing here executes the layer; it only counts.
"""

from __future__ import annotations

MIXTRAL = dict(layers=32, d=4096, f=14336, E=8, k=2)
PEAK_BF16_FLOPS = 2.5e15      # MI355X dense bf16 MFMA, published
PEAK_FP32_FLOPS = 157.3e12    # MI355X fp32 vector, published
PEAK_HBM_BYTES = 8.0e12       # MI355X HBM3E, published


def projection_params(d: int, f: int) -> int:
    """Parameters of one projection matrix (gate, up or down)."""
    return d * f


def expert_params(d: int, f: int, layers: int = 1) -> int:
    """Parameters of one expert's three projections, over ``layers`` layers."""
    return 3 * d * f * layers


def ffn_params(d: int, f: int, E: int, layers: int = 1) -> int:
    """All expert parameters (E experts per layer)."""
    return E * expert_params(d, f, layers)


def active_ffn_params(d: int, f: int, k: int, layers: int = 1) -> int:
    """Expert parameters one token touches (k experts per layer)."""
    return k * expert_params(d, f, layers)


def router_flops_per_token(d: int, E: int) -> int:
    return 2 * d * E


def expert_flops_per_token(d: int, f: int, k: int) -> int:
    """Multiply-adds of k SwiGLU experts, counted as 2 flops each."""
    return 2 * k * 3 * d * f


def up_flops_per_slot(d: int, f: int) -> int:
    """Gate and up projections of one (token, expert) slot."""
    return 2 * 2 * d * f


def down_flops_per_slot(d: int, f: int) -> int:
    return 2 * d * f


def layer_flops(T: int, d: int, f: int, E: int, k: int) -> int:
    """Whole layer: router + k experts per token."""
    return T * (router_flops_per_token(d, E) + expert_flops_per_token(d, f, k))


def expert_weight_bytes(d: int, f: int, n_experts: int, elem_bytes: int = 2) -> int:
    """Bytes of the three matrices of ``n_experts`` experts."""
    return n_experts * 3 * d * f * elem_bytes


def decode_layer_bytes(T: int, d: int, f: int, E: int, k: int, n_touched: int, elem_bytes: int = 2) -> int:
    """Minimum HBM traffic of one layer when the weights dominate: every
    touched expert's weights once, the router matrix, x in and y out."""
    return (expert_weight_bytes(d, f, n_touched, elem_bytes) + E * d * elem_bytes
            + 2 * T * d * elem_bytes)


def up_bytes(T: int, d: int, f: int, k: int, n_touched: int, elem_bytes: int = 2) -> int:
    """Algorithmic HBM bytes of the up projection (gate + up + SwiGLU) over
    one layer: each token row read once per slot, the touched experts' gate
    and up matrices read once, h [T*k, f] written once."""
    return (T * k * d + n_touched * 2 * f * d + T * k * f) * elem_bytes


def down_bytes(T: int, d: int, f: int, k: int, n_touched: int, elem_bytes: int = 2, out_bytes: int = 4) -> int:
    """Algorithmic HBM bytes of the down projection: h read once, the
    touched experts' down matrices read once, fp32 y_rows [T*k, d] written."""
    return (T * k * f + n_touched * d * f) * elem_bytes + T * k * d * out_bytes


# Row heights of the prefill GEMM's tile paths: an m-tile with r rows left runs
# on the smallest of these that holds r (thin, small, medium, large, full).
PREFILL_TILE_ROWS = (32, 64, 128, 160, 256)


def prefill_rows_issued(counts, tile_rows: int = 256, tail_rows: int = 32, group_rows: int = 16,
                        tile_heights=PREFILL_TILE_ROWS):
    """Rows the prefill path runs through the matrix cores for these
    per-expert counts: each expert's rows in m-tiles of ``tile_rows``; an
    m-tile with r < tile_rows rows issues the smallest of ``tile_heights``
    that holds r, except a last tile of at most ``tail_rows`` rows after at
    least one full tile, which goes to the streaming kernels in token groups
    of ``group_rows``.  Returns (rows needed, rows issued in GEMM tiles, rows
    issued in tails); the padding waste is issued / needed - 1."""
    needed = gemm = tails = 0
    for c in counts:
        c = int(c)
        needed += c
        if c == 0:
            continue
        tiles = -(-c // tile_rows)
        last = c - (tiles - 1) * tile_rows
        if tiles >= 2 and last <= tail_rows:
            gemm += (tiles - 1) * tile_rows
            tails += -(-last // group_rows) * group_rows
        else:
            gemm += (tiles - 1) * tile_rows + min(h for h in tile_heights if h >= last)
    return needed, gemm, tails


def prefill_gemm_rows(counts, tile_rows: int = 256, tail_rows: int = 32) -> int:
    """Rows (unpadded) the prefill GEMM launch computes itself: every row
    but an expert's short tail (a last tile of at most ``tail_rows`` rows
    after at least one full tile), which its own launch computes."""
    rows = 0
    for c in counts:
        c = int(c)
        tiles = -(-c // tile_rows)
        last = c - (tiles - 1) * tile_rows
        rows += c - (last if tiles >= 2 and last <= tail_rows else 0)
    return rows
