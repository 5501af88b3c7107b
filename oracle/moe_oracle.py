"""CPU oracle for the MoE variable-size grouped GEMM.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import or call this
module: only the tests, the smoke check and the benchmark's CPU-baseline leg
use it.  It shares no code with the HIP library.

It is the plain, slow, obviously correct definition of every result the HIP
path computes, written from three pages:

  [GG]   "Grouped GEMM for MoE, in depth" (aicassindra.com engineering article)
  [CARD] "grouped-gemm-moe" (model card of a published grouped GEMM kernel)
  [NOTE] "Grouped GEMM" (scholia-log study notes on MoE variable-length matmul)

Conventions:
  * an assignment is one (token, slot) pair of expert_ids [T, k]; it is numbered
    s = t*k + j (row-major flatten), as the card's usage example builds the ids;
  * expert weights are stored (E, N, K) like nn.Linear ([GG] "Data layout,
    offsets and alignment"), so the forward multiplies a row by W[e] transposed;
  * offsets are int32 END offsets: offs[e] = end of group e ([GG] "Data layout,
    offsets and alignment": counts [3,0,5] give offsets [3,3,8]);
  * floating point is evaluated in float64 by default (``acc``).  [GG]'s loop
    reference casts to fp32; ``acc=np.float32`` follows it literally.  The
    float64 default makes a parity tolerance measure the GPU's rounding alone.

Parity pins: every function here is checked in tests/ against something other
than itself (page examples, closed forms, brute force, finite differences,
identities).  Exact low-order bits of GPU float results under atomics and the
order of tiles inside one expert are not pinned (they are not part of the
result).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np


def _cdiv(a, b):
    return -(-np.asarray(a, dtype=np.int64) // b)


# ----------------------------------------------------------------------------
# Routing schedule
# ----------------------------------------------------------------------------
@dataclass
class Schedule:
    E: int
    k: int
    counts: np.ndarray        # [E] int64: rows per expert (m_e)
    offsets: np.ndarray       # [E] int32 end offsets
    starts: np.ndarray        # [E] int64 start offsets
    perm: np.ndarray          # [R] int64 assignment id s of row r
    row_to_token: np.ndarray  # [R] int64
    row_weight: np.ndarray    # [R] routing weight of the row (dtype of the input weights)
    n_invalid: int            # assignments whose id is outside [0, E)


def routing_schedule(expert_ids: np.ndarray, topk_weights: Optional[np.ndarray], E: int) -> Schedule:
    """Sort the assignments by expert and derive the row maps.

    [GG] "Data layout, offsets and alignment": a stable argsort of the per-copy
    expert index groups the rows by expert; bincount gives the per-expert
    counts and an int32 cumulative sum gives the end offsets.
    [CARD] "How it works": from the sorted order come the token of each row,
    the weight of each row and the size of each expert's group.
    Ids outside [0, E) belong to no expert: they are excluded and counted.
    """
    expert_ids = np.asarray(expert_ids)
    T, k = expert_ids.shape
    ids = expert_ids.reshape(-1).astype(np.int64)
    valid = (ids >= 0) & (ids < E)
    s_valid = np.nonzero(valid)[0]
    order = np.argsort(ids[s_valid], kind="stable")
    perm = s_valid[order]
    counts = np.bincount(ids[valid], minlength=E).astype(np.int64)
    offsets = np.cumsum(counts).astype(np.int32)
    starts = offsets.astype(np.int64) - counts
    if topk_weights is None:
        row_weight = np.ones(perm.shape[0], dtype=np.float32)
    else:
        row_weight = np.asarray(topk_weights).reshape(-1)[perm]
    return Schedule(E, k, counts, offsets, starts, perm, perm // k, row_weight,
                    int((~valid).sum()))


@dataclass
class RankSchedule:
    """Rows of the assignments ordered by (rank, expert, s), where the rank of
    an assignment is the number of valid assignments of its token in earlier
    slots.  Group p*E + e holds the rank-p assignments routed to expert e.  A
    token with no valid assignment has one row in group 0 (rank 0, expert 0)
    at its last slot's s, with weight 0 and assignment -1."""
    E: int
    k: int
    counts: np.ndarray        # [k*E] int64 rows per (rank, expert) group
    offsets: np.ndarray       # [k*E] int32 END offsets
    row_to_assign: np.ndarray  # [rows] int64, -1 for a token's row with no valid assignment
    row_to_token: np.ndarray   # [rows] int64
    row_weight: np.ndarray     # [rows] float32


def rank_schedule(expert_ids: np.ndarray, topk_weights: Optional[np.ndarray], E: int) -> RankSchedule:
    """The rank-ordered view of the assignments (a layout of this library, not
    of the pages): each token's contributions numbered by slot among its valid
    ones, so that the rows of one rank hold every token at most once and the
    rank-0 rows hold every token exactly once."""
    expert_ids = np.asarray(expert_ids)
    T, k = expert_ids.shape
    ids = expert_ids.astype(np.int64)
    valid = (ids >= 0) & (ids < E)
    rank = np.cumsum(valid, axis=1) - valid            # valid slots before each one
    dead = ~valid.any(axis=1)                           # tokens with no valid assignment
    key = np.where(valid, rank * E + ids, -1)
    key[dead, k - 1] = 0
    flat = key.reshape(-1)
    s_in = np.nonzero(flat >= 0)[0]
    order = s_in[np.argsort(flat[s_in], kind="stable")]
    counts = np.bincount(flat[s_in], minlength=k * E).astype(np.int64)
    offsets = np.cumsum(counts).astype(np.int32)
    vflat = valid.reshape(-1)
    assign = np.where(vflat[order], order, -1)
    w = np.ones(T * k, dtype=np.float32) if topk_weights is None else \
        np.asarray(topk_weights, dtype=np.float32).reshape(-1)
    weight = np.where(vflat[order], w[order], np.float32(0)).astype(np.float32)
    return RankSchedule(E, k, counts, offsets, assign, order // k, weight)


def group_rows(offsets: np.ndarray) -> list:
    """Row ranges of each group from END offsets ([GG] "Data layout, offsets and
    alignment"): group e owns rows [offs[e-1], offs[e]), with offs[-1] := 0."""
    offs = np.asarray(offsets, dtype=np.int64)
    prev = np.concatenate([[0], offs[:-1]])
    return [range(int(a), int(b)) for a, b in zip(prev, offs)]


# ----------------------------------------------------------------------------
# Tile space ([GG] "Problem descriptors and the tile scheduler")
# ----------------------------------------------------------------------------
@dataclass
class TileSpace:
    BM: int
    BN: int
    tiles_n: int
    tiles: np.ndarray       # [E] int64
    tile_start: np.ndarray  # [E] int64, exclusive prefix
    total: int


def tile_space(counts: np.ndarray, N: int, BM: int, BN: int) -> TileSpace:
    """Group g contributes ceil(M_g/BM) * ceil(N/BN) output tiles; an exclusive
    prefix sum gives each group's first tile; the total is one flat space."""
    tiles_n = int(_cdiv(N, BN))
    tiles = _cdiv(counts, BM) * tiles_n
    tile_start = np.concatenate([[0], np.cumsum(tiles)[:-1]]).astype(np.int64)
    total = int(tile_start[-1] + tiles[-1]) if len(tiles) else 0
    return TileSpace(BM, BN, tiles_n, tiles.astype(np.int64), tile_start, total)


def tile_owner(ts: TileSpace, tau) -> np.ndarray:
    """Owning group of tile index tau: the upper bound of tau in the start
    prefix, minus one.  With empty groups several starts are equal; the upper
    bound picks the last of them, the only one that owns tiles there."""
    return np.searchsorted(ts.tile_start, np.asarray(tau), side="right") - 1


def tile_coords(ts: TileSpace, counts: np.ndarray, offsets: np.ndarray, tau: int):
    """(group, row block, column block, first row, rows) of tile tau.

    Inside a group the walk is column-block-major: consecutive tile indices
    share one column block of the group's weights and step over row blocks
    ([GG] "Problem descriptors and the tile scheduler", on reusing B_g from
    L2).  The last row block of a group is ragged; its rows past the group end
    are masked.
    """
    g = int(tile_owner(ts, tau))
    local = int(tau) - int(ts.tile_start[g])
    mblocks = int(_cdiv(counts[g], ts.BM))
    nb, mb = divmod(local, mblocks)
    start = 0 if g == 0 else int(offsets[g - 1])
    row0 = start + mb * ts.BM
    rows = min(ts.BM, int(counts[g]) - mb * ts.BM)
    return g, mb, nb, row0, rows


# ----------------------------------------------------------------------------
# Masked fixed-capacity layout ([NOTE] section 5, "Masked" decode layout)
# ----------------------------------------------------------------------------
@dataclass
class MaskedSchedule:
    E: int
    capacity: int
    masked_m: np.ndarray     # [E] valid rows per expert = min(m_e, capacity)
    slot_assign: np.ndarray  # [E, capacity] assignment id or -1
    slot_token: np.ndarray   # [E, capacity] token or -1
    slot_weight: np.ndarray  # [E, capacity] routing weight, 0 for empty slots
    n_invalid: int
    n_dropped: int


def masked_schedule(expert_ids, topk_weights, E: int, capacity: int) -> MaskedSchedule:
    """Each expert reserves ``capacity`` row slots; its assignments fill them in
    ascending assignment order and the valid rows are the prefix
    0 .. min(m_e, capacity)-1.  Assignments beyond the capacity are dropped (the
    fixed-capacity approach drops tokens, [NOTE] section 2) and counted."""
    expert_ids = np.asarray(expert_ids)
    T, k = expert_ids.shape
    ids = expert_ids.reshape(-1).astype(np.int64)
    w = None if topk_weights is None else np.asarray(topk_weights).reshape(-1)
    slot_assign = np.full((E, capacity), -1, dtype=np.int64)
    fill = np.zeros(E, dtype=np.int64)
    n_invalid = n_dropped = 0
    for s in range(ids.shape[0]):
        e = ids[s]
        if e < 0 or e >= E:
            n_invalid += 1
            continue
        if fill[e] < capacity:
            slot_assign[e, fill[e]] = s
        else:
            n_dropped += 1
        fill[e] += 1
    valid = slot_assign >= 0
    slot_token = np.where(valid, slot_assign // k, -1)
    slot_weight = np.zeros((E, capacity), dtype=np.float64 if w is None else w.dtype)
    if w is None:
        slot_weight[valid] = 1.0
    else:
        slot_weight[valid] = w[slot_assign[valid]]
    return MaskedSchedule(E, capacity, np.minimum(fill, capacity), slot_assign, slot_token,
                          slot_weight, n_invalid, n_dropped)


# ----------------------------------------------------------------------------
# Products
# ----------------------------------------------------------------------------
def grouped_gemm(A: np.ndarray, W: np.ndarray, offsets: np.ndarray, *, acc=np.float64,
                 out: Optional[np.ndarray] = None) -> np.ndarray:
    """Bare grouped GEMM: rows already grouped by expert; for every group e,
    C[rows of e] = A[rows of e] @ W[e]^T ([GG] loop reference in "Data layout,
    offsets and alignment"; [CARD] "How it works", the kernel with the maps
    omitted).  Rows at or past offs[E-1] are not written (``out`` keeps them)."""
    A = np.asarray(A)
    M = A.shape[0]
    N = W.shape[1]
    C = np.zeros((M, N), dtype=acc) if out is None else np.array(out, dtype=acc, copy=True)
    for e, rows in enumerate(group_rows(offsets)):
        if len(rows) == 0:
            continue
        C[rows.start:rows.stop] = A[rows.start:rows.stop].astype(acc) @ W[e].astype(acc).T
    return C


def moe_forward_explicit(x, W, expert_ids, topk_weights, E: int, *, acc=np.float64) -> np.ndarray:
    """The unfused path: gather the token copies in expert order, run the bare
    grouped GEMM, then un-permute and combine by routing weight ([GG] "Data
    layout, offsets and alignment"; [NOTE] 4.1 permute, 4.3 un-permute with
    gating weights; [CARD] "Correctness", the explicit gather -> grouped GEMM ->
    scatter path).  The weight scales the fp32/fp64 product, not the input.
    Contributions are added to y in ascending sorted-row order."""
    sch = routing_schedule(expert_ids, topk_weights, E)
    T = x.shape[0]
    N = W.shape[1]
    xs = np.asarray(x)[sch.row_to_token]                 # [S, K] permuted copies
    ys = grouped_gemm(xs, W, sch.offsets, acc=acc)       # [S, N]
    y = np.zeros((T, N), dtype=acc)
    np.add.at(y, sch.row_to_token, sch.row_weight.astype(acc)[:, None] * ys)
    return y


def moe_forward(x, W, expert_ids, topk_weights, E: int, *, acc=np.float64) -> np.ndarray:
    """The fused form ([CARD] intro and "How it works"): for each expert, gather
    its token rows, multiply by its weights, scale by the routing weight and add
    into the token's output row; nothing of shape [S, K] or [S, N] is built.

    y[t, n] = sum_j w[t, j] * sum_k x[t, k] * W[ids[t, j], n, k].
    Experts are visited in ascending order and each expert's assignments in
    ascending s, which is the explicit path's order, so the two agree bit for
    bit in any precision ([CARD] "Correctness": the fusion is exact)."""
    expert_ids = np.asarray(expert_ids)
    T, k = expert_ids.shape
    ids = expert_ids.reshape(-1)
    wflat = None if topk_weights is None else np.asarray(topk_weights).reshape(-1)
    N = W.shape[1]
    y = np.zeros((T, N), dtype=acc)
    for e in range(E):
        s_e = np.nonzero(ids == e)[0]
        if s_e.size == 0:
            continue
        tok = s_e // k
        z = np.asarray(x)[tok].astype(acc) @ W[e].astype(acc).T
        we = np.ones(s_e.size, dtype=acc) if wflat is None else wflat[s_e].astype(acc)
        np.add.at(y, tok, we[:, None] * z)
    return y


def moe_backward(dY, x, W, expert_ids, topk_weights, E: int, *, acc=np.float64, dw_experts=None):
    """Gradients of L = sum(dY * y) for the fused layer.

    [GG] "The backward pass": with Y_g = X_g W_g, the input gradient is
    dY_g W_g^T (the forward pattern with the weights read transposed) and the
    weight gradient is X_g^T dY_g, a reduction over the group's rows; an
    expert with no rows gets an exact zero gradient.  In (E, N, K) storage the
    weight gradient of expert e is sum over its rows of (w * dY[t])^T x[t].
    [CARD] "How it works": the token gradient is scattered with the routing
    weight like the forward; for assignment s of token t to expert e,
    d_w[s] = <dY[t], x[t] W[e]^T> (the product before the weight multiplies it).

    Returns dX [T, K], dW [E, N, K], d_w [T, k].  With ``dw_experts`` (a list
    of expert ids) dW is instead a dict holding dW[e] for those experts only
    (the full [E, N, K] array is not formed).
    """
    expert_ids = np.asarray(expert_ids)
    T, k = expert_ids.shape
    ids = expert_ids.reshape(-1)
    wflat = None if topk_weights is None else np.asarray(topk_weights).reshape(-1)
    K = x.shape[1]
    N = W.shape[1]
    dX = np.zeros((T, K), dtype=acc)
    if dw_experts is None:
        dW = np.zeros((E, N, K), dtype=acc)
    else:
        dW = {int(e): np.zeros((N, K), dtype=acc) for e in dw_experts}
    d_w = np.zeros(T * k, dtype=acc)
    xa = np.asarray(x)
    dYa = np.asarray(dY)
    for e in range(E):
        s_e = np.nonzero(ids == e)[0]
        if s_e.size == 0:
            continue                      # dW[e] stays exactly zero
        tok = s_e // k
        We = W[e].astype(acc)            # [N, K]
        we = np.ones(s_e.size, dtype=acc) if wflat is None else wflat[s_e].astype(acc)
        g_rows = dYa[tok].astype(acc)    # [m_e, N]
        x_rows = xa[tok].astype(acc)     # [m_e, K]
        G = g_rows @ We                  # unweighted input gradient per assignment
        np.add.at(dX, tok, we[:, None] * G)
        if dw_experts is None or e in dW:
            dW[e] = (we[:, None] * g_rows).T @ x_rows
        Z = x_rows @ We.T                # unweighted forward product per assignment
        d_w[s_e] = np.sum(g_rows * Z, axis=1)
    return dX, dW, d_w.reshape(T, k)


def grouped_weight_grad(X, dY, offsets, E: int, *, acc=np.float64) -> np.ndarray:
    """Weight gradient of the bare grouped GEMM with rows already grouped:
    dW[e] = (dY[rows of e])^T X[rows of e], stored (E, N, K); zero for an empty
    group ([GG] "The backward pass", the variable-K grouped GEMM)."""
    K = X.shape[1]
    N = dY.shape[1]
    dW = np.zeros((E, N, K), dtype=acc)
    for e, rows in enumerate(group_rows(offsets)):
        if len(rows) == 0:
            continue
        dW[e] = np.asarray(dY[rows.start:rows.stop]).astype(acc).T @ np.asarray(X[rows.start:rows.stop]).astype(acc)
    return dW


def masked_forward(x, W, ms: MaskedSchedule, T: int, *, acc=np.float64) -> np.ndarray:
    """Decode forward on the masked layout: for every expert, only the valid row
    prefix of its slots contributes; each valid slot adds its routing-weighted
    product to its token's output row ([NOTE] section 5, masked layout)."""
    N = W.shape[1]
    y = np.zeros((T, N), dtype=acc)
    for e in range(ms.E):
        m = int(ms.masked_m[e])
        if m == 0:
            continue
        tok = ms.slot_token[e, :m]
        z = np.asarray(x)[tok].astype(acc) @ W[e].astype(acc).T
        np.add.at(y, tok, ms.slot_weight[e, :m].astype(acc)[:, None] * z)
    return y


# ----------------------------------------------------------------------------
# Gated expert FFN ([GG] "Choosing an implementation": the gated FFN's two
# up-projections, gate and up, form one grouped GEMM with the output width
# doubled, and the activation belongs in that GEMM's epilogue)
#
# Readings (the page names neither the activation nor the weight layout):
#   * the activation is SiLU on the gate times the up projection,
#     h = silu(x W_gate^T) * (x W_up^T), silu(z) = z / (1 + exp(-z));
#   * the doubled weight is W_gu [E, 2F, K]: rows 0 .. F-1 are the gate
#     projection, rows F .. 2F-1 the up projection;
#   * the down projection W_down [E, N, F] is the fused forward of the layer
#     applied to h: y[t] = sum_j w[t, j] * h[s] W_down[e]^T with s = t*k + j.
# ----------------------------------------------------------------------------
def round_bf16(a) -> np.ndarray:
    """Values rounded to bfloat16 (float64 -> float32 -> the nearest value with
    an 8-bit significand, ties to even), returned as float64.  The gated FFN's
    intermediate h is a bf16 tensor of the path; ``round_h=True`` applies this
    to h where the oracle forms it."""
    f = np.asarray(a, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def silu(z):
    """SiLU (sigmoid-weighted linear unit): z / (1 + exp(-z)), in float64."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def gated_activation(gu, *, acc=np.float64, round_h=False):
    """h = silu(gate) * up for a row block gu = [gate | up] of width 2F
    (rounded to bf16 with ``round_h``)."""
    F = gu.shape[1] // 2
    h = silu(gu[:, :F]) * np.asarray(gu[:, F:], dtype=np.float64)
    return (round_bf16(h) if round_h else h).astype(acc)


def gated_ffn_forward(x, W_gu, W_down, expert_ids, topk_weights, E: int, *, acc=np.float64,
                      round_h=False):
    """Fused gated expert FFN: for each expert, gather its token rows, run the
    doubled up-projection, apply silu(gate) * up, project down and add the
    routing-weighted result into each token's output row.  Returns y [T, N]."""
    expert_ids = np.asarray(expert_ids)
    T, k = expert_ids.shape
    ids = expert_ids.reshape(-1)
    wflat = None if topk_weights is None else np.asarray(topk_weights).reshape(-1)
    N = W_down.shape[1]
    y = np.zeros((T, N), dtype=acc)
    for e in range(E):
        s_e = np.nonzero(ids == e)[0]
        if s_e.size == 0:
            continue
        tok = s_e // k
        gu = np.asarray(x)[tok].astype(acc) @ W_gu[e].astype(acc).T
        z = gated_activation(gu, acc=acc, round_h=round_h) @ W_down[e].astype(acc).T
        we = np.ones(s_e.size, dtype=acc) if wflat is None else wflat[s_e].astype(acc)
        np.add.at(y, tok, we[:, None] * z)
    return y


def gated_intermediate(x, W_gu, expert_ids, E: int, *, acc=np.float64, round_h=False) -> np.ndarray:
    """The intermediate h [R, F] in the routing schedule's row order (the
    explicit path: gather the token copies, one grouped GEMM over the doubled
    weights, then the activation).  Rows past the routed rows stay zero."""
    sch = routing_schedule(expert_ids, None, E)
    xs = np.asarray(x)[sch.row_to_token]
    gu = grouped_gemm(xs, W_gu, sch.offsets, acc=acc)
    h = np.zeros((np.asarray(expert_ids).size, W_gu.shape[1] // 2), dtype=acc)
    h[:xs.shape[0]] = gated_activation(gu, acc=acc, round_h=round_h)
    return h


def gated_ffn_forward_explicit(x, W_gu, W_down, expert_ids, topk_weights, E: int, *,
                               acc=np.float64) -> np.ndarray:
    """Unfused gated FFN: h in schedule row order, the bare grouped GEMM with the
    down weights, then the weighted un-permute ([NOTE] 4.3)."""
    sch = routing_schedule(expert_ids, topk_weights, E)
    h = gated_intermediate(x, W_gu, expert_ids, E, acc=acc)[:sch.row_to_token.size]
    z = grouped_gemm(h, W_down, sch.offsets, acc=acc)
    y = np.zeros((np.asarray(x).shape[0], W_down.shape[1]), dtype=acc)
    np.add.at(y, sch.row_to_token, sch.row_weight.astype(acc)[:, None] * z)
    return y


def gated_ffn_backward(dY, x, W_gu, W_down, expert_ids, topk_weights, E: int, *, acc=np.float64,
                       round_h=False):
    """Gradients of L = sum(dY * y) for the gated FFN, by the chain rule per
    expert.  With z = h W_down^T, h = silu(g) * u, (g | u) = x W_gu^T:
      dh = w * dY W_down;  dg = dh * u * silu'(g),  du = dh * silu(g),
      silu'(g) = s (1 + g (1 - s)) with s = 1 / (1 + exp(-g));
      dX[t] += (dg | du) W_gu;  dW_gu[e] = sum (dg | du)^T x;
      dW_down[e] = sum (w dY)^T h;  d_w[s] = dY[t] . z[s] (the unweighted
      down-projection output).
    Returns dX [T, K], dW_gu [E, 2F, K], dW_down [E, N, F], d_w [T, k]."""
    expert_ids = np.asarray(expert_ids)
    T, k = expert_ids.shape
    ids = expert_ids.reshape(-1)
    wflat = None if topk_weights is None else np.asarray(topk_weights).reshape(-1)
    F = W_gu.shape[1] // 2
    K = np.asarray(x).shape[1]
    N = W_down.shape[1]
    dX = np.zeros((T, K), dtype=acc)
    dWgu = np.zeros((E, 2 * F, K), dtype=acc)
    dWd = np.zeros((E, N, F), dtype=acc)
    d_w = np.zeros(T * k, dtype=acc)
    for e in range(E):
        s_e = np.nonzero(ids == e)[0]
        if s_e.size == 0:
            continue
        tok = s_e // k
        xe = np.asarray(x)[tok].astype(acc)
        gu = xe @ W_gu[e].astype(acc).T
        g, u = gu[:, :F].astype(np.float64), gu[:, F:].astype(np.float64)
        sg = 1.0 / (1.0 + np.exp(-g))
        h = g * sg * u
        h = (round_bf16(h) if round_h else h).astype(acc)
        we = np.ones(s_e.size, dtype=acc) if wflat is None else wflat[s_e].astype(acc)
        dYe = np.asarray(dY)[tok].astype(acc)
        Wd = W_down[e].astype(acc)
        d_w[s_e] = np.sum(dYe * (h @ Wd.T), axis=1)
        dh = we[:, None] * (dYe @ Wd)
        dg = (dh * u * sg * (1.0 + g * (1.0 - sg))).astype(acc)
        du = (dh * g * sg).astype(acc)
        dgu = np.concatenate([dg, du], axis=1)
        np.add.at(dX, tok, dgu @ W_gu[e].astype(acc))
        dWgu[e] = dgu.T @ xe
        dWd[e] = (we[:, None] * dYe).T @ h
    return dX, dWgu, dWd, d_w.reshape(T, k)


def gated_ffn_backward_rows(dY, x, W_gu, W_down, expert_ids, topk_weights, tokens, *,
                            acc=np.float64, round_h=False):
    """dX[t] and d_w[t, :] of the gated FFN for the listed tokens only."""
    expert_ids = np.asarray(expert_ids)
    k = expert_ids.shape[1]
    F = W_gu.shape[1] // 2
    dX = np.zeros((len(tokens), np.asarray(x).shape[1]), dtype=acc)
    dw = np.zeros((len(tokens), k), dtype=acc)
    for i, t in enumerate(tokens):
        xt = np.asarray(x)[t].astype(acc)
        gy = np.asarray(dY)[t].astype(acc)
        for j in range(k):
            e = int(expert_ids[t, j])
            w = 1.0 if topk_weights is None else float(topk_weights[t, j])
            gu = W_gu[e].astype(acc) @ xt
            g, u = gu[:F], gu[F:]
            sg = 1.0 / (1.0 + np.exp(-g))
            h = round_bf16(g * sg * u) if round_h else g * sg * u
            Wd = W_down[e].astype(acc)
            dw[i, j] = gy @ (Wd @ h)
            dh = w * (gy @ Wd)
            dgu = np.concatenate([dh * u * sg * (1.0 + g * (1.0 - sg)), dh * g * sg])
            dX[i] += dgu @ W_gu[e].astype(acc)
    return dX, dw


def gated_weight_grad_entries(dY, x, W_gu, W_down, expert_ids, topk_weights, E: int,
                              gu_entries, down_entries, *, acc=np.float64, round_h=False):
    """Listed entries of dW_gu [(e, j, k)] and dW_down [(e, n, f)], from sums
    over the expert's assignments."""
    expert_ids = np.asarray(expert_ids)
    kk = expert_ids.shape[1]
    ids = expert_ids.reshape(-1)
    wflat = None if topk_weights is None else np.asarray(topk_weights).reshape(-1)
    F = W_gu.shape[1] // 2
    cache = {}

    def rows(e):
        if e not in cache:
            s_e = np.nonzero(ids == e)[0]
            tok = s_e // kk
            xe = np.asarray(x)[tok].astype(acc)
            gu = xe @ W_gu[e].astype(acc).T
            g, u = gu[:, :F], gu[:, F:]
            sg = 1.0 / (1.0 + np.exp(-g))
            h = round_bf16(g * sg * u) if round_h else g * sg * u
            we = np.ones(s_e.size, dtype=acc) if wflat is None else wflat[s_e].astype(acc)
            dYe = np.asarray(dY)[tok].astype(acc)
            dh = we[:, None] * (dYe @ W_down[e].astype(acc))
            dgu = np.concatenate([dh * u * sg * (1.0 + g * (1.0 - sg)), dh * g * sg], axis=1)
            cache[e] = (xe, h, we, dYe, dgu)
        return cache[e]

    out_gu = np.zeros(len(gu_entries), dtype=acc)
    for i, (e, j, kc) in enumerate(gu_entries):
        xe, _, _, _, dgu = rows(e)
        out_gu[i] = np.sum(dgu[:, j] * xe[:, kc])
    out_d = np.zeros(len(down_entries), dtype=acc)
    for i, (e, n, f) in enumerate(down_entries):
        _, h, we, dYe, _ = rows(e)
        out_d[i] = np.sum(we * dYe[:, n] * h[:, f])
    return out_gu, out_d


def masked_gated_ffn(x, W_gu, W_down, ms: MaskedSchedule, T: int, *, acc=np.float64, round_h=False):
    """Gated FFN on the masked layout.  Returns (y [T, N], h [E*capacity, F]);
    h rows of empty slots are zero (the library leaves them unwritten)."""
    F = W_gu.shape[1] // 2
    y = np.zeros((T, W_down.shape[1]), dtype=acc)
    h = np.zeros((ms.E * ms.capacity, F), dtype=acc)
    for e in range(ms.E):
        m = int(ms.masked_m[e])
        if m == 0:
            continue
        tok = ms.slot_token[e, :m]
        he = gated_activation(np.asarray(x)[tok].astype(acc) @ W_gu[e].astype(acc).T, acc=acc,
                              round_h=round_h)
        h[e * ms.capacity:e * ms.capacity + m] = he
        z = he @ W_down[e].astype(acc).T
        np.add.at(y, tok, ms.slot_weight[e, :m].astype(acc)[:, None] * z)
    return y, h


# ----------------------------------------------------------------------------
# FP8 grouped GEMM with scales that travel with each group ([GG] "Choosing an
# implementation": FP8 adds per-group or per-block scale factors carried with
# every group)
#
# Readings (the page fixes neither the format nor the scale granularity):
#   * operands are 8-bit floats in the E4M3 encoding without infinities
#     (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0
#     holds subnormals m/8 * 2^-6; exponent 15 with mantissa 7 is NaN; largest
#     finite value 448);
#   * a token row t carries one scale sx[t]; expert e carries one scale per
#     output channel sw[e, n] (per-group scales); the value of an operand is
#     its decoded 8-bit float times its scale;
#   * the layer is then the fused forward on the scaled values:
#     y[t, n] = sum_j w[t, j] * sum_k (sx[t] qx[t, k]) * (sw[e, n] qW[e, n, k]).
# ----------------------------------------------------------------------------
def decode_e4m3(bits) -> np.ndarray:
    """Value of each E4M3 code (uint8) as float64, from the field definition."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    exp = (b >> 3) & 0xF
    man = b & 0x7
    val = np.where(exp == 0, man / 8.0 * 2.0 ** -6, (1.0 + man / 8.0) * 2.0 ** (exp - 7))
    val = np.where((exp == 15) & (man == 7), np.nan, val)
    return sign * val


def moe_forward_fp8(xq, x_scale, Wq, w_scale, expert_ids, topk_weights, E: int, *,
                    acc=np.float64) -> np.ndarray:
    """Fused forward of 8-bit operands: decode, apply the per-token and the
    per-group-per-channel scales, then the fused forward of the layer."""
    x = decode_e4m3(xq) * np.asarray(x_scale, dtype=np.float64)[:, None]
    W = decode_e4m3(Wq) * np.asarray(w_scale, dtype=np.float64)[:, :, None]
    return moe_forward(x, W, expert_ids, topk_weights, E, acc=acc)


def masked_forward_fp8(xq, x_scale, Wq, w_scale, ms: MaskedSchedule, T: int, *,
                       acc=np.float64) -> np.ndarray:
    """Decode forward of 8-bit operands on the masked layout."""
    x = decode_e4m3(xq) * np.asarray(x_scale, dtype=np.float64)[:, None]
    W = decode_e4m3(Wq) * np.asarray(w_scale, dtype=np.float64)[:, :, None]
    return masked_forward(x, W, ms, T, acc=acc)


# Per-block scales (the other reading of "per-group or per-block"): every run of
# 32 consecutive reduction elements of a token row and of an expert's weight
# row carries its own power-of-two scale, an 8-bit exponent code E8M0 (value
# 2^(c - 127), code 255 = NaN).  The operand value is the E4M3 value times its
# block's scale.
MX_BLOCK = 32


def decode_e8m0(codes) -> np.ndarray:
    """2^(c - 127) for each E8M0 code (NaN for 255), float64."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.float64)
    return np.where(c == 255, np.nan, np.exp2(c - 127.0))


def mx_values(q, scales) -> np.ndarray:
    """Values of E4M3 codes q [..., K] with per-32-element scales [..., K/32]."""
    s = np.repeat(decode_e8m0(scales), MX_BLOCK, axis=-1)
    return decode_e4m3(q) * s


def moe_forward_mx(xq, x_bs, Wq, w_bs, expert_ids, topk_weights, E: int, *, acc=np.float64):
    """Fused forward of 8-bit operands with per-32-element block scales."""
    return moe_forward(mx_values(xq, x_bs), mx_values(Wq, w_bs), expert_ids, topk_weights, E,
                       acc=acc)


def masked_forward_mx(xq, x_bs, Wq, w_bs, ms: MaskedSchedule, T: int, *, acc=np.float64):
    return masked_forward(mx_values(xq, x_bs), mx_values(Wq, w_bs), ms, T, acc=acc)


def moe_forward_fp8_rows(xq, x_scale, Wq, w_scale, expert_ids, topk_weights, tokens, *,
                         acc=np.float64) -> np.ndarray:
    """y[t, :] of the 8-bit forward for the listed tokens only."""
    expert_ids = np.asarray(expert_ids)
    out = np.zeros((len(tokens), Wq.shape[1]), dtype=acc)
    for i, t in enumerate(tokens):
        xt = decode_e4m3(xq[t]) * float(x_scale[t])
        for j in range(expert_ids.shape[1]):
            e = int(expert_ids[t, j])
            w = 1.0 if topk_weights is None else float(topk_weights[t, j])
            We = decode_e4m3(Wq[e]) * np.asarray(w_scale[e], dtype=np.float64)[:, None]
            out[i] += acc(w) * (We @ xt)
    return out


# ----------------------------------------------------------------------------
# Sampled evaluation for full-size parity checks
# ----------------------------------------------------------------------------
def gated_intermediate_rows(x, W_gu, expert_ids, E: int, rows, *, acc=np.float64,
                            round_h=False) -> np.ndarray:
    """Rows of h [R, F] for the listed schedule rows only: row r is the r-th
    assignment s in (expert, s) order, h[r] = silu(W_gate[e] x[t]) * (W_up[e] x[t])."""
    sch = routing_schedule(expert_ids, None, E)
    ids = np.asarray(expert_ids).reshape(-1)
    F = W_gu.shape[1] // 2
    out = np.zeros((len(rows), F), dtype=acc)
    for i, r in enumerate(rows):
        s = int(sch.perm[r])
        gu = W_gu[int(ids[s])].astype(acc) @ np.asarray(x)[int(sch.row_to_token[r])].astype(acc)
        h = silu(gu[:F]) * gu[F:]
        out[i] = (round_bf16(h) if round_h else h).astype(acc)
    return out


def gated_ffn_rows(x, W_gu, W_down, expert_ids, topk_weights, tokens, *, acc=np.float64,
                   round_h=False):
    """y[t, :] of the gated FFN for the listed tokens only, from the definition
    y[t] = sum_j w[t, j] * W_down[e] (silu(W_gate[e] x[t]) * (W_up[e] x[t]))."""
    expert_ids = np.asarray(expert_ids)
    F = W_gu.shape[1] // 2
    out = np.zeros((len(tokens), W_down.shape[1]), dtype=acc)
    for i, t in enumerate(tokens):
        xt = np.asarray(x)[t].astype(acc)
        for j in range(expert_ids.shape[1]):
            e = int(expert_ids[t, j])
            w = 1.0 if topk_weights is None else float(topk_weights[t, j])
            gu = W_gu[e].astype(acc) @ xt
            h = silu(gu[:F]) * gu[F:]
            h = (round_bf16(h) if round_h else h).astype(acc)
            out[i] += acc(w) * (W_down[e].astype(acc) @ h)
    return out


def moe_forward_rows(x, W, expert_ids, topk_weights, tokens, *, acc=np.float64) -> np.ndarray:
    """y[t, :] for the listed tokens only, straight from the definition
    y[t] = sum_j w[t, j] * (x[t] @ W[ids[t, j]]^T)."""
    expert_ids = np.asarray(expert_ids)
    out = np.zeros((len(tokens), W.shape[1]), dtype=acc)
    for i, t in enumerate(tokens):
        xt = np.asarray(x)[t].astype(acc)
        for j in range(expert_ids.shape[1]):
            e = int(expert_ids[t, j])
            w = 1.0 if topk_weights is None else float(topk_weights[t, j])
            out[i] += acc(w) * (W[e].astype(acc) @ xt)
    return out


def moe_backward_rows(dY, x, W, expert_ids, topk_weights, tokens, *, acc=np.float64):
    """dX[t, :] and d_w[t, :] for the listed tokens only, from the definitions
    dX[t] = sum_j w[t, j] * dY[t] @ W[e_tj],  d_w[t, j] = dY[t] . (W[e_tj] @ x[t])."""
    expert_ids = np.asarray(expert_ids)
    k = expert_ids.shape[1]
    dX = np.zeros((len(tokens), W.shape[2]), dtype=acc)
    dw = np.zeros((len(tokens), k), dtype=acc)
    for i, t in enumerate(tokens):
        g = np.asarray(dY)[t].astype(acc)
        xt = np.asarray(x)[t].astype(acc)
        for j in range(k):
            e = int(expert_ids[t, j])
            We = W[e].astype(acc)
            w = 1.0 if topk_weights is None else float(topk_weights[t, j])
            dX[i] += acc(w) * (g @ We)
            dw[i, j] = g @ (We @ xt)
    return dX, dw


def weight_grad_entries(dY, x, expert_ids, topk_weights, E: int, entries, *, acc=np.float64) -> np.ndarray:
    """dW[e, n, k] for listed (e, n, k) triples, from the definition
    sum over assignments s routed to e of w_s * dY[t_s, n] * x[t_s, k]."""
    expert_ids = np.asarray(expert_ids)
    kk = expert_ids.shape[1]
    ids = expert_ids.reshape(-1)
    wflat = None if topk_weights is None else np.asarray(topk_weights).reshape(-1)
    members = {}
    out = np.zeros(len(entries), dtype=acc)
    for i, (e, n, kc) in enumerate(entries):
        if e not in members:
            members[e] = np.nonzero(ids == e)[0]
        s_e = members[e]
        if s_e.size == 0:
            continue
        tok = s_e // kk
        we = np.ones(s_e.size, dtype=acc) if wflat is None else wflat[s_e].astype(acc)
        out[i] = np.sum(we * np.asarray(dY)[tok, n].astype(acc) * np.asarray(x)[tok, kc].astype(acc))
    return out
