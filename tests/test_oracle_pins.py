"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these tests re-types the oracle's own formula: each compares it with a
value printed on a page, a brute-force evaluation in plain Python, a closed
form, a finite difference or an identity the definitions imply.
"""
import json
import math
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _ids_from_counts(counts, k=1, seed=0):
    """Assignments whose per-expert counts are ``counts``, shuffled, as [T, k]."""
    rng = np.random.default_rng(seed)
    ids = np.repeat(np.arange(len(counts)), counts)
    rng.shuffle(ids)
    return ids.reshape(-1, k).astype(np.int32)


# ----------------------------------------------------------------------------
# Offsets and schedule
# ----------------------------------------------------------------------------
def test_offsets_page_examples():
    g = _load("offsets_examples.json")
    c0 = g["cases"][0]
    sch = O.routing_schedule(_ids_from_counts(c0["counts"]), None, len(c0["counts"]))
    assert sch.offsets.dtype == np.int32
    assert sch.offsets.tolist() == c0["end_offsets"]
    assert [list(r) for r in O.group_rows(sch.offsets)] == c0["group_rows"]
    c1 = g["cases"][1]
    sch = O.routing_schedule(_ids_from_counts(c1["counts"]), None, len(c1["counts"]))
    assert int(sch.offsets[-1]) == c1["total_rows"]
    assert sch.counts.tolist() == c1["counts"]


def test_sorted_rows_brute_force():
    """Rows are grouped by expert and, within an expert, in ascending assignment
    order (a stable sort); row -> token is s div k; row weight is w[s]."""
    rng = np.random.default_rng(3)
    T, k, E = 37, 3, 6
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    sch = O.routing_schedule(ids, w, E)
    expect = []
    for e in range(E):
        for t in range(T):
            for j in range(k):
                if ids[t, j] == e:
                    expect.append((t * k + j, t, w[t, j]))
    assert sch.perm.tolist() == [a for a, _, _ in expect]
    assert sch.row_to_token.tolist() == [b for _, b, _ in expect]
    assert sch.row_weight.tolist() == [c for _, _, c in expect]
    for e, rows in enumerate(O.group_rows(sch.offsets)):
        assert all(ids.reshape(-1)[sch.perm[r]] == e for r in rows)


@settings(max_examples=60, deadline=None)
@given(st.lists(st.integers(min_value=0, max_value=9), min_size=1, max_size=12),
       st.integers(min_value=1, max_value=4))
def test_sum_of_group_sizes(counts, k):
    """Sum over experts of m_e equals tokens * top_k when no assignment is lost
    (study notes, section 1)."""
    total = sum(counts)
    pad = (-total) % k
    counts = list(counts)
    counts[0] += pad
    ids = _ids_from_counts(counts, k=k, seed=total)
    sch = O.routing_schedule(ids, None, len(counts))
    assert int(sch.counts.sum()) == ids.shape[0] * k
    assert sch.counts.tolist() == counts


def test_out_of_range_ids_are_excluded():
    ids = np.array([[0, 5], [-1, 1], [1, 0]], dtype=np.int32)
    sch = O.routing_schedule(ids, None, 2)
    assert sch.n_invalid == 2
    assert sch.counts.tolist() == [2, 2]
    assert sch.perm.tolist() == [0, 5, 3, 4]


# ----------------------------------------------------------------------------
# Tile space: the page's worked example
# ----------------------------------------------------------------------------
def test_worked_example_balanced():
    g = _load("worked_example.json")
    b = g["balanced"]
    counts = np.full(g["experts"], b["rows_per_expert"])
    ts = O.tile_space(counts, g["N"], g["BM"], g["BN"])
    assert ts.tiles_n == b["col_blocks"]
    assert (ts.tiles == b["tiles_per_expert"]).all()
    assert ts.total == b["total_tiles"]
    assert ts.total / g["gpu_sms"] == pytest.approx(b["waves_exact"], abs=0.05)
    assert math.ceil(ts.total / g["gpu_sms"]) == b["waves"]
    S = g["tokens"] * g["top_k"]
    assert int(counts.sum()) == S
    assert 2 * S * g["K"] * g["N"] / 1e9 == pytest.approx(g["useful_gflop_approx"], rel=0.01)


@pytest.mark.parametrize("key", ["skewed", "skewed_bm64"])
def test_worked_example_skewed(key):
    g = _load("worked_example.json")
    case = g[key]
    BM = case.get("BM", g["BM"])
    counts = np.concatenate([np.full(n, rows) for n, rows in g["skewed"]["groups"]])
    assert int(counts.sum()) == g["tokens"] * g["top_k"]
    ts = O.tile_space(counts, g["N"], BM, g["BN"])
    row_blocks = ts.tiles // ts.tiles_n
    per_group = []
    i = 0
    for n, _ in g["skewed"]["groups"]:
        per_group.append(int(row_blocks[i]))
        i += n
    assert per_group == case["row_blocks_per_group"]
    assert int(row_blocks.sum()) == case["row_blocks"]
    computed = int(row_blocks.sum()) * BM
    assert computed == case["computed_rows"]
    useful = 100.0 * counts.sum() / computed
    assert round(useful) == case["useful_percent"]
    if key == "skewed":
        assert ts.total == case["total_tiles"]
        assert math.ceil(ts.total / g["gpu_sms"]) == case["waves"]
        bal = O.tile_space(np.full(64, 256), g["N"], BM, g["BN"])
        assert ts.total / bal.total == pytest.approx(case["cost_ratio_approx"], abs=0.01)


@settings(max_examples=80, deadline=None)
@given(st.lists(st.sampled_from([0, 0, 0, 1, 2, 5, 31, 32, 33, 64, 100]), min_size=1, max_size=10),
       st.sampled_from([1, 7, 32, 130]), st.sampled_from([16, 32, 64]), st.sampled_from([16, 64]))
def test_tile_owner_brute_force(counts, N, BM, BN):
    """Owner of every tile = the unique group whose tile range contains it; the
    coordinates enumerate every (row block, column block) of every group once."""
    counts = np.array(counts)
    offsets = np.cumsum(counts).astype(np.int32)
    ts = O.tile_space(counts, N, BM, BN)
    seen = set()
    for tau in range(ts.total):
        owners = [e for e in range(len(counts)) if ts.tile_start[e] <= tau < ts.tile_start[e] + ts.tiles[e]]
        assert len(owners) == 1
        assert int(O.tile_owner(ts, tau)) == owners[0]
        g, mb, nb, row0, rows = O.tile_coords(ts, counts, offsets, tau)
        assert 1 <= rows <= BM
        assert row0 >= (0 if g == 0 else offsets[g - 1]) and row0 + rows <= offsets[g]
        assert 0 <= nb < ts.tiles_n
        seen.add((g, mb, nb))
    expect = {(e, mb, nb) for e in range(len(counts)) for mb in range(-(-counts[e] // BM))
              for nb in range(ts.tiles_n)}
    assert seen == expect


def test_column_block_major_walk():
    """Consecutive tiles of one group share a column block and step over row blocks."""
    counts = np.array([300, 0, 130])
    offsets = np.cumsum(counts).astype(np.int32)
    ts = O.tile_space(counts, 256, 128, 128)
    coords = [O.tile_coords(ts, counts, offsets, t)[:3] for t in range(ts.total)]
    assert coords[:6] == [(0, 0, 0), (0, 1, 0), (0, 2, 0), (0, 0, 1), (0, 1, 1), (0, 2, 1)]
    assert coords[6:] == [(2, 0, 0), (2, 1, 0), (2, 0, 1), (2, 1, 1)]


# ----------------------------------------------------------------------------
# Products: brute force, closed forms, textbook reductions
# ----------------------------------------------------------------------------
def _brute_grouped(A, W, offsets):
    M = len(A)
    N = len(W[0])
    K = len(A[0])
    C = [[0.0] * N for _ in range(M)]
    prev = 0
    for e, end in enumerate(offsets):
        for r in range(prev, end):
            for n in range(N):
                s = 0.0
                for kk in range(K):
                    s += float(A[r][kk]) * float(W[e][n][kk])
                C[r][n] = s
        prev = end
    return np.array(C)


def _dot_bound(a, b):
    return len(a) * 2.0 ** -52 * np.sum(np.abs(a * b))


@pytest.mark.parametrize("counts", [[3, 0, 5], [0, 1, 4], [2, 2, 0], [0, 0, 6], [1]])
def test_grouped_gemm_brute_force(counts):
    rng = np.random.default_rng(sum(counts))
    M, K, N = sum(counts), 7, 5
    A = rng.standard_normal((M + 2, K))
    W = rng.standard_normal((len(counts), N, K))
    offsets = np.cumsum(counts).astype(np.int32)
    out = np.full((M + 2, N), -7.0)
    C = O.grouped_gemm(A, W, offsets, out=out)
    B = _brute_grouped(A.tolist(), W.tolist(), offsets.tolist())
    assert np.allclose(C[:M], B[:M], rtol=0, atol=1e-12)
    assert (C[M:] == -7.0).all()


def _brute_moe(x, W, ids, w):
    T, k = ids.shape
    N, K = W.shape[1], W.shape[2]
    y = np.zeros((T, N))
    for t in range(T):
        for n in range(N):
            tot = 0.0
            for j in range(k):
                e = ids[t, j]
                s = 0.0
                for kk in range(K):
                    s += float(x[t, kk]) * float(W[e, n, kk])
                tot += float(w[t, j]) * s
            y[t, n] = tot
    return y


def _tiny_routed(seed, T=5, k=2, E=3, K=7, N=5, empty=1):
    rng = np.random.default_rng(seed)
    live = [e for e in range(E) if e != empty]
    ids = np.array([rng.choice(live, size=k, replace=False) for _ in range(T)], dtype=np.int32)
    x = rng.standard_normal((T, K)).astype(np.float32)
    W = rng.standard_normal((E, N, K)).astype(np.float32)
    w = rng.random((T, k)).astype(np.float32)
    return x, W, ids, w


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_moe_forward_brute_force(seed):
    x, W, ids, w = _tiny_routed(seed)
    y = O.moe_forward(x, W, ids, w, 3)
    y_explicit = O.moe_forward_explicit(x, W, ids, w, 3)
    ref = _brute_moe(x, W, ids, w)
    assert np.abs(y - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())
    assert np.abs(y_explicit - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def test_single_expert_is_plain_matmul():
    """E=1, k=1, weight 1: the layer is x @ W[0]^T."""
    rng = np.random.default_rng(11)
    T, K, N = 19, 13, 9
    x = rng.standard_normal((T, K))
    W = rng.standard_normal((1, N, K))
    ids = np.zeros((T, 1), dtype=np.int32)
    y = O.moe_forward(x, W, ids, None, 1)
    assert np.allclose(y, np.matmul(x, W[0].T), rtol=1e-13, atol=1e-13)
    C = O.grouped_gemm(x, W, np.array([T], dtype=np.int32))
    assert np.allclose(C, np.matmul(x, W[0].T), rtol=1e-13, atol=1e-13)


def test_rank_one_closed_form():
    """W[e] = u_e v_e^T in (E, N, K) storage with K != N gives
    y[t] = sum_j w[t,j] * (v_{e} . x[t]) * u_{e}: a transposed operand or a
    dropped weight cannot produce it."""
    rng = np.random.default_rng(5)
    T, K, N, E, k = 11, 6, 4, 3, 2
    u = rng.standard_normal((E, N))
    v = rng.standard_normal((E, K))
    W = np.einsum("en,ek->enk", u, v)
    x = rng.standard_normal((T, K))
    ids = np.array([rng.choice(E, size=k, replace=False) for _ in range(T)], dtype=np.int32)
    w = rng.random((T, k))
    y = O.moe_forward(x, W, ids, w, E)
    expect = np.zeros((T, N))
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            expect[t] += w[t, j] * float(v[e] @ x[t]) * u[e]
    assert np.allclose(y, expect, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("acc", [np.float32, np.float64])
def test_fused_equals_explicit_bitwise(acc):
    """The card's 'Correctness' section: the fused forward equals the explicit
    gather -> grouped GEMM -> scatter path bit for bit in fp32."""
    rng = np.random.default_rng(21)
    T, K, N, E, k = 64, 24, 16, 5, 2
    ids = np.array([rng.choice([0, 1, 3, 4], size=k, replace=False) for _ in range(T)], dtype=np.int32)
    x = rng.standard_normal((T, K)).astype(np.float32)
    W = rng.standard_normal((E, N, K)).astype(np.float32)
    w = rng.random((T, k)).astype(np.float32)
    a = O.moe_forward(x, W, ids, w, E, acc=acc)
    b = O.moe_forward_explicit(x, W, ids, w, E, acc=acc)
    assert a.dtype == acc and np.array_equal(a, b)


def test_empty_and_single_row_experts():
    """'What to do next', step 2: an empty expert and a single-row expert."""
    rng = np.random.default_rng(8)
    T, K, N, E = 9, 5, 3, 4
    ids = np.array([[0], [0], [2], [0], [0], [3], [3], [0], [3]], dtype=np.int32)   # expert 1 empty, 2 single
    x = rng.standard_normal((T, K))
    W = rng.standard_normal((E, N, K))
    y = O.moe_forward(x, W, ids, None, E)
    assert np.allclose(y[2], W[2] @ x[2], rtol=1e-13, atol=1e-13)
    W2 = W.copy()
    W2[1] = np.nan                      # an empty expert's weights are never read
    y2 = O.moe_forward(x, W2, ids, None, E)
    assert np.array_equal(y, y2)


# ----------------------------------------------------------------------------
# Backward: finite differences, identities, exact zeros
# ----------------------------------------------------------------------------
def _loss(dY, x, W, ids, w, E):
    return float(np.sum(dY * O.moe_forward(x, W, ids, w, E)))


def test_backward_finite_differences():
    """y is linear in each of x, W and w separately, so a central difference in
    float64 has no truncation error and must match the analytic gradients up to
    rounding (the card: the backward agrees with finite differences)."""
    rng = np.random.default_rng(13)
    T, K, N, E, k = 6, 5, 4, 3, 2
    ids = np.array([rng.choice(E, size=k, replace=False) for _ in range(T)], dtype=np.int32)
    x = rng.standard_normal((T, K))
    W = rng.standard_normal((E, N, K))
    w = rng.random((T, k))
    dY = rng.standard_normal((T, N))
    dX, dW, d_w = O.moe_backward(dY, x, W, ids, w, E)
    h = 0.5

    def fd(arr, idx, f):
        a = arr.copy(); a[idx] += h
        b = arr.copy(); b[idx] -= h
        return (f(a) - f(b)) / (2 * h)

    for idx in np.ndindex(x.shape):
        assert fd(x, idx, lambda a: _loss(dY, a, W, ids, w, E)) == pytest.approx(dX[idx], abs=1e-12)
    for idx in np.ndindex(W.shape):
        assert fd(W, idx, lambda a: _loss(dY, x, a, ids, w, E)) == pytest.approx(dW[idx], abs=1e-12)
    for idx in np.ndindex(w.shape):
        assert fd(w, idx, lambda a: _loss(dY, x, W, ids, a, E)) == pytest.approx(d_w[idx], abs=1e-12)


def test_backward_euler_identities():
    """L = <dY, y> is linear in x, in W and in w, so
    <dX, x> = <dW, W> = sum(w * d_w) = L."""
    rng = np.random.default_rng(17)
    T, K, N, E, k = 40, 12, 9, 6, 3
    ids = np.array([rng.choice(E, size=k, replace=False) for _ in range(T)], dtype=np.int32)
    x = rng.standard_normal((T, K))
    W = rng.standard_normal((E, N, K))
    w = rng.random((T, k))
    dY = rng.standard_normal((T, N))
    L = float(np.sum(dY * O.moe_forward(x, W, ids, w, E)))
    dX, dW, d_w = O.moe_backward(dY, x, W, ids, w, E)
    assert float(np.sum(dX * x)) == pytest.approx(L, rel=1e-12)
    assert float(np.sum(dW * W)) == pytest.approx(L, rel=1e-12)
    assert float(np.sum(d_w * w)) == pytest.approx(L, rel=1e-12)


def test_weight_grad_of_empty_expert_is_exact_zero():
    """'The backward pass' and 'What to do next', step 6."""
    x, W, ids, w = _tiny_routed(4, T=8, E=4, empty=2)
    dY = np.random.default_rng(4).standard_normal((8, W.shape[1]))
    _, dW, _ = O.moe_backward(dY, x, W, ids, w, 4)
    assert np.all(dW[2] == 0.0) and not np.signbit(dW[2]).any()
    assert np.abs(dW[[0, 1, 3]]).max() > 0


def test_backward_brute_force_entries():
    """Sampled-entry evaluators agree with plain Python loops over the definition."""
    x, W, ids, w = _tiny_routed(9, T=6, k=2, E=3, K=4, N=3, empty=1)
    dY = np.random.default_rng(9).standard_normal((6, 3))
    dX, dW, d_w = O.moe_backward(dY, x, W, ids, w, 3)
    T, k = ids.shape
    bx = np.zeros_like(dX)
    bw = np.zeros_like(dW)
    bd = np.zeros_like(d_w)
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            for kk in range(x.shape[1]):
                bx[t, kk] += w[t, j] * sum(dY[t, n] * W[e, n, kk] for n in range(3))
            for n in range(3):
                for kk in range(x.shape[1]):
                    bw[e, n, kk] += w[t, j] * dY[t, n] * x[t, kk]
            bd[t, j] = sum(dY[t, n] * sum(x[t, kk] * W[e, n, kk] for kk in range(x.shape[1])) for n in range(3))
    assert np.allclose(dX, bx, atol=1e-12) and np.allclose(dW, bw, atol=1e-12) and np.allclose(d_w, bd, atol=1e-12)
    toks = [0, 3, 5]
    rx, rd = O.moe_backward_rows(dY, x, W, ids, w, toks)
    assert np.allclose(rx, bx[toks], atol=1e-12) and np.allclose(rd, bd[toks], atol=1e-12)
    ent = [(0, 1, 2), (1, 0, 0), (2, 2, 3)]
    assert np.allclose(O.weight_grad_entries(dY, x, ids, w, 3, ent), [bw[e] [n][kk] for e, n, kk in ent], atol=1e-12)
    ry = O.moe_forward_rows(x, W, ids, w, toks)
    assert np.allclose(ry, _brute_moe(x, W, ids, w)[toks], atol=1e-12)


def test_grouped_weight_grad_brute_force():
    rng = np.random.default_rng(31)
    counts = [3, 0, 1, 4]
    M, K, N = sum(counts), 5, 3
    X = rng.standard_normal((M, K))
    dY = rng.standard_normal((M, N))
    offsets = np.cumsum(counts).astype(np.int32)
    dW = O.grouped_weight_grad(X, dY, offsets, 4)
    prev = 0
    for e, end in enumerate(offsets):
        for n in range(N):
            for kk in range(K):
                s = sum(dY[r, n] * X[r, kk] for r in range(prev, end))
                assert dW[e, n, kk] == pytest.approx(s, abs=1e-12)
        prev = end
    assert np.all(dW[1] == 0)


# ----------------------------------------------------------------------------
# Masked layout
# ----------------------------------------------------------------------------
def test_masked_equals_contiguous_without_overflow():
    rng = np.random.default_rng(41)
    T, K, N, E, k = 30, 8, 6, 7, 3
    ids = np.array([rng.choice(E, size=k, replace=False) for _ in range(T)], dtype=np.int32)
    x = rng.standard_normal((T, K))
    W = rng.standard_normal((E, N, K))
    w = rng.random((T, k))
    ms = O.masked_schedule(ids, w, E, capacity=T)
    assert ms.n_dropped == 0
    assert np.allclose(O.masked_forward(x, W, ms, T), O.moe_forward(x, W, ids, w, E), rtol=1e-13, atol=1e-13)


def test_masked_overflow_drops_latest_assignments():
    ids = np.array([[0, 1], [0, 2], [0, 1], [1, 0]], dtype=np.int32)
    ms = O.masked_schedule(ids, None, 3, capacity=2)
    assert ms.masked_m.tolist() == [2, 2, 1]
    assert ms.slot_assign.tolist() == [[0, 2], [1, 5], [3, -1]]
    assert ms.n_dropped == 3       # s=4, 7 (expert 0) and s=6 (expert 1)
    assert ms.slot_token.tolist() == [[0, 1], [0, 2], [1, -1]]
    assert ms.slot_weight.tolist() == [[1, 1], [1, 1], [1, 0]]


# ----------------------------------------------------------------------------
# Gated expert FFN
# ----------------------------------------------------------------------------
def test_silu_against_library_and_closed_forms():
    """silu(z) = z * expit(z) (scipy's logistic function); silu(0) = 0,
    silu(1) = 1 / (1 + e^-1); it tends to z for large z and to 0 for very
    negative z."""
    from scipy.special import expit
    z = np.linspace(-40.0, 40.0, 2001)
    assert np.allclose(O.silu(z), z * expit(z), rtol=1e-14, atol=1e-300)
    assert O.silu(0.0) == 0.0
    assert abs(float(O.silu(1.0)) - 1.0 / (1.0 + math.exp(-1.0))) <= 1e-16
    assert float(O.silu(800.0)) == 800.0
    assert abs(float(O.silu(-800.0))) == 0.0


def test_gated_ffn_reduces_to_dense_swiglu():
    """E = 1, k = 1, weight 1: a dense gated MLP, computed with torch's own
    SiLU in float64: y = (silu(x Wg^T) * (x Wu^T)) Wd^T."""
    import torch
    rng = np.random.default_rng(61)
    T, K, F, N = 13, 11, 7, 5
    x = rng.standard_normal((T, K))
    Wgu = rng.standard_normal((1, 2 * F, K))
    Wd = rng.standard_normal((1, N, F))
    ids = np.zeros((T, 1), dtype=np.int32)
    y = O.gated_ffn_forward(x, Wgu, Wd, ids, None, 1)
    xt = torch.from_numpy(x)
    g = xt @ torch.from_numpy(Wgu[0, :F]).T
    u = xt @ torch.from_numpy(Wgu[0, F:]).T
    ref = (torch.nn.functional.silu(g) * u) @ torch.from_numpy(Wd[0]).T
    assert np.allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_gated_gate_and_up_halves():
    """x[:, 0] = 1 and x[:, 1] = v_t; the up rows select column 0 (u = 1), the
    gate rows give g = a[e, f] * v_t, and W_down is the identity, so
    y[t, f] = sum_j w[t, j] * silu(a[e_tj, f] * v_t) exactly (scipy's expit).
    Swapping the gate and up halves gives silu(1) * g instead."""
    from scipy.special import expit
    rng = np.random.default_rng(62)
    T, E, k, F = 17, 4, 2, 6
    K = 3
    v = rng.standard_normal(T) * 3
    x = np.zeros((T, K))
    x[:, 0] = 1.0
    x[:, 1] = v
    x[:, 2] = rng.standard_normal(T)          # never read by a nonzero weight
    a = rng.standard_normal((E, F))
    Wgu = np.zeros((E, 2 * F, K))
    Wgu[:, :F, 1] = a
    Wgu[:, F:, 0] = 1.0
    Wd = np.broadcast_to(np.eye(F), (E, F, F)).copy()
    ids = np.array([rng.choice(E, size=k, replace=False) for _ in range(T)], dtype=np.int32)
    w = rng.random((T, k))
    y = O.gated_ffn_forward(x, Wgu, Wd, ids, w, E)
    expect = np.zeros((T, F))
    for t in range(T):
        for j in range(k):
            z = a[ids[t, j]] * v[t]
            expect[t] += w[t, j] * z * expit(z)
    assert np.allclose(y, expect, rtol=1e-13, atol=1e-13)


def _brute_gated(x, Wgu, Wd, ids, w):
    T, k = ids.shape
    F = Wgu.shape[1] // 2
    N = Wd.shape[1]
    K = x.shape[1]
    y = [[0.0] * N for _ in range(T)]
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            h = []
            for f in range(F):
                g = sum(float(x[t, c]) * float(Wgu[e, f, c]) for c in range(K))
                u = sum(float(x[t, c]) * float(Wgu[e, F + f, c]) for c in range(K))
                h.append(g / (1.0 + math.exp(-g)) * u)
            for n in range(N):
                y[t][n] += float(w[t, j]) * sum(h[f] * float(Wd[e, n, f]) for f in range(F))
    return np.array(y)


@pytest.mark.parametrize("seed", [0, 1])
def test_gated_ffn_brute_force(seed):
    """Plain Python loops on a tiny routed case with an empty expert and
    F != N != K; the fused and the explicit oracle forms both match."""
    rng = np.random.default_rng(70 + seed)
    T, K, F, N, E, k = 5, 7, 3, 4, 3, 2
    ids = np.array([rng.choice([0, 2], size=k, replace=False) for _ in range(T)], dtype=np.int32)
    x = rng.standard_normal((T, K))
    Wgu = rng.standard_normal((E, 2 * F, K))
    Wd = rng.standard_normal((E, N, F))
    w = rng.random((T, k))
    ref = _brute_gated(x, Wgu, Wd, ids, w)
    for y in (O.gated_ffn_forward(x, Wgu, Wd, ids, w, E),
              O.gated_ffn_forward_explicit(x, Wgu, Wd, ids, w, E),
              O.gated_ffn_rows(x, Wgu, Wd, ids, w, range(T))):
        assert np.abs(y - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def test_gated_intermediate_rows_brute_force():
    """h row r belongs to the r-th assignment in (expert, s) order."""
    rng = np.random.default_rng(75)
    T, K, F, E, k = 6, 5, 4, 3, 2
    ids = np.array([rng.choice(E, size=k, replace=False) for _ in range(T)], dtype=np.int32)
    x = rng.standard_normal((T, K))
    Wgu = rng.standard_normal((E, 2 * F, K))
    h = O.gated_intermediate(x, Wgu, ids, E)
    order = sorted(range(T * k), key=lambda s: (ids.reshape(-1)[s], s))
    for r, s in enumerate(order):
        t, e = s // k, int(ids.reshape(-1)[s])
        for f in range(F):
            g = sum(x[t, c] * Wgu[e, f, c] for c in range(K))
            u = sum(x[t, c] * Wgu[e, F + f, c] for c in range(K))
            assert abs(h[r, f] - g / (1.0 + math.exp(-g)) * u) <= 1e-12 * max(1.0, abs(h[r, f]))
    sel = [0, 5, 11]
    assert np.allclose(O.gated_intermediate_rows(x, Wgu, ids, E, sel), h[sel], rtol=1e-12, atol=1e-12)


def test_gated_ffn_homogeneity():
    """y is linear in the up half, in W_down and in the routing weights (exact
    under power-of-two scaling), but not in the gate half."""
    rng = np.random.default_rng(77)
    T, K, F, N, E, k = 9, 6, 5, 4, 3, 2
    ids = np.array([rng.choice(E, size=k, replace=False) for _ in range(T)], dtype=np.int32)
    x = rng.standard_normal((T, K))
    Wgu = rng.standard_normal((E, 2 * F, K))
    Wd = rng.standard_normal((E, N, F))
    w = rng.random((T, k))
    y = O.gated_ffn_forward(x, Wgu, Wd, ids, w, E)
    up2 = Wgu.copy()
    up2[:, F:] *= 2
    assert np.array_equal(O.gated_ffn_forward(x, up2, Wd, ids, w, E), 2 * y)
    assert np.array_equal(O.gated_ffn_forward(x, Wgu, 4 * Wd, ids, w, E), 4 * y)
    assert np.array_equal(O.gated_ffn_forward(x, Wgu, Wd, ids, 0.5 * w, E), 0.5 * y)
    g2 = Wgu.copy()
    g2[:, :F] *= 2
    assert not np.allclose(O.gated_ffn_forward(x, g2, Wd, ids, w, E), 2 * y)


def test_masked_gated_equals_contiguous_without_overflow():
    rng = np.random.default_rng(79)
    T, K, F, N, E, k = 20, 6, 5, 7, 6, 3
    ids = np.array([rng.choice(E, size=k, replace=False) for _ in range(T)], dtype=np.int32)
    x = rng.standard_normal((T, K))
    Wgu = rng.standard_normal((E, 2 * F, K))
    Wd = rng.standard_normal((E, N, F))
    w = rng.random((T, k))
    ms = O.masked_schedule(ids, w, E, capacity=T)
    y, h = O.masked_gated_ffn(x, Wgu, Wd, ms, T)
    assert np.allclose(y, _brute_gated(x, Wgu, Wd, ids, w), rtol=1e-12, atol=1e-12)
    hc = O.gated_intermediate(x, Wgu, ids, E)
    sch = O.routing_schedule(ids, None, E)
    for e in range(E):
        m = int(ms.masked_m[e])
        start = int(sch.starts[e])
        assert np.array_equal(h[e * T:e * T + m], hc[start:start + m])
        assert np.all(h[e * T + m:(e + 1) * T] == 0)


# ----------------------------------------------------------------------------
# FP8 operands with per-token and per-group-per-channel scales
# ----------------------------------------------------------------------------
def test_e4m3_decode_against_torch():
    """All 256 codes decode as torch's float8_e4m3fn does (NaN codes too)."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.decode_e4m3(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert O.decode_e4m3(0x7E) == 448.0 and O.decode_e4m3(0x01) == 2.0 ** -9
    assert O.decode_e4m3(0x38) == 1.0 and O.decode_e4m3(0xB8) == -1.0


def _tiny_fp8(seed, T=9, K=16, N=6, E=3, k=2):
    rng = np.random.default_rng(seed)
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    xq = rng.choice(codes, size=(T, K)).astype(np.uint8)
    Wq = rng.choice(codes, size=(E, N, K)).astype(np.uint8)
    ids = np.array([rng.choice(E, size=k, replace=False) for _ in range(T)], dtype=np.int32)
    w = rng.random((T, k))
    return rng, xq, Wq, ids, w


def test_fp8_forward_brute_force():
    """Plain Python loops over decoded codes (via torch's decoder) and scales."""
    import torch
    rng, xq, Wq, ids, w = _tiny_fp8(81)
    T, K = xq.shape
    E, N, _ = Wq.shape
    sx = rng.random(T) + 0.5
    sw = rng.random((E, N)) + 0.5
    dec = lambda a: torch.from_numpy(np.ascontiguousarray(a)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    xv, Wv = dec(xq), dec(Wq)
    ref = np.zeros((T, N))
    for t in range(T):
        for j in range(ids.shape[1]):
            e = ids[t, j]
            for n in range(N):
                dot = sum(float(xv[t, c]) * float(Wv[e, n, c]) for c in range(K))
                ref[t, n] += w[t, j] * sx[t] * sw[e, n] * dot
    y = O.moe_forward_fp8(xq, sx, Wq, sw, ids, w, E)
    assert np.abs(y - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())
    rows = O.moe_forward_fp8_rows(xq, sx, Wq, sw, ids, w, range(T))
    assert np.abs(rows - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def test_fp8_power_of_two_scales_are_exact():
    """With sx = 2^a and sw[e, n] = 2^b[n], y equals 2^(a + b[n]) times the
    unscaled result exactly, column by column: a scale indexed by the
    reduction dimension (or transposed) breaks this."""
    rng, xq, Wq, ids, w = _tiny_fp8(82, K=16, N=5)
    T = xq.shape[0]
    E, N, _ = Wq.shape
    y1 = O.moe_forward_fp8(xq, np.ones(T), Wq, np.ones((E, N)), ids, w, E)
    b = rng.integers(-3, 4, size=N)
    sw = np.broadcast_to(2.0 ** b, (E, N)).copy()
    y2 = O.moe_forward_fp8(xq, np.full(T, 4.0), Wq, sw, ids, w, E)
    assert np.array_equal(y2, y1 * 4.0 * 2.0 ** b[None, :])


def test_fp8_masked_equals_contiguous():
    rng, xq, Wq, ids, w = _tiny_fp8(83, T=20, K=32, N=7, E=5, k=3)
    T = xq.shape[0]
    E, N, _ = Wq.shape
    sx = rng.random(T) + 0.5
    sw = rng.random((E, N)) + 0.5
    ms = O.masked_schedule(ids, w, E, capacity=T)
    a = O.masked_forward_fp8(xq, sx, Wq, sw, ms, T)
    b = O.moe_forward_fp8(xq, sx, Wq, sw, ids, w, E)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-13)


def _gated_case(seed, T=7, K=6, F=4, N=5, E=3, k=2):
    rng = np.random.default_rng(seed)
    ids = np.array([rng.choice([0, 2], size=k, replace=False) for _ in range(T)], dtype=np.int32)
    x = rng.standard_normal((T, K))
    Wgu = rng.standard_normal((E, 2 * F, K))
    Wd = rng.standard_normal((E, N, F))
    w = rng.random((T, k))
    dY = rng.standard_normal((T, N))
    return x, Wgu, Wd, ids, w, dY


def test_gated_backward_finite_differences():
    """Central differences of L = sum(dY * y) in float64 (h = 1e-6; y is
    smooth, so the truncation error is O(h^2)) against every gradient."""
    x, Wgu, Wd, ids, w, dY = _gated_case(91)
    E = 3
    L = lambda x_, Wgu_, Wd_, w_: float(np.sum(dY * O.gated_ffn_forward(x_, Wgu_, Wd_, ids, w_, E)))
    dX, dWgu, dWd, d_w = O.gated_ffn_backward(dY, x, Wgu, Wd, ids, w, E)
    eps = 1e-6

    def fd(arr, idx, which):
        p_, m_ = arr.copy(), arr.copy()
        p_[idx] += eps
        m_[idx] -= eps
        args_p = [x, Wgu, Wd, w]
        args_m = [x, Wgu, Wd, w]
        args_p[which], args_m[which] = p_, m_
        return (L(*args_p) - L(*args_m)) / (2 * eps)

    for idx in [(0, 0), (3, 5), (6, 2)]:
        assert abs(fd(x, idx, 0) - dX[idx]) <= 1e-6 * max(1.0, abs(dX[idx]))
    for idx in [(0, 0, 0), (2, 1, 3), (2, 6, 5), (0, 7, 1)]:   # gate rows and up rows
        assert abs(fd(Wgu, idx, 1) - dWgu[idx]) <= 1e-6 * max(1.0, abs(dWgu[idx]))
    for idx in [(0, 0, 0), (2, 4, 3)]:
        assert abs(fd(Wd, idx, 2) - dWd[idx]) <= 1e-6 * max(1.0, abs(dWd[idx]))
    for idx in [(0, 0), (4, 1)]:
        assert abs(fd(w, idx, 3) - d_w[idx]) <= 1e-6 * max(1.0, abs(d_w[idx]))
    assert np.all(dWgu[1] == 0) and np.all(dWd[1] == 0)      # expert 1 has no rows


def test_gated_backward_identities():
    """y is linear in W_down, in the up half of W_gu and in w, so
    <dW_down, W_down> = <dW_up, W_up> = sum w * d_w = <dY, y>."""
    x, Wgu, Wd, ids, w, dY = _gated_case(92, T=11, K=5, F=3, N=4)
    E, F = 3, 3
    y = O.gated_ffn_forward(x, Wgu, Wd, ids, w, E)
    dX, dWgu, dWd, d_w = O.gated_ffn_backward(dY, x, Wgu, Wd, ids, w, E)
    Lv = float(np.sum(dY * y))
    assert abs(float(np.sum(dWd * Wd)) - Lv) <= 1e-12 * max(1.0, abs(Lv))
    assert abs(float(np.sum(dWgu[:, F:] * Wgu[:, F:])) - Lv) <= 1e-12 * max(1.0, abs(Lv))
    assert abs(float(np.sum(w * d_w)) - Lv) <= 1e-12 * max(1.0, abs(Lv))


def test_gated_backward_sampled_forms_agree():
    x, Wgu, Wd, ids, w, dY = _gated_case(93)
    E = 3
    dX, dWgu, dWd, d_w = O.gated_ffn_backward(dY, x, Wgu, Wd, ids, w, E)
    rx, rw = O.gated_ffn_backward_rows(dY, x, Wgu, Wd, ids, w, range(x.shape[0]))
    assert np.allclose(rx, dX, rtol=1e-12, atol=1e-12) and np.allclose(rw, d_w, rtol=1e-12, atol=1e-12)
    ge = [(0, 0, 0), (2, 7, 5), (2, 3, 1)]
    de = [(0, 4, 3), (2, 0, 0)]
    eg, ed = O.gated_weight_grad_entries(dY, x, Wgu, Wd, ids, w, E, ge, de)
    assert np.allclose(eg, [dWgu[i] for i in ge], rtol=1e-12, atol=1e-12)
    assert np.allclose(ed, [dWd[i] for i in de], rtol=1e-12, atol=1e-12)


def test_round_bf16_against_torch():
    """The oracle's bf16 rounding equals torch's float32 -> bfloat16 conversion
    (round to nearest, ties to even) on random values, ties and extremes."""
    import torch
    rng = np.random.default_rng(95)
    v = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.integers(-6, 6, 4000),
                        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -1.0 - 2.0 ** -8, 0.0, 448.0])])
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_bf16(v), ref)
    assert O.round_bf16(1.0 + 2.0 ** -8) == 1.0 and O.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6


def test_e8m0_decode_closed_form():
    c = np.arange(256, dtype=np.uint8)
    v = O.decode_e8m0(c)
    assert np.isnan(v[255]) and v[127] == 1.0 and v[128] == 2.0 and v[0] == 2.0 ** -127
    assert np.array_equal(v[:255], [math.ldexp(1.0, int(i) - 127) for i in range(255)])


def test_mx_forward_brute_force_and_block_structure():
    """Each 32-element block of x and W takes its own scale: brute force over
    blocks, and a scale change in one block moves only that block's terms."""
    import torch
    rng, xq, Wq, ids, w = _tiny_fp8(84, T=6, K=64, N=5, E=3, k=2)
    T, K = xq.shape
    E, N, _ = Wq.shape
    xs = rng.integers(120, 134, size=(T, K // 32)).astype(np.uint8)
    ws = rng.integers(120, 134, size=(E, N, K // 32)).astype(np.uint8)
    dec = lambda a: torch.from_numpy(np.ascontiguousarray(a)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    xv, Wv = dec(xq), dec(Wq)
    ref = np.zeros((T, N))
    for t in range(T):
        for j in range(2):
            e = ids[t, j]
            for n in range(N):
                tot = 0.0
                for b in range(K // 32):
                    sc = 2.0 ** (int(xs[t, b]) - 127) * 2.0 ** (int(ws[e, n, b]) - 127)
                    tot += sc * sum(float(xv[t, c]) * float(Wv[e, n, c]) for c in range(32 * b, 32 * b + 32))
                ref[t, n] += w[t, j] * tot
    y = O.moe_forward_mx(xq, xs, Wq, ws, ids, w, E)
    assert np.abs(y - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())
    # raising block 1's scale of every x row by 2^3 multiplies exactly that block's part by 8
    xs2 = xs.copy()
    xs2[:, 1] += 3
    y2 = O.moe_forward_mx(xq, xs2, Wq, ws, ids, w, E)
    only0 = xs.copy()
    only0[:, 1] = 0                     # 2^-127: block 1 contributes nothing measurable
    y0 = O.moe_forward_mx(xq, only0, Wq, ws, ids, w, E)
    assert np.allclose(y2 - y0, 8 * (y - y0), rtol=1e-12, atol=1e-12)


def test_mx_masked_equals_contiguous():
    """Masked layout with room for every assignment: the block-scaled decode
    forward equals the contiguous block-scaled forward ("Grouped GEMM" notes,
    section 5: the two layouts hold the same rows)."""
    rng, xq, Wq, ids, w = _tiny_fp8(85, T=20, K=64, N=7, E=5, k=3)
    T, K = xq.shape
    E, N, _ = Wq.shape
    xs = rng.integers(118, 136, size=(T, K // 32)).astype(np.uint8)
    ws = rng.integers(118, 136, size=(E, N, K // 32)).astype(np.uint8)
    ms = O.masked_schedule(ids, w, E, capacity=T)
    a = O.masked_forward_mx(xq, xs, Wq, ws, ms, T)
    b = O.moe_forward_mx(xq, xs, Wq, ws, ids, w, E)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-13)


def test_mx_masked_overflow_brute_force():
    """Masked block-scaled forward with a capacity below the busiest expert's
    load, against plain loops: per expert, the assignments taken in ascending
    s = t*k + j keep a slot while fewer than `capacity` came before them; each
    kept one adds w * sum over 32-element blocks of (block scales) x (decoded
    code products) to its token's row; dropped ones add nothing."""
    import torch
    rng, xq, Wq, ids, w = _tiny_fp8(86, T=14, K=64, N=4, E=3, k=2)
    T, K = xq.shape
    E, N, _ = Wq.shape
    cap = 5
    xs = rng.integers(120, 134, size=(T, K // 32)).astype(np.uint8)
    ws = rng.integers(120, 134, size=(E, N, K // 32)).astype(np.uint8)
    dec = lambda a: torch.from_numpy(np.ascontiguousarray(a)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    xv, Wv = dec(xq), dec(Wq)
    seen = [0] * E
    ref = np.zeros((T, N))
    dropped = 0
    for t in range(T):
        for j in range(2):
            e = int(ids[t, j])
            if seen[e] >= cap:
                dropped += 1
                continue
            seen[e] += 1
            for n in range(N):
                tot = 0.0
                for b in range(K // 32):
                    sc = 2.0 ** (int(xs[t, b]) - 127) * 2.0 ** (int(ws[e, n, b]) - 127)
                    tot += sc * sum(float(xv[t, c]) * float(Wv[e, n, c]) for c in range(32 * b, 32 * b + 32))
                ref[t, n] += w[t, j] * tot
    assert dropped > 0, "the case must overflow"
    ms = O.masked_schedule(ids, w, E, capacity=cap)
    y = O.masked_forward_mx(xq, xs, Wq, ws, ms, T)
    assert np.abs(y - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def test_backward_selected_experts_match_full():
    """The per-expert weight gradients of moe_backward's dw_experts form are
    the same numbers as its full form (the same loop, dW kept for the listed
    experts only); an expert with no rows gives exact zeros."""
    rng = np.random.default_rng(97)
    T, K, N, E, k = 13, 7, 5, 4, 2
    ids = np.array([rng.choice([0, 1, 3], size=k, replace=False) for _ in range(T)], dtype=np.int32)
    x, W, dY = rng.standard_normal((T, K)), rng.standard_normal((E, N, K)), rng.standard_normal((T, N))
    w = rng.random((T, k))
    dX, dW, dw = O.moe_backward(dY, x, W, ids, w, E)
    dX2, dWs, dw2 = O.moe_backward(dY, x, W, ids, w, E, dw_experts=[3, 2])
    assert np.array_equal(dX, dX2) and np.array_equal(dw, dw2)
    assert set(dWs) == {2, 3} and np.array_equal(dWs[3], dW[3]) and np.all(dWs[2] == 0)


# ----------------------------------------------------------------------------
# Rank-ordered view (the layout the rank-by-rank combine runs on)
# ----------------------------------------------------------------------------
def _rank_brute(ids, w, E):
    """Plain loops: rank = valid slots of the token before this one; rows sorted
    by (rank * E + expert, s); a token with no valid slot contributes one row
    (rank 0, expert 0) at its last slot."""
    T, k = ids.shape
    rows = []
    for t in range(T):
        nvalid = 0
        for j in range(k):
            e = int(ids[t, j])
            if 0 <= e < E:
                rows.append((nvalid * E + e, t * k + j, t * k + j, float(w[t, j])))
                nvalid += 1
        if nvalid == 0:
            rows.append((0, t * k + k - 1, -1, 0.0))
    rows.sort(key=lambda r: (r[0], r[1]))
    counts = [0] * (k * E)
    for key, *_ in rows:
        counts[key] += 1
    return counts, [r[2] for r in rows], [r[1] // k for r in rows], [r[3] for r in rows]


@pytest.mark.parametrize("seed,T,k,E,bad", [(1, 40, 2, 5, 0.0), (2, 31, 3, 4, 0.2), (3, 17, 1, 6, 0.3),
                                            (4, 25, 4, 3, 0.5)])
def test_rank_schedule_brute_force(seed, T, k, E, bad):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    ids[rng.random((T, k)) < bad] = -3          # excluded ids, some tokens left with none
    w = rng.random((T, k)).astype(np.float32)
    rs = O.rank_schedule(ids, w, E)
    counts, assign, tok, wt = _rank_brute(ids, w, E)
    assert list(rs.counts) == counts
    assert list(rs.offsets) == list(np.cumsum(counts))
    assert list(rs.row_to_assign) == assign and list(rs.row_to_token) == tok
    assert np.array_equal(rs.row_weight, np.array(wt, dtype=np.float32))


def test_rank_schedule_rank_groups_hold_each_token_once():
    """Rank 0 rows hold every token exactly once; any rank holds a token at
    most once; the valid rows are the canonical schedule's rows."""
    rng = np.random.default_rng(5)
    T, k, E = 200, 3, 7
    ids = np.array([rng.choice(E, size=k, replace=True) for _ in range(T)], dtype=np.int32)
    ids[rng.random((T, k)) < 0.15] = E + 4
    rs = O.rank_schedule(ids, None, E)
    starts = np.concatenate([[0], rs.offsets])
    for p in range(k):
        toks = rs.row_to_token[starts[p * E]:starts[(p + 1) * E]]
        assert len(set(toks.tolist())) == len(toks)
        if p == 0:
            assert sorted(toks.tolist()) == list(range(T))
    sch = O.routing_schedule(ids, None, E)
    real = rs.row_to_assign[rs.row_to_assign >= 0]
    assert sorted(real.tolist()) == sorted(sch.perm.tolist())
