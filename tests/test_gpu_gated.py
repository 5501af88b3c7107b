"""GPU parity of the gated expert FFN (moe_gated_ffn_fwd / _bwd) against the oracle.

The intermediate h (bf16, schedule row order), the output y (fp32) and the
gradients are compared with the bf16 tolerances: max relative error <= 1e-2
and relative Frobenius error <= 3e-3 (normwise).  The forward and the
backward's dX, dW_gu and d_topk are checked against the exact (float64)
oracle.  dW_down = sum over rows of (w dY)^T h is checked against the oracle
that rounds h to bf16 where it forms it: h is a bf16 tensor of the path by the
call's contract (the forward stores it, the backward takes it back), and that
rounding alone puts dW_down near the Frobenius bound of the exact product.
Both margins are logged.  Rows of h the call must not write keep a sentinel.
"""
import numpy as np
import pytest
import torch

from moe_variable_size_amd import api
from moe_variable_size_amd import workloads as WL
from oracle import moe_oracle as O
from tests.gpu_util import assert_close, dev, host, log, max_rel, rel_fro

pytestmark = pytest.mark.gpu

SENTINEL = 7.0


def _small(T, K, F, N, E, k, seed, empty=()):
    g = WL.gated("small_gated", T, K, F, N, E, k, seed=seed)
    if empty:
        live = [e for e in range(E) if e not in empty]
        rng = np.random.default_rng(seed)
        g.expert_ids = np.array([rng.choice(live, size=k, replace=False) for _ in range(T)],
                                dtype=np.int32)
    return g


def _run(g, layout=api.MOE_LAYOUT_CONTIGUOUS, cap=0):
    sch = api.moe_build_schedule(dev(g.expert_ids), dev(g.topk_weights), g.E, layout=layout,
                                 capacity=cap)
    h0 = torch.full((sch.c.R, g.F), SENTINEL, dtype=torch.bfloat16, device="cuda")
    y0 = torch.full((g.T, g.N), float("nan"), dtype=torch.float32, device="cuda")  # y is overwritten
    y, h = api.moe_gated_ffn_fwd(dev(g.x), dev(g.W_gu), dev(g.W_down), sch, h=h0, y=y0)
    torch.cuda.synchronize()
    return host(y), host(h)


@pytest.mark.parametrize("T,K,F,N,E,k,empty", [
    (333, 136, 200, 72, 7, 2, (3,)),     # ragged K, F and N; an empty expert
    (129, 64, 128, 192, 3, 1, ()),
    (1030, 256, 384, 256, 8, 2, ()),     # 48 tiles: the last round splits into row halves
    (64, 72, 8, 16, 5, 3, (0, 4)),       # F = 8: one partial gate/up block
])
def test_gated_contiguous(T, K, F, N, E, k, empty):
    g = _small(T, K, F, N, E, k, seed=T + K + F, empty=empty)
    log(f"gated contiguous T={T} K={K} F={F} N={N} E={E} k={k} empty={empty}")
    y, h = _run(g)
    ref_y = O.gated_ffn_forward(g.x.values, g.W_gu.values, g.W_down.values, g.expert_ids,
                                g.topk_weights, E)
    ref_h = O.gated_intermediate(g.x.values, g.W_gu.values, g.expert_ids, E)
    assert_close(h, ref_h, "bf16", "h")
    assert_close(y, ref_y, "bf16", "y")


@pytest.mark.parametrize("T,K,F,N,E,k,cap", [
    (128, 512, 256, 384, 16, 4, 64),     # 64-row decode tiles
    (97, 128, 136, 64, 11, 4, 3),        # overflowing capacity, 64-row tiles
    (300, 96, 128, 128, 6, 2, 130),      # capacity above 64: 256-row tiles
])
def test_gated_masked(T, K, F, N, E, k, cap):
    g = _small(T, K, F, N, E, k, seed=T + cap)
    log(f"gated masked T={T} K={K} F={F} N={N} E={E} k={k} cap={cap}")
    y, h = _run(g, api.MOE_LAYOUT_MASKED, cap)
    ms = O.masked_schedule(g.expert_ids, g.topk_weights, E, cap)
    ref_y, ref_h = O.masked_gated_ffn(g.x.values, g.W_gu.values, g.W_down.values, ms, T)
    valid = (ms.slot_assign.reshape(-1) >= 0)
    assert_close(h[valid], ref_h[valid], "bf16", "h valid slots")
    assert (h[~valid] == SENTINEL).all(), "empty slots of h were written"
    assert_close(y, ref_y, "bf16", "y")


def test_gated_page_example_sampled():
    """The balanced step of the page's worked example at full size; y checked
    on sampled tokens, h on sampled schedule rows (oracle's own schedule)."""
    g = WL.gated_page_example()
    log(f"gated full size {g.name}")
    y, h = _run(g)
    rng = np.random.default_rng(5)
    toks = np.sort(rng.choice(g.T, size=12, replace=False))
    ref_y = O.gated_ffn_rows(g.x.values, g.W_gu.values, g.W_down.values, g.expert_ids,
                             g.topk_weights, toks)
    assert_close(y[toks], ref_y, "bf16", "y sampled tokens")
    rows = np.sort(rng.choice(g.S, size=12, replace=False))
    ref_h = O.gated_intermediate_rows(g.x.values, g.W_gu.values, g.expert_ids, g.E, rows)
    assert_close(h[rows], ref_h, "bf16", "h sampled rows")


# ----------------------------------------------------------------------------
# backward
# ----------------------------------------------------------------------------
def _bwd(g, dY, layout=api.MOE_LAYOUT_CONTIGUOUS, cap=0):
    sch = api.moe_build_schedule(dev(g.expert_ids), dev(g.topk_weights), g.E, layout=layout,
                                 capacity=cap)
    y, h, gu = api.moe_gated_ffn_fwd(dev(g.x), dev(g.W_gu), dev(g.W_down), sch, save_gu=True)
    dX, dWgu, dWd, dT = api.moe_gated_ffn_bwd(dev(dY), dev(g.x), dev(g.W_gu), dev(g.W_down), sch,
                                              gu, h)
    torch.cuda.synchronize()
    return host(dX), host(dWgu), host(dWd), host(dT)


def _margins(pairs):
    """Log max_rel / rel_fro of each gradient against the exact oracle and
    against the oracle that rounds h to bf16 as the kernels store it."""
    for name, got, exact, rounded in pairs:
        log(f"  {name}: exact oracle max_rel {max_rel(got, exact):.3e} rel_fro {rel_fro(got, exact):.3e}"
            f" | h-rounded oracle max_rel {max_rel(got, rounded):.3e} rel_fro {rel_fro(got, rounded):.3e}")


def _dy(g, seed):
    rng = np.random.default_rng(seed)
    return WL._make(rng.standard_normal((g.T, g.N), dtype=np.float32), True)


@pytest.mark.parametrize("T,K,F,N,E,k,empty", [
    (333, 136, 200, 72, 7, 2, (3,)),
    (1030, 256, 384, 256, 8, 2, ()),
    (64, 72, 8, 16, 5, 3, (0, 4)),
])
def test_gated_backward_contiguous(T, K, F, N, E, k, empty):
    g = _small(T, K, F, N, E, k, seed=T + 2 * K, empty=empty)
    dY = _dy(g, T)
    log(f"gated bwd T={T} K={K} F={F} N={N} E={E} k={k} empty={empty}")
    dX, dWgu, dWd, dT = _bwd(g, dY)
    rx, rgu, rd, rt = O.gated_ffn_backward(dY.values, g.x.values, g.W_gu.values, g.W_down.values,
                                           g.expert_ids, g.topk_weights, E, round_h=True)
    ex = O.gated_ffn_backward(dY.values, g.x.values, g.W_gu.values, g.W_down.values,
                              g.expert_ids, g.topk_weights, E)
    _margins(zip(("dX", "dW_gu", "dW_down", "d_topk"), (dX, dWgu, dWd, dT), ex, (rx, rgu, rd, rt)))
    assert_close(dX, ex[0], "bf16", "dX")
    assert_close(dWgu, ex[1], "bf16", "dW_gu")
    assert_close(dWd, rd, "bf16", "dW_down (h as stored, bf16)")
    assert_close(dT, ex[3], "bf16", "d_topk")
    for e in empty:
        assert (dWgu[e] == 0).all() and (dWd[e] == 0).all()


@pytest.mark.parametrize("T,K,F,N,E,k,cap", [
    (128, 512, 256, 384, 16, 4, 64),
    (97, 128, 136, 64, 11, 4, 3),        # overflow: dropped assignments get nothing
    (300, 96, 128, 128, 6, 2, 130),
])
def test_gated_backward_masked(T, K, F, N, E, k, cap):
    g = _small(T, K, F, N, E, k, seed=T + 3 * cap)
    dY = _dy(g, cap)
    log(f"gated bwd masked T={T} K={K} F={F} N={N} E={E} k={k} cap={cap}")
    dX, dWgu, dWd, dT = _bwd(g, dY, api.MOE_LAYOUT_MASKED, cap)
    ms = O.masked_schedule(g.expert_ids, g.topk_weights, E, cap)
    kept = np.full(T * k, -1, dtype=np.int32)        # ids of the assignments that hold a slot
    flat = g.expert_ids.reshape(-1)
    for s in ms.slot_assign[ms.slot_assign >= 0]:
        kept[s] = flat[s]
    rx, rgu, rd, rt = O.gated_ffn_backward(dY.values, g.x.values, g.W_gu.values, g.W_down.values,
                                           kept.reshape(T, k), g.topk_weights, E, round_h=True)
    ex = O.gated_ffn_backward(dY.values, g.x.values, g.W_gu.values, g.W_down.values,
                              kept.reshape(T, k), g.topk_weights, E)
    _margins(zip(("dX", "dW_gu", "dW_down", "d_topk"), (dX, dWgu, dWd, dT), ex, (rx, rgu, rd, rt)))
    assert_close(dX, ex[0], "bf16", "dX")
    assert_close(dWgu, ex[1], "bf16", "dW_gu")
    assert_close(dWd, rd, "bf16", "dW_down (h as stored, bf16)")
    assert_close(dT, ex[3], "bf16", "d_topk")


def test_gated_backward_page_example_sampled():
    g = WL.gated_page_example()
    dY = _dy(g, 11)
    log(f"gated bwd full size {g.name}")
    dX, dWgu, dWd, dT = _bwd(g, dY)
    rng = np.random.default_rng(6)
    toks = np.sort(rng.choice(g.T, size=8, replace=False))
    rx, rt = O.gated_ffn_backward_rows(dY.values, g.x.values, g.W_gu.values, g.W_down.values,
                                       g.expert_ids, g.topk_weights, toks, round_h=True)
    ex, et = O.gated_ffn_backward_rows(dY.values, g.x.values, g.W_gu.values, g.W_down.values,
                                       g.expert_ids, g.topk_weights, toks)
    _margins([("dX sampled", dX[toks], ex, rx), ("d_topk sampled", dT[toks], et, rt)])
    assert_close(dX[toks], ex, "bf16", "dX sampled tokens")
    assert_close(dT[toks], et, "bf16", "d_topk sampled tokens")
    es = [int(e) for e in rng.choice(g.E, size=2, replace=False)]
    ge = [(e, int(j), int(kk)) for e in es for j, kk in zip(rng.integers(0, 2 * g.F, 16),
                                                             rng.integers(0, g.K, 16))]
    de = [(e, int(n), int(f)) for e in es for n, f in zip(rng.integers(0, g.N, 16),
                                                           rng.integers(0, g.F, 16))]
    rgu, rd = O.gated_weight_grad_entries(dY.values, g.x.values, g.W_gu.values, g.W_down.values,
                                          g.expert_ids, g.topk_weights, g.E, ge, de, round_h=True)
    egu, ed = O.gated_weight_grad_entries(dY.values, g.x.values, g.W_gu.values, g.W_down.values,
                                          g.expert_ids, g.topk_weights, g.E, ge, de)
    _margins([("dW_gu sampled", np.array([dWgu[i] for i in ge]), egu, rgu),
              ("dW_down sampled", np.array([dWd[i] for i in de]), ed, rd)])
    assert_close(np.array([dWgu[i] for i in ge]), egu, "bf16", "dW_gu sampled entries")
    assert_close(np.array([dWd[i] for i in de]), rd, "bf16", "dW_down sampled entries (h as stored)")
