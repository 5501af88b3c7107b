"""GPU parity of the gated expert FFN on its vector-ALU path: fp32 inputs, and
bf16 inputs whose K, F or N is not a multiple of 8.

fp32: the intermediate h stays fp32, so every result is compared with the
exact (float64) oracle at the fp32 tolerances (max relative error <= 1e-4,
see tests/gpu_util.py).  bf16 with odd sizes: as on the matrix-core path, h
is stored bf16, so dW_down is compared with the oracle that rounds h where it
forms it, everything else with the exact oracle at the bf16 tolerances.
Empty masked slots of h keep a sentinel.
"""
import numpy as np
import pytest
import torch

from moe_variable_size_amd import api
from moe_variable_size_amd import workloads as WL
from oracle import moe_oracle as O
from tests.gpu_util import assert_close, dev, host, log

pytestmark = pytest.mark.gpu

SENTINEL = 7.0


def _case(T, K, F, N, E, k, seed, bf16, empty=()):
    g = WL.gated("gated_generic", T, K, F, N, E, k, seed=seed, bf16=bf16)
    if empty:
        live = [e for e in range(E) if e not in empty]
        rng = np.random.default_rng(seed)
        g.expert_ids = np.array([rng.choice(live, size=k, replace=False) for _ in range(T)],
                                dtype=np.int32)
    rng = np.random.default_rng(seed + 1)
    dY = WL._make(rng.standard_normal((T, N), dtype=np.float32), bf16)
    return g, dY


def _run(g, dY, bf16, layout=api.MOE_LAYOUT_CONTIGUOUS, cap=0):
    sch = api.moe_build_schedule(dev(g.expert_ids), dev(g.topk_weights), g.E, layout=layout,
                                 capacity=cap)
    dt = torch.bfloat16 if bf16 else torch.float32
    h0 = torch.full((sch.c.R, g.F), SENTINEL, dtype=dt, device="cuda")
    y, h, gu = api.moe_gated_ffn_fwd(dev(g.x, bf16), dev(g.W_gu, bf16), dev(g.W_down, bf16), sch,
                                     h=h0, save_gu=True)
    dX, dWgu, dWd, dT = api.moe_gated_ffn_bwd(dev(dY, bf16), dev(g.x, bf16), dev(g.W_gu, bf16),
                                              dev(g.W_down, bf16), sch, gu, h)
    torch.cuda.synchronize()
    return [host(t) for t in (y, h, dX, dWgu, dWd, dT)]


@pytest.mark.parametrize("T,K,F,N,E,k,bf16,empty", [
    (333, 37, 13, 29, 7, 2, False, (3,)),     # fp32, every size odd, an empty expert
    (400, 136, 200, 72, 5, 2, False, ()),     # fp32, sizes the matrix cores would take
    (129, 300, 70, 130, 3, 1, False, ()),     # fp32, several tiles each way
    (64, 72, 8, 16, 5, 3, False, (0, 4)),
    (333, 37, 13, 29, 7, 2, True, (3,)),      # bf16, odd sizes
    (200, 136, 100, 70, 6, 2, True, ()),      # bf16, F and N not multiples of 8
])
def test_gated_generic_contiguous(T, K, F, N, E, k, bf16, empty):
    g, dY = _case(T, K, F, N, E, k, seed=T + K + F + N, bf16=bf16, empty=empty)
    log(f"gated generic T={T} K={K} F={F} N={N} E={E} k={k} bf16={bf16} empty={empty}")
    y, h, dX, dWgu, dWd, dT = _run(g, dY, bf16)
    tol = "bf16" if bf16 else "f32"
    ref_y = O.gated_ffn_forward(g.x.values, g.W_gu.values, g.W_down.values, g.expert_ids,
                                g.topk_weights, E)
    ref_h = O.gated_intermediate(g.x.values, g.W_gu.values, g.expert_ids, E)
    assert_close(h, ref_h, tol, "h")
    assert_close(y, ref_y, tol, "y")
    ex = O.gated_ffn_backward(dY.values, g.x.values, g.W_gu.values, g.W_down.values,
                              g.expert_ids, g.topk_weights, E)
    rd = O.gated_ffn_backward(dY.values, g.x.values, g.W_gu.values, g.W_down.values,
                              g.expert_ids, g.topk_weights, E, round_h=True)[2] if bf16 else ex[2]
    assert_close(dX, ex[0], tol, "dX")
    assert_close(dWgu, ex[1], tol, "dW_gu")
    assert_close(dWd, rd, tol, "dW_down")
    assert_close(dT, ex[3], tol, "d_topk")
    for e in empty:
        assert (dWgu[e] == 0).all() and (dWd[e] == 0).all()


@pytest.mark.parametrize("T,K,F,N,E,k,cap", [
    (97, 44, 21, 35, 11, 4, 3),        # overflowing capacity
    (300, 96, 40, 50, 6, 2, 130),
])
def test_gated_generic_masked_fp32(T, K, F, N, E, k, cap):
    g, dY = _case(T, K, F, N, E, k, seed=T + cap, bf16=False)
    log(f"gated generic masked T={T} K={K} F={F} N={N} E={E} k={k} cap={cap}")
    y, h, dX, dWgu, dWd, dT = _run(g, dY, False, api.MOE_LAYOUT_MASKED, cap)
    ms = O.masked_schedule(g.expert_ids, g.topk_weights, E, cap)
    ref_y, ref_h = O.masked_gated_ffn(g.x.values, g.W_gu.values, g.W_down.values, ms, T)
    valid = ms.slot_assign.reshape(-1) >= 0
    assert_close(h[valid], ref_h[valid], "f32", "h valid slots")
    assert (h[~valid] == SENTINEL).all(), "empty slots of h were written"
    assert_close(y, ref_y, "f32", "y")
    kept = np.full(T * k, -1, dtype=np.int32)
    flat = g.expert_ids.reshape(-1)
    for s in ms.slot_assign[ms.slot_assign >= 0]:
        kept[s] = flat[s]
    ex = O.gated_ffn_backward(dY.values, g.x.values, g.W_gu.values, g.W_down.values,
                              kept.reshape(T, k), g.topk_weights, E)
    assert_close(dX, ex[0], "f32", "dX")
    assert_close(dWgu, ex[1], "f32", "dW_gu")
    assert_close(dWd, ex[2], "f32", "dW_down")
    assert_close(dT, ex[3], "f32", "d_topk")
