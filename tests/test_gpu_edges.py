"""Degenerate shapes on the GPU for the later entry points (gated FFN forward
and backward, 8-bit forward): one token, one expert, the smallest reduction,
one output column, mostly empty experts.  Oracle as in the other parity tests."""
import numpy as np
import pytest
import torch

from moe_variable_size_amd import api
from moe_variable_size_amd import workloads as WL
from oracle import moe_oracle as O
from tests.gpu_util import assert_close, dev, host, log

pytestmark = pytest.mark.gpu


def _ids(T, E, k, live, seed):
    rng = np.random.default_rng(seed)
    return np.array([rng.choice(live, size=k, replace=False) for _ in range(T)], dtype=np.int32)


@pytest.mark.parametrize("T,K,F,N,E,k,live", [
    (1, 8, 8, 8, 1, 1, [0]),               # one token, one expert, one 8-wide stage
    (48, 16, 8, 24, 6, 2, [1, 4]),         # four of six experts empty (the two live ones get
                                           # 48 rows each: with only a few rows a dW entry is a
                                           # sum of a few products and its two bf16 roundings,
                                           # w*dY and the output, do not average below 3e-3)
    (5, 200, 16, 8, 3, 3, [0, 1, 2]),      # k = E: every token in every expert
])
def test_gated_edges(T, K, F, N, E, k, live):
    g = WL.gated("edge_gated", T, K, F, N, E, k, seed=T * 7 + K)
    g.expert_ids = _ids(T, E, k, live, T + K)
    rng = np.random.default_rng(T)
    dY = WL._make(rng.standard_normal((T, N), dtype=np.float32), True)
    log(f"gated edge T={T} K={K} F={F} N={N} E={E} k={k}")
    sch = api.moe_build_schedule(dev(g.expert_ids), dev(g.topk_weights), E)
    y, h, gu = api.moe_gated_ffn_fwd(dev(g.x), dev(g.W_gu), dev(g.W_down), sch, save_gu=True)
    dX, dWgu, dWd, dT = api.moe_gated_ffn_bwd(dev(dY), dev(g.x), dev(g.W_gu), dev(g.W_down), sch,
                                              gu, h)
    torch.cuda.synchronize()
    ry = O.gated_ffn_forward(g.x.values, g.W_gu.values, g.W_down.values, g.expert_ids,
                             g.topk_weights, E, round_h=True)
    assert_close(host(y), ry, "bf16", "y")
    rx, rgu, rd, rt = O.gated_ffn_backward(dY.values, g.x.values, g.W_gu.values, g.W_down.values,
                                           g.expert_ids, g.topk_weights, E, round_h=True)
    assert_close(host(dX), rx, "bf16", "dX")
    assert_close(host(dWgu), rgu, "bf16", "dW_gu")
    assert_close(host(dWd), rd, "bf16", "dW_down")
    assert_close(host(dT), rt, "bf16", "d_topk")
    for e in range(E):
        if e not in live:
            assert (host(dWgu)[e] == 0).all() and (host(dWd)[e] == 0).all()


@pytest.mark.parametrize("T,K,N,E,k,live", [
    (1, 16, 1, 1, 1, [0]),                 # one token, one expert, one output column
    (7, 16, 40, 9, 2, [2, 8]),
    (64, 4096, 8, 4, 4, [0, 1, 2, 3]),     # long reduction, narrow output
])
def test_fp8_edges(T, K, N, E, k, live):
    r = WL.routed("edge_fp8", T, K, N, E, k, seed=T + K + N)
    r.expert_ids = _ids(T, E, k, live, T * 3 + N)
    f = WL.fp8_routed(r)
    log(f"fp8 edge T={T} K={K} N={N} E={E} k={k}")
    sch = api.moe_build_schedule(dev(f.expert_ids), dev(f.topk_weights), E)
    u8 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    y = api.moe_fused_fwd_fp8(u8(f.xq), u8(f.x_scale), u8(f.Wq), u8(f.w_scale), sch)
    torch.cuda.synchronize()
    ref = O.moe_forward_fp8(f.xq, f.x_scale, f.Wq, f.w_scale, f.expert_ids, f.topk_weights, E)
    assert_close(host(y), ref, "f32", "y")
