"""Per-launch choice of the tile height on the device: workloads of small
experts, where the routed kernels take 128-row tiles, checked against the
oracle in the forward, the backward and the gated FFN.

The choice is made inside the kernels from the schedule's row-block totals;
the test states which height the estimate picks for each case (256-row tiles
estimate rb256 * tiles_n / G rounds, 128-row tiles 0.75 * rb128 * tiles_n / G,
each at least one round) so that the cases cover the 128-row path with whole
tiles and with its 2- and 4-way splits of a last partial round.
"""
import numpy as np
import pytest
import torch

from moe_variable_size_amd import api
from moe_variable_size_amd import workloads as WL
from oracle import moe_oracle as O
from tests.gpu_util import assert_close, dev, host, log

pytestmark = pytest.mark.gpu

G = 256   # persistent workgroups (one per compute unit of an MI355X)


def _picks_128(counts, ncols):
    tn = -(-ncols // 256)
    rb256 = int((-(-counts // 256)).sum())
    rb128 = int((-(-counts // 128)).sum())
    return 0.75 * max(rb128 * tn / G, 1.0) < max(rb256 * tn / G, 1.0), rb128 * tn


# (T, K, N, E, k): ~T*k/E rows per expert, all below 128
CASES = [
    (1536, 256, 768, 40, 2),    # forward 120 tiles of 128 x 256 (2-way split), dX 40 (4-way)
    (640, 512, 256, 40, 3),     # forward 40 tiles (4-way split), dX 80 (2-way)
    (3200, 384, 2560, 64, 2),   # forward 640 tiles: two rounds and a split last round
]


@pytest.mark.parametrize("T,K,N,E,k", CASES)
def test_small_experts_forward_and_backward(T, K, N, E, k):
    r = WL.routed("small_experts", T, K, N, E, k, seed=T + E, weights="uniform")
    counts = np.bincount(r.expert_ids.ravel(), minlength=E)
    assert counts.max() <= 128
    for ncols in (N, K):
        pick, tiles = _picks_128(counts, ncols)
        assert pick, (ncols, tiles)
    log(f"small experts T={T} K={K} N={N} E={E} k={k}")
    sch = api.moe_build_schedule(dev(r.expert_ids), dev(r.topk_weights), E)
    y = api.moe_fused_fwd(dev(r.x), dev(r.W), sch)
    dX, dW, dT = api.moe_fused_bwd(dev(r.dY), dev(r.x), dev(r.W), sch)
    torch.cuda.synchronize()
    assert_close(host(y), O.moe_forward(r.x.values, r.W.values, r.expert_ids, r.topk_weights, E),
                 "bf16", "y")
    rx, rw, rt = O.moe_backward(r.dY.values, r.x.values, r.W.values, r.expert_ids, r.topk_weights, E)
    assert_close(host(dX), rx, "bf16", "dX")
    assert_close(host(dW), rw, "bf16", "dW")
    assert_close(host(dT), rt, "bf16", "d_topk")


def test_small_experts_gated():
    T, K, F, N, E, k = 1536, 256, 384, 256, 40, 2
    g = WL.gated("small_experts_gated", T, K, F, N, E, k, seed=5)
    counts = np.bincount(g.expert_ids.ravel(), minlength=E)
    assert _picks_128(counts, N)[0]
    log(f"small experts gated T={T} K={K} F={F} N={N} E={E}")
    sch = api.moe_build_schedule(dev(g.expert_ids), dev(g.topk_weights), E)
    y, h = api.moe_gated_ffn_fwd(dev(g.x), dev(g.W_gu), dev(g.W_down), sch)
    torch.cuda.synchronize()
    assert_close(host(h), O.gated_intermediate(g.x.values, g.W_gu.values, g.expert_ids, E), "bf16", "h")
    assert_close(host(y), O.gated_ffn_forward(g.x.values, g.W_gu.values, g.W_down.values,
                                              g.expert_ids, g.topk_weights, E), "bf16", "y")
