"""The two ways the fused forward and the input gradient combine a token's k
contributions, each forced and checked against the oracle: atomic adds into a
zeroed output, and the ranked combine over the schedule's rank-ordered view
(one launch; rank 0 stores, a later rank waits for the earlier one in its
column block, then reads, adds and stores; the counters must be back at zero
and no wait may have given up).  Cases cover k = 1..4,
ids outside [0, E) (tokens with some or all slots excluded), empty experts,
ragged K and N, sub-tiles of a last partial round and the config-2 layer."""
import numpy as np
import pytest
import torch

from moe_variable_size_amd import api
from moe_variable_size_amd import workloads as WL
from oracle import moe_oracle as O
from tests.gpu_util import assert_close, dev, host, log

pytestmark = pytest.mark.gpu

MODES = {"atomic": api.MOE_COMBINE_ATOMIC, "ranked": api.MOE_COMBINE_RANKED}


def _case(T, K, N, E, k, seed, bad=0.0):
    r = WL.routed("combine_case", T, K, N, E, k, seed=seed)
    if bad:
        rng = np.random.default_rng(seed + 1)
        ids = r.expert_ids.copy()
        ids[rng.random(ids.shape) < bad] = E + 2      # excluded: some tokens keep no slot
        r.expert_ids = ids
    return r


def _run(r, mode):
    api.moe_set_combine(MODES[mode])
    try:
        sch = api.moe_build_schedule(dev(r.expert_ids), dev(r.topk_weights), r.E)
        y = torch.full((r.T, r.N), float("nan"), dtype=torch.float32, device="cuda")
        dX = torch.full((r.T, r.K), float("nan"), dtype=torch.float32, device="cuda")
        dT = torch.full((r.T, r.k), float("nan"), dtype=torch.float32, device="cuda")
        api.moe_fused_fwd(dev(r.x), dev(r.W), sch, y=y)
        _, dW, _ = api.moe_fused_bwd(dev(r.dY), dev(r.x), dev(r.W), sch, out_dX=dX, out_dtopk=dT)
        torch.cuda.synchronize()
    finally:
        api.moe_set_combine(api.MOE_COMBINE_AUTO)
    # the view is built only when the mode at build time can use it
    if mode == "ranked":
        assert sch.phases == r.k
        sync = sch.phase_sync.cpu().numpy()
        assert (sync == 0).all(), f"ranked counters not reset / waits gave up: {np.nonzero(sync)[0][:8]}"
    else:
        assert sch.phases == 0
    return host(y), host(dX), host(dW), host(dT)


@pytest.mark.parametrize("mode", ["atomic", "ranked"])
@pytest.mark.parametrize("T,K,N,E,k,bad", [
    (700, 256, 320, 6, 2, 0.0),
    (333, 136, 200, 7, 3, 0.0),          # ragged K and N, three ranks
    (129, 128, 192, 3, 1, 0.0),          # one rank: stores only
    (901, 264, 136, 9, 4, 0.25),         # excluded ids: ranks shift, some tokens keep none
    (2000, 1536, 256, 8, 2, 0.0),        # sub-tiles of the last partial round
])
def test_combine_modes_match_oracle(mode, T, K, N, E, k, bad):
    r = _case(T, K, N, E, k, seed=T + K, bad=bad)
    log(f"combine {mode} T={T} K={K} N={N} E={E} k={k} bad={bad}")
    y, dX, dW, dT = _run(r, mode)
    ry = O.moe_forward(r.x.values, r.W.values, r.expert_ids, r.topk_weights, E)
    rx, rW, rt = O.moe_backward(r.dY.values, r.x.values, r.W.values, r.expert_ids, r.topk_weights, E)
    valid = (r.expert_ids >= 0) & (r.expert_ids < E)
    rt = np.where(valid, rt, 0.0)                     # excluded assignments get 0
    assert_close(y, ry, "bf16", "y")
    assert_close(dX, rx, "bf16", "dX")
    assert_close(dW, rW, "bf16", "dW")
    assert_close(dT, rt, "bf16", "d_topk")
    dead = ~valid.any(axis=1)
    if dead.any():
        assert (y[dead] == 0).all() and (dX[dead] == 0).all()


def test_combine_modes_agree_on_config2():
    """The config-2 layer both ways: each within the bf16 bar of the oracle;
    with k = 2 the two fp32 sums 0 + a + b and a + b are the same number, so
    the two modes agree to the products' own rounding."""
    r = WL.config2()
    log(f"combine both modes {r.name}")
    ya, xa, Wa, ta = _run(r, "atomic")
    yr, xr, Wr, tr = _run(r, "ranked")
    ry = O.moe_forward(r.x.values, r.W.values, r.expert_ids, r.topk_weights, r.E)
    assert_close(ya, ry, "bf16", "y atomic")
    assert_close(yr, ry, "bf16", "y ranked")
    assert_close(yr, ya.astype(np.float64), "f32", "y ranked vs atomic")
    assert_close(xr, xa.astype(np.float64), "f32", "dX ranked vs atomic")
    assert_close(tr, ta.astype(np.float64), "f32", "d_topk ranked vs atomic")


def test_ranked_forward_is_deterministic():
    """Rank order fixes the fp32 summation order: two runs are bit-identical
    (k = 4)."""
    r = _case(1500, 512, 384, 12, 4, seed=77)
    a = _run(r, "ranked")
    b = _run(r, "ranked")
    assert np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32))
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
