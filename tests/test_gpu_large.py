"""Outputs past 2^31 and 2^32 bytes.

Inputs (x, dY, each expert's weight slice) are read through 32-bit buffer
offsets and stay below 2^31 bytes; the fp32 outputs y and dX are written by
the atomic scatter-combine with 64-bit addresses and may be larger.  Each
test compares sampled token rows, the last ones (the highest addresses)
among them, with the oracle's definition evaluated on those rows alone (the
forward and the input gradient of a token depend on that token's rows only).
The ranked combine reads outputs back with 32-bit offsets: forced, it refuses
a large output before launching anything.
"""
import numpy as np
import pytest
import torch

from moe_variable_size_amd import api
from moe_variable_size_amd import workloads as WL
from moe_variable_size_amd._lib import MoeError
from oracle import moe_oracle as O
from tests.gpu_util import assert_close, dev, host, log

pytestmark = pytest.mark.gpu


def _sample_tokens(T, seed):
    rng = np.random.default_rng(seed)
    body = rng.choice(T - 16, size=48, replace=False)
    return np.sort(np.concatenate([body, np.arange(T - 16, T)]))


@pytest.mark.parametrize("k", [1, 2])
def test_forward_output_past_4gib(k):
    """y [65536, 16448] fp32 = 4.31 GB: rows past byte 2^32 included.  With
    k = 1 the automatic combine would be the ranked one; at this size it takes
    the atomic scatter."""
    T, K, N, E = 65536, 64, 16448, 4
    r = WL.routed("y_past_4gib", T, K, N, E, k, seed=4242 + k, with_dy=False)
    assert T * N * 4 > 1 << 32
    log(f"forward T={T} K={K} N={N} E={E} k={k}: y {T * N * 4 / 1e9:.2f} GB")
    sch = api.moe_build_schedule(dev(r.expert_ids), dev(r.topk_weights), E)
    y = api.moe_fused_fwd(dev(r.x), dev(r.W), sch)
    torch.cuda.synchronize()
    toks = _sample_tokens(T, 7 + k)
    got = y[torch.from_numpy(toks).cuda()].cpu().numpy()
    del y
    ref = O.moe_forward(r.x.values[toks], r.W.values, r.expert_ids[toks], r.topk_weights[toks], E)
    assert_close(got, ref, "bf16", f"y rows (k={k})")


def test_input_grad_output_past_2gib():
    """dX [65536, 8200] fp32 = 2.15 GB (x itself, bf16, stays below 2^31
    bytes).  Only dX is asked for, so x is not read."""
    T, K, N, E, k = 65536, 8200, 64, 4, 2
    r = WL.routed("dx_past_2gib", T, K, N, E, k, seed=4343, with_x=False)
    assert T * K * 4 > 1 << 31 and T * K * 2 < 1 << 31
    log(f"input gradient T={T} K={K} N={N} E={E} k={k}: dX {T * K * 4 / 1e9:.2f} GB")
    sch = api.moe_build_schedule(dev(r.expert_ids), dev(r.topk_weights), E)
    x = torch.zeros((T, K), dtype=torch.bfloat16, device="cuda")
    dX, _, _ = api.moe_fused_bwd(dev(r.dY), x, dev(r.W), sch, dw=False, dtopk=False)
    torch.cuda.synchronize()
    toks = _sample_tokens(T, 11)
    got = dX[torch.from_numpy(toks).cuda()].cpu().numpy()
    del dX, x
    rx, _, _ = O.moe_backward(r.dY.values[toks], np.zeros((toks.size, K), np.float32), r.W.values,
                              r.expert_ids[toks], r.topk_weights[toks], E, dw_experts=[])
    assert_close(got, rx, "bf16", "dX rows")


def test_forced_ranked_refuses_large_output():
    """Ranked combine forced and y of 2^31 bytes or more: MOE_ERR_LIMIT before
    any launch; the atomic combine takes the same call."""
    T, K, N, E, k = 65536, 64, 8256, 4, 1
    r = WL.routed("ranked_large", T, K, N, E, k, seed=4444, with_dy=False)
    assert T * N * 4 >= 1 << 31
    ids, w = dev(r.expert_ids), dev(r.topk_weights)
    try:
        api.moe_set_combine(api.MOE_COMBINE_RANKED)
        sch = api.moe_build_schedule(ids, w, E)
        assert sch.phases == k
        with pytest.raises(MoeError) as ei:
            api.moe_fused_fwd(dev(r.x), dev(r.W), sch)
        assert ei.value.status == 7
        api.moe_set_combine(api.MOE_COMBINE_ATOMIC)
        y = api.moe_fused_fwd(dev(r.x), dev(r.W), sch)
        torch.cuda.synchronize()
    finally:
        api.moe_set_combine(api.MOE_COMBINE_AUTO)
    toks = _sample_tokens(T, 13)
    got = y[torch.from_numpy(toks).cuda()].cpu().numpy()
    del y
    ref = O.moe_forward(r.x.values[toks], r.W.values, r.expert_ids[toks], r.topk_weights[toks], E)
    assert_close(got, ref, "bf16", "y rows (atomic)")
