"""Seeded sweep of ragged shapes through the fused forward and backward.

Each case draws T, K, N (multiples of 8, rarely of a tile), E, k, empty
experts, routing weights or none, and the layout (contiguous, or masked with a
capacity that may drop assignments) from its own seed, runs schedule +
forward + backward on the GPU and compares y, dX, dW and d_topk with the
oracle's definitions.  With the masked layout the reference routing keeps
only the assignments that hold a slot (the oracle's masked schedule decides
which), the others contributing nothing.
"""
import numpy as np
import pytest
import torch

from moe_variable_size_amd import api
from moe_variable_size_amd import workloads as WL
from oracle import moe_oracle as O
from tests.gpu_util import assert_close, dev, host, log

pytestmark = pytest.mark.gpu


def _case(seed):
    rng = np.random.default_rng(9000 + seed)
    T = int(rng.integers(1, 700))
    K = 8 * int(rng.integers(1, 72))
    N = 8 * int(rng.integers(1, 72))
    E = int(rng.integers(1, 40))
    k = int(rng.integers(1, min(E, 8) + 1))
    masked = bool(rng.random() < 0.3)
    weighted = bool(rng.random() < 0.8)
    n_empty = int(rng.integers(0, max(1, E - k) + 1)) if E > k else 0
    empty = tuple(sorted(int(e) for e in rng.choice(E, size=n_empty, replace=False)))
    cap = int(rng.integers(1, 2 * max(1, T * k // max(1, E - len(empty))) + 2)) if masked else 0
    return T, K, N, E, k, masked, weighted, empty, cap


@pytest.mark.parametrize("seed", range(20))
def test_sweep(seed):
    T, K, N, E, k, masked, weighted, empty, cap = _case(seed)
    r = WL.routed(f"sweep{seed}", T, K, N, E, k, seed=7000 + seed,
                  weights="uniform" if weighted else "ones")
    if empty:
        live = [e for e in range(E) if e not in empty]
        rng = np.random.default_rng(seed)
        r.expert_ids = np.array([rng.choice(live, size=k, replace=False) for _ in range(T)], dtype=np.int32)
    layout = api.MOE_LAYOUT_MASKED if masked else api.MOE_LAYOUT_CONTIGUOUS
    log(f"sweep seed={seed}: T={T} K={K} N={N} E={E} k={k} empty={empty} "
        f"weighted={weighted} masked={masked} cap={cap}")
    tw = None if r.topk_weights is None else dev(r.topk_weights)
    sch = api.moe_build_schedule(dev(r.expert_ids), tw, E, layout=layout, capacity=cap)
    y = api.moe_fused_fwd(dev(r.x), dev(r.W), sch)
    dX, dW, dT = api.moe_fused_bwd(dev(r.dY), dev(r.x), dev(r.W), sch)
    torch.cuda.synchronize()
    ids = r.expert_ids
    if masked:
        ms = O.masked_schedule(r.expert_ids, r.topk_weights, E, cap)
        kept = np.full(T * k, -1, dtype=np.int32)
        flat = r.expert_ids.reshape(-1)
        for s in ms.slot_assign[ms.slot_assign >= 0]:
            kept[s] = flat[s]
        ids = kept.reshape(T, k)
        assert int(sch.status[1].item()) == ms.n_dropped
    ref_y = O.moe_forward(r.x.values, r.W.values, ids, r.topk_weights, E)
    rx, rw, rt = O.moe_backward(r.dY.values, r.x.values, r.W.values, ids, r.topk_weights, E)
    assert_close(host(y), ref_y, "bf16", "y")
    assert_close(host(dX), rx, "bf16", "dX")
    assert_close(host(dW), rw, "bf16", "dW")
    assert_close(host(dT), rt, "bf16", "d_topk")
    counts = np.bincount(ids[ids >= 0].ravel(), minlength=E)
    got_dw = host(dW)
    for e in np.nonzero(counts == 0)[0]:
        assert (got_dw[e] == 0).all(), f"dW[{e}] of an expert without rows"
