"""GPU parity of the gated expert FFN (moe_gated_ffn_fwd) against the oracle.

The intermediate h (bf16, schedule row order) and the output y (fp32) are both
compared, with the bf16 tolerances: max relative error <= 1e-2 and relative
Frobenius error <= 3e-3 (normwise).  Rows of h the call must not write keep a
sentinel.
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
    y, h = api.moe_gated_ffn_fwd(dev(g.x), dev(g.W_gu), dev(g.W_down), sch, h=h0)
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
