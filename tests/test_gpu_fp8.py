"""GPU parity of the 8-bit forward (moe_fused_fwd_fp8) against the oracle.

Both sides read the same E4M3 codes and scales; products of two E4M3 values
are exact in fp32, so the only differences are fp32 accumulation order and the
atomic combine: the fp32 bar applies (max relative error <= 1e-4, normwise).
"""
import numpy as np
import pytest
import torch

from moe_variable_size_amd import api
from moe_variable_size_amd import workloads as WL
from oracle import moe_oracle as O
from tests.gpu_util import assert_close, dev, host, log

pytestmark = pytest.mark.gpu


def _u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _run(f, layout=api.MOE_LAYOUT_CONTIGUOUS, cap=0):
    sch = api.moe_build_schedule(dev(f.expert_ids), dev(f.topk_weights), f.E, layout=layout,
                                 capacity=cap)
    y0 = torch.full((f.T, f.N), float("nan"), dtype=torch.float32, device="cuda")  # overwritten
    y = api.moe_fused_fwd_fp8(_u8(f.xq), _u8(f.x_scale), _u8(f.Wq), _u8(f.w_scale), sch, y=y0)
    torch.cuda.synchronize()
    return sch, host(y)


def _small(T, K, N, E, k, seed, empty=(), cap=0):
    r = WL.routed("small_fp8", T, K, N, E, k, seed=seed, capacity=cap)
    if empty:
        live = [e for e in range(E) if e not in empty]
        rng = np.random.default_rng(seed)
        r.expert_ids = np.array([rng.choice(live, size=k, replace=False) for _ in range(T)],
                                dtype=np.int32)
    return WL.fp8_routed(r)


@pytest.mark.parametrize("T,K,N,E,k,empty", [
    (333, 144, 200, 7, 2, (3,)),     # two stages, the second 16 bytes deep; ragged N; empty expert
    (129, 128, 192, 3, 1, ()),
    (1030, 512, 768, 8, 2, ()),      # 51 tiles of 128 x 256: 4-way split of the last round
    (4000, 256, 520, 8, 2, ()),      # several rounds, partial last column block
])
def test_fp8_contiguous(T, K, N, E, k, empty):
    f = _small(T, K, N, E, k, seed=T + K, empty=empty)
    log(f"fp8 fwd T={T} K={K} N={N} E={E} k={k} empty={empty}")
    _, y = _run(f)
    ref = O.moe_forward_fp8(f.xq, f.x_scale, f.Wq, f.w_scale, f.expert_ids, f.topk_weights, E)
    assert_close(y, ref, "f32", "y")


@pytest.mark.parametrize("T,K,N,E,k,cap", [
    (128, 512, 384, 16, 4, 64),      # 64-row decode tiles
    (97, 128, 136, 11, 4, 3),        # overflowing capacity
    (300, 96 + 16, 128, 6, 2, 130),  # capacity above 64: 128-row tiles
])
def test_fp8_masked(T, K, N, E, k, cap):
    f = _small(T, K, N, E, k, seed=T + cap, cap=cap)
    log(f"fp8 masked T={T} K={K} N={N} E={E} k={k} cap={cap}")
    sch, y = _run(f, api.MOE_LAYOUT_MASKED, cap)
    ms = O.masked_schedule(f.expert_ids, f.topk_weights, E, cap)
    ref = O.masked_forward_fp8(f.xq, f.x_scale, f.Wq, f.w_scale, ms, T)
    assert_close(y, ref, "f32", "masked y")
    assert int(sch.status[1].item()) == ms.n_dropped


def test_fp8_config2():
    f = WL.fp8_routed(WL.config2(with_dy=False))
    log(f"fp8 fwd {f.name}")
    _, y = _run(f)
    ref = O.moe_forward_fp8(f.xq, f.x_scale, f.Wq, f.w_scale, f.expert_ids, f.topk_weights, f.E)
    assert_close(y, ref, "f32", "config2 fp8 y")


def test_fp8_config5_decode():
    r = WL.config5()
    f = WL.fp8_routed(r)
    log(f"fp8 decode {f.name}")
    _, y = _run(f, api.MOE_LAYOUT_MASKED, r.capacity)
    ms = O.masked_schedule(f.expert_ids, f.topk_weights, f.E, r.capacity)
    ref = O.masked_forward_fp8(f.xq, f.x_scale, f.Wq, f.w_scale, ms, f.T)
    assert_close(y, ref, "f32", "config5 fp8 y")


# ----------------------------------------------------------------------------
# per-block (E8M0, 32 elements) scales
# ----------------------------------------------------------------------------
def _run_mx(f, layout=api.MOE_LAYOUT_CONTIGUOUS, cap=0):
    sch = api.moe_build_schedule(dev(f.expert_ids), dev(f.topk_weights), f.E, layout=layout,
                                 capacity=cap)
    y0 = torch.full((f.T, f.N), float("nan"), dtype=torch.float32, device="cuda")  # overwritten
    y = api.moe_fused_fwd_mx(_u8(f.xq), _u8(f.x_bs), _u8(f.Wq), _u8(f.w_bs), sch, y=y0)
    torch.cuda.synchronize()
    return sch, host(y)


@pytest.mark.parametrize("T,K,N,E,k,empty", [
    (333, 256, 200, 7, 2, (3,)),
    (1030, 512, 768, 8, 2, ()),
    (4000, 128, 520, 8, 2, ()),
])
def test_mx_contiguous(T, K, N, E, k, empty):
    r = WL.routed("small_mx", T, K, N, E, k, seed=T + 5 * K)
    if empty:
        live = [e for e in range(E) if e not in empty]
        rng = np.random.default_rng(T)
        r.expert_ids = np.array([rng.choice(live, size=k, replace=False) for _ in range(T)],
                                dtype=np.int32)
    f = WL.mx_routed(r)
    log(f"mx fwd T={T} K={K} N={N} E={E} k={k} empty={empty}")
    _, y = _run_mx(f)
    ref = O.moe_forward_mx(f.xq, f.x_bs, f.Wq, f.w_bs, f.expert_ids, f.topk_weights, E)
    assert_close(y, ref, "f32", "y")


@pytest.mark.parametrize("T,K,N,E,k,cap", [(128, 512, 384, 16, 4, 64), (97, 128, 136, 11, 4, 3)])
def test_mx_masked(T, K, N, E, k, cap):
    r = WL.routed("small_mx", T, K, N, E, k, seed=T + cap, capacity=cap)
    f = WL.mx_routed(r)
    log(f"mx masked T={T} K={K} N={N} E={E} k={k} cap={cap}")
    sch, y = _run_mx(f, api.MOE_LAYOUT_MASKED, cap)
    ms = O.masked_schedule(f.expert_ids, f.topk_weights, E, cap)
    ref = O.masked_forward_mx(f.xq, f.x_bs, f.Wq, f.w_bs, ms, T)
    assert_close(y, ref, "f32", "masked y")


def test_mx_config2():
    f = WL.mx_routed(WL.config2(with_dy=False))
    log(f"mx fwd {f.name}")
    _, y = _run_mx(f)
    ref = O.moe_forward_mx(f.xq, f.x_bs, f.Wq, f.w_bs, f.expert_ids, f.topk_weights, f.E)
    assert_close(y, ref, "f32", "config2 mx y")


def test_mx_config5_decode():
    r = WL.config5()
    f = WL.mx_routed(r)
    log(f"mx decode {f.name}")
    _, y = _run_mx(f, api.MOE_LAYOUT_MASKED, r.capacity)
    ms = O.masked_schedule(f.expert_ids, f.topk_weights, f.E, r.capacity)
    ref = O.masked_forward_mx(f.xq, f.x_bs, f.Wq, f.w_bs, ms, f.T)
    assert_close(y, ref, "f32", "config5 mx y")
