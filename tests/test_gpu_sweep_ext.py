"""Seeded sweeps of ragged shapes through the 8-bit forwards, the gated FFN,
the bare grouped GEMM and the fp32 step.

Each case draws its sizes, expert count, top-k, experts left without rows and
the layout (contiguous, or masked with a capacity that may drop assignments)
from its own seed, runs the path on the GPU with its outputs prefilled with NaN
(every call overwrites them) and compares with the oracle:
  - E4M3 forward (per-token and per-channel scales): K a multiple of 16, any N;
  - block-scaled 8-bit forward (E8M0 per 32 elements): K a multiple of 128;
  - gated expert FFN forward and backward on the matrix cores (K, F, N
    multiples of 8): y and the gradients against the exact oracle, dW_down
    against the oracle with h rounded to bf16 as the call stores it.
With the masked layout the reference keeps only the assignments that hold a
slot (the oracle's masked schedule decides which).
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


def _routing(rng, T, E, k):
    """Top-k distinct experts per token drawn from the live ones (some experts
    may be left without rows), the layout and the capacity."""
    n_empty = int(rng.integers(0, E - k + 1)) if E > k else 0
    empty = sorted(int(e) for e in rng.choice(E, size=n_empty, replace=False))
    live = [e for e in range(E) if e not in empty]
    ids = np.array([rng.choice(live, size=k, replace=False) for _ in range(T)], dtype=np.int32)
    masked = bool(rng.random() < 0.35)
    cap = int(rng.integers(1, 2 * max(1, T * k // len(live)) + 2)) if masked else 0
    return ids, empty, masked, cap


def _kept(ids, weights, E, cap):
    """ids with the assignments that hold no masked slot set to -1."""
    ms = O.masked_schedule(ids, weights, E, cap)
    kept = np.full(ids.size, -1, dtype=np.int32)
    flat = ids.reshape(-1)
    for s in ms.slot_assign[ms.slot_assign >= 0]:
        kept[s] = flat[s]
    return ms, kept.reshape(ids.shape)


def _schedule(ids, weights, E, masked, cap):
    layout = api.MOE_LAYOUT_MASKED if masked else api.MOE_LAYOUT_CONTIGUOUS
    return api.moe_build_schedule(dev(ids), dev(weights), E, layout=layout, capacity=cap)


def _nan(shape):
    return torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")


@pytest.mark.parametrize("seed", range(10))
def test_sweep_fp8(seed):
    rng = np.random.default_rng(12000 + seed)
    T = int(rng.integers(1, 600))
    K = 16 * int(rng.integers(1, 40))
    N = int(rng.integers(1, 400))
    E = int(rng.integers(1, 33))
    k = int(rng.integers(1, min(E, 6) + 1))
    ids, empty, masked, cap = _routing(rng, T, E, k)
    r = WL.routed(f"sweep_fp8_{seed}", T, K, N, E, k, seed=12500 + seed, with_dy=False)
    r.expert_ids = ids
    f = WL.fp8_routed(r)
    log(f"fp8 sweep seed={seed}: T={T} K={K} N={N} E={E} k={k} empty={empty} masked={masked} cap={cap}")
    sch = _schedule(ids, f.topk_weights, E, masked, cap)
    y = api.moe_fused_fwd_fp8(_u8(f.xq), _u8(f.x_scale), _u8(f.Wq), _u8(f.w_scale), sch,
                              y=_nan((T, N)))
    torch.cuda.synchronize()
    if masked:
        ms, _ = _kept(ids, f.topk_weights, E, cap)
        ref = O.masked_forward_fp8(f.xq, f.x_scale, f.Wq, f.w_scale, ms, T)
        assert int(sch.status[1].item()) == ms.n_dropped
    else:
        ref = O.moe_forward_fp8(f.xq, f.x_scale, f.Wq, f.w_scale, ids, f.topk_weights, E)
    assert_close(host(y), ref, "f32", "y")


@pytest.mark.parametrize("seed", range(6))
def test_sweep_mx(seed):
    rng = np.random.default_rng(13000 + seed)
    T = int(rng.integers(1, 500))
    K = 128 * int(rng.integers(1, 5))
    N = int(rng.integers(1, 300))
    E = int(rng.integers(1, 25))
    k = int(rng.integers(1, min(E, 4) + 1))
    ids, empty, masked, cap = _routing(rng, T, E, k)
    r = WL.routed(f"sweep_mx_{seed}", T, K, N, E, k, seed=13500 + seed, with_dy=False)
    r.expert_ids = ids
    f = WL.mx_routed(r)
    log(f"mx sweep seed={seed}: T={T} K={K} N={N} E={E} k={k} empty={empty} masked={masked} cap={cap}")
    sch = _schedule(ids, f.topk_weights, E, masked, cap)
    y = api.moe_fused_fwd_mx(_u8(f.xq), _u8(f.x_bs), _u8(f.Wq), _u8(f.w_bs), sch, y=_nan((T, N)))
    torch.cuda.synchronize()
    if masked:
        ms, _ = _kept(ids, f.topk_weights, E, cap)
        ref = O.masked_forward_mx(f.xq, f.x_bs, f.Wq, f.w_bs, ms, T)
    else:
        ref = O.moe_forward_mx(f.xq, f.x_bs, f.Wq, f.w_bs, ids, f.topk_weights, E)
    assert_close(host(y), ref, "f32", "y")


@pytest.mark.parametrize("seed", range(6))
def test_sweep_gated(seed):
    rng = np.random.default_rng(14000 + seed)
    T = int(rng.integers(1, 400))
    K = 8 * int(rng.integers(1, 40))
    F = 8 * int(rng.integers(1, 40))
    N = 8 * int(rng.integers(1, 40))
    E = int(rng.integers(1, 20))
    k = int(rng.integers(1, min(E, 4) + 1))
    ids, empty, masked, cap = _routing(rng, T, E, k)
    g = WL.gated(f"sweep_gated_{seed}", T, K, F, N, E, k, seed=14500 + seed)
    g.expert_ids = ids
    dY = WL._make(np.random.default_rng(14900 + seed).standard_normal((T, N), dtype=np.float32), True)
    log(f"gated sweep seed={seed}: T={T} K={K} F={F} N={N} E={E} k={k} empty={empty} "
        f"masked={masked} cap={cap}")
    sch = _schedule(ids, g.topk_weights, E, masked, cap)
    y, h, gu = api.moe_gated_ffn_fwd(dev(g.x), dev(g.W_gu), dev(g.W_down), sch, save_gu=True,
                                     y=_nan((T, N)))
    dX, dWgu, dWd, dT = api.moe_gated_ffn_bwd(dev(dY), dev(g.x), dev(g.W_gu), dev(g.W_down), sch,
                                              gu, h)
    torch.cuda.synchronize()
    ref_ids = _kept(ids, g.topk_weights, E, cap)[1] if masked else ids
    ry = O.gated_ffn_forward(g.x.values, g.W_gu.values, g.W_down.values, ref_ids,
                             g.topk_weights, E)
    ex = O.gated_ffn_backward(dY.values, g.x.values, g.W_gu.values, g.W_down.values, ref_ids,
                              g.topk_weights, E)
    rd = O.gated_ffn_backward(dY.values, g.x.values, g.W_gu.values, g.W_down.values, ref_ids,
                              g.topk_weights, E, round_h=True)[2]
    assert_close(host(y), ry, "bf16", "y")
    assert_close(host(dX), ex[0], "bf16", "dX")
    assert_close(host(dWgu), ex[1], "bf16", "dW_gu")
    assert_close(host(dWd), rd, "bf16", "dW_down (h as stored, bf16)")
    assert_close(host(dT), ex[3], "bf16", "d_topk")
    counts = np.bincount(ref_ids[ref_ids >= 0].ravel(), minlength=E)
    got_gu, got_d = host(dWgu), host(dWd)
    for e in np.nonzero(counts == 0)[0]:
        assert (got_gu[e] == 0).all() and (got_d[e] == 0).all(), f"dW of expert {e} without rows"


@pytest.mark.parametrize("seed", range(8))
def test_sweep_grouped_gemm(seed):
    """Bare grouped GEMM over drawn group sizes (empty groups included) and
    input / output dtypes; sizes not a multiple of 8 take the vector ALUs.
    Rows past the last offset keep what the caller left there."""
    rng = np.random.default_rng(15000 + seed)
    E = int(rng.integers(1, 24))
    counts = [int(c) if rng.random() > 0.25 else 0 for c in rng.integers(0, 300, size=E)]
    odd = bool(rng.random() < 0.3)
    K = int(rng.integers(1, 400)) if odd else 8 * int(rng.integers(1, 50))
    N = int(rng.integers(1, 400)) if odd else 8 * int(rng.integers(1, 50))
    bf16 = bool(rng.random() < 0.7)
    out = "bf16" if bf16 and rng.random() < 0.4 else "f32"
    M = sum(counts) + 5
    A = WL._make(rng.standard_normal((M, K), dtype=np.float32), bf16)
    W = WL._make(rng.standard_normal((E, N, K), dtype=np.float32) / np.sqrt(K), bf16)
    offs = np.cumsum(counts).astype(np.int32)
    log(f"grouped_gemm sweep seed={seed}: counts={counts} K={K} N={N} bf16={bf16} out={out}")
    od = torch.float32 if out == "f32" else torch.bfloat16
    C0 = torch.full((M, N), 7.0, dtype=od, device="cuda")
    C = api.grouped_gemm(dev(A), dev(W), dev(offs), out=C0, out_dtype=od)
    torch.cuda.synchronize()
    got = host(C)
    nv = int(offs[-1])
    ref = O.grouped_gemm(A.values, W.values, offs)
    assert_close(got[:nv], ref[:nv], "bf16" if (bf16 or out == "bf16") else "f32", "C")
    assert (got[nv:] == 7.0).all()


@pytest.mark.parametrize("seed", range(6))
def test_sweep_fp32_step(seed):
    """fp32 inputs (exact fp32 products on the vector ALUs) at any sizes:
    forward and backward against the oracle at the fp32 bar."""
    rng = np.random.default_rng(16000 + seed)
    T = int(rng.integers(1, 300))
    K = int(rng.integers(1, 200))
    N = int(rng.integers(1, 200))
    E = int(rng.integers(1, 16))
    k = int(rng.integers(1, min(E, 4) + 1))
    ids, empty, masked, cap = _routing(rng, T, E, k)
    r = WL.routed(f"sweep_f32_{seed}", T, K, N, E, k, seed=16500 + seed, bf16=False)
    r.expert_ids = ids
    log(f"fp32 sweep seed={seed}: T={T} K={K} N={N} E={E} k={k} empty={empty} masked={masked} cap={cap}")
    sch = _schedule(ids, r.topk_weights, E, masked, cap)
    y = api.moe_fused_fwd(dev(r.x), dev(r.W), sch, y=_nan((T, N)))
    dX, dW, dT = api.moe_fused_bwd(dev(r.dY), dev(r.x), dev(r.W), sch)
    torch.cuda.synchronize()
    ref_ids = _kept(ids, r.topk_weights, E, cap)[1] if masked else ids
    ry = O.moe_forward(r.x.values, r.W.values, ref_ids, r.topk_weights, E)
    rx, rw, rt = O.moe_backward(r.dY.values, r.x.values, r.W.values, ref_ids, r.topk_weights, E)
    assert_close(host(y), ry, "f32", "y")
    assert_close(host(dX), rx, "f32", "dX")
    assert_close(host(dW), rw, "f32", "dW")
    assert_close(host(dT), rt, "f32", "d_topk")
