"""GPU parity of the grouped GEMM entry points against the CPU oracle.

fp32 path: max relative error <= 1e-4.  bf16 path: max relative error <= 1e-2
and relative Frobenius error <= 3e-3 (normwise, see tests/gpu_util.py).
Integer results are compared bit for bit elsewhere (test_gpu_schedule.py).
"""
import numpy as np
import pytest
import torch

from moe_variable_size_amd import api
from moe_variable_size_amd import workloads as WL
from oracle import moe_oracle as O
from tests.gpu_util import assert_close, dev, host, log

pytestmark = pytest.mark.gpu


# ----------------------------------------------------------------------------
# bare grouped GEMM
# ----------------------------------------------------------------------------
def test_config1_bare_fp32():
    g = WL.config1()
    log(f"grouped_gemm fp32 {g.name}")
    offs = np.cumsum(g.group_sizes).astype(np.int32)
    C = api.grouped_gemm(dev(g.A), dev(g.W), dev(offs))
    torch.cuda.synchronize()
    ref = O.grouped_gemm(g.A.values, g.W.values, offs)
    assert_close(host(C), ref, "f32", "config1 C")


@pytest.mark.parametrize("counts,K,N,bf16,out", [
    ([40, 0, 88, 128], 128, 128, True, "f32"),
    ([0, 1, 300, 0, 513, 7], 200, 264, True, "bf16"),
    ([3, 0, 5], 64, 8, True, "f32"),
    ([0, 0, 1000], 72, 520, True, "f32"),
    ([17, 0, 30], 13, 7, True, "f32"),      # K, N not multiples of 8 (vector ALU path)
    ([17, 0, 30, 1], 13, 7, False, "f32"),
    ([129, 0, 64], 96, 100, False, "f32"),
])
def test_bare_grouped_gemm(counts, K, N, bf16, out):
    rng = np.random.default_rng(sum(counts) + K + N)
    E = len(counts)
    M = sum(counts) + 3                      # rows past offsets[E-1] are left untouched
    A = WL._make(rng.standard_normal((M, K), dtype=np.float32), bf16)
    W = WL._make(rng.standard_normal((E, N, K), dtype=np.float32) / np.sqrt(K), bf16)
    offs = np.cumsum(counts).astype(np.int32)
    log(f"grouped_gemm counts={counts} K={K} N={N} bf16={bf16} out={out}")
    od = torch.float32 if out == "f32" else torch.bfloat16
    C0 = torch.full((M, N), 7.0, dtype=od, device="cuda")
    C = api.grouped_gemm(dev(A), dev(W), dev(offs), out=C0, out_dtype=od)
    torch.cuda.synchronize()
    ref = O.grouped_gemm(A.values, W.values, offs)
    got = host(C)
    nv = int(offs[-1])
    assert_close(got[:nv], ref[:nv], "bf16" if (bf16 or out == "bf16") else "f32", "C")
    assert (got[nv:] == 7.0).all()


# ----------------------------------------------------------------------------
# fused forward
# ----------------------------------------------------------------------------
def _routed_small(T, K, N, E, k, seed, bf16=True, empty=(), weights="uniform"):
    r = WL.routed("small", T, K, N, E, k, seed=seed, bf16=bf16, weights=weights)
    if empty:
        live = [e for e in range(E) if e not in empty]
        rng = np.random.default_rng(seed)
        r.expert_ids = np.array([rng.choice(live, size=k, replace=False) for _ in range(T)], dtype=np.int32)
    return r


def _fwd(r, layout=api.MOE_LAYOUT_CONTIGUOUS, cap=0):
    sch = api.moe_build_schedule(dev(r.expert_ids), None if r.topk_weights is None else dev(r.topk_weights),
                                 r.E, layout=layout, capacity=cap)
    y = api.moe_fused_fwd(dev(r.x), dev(r.W), sch)
    torch.cuda.synchronize()
    return sch, host(y)


@pytest.mark.parametrize("T,K,N,E,k,bf16,empty", [
    (300, 128, 96, 6, 2, False, (1, 4)),
    (1, 64, 64, 3, 1, False, ()),
    (700, 256, 320, 5, 2, True, (0,)),
    (257, 512, 264, 9, 3, True, (2, 3, 8)),
    (1030, 2048, 512, 8, 2, True, ()),
    (50, 40, 24, 4, 4, True, ()),
    (333, 136, 200, 7, 2, True, (3,)),        # three stages, the last one partial
    (129, 192, 128, 3, 1, True, ()),          # three whole stages
    (90, 104, 72, 4, 2, True, ()),            # two stages, the last one partial
    (1030, 512, 768, 8, 2, True, ()),         # 48 tiles: 128 x 128 sub-tiles of the last round
    (2000, 256, 1536, 8, 2, True, ()),        # 96 tiles: 128 x 256 sub-tiles of the last round
    (64, 30, 17, 5, 2, True, (1,)),           # vector ALU path for bf16
])
def test_fused_forward_small(T, K, N, E, k, bf16, empty):
    r = _routed_small(T, K, N, E, k, seed=T + K, bf16=bf16, empty=empty)
    log(f"fused fwd T={T} K={K} N={N} E={E} k={k} bf16={bf16}")
    _, y = _fwd(r)
    ref = O.moe_forward(r.x.values, r.W.values, r.expert_ids, r.topk_weights, E)
    assert_close(y, ref, "bf16" if bf16 else "f32", "y")


def test_fused_equals_explicit_fp32_bitwise():
    """fp32, k <= 2: the fused forward equals gather -> bare grouped GEMM ->
    weighted scatter bit for bit, and repeats bit for bit (the card's
    "Correctness": the fusion is exact)."""
    r = _routed_small(513, 96, 72, 7, 2, seed=5, bf16=False, empty=(3,))
    sch, y = _fwd(r)
    _, y2 = _fwd(r)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))
    x = dev(r.x)
    r2t = sch.row_to_token.long()
    nrow = int(sch.offsets[-1].item())
    xs = x[r2t[:nrow]].contiguous()
    ys = api.grouped_gemm(xs, dev(r.W), sch.offsets.clone())
    yy = torch.zeros_like(torch.from_numpy(y)).cuda()
    yy.index_add_(0, r2t[:nrow], ys * sch.row_weight[:nrow, None])
    torch.cuda.synchronize()
    assert np.array_equal(host(yy).view(np.uint32), y.view(np.uint32))


def test_fused_forward_config2():
    r = WL.config2(with_dy=False)
    log(f"fused fwd {r.name}")
    _, y = _fwd(r)
    ref = O.moe_forward(r.x.values, r.W.values, r.expert_ids, r.topk_weights, r.E)
    assert_close(y, ref, "bf16", "config2 y")


@pytest.mark.slow
def test_fused_forward_config3():
    r = WL.config3(with_dy=False)
    log(f"fused fwd {r.name}")
    _, y = _fwd(r)
    ref = O.moe_forward(r.x.values, r.W.values, r.expert_ids, r.topk_weights, r.E)
    assert_close(y, ref, "bf16", "config3 y")


# ----------------------------------------------------------------------------
# masked decode
# ----------------------------------------------------------------------------
def test_masked_decode_config5():
    r = WL.config5()
    log(f"masked fwd {r.name}")
    sch, y = _fwd(r, api.MOE_LAYOUT_MASKED, r.capacity)
    ms = O.masked_schedule(r.expert_ids, r.topk_weights, r.E, r.capacity)
    assert ms.n_dropped == 0
    ref = O.masked_forward(r.x.values, r.W.values, ms, r.T)
    assert_close(y, ref, "bf16", "config5 y")
    # no overflow: masked layout gives the contiguous result
    _, yc = _fwd(r)
    assert_close(yc, ref, "bf16", "config5 contiguous y")


@pytest.mark.parametrize("cap,bf16", [(2, True), (5, False), (64, True), (100, True)])
def test_masked_with_overflow(cap, bf16):
    r = _routed_small(90, 64, 136, 6, 3, seed=cap, bf16=bf16)
    log(f"masked fwd cap={cap} bf16={bf16}")
    sch, y = _fwd(r, api.MOE_LAYOUT_MASKED, cap)
    ms = O.masked_schedule(r.expert_ids, r.topk_weights, r.E, cap)
    ref = O.masked_forward(r.x.values, r.W.values, ms, r.T)
    assert_close(y, ref, "bf16" if bf16 else "f32", "masked y")
    assert int(sch.status[1].item()) == ms.n_dropped


# ----------------------------------------------------------------------------
# backward
# ----------------------------------------------------------------------------
def _bwd(r, layout=api.MOE_LAYOUT_CONTIGUOUS, cap=0):
    sch = api.moe_build_schedule(dev(r.expert_ids), None if r.topk_weights is None else dev(r.topk_weights),
                                 r.E, layout=layout, capacity=cap)
    dX, dW, dT = api.moe_fused_bwd(dev(r.dY), dev(r.x), dev(r.W), sch)
    torch.cuda.synchronize()
    return host(dX), host(dW), host(dT)


@pytest.mark.parametrize("T,K,N,E,k,bf16,empty", [
    (300, 64, 96, 6, 2, False, (1, 4)),
    (700, 256, 512, 5, 2, True, (0,)),
    (257, 512, 264, 9, 3, True, (2, 3, 8)),
    (600, 320, 1024, 4, 1, True, ()),
    (333, 200, 136, 7, 2, True, (3,)),       # dX reduction: three stages, the last partial
    (129, 128, 192, 3, 1, True, ()),         # dX reduction: three whole stages
    (2000, 1536, 256, 8, 2, True, ()),       # 96 dX tiles: 128 x 256 sub-tiles of the last round
    (64, 30, 17, 5, 2, True, (1,)),          # vector ALU path for bf16
])
def test_backward_small(T, K, N, E, k, bf16, empty):
    r = _routed_small(T, K, N, E, k, seed=T + N, bf16=bf16, empty=empty)
    log(f"fused bwd T={T} K={K} N={N} E={E} k={k} bf16={bf16}")
    dX, dW, dT = _bwd(r)
    rx, rw, rt = O.moe_backward(r.dY.values, r.x.values, r.W.values, r.expert_ids, r.topk_weights, E)
    dt = "bf16" if bf16 else "f32"
    assert_close(dX, rx, dt, "dX")
    assert_close(dW, rw, dt, "dW")
    assert_close(dT, rt, dt, "d_topk")
    for e in empty:
        assert (dW[e] == 0).all()


def test_backward_empty_expert_overwrites_garbage():
    """dW of an expert with no rows is written as exact zeros over a NaN-filled
    buffer ([GG] "The backward pass" and "Failure modes": stale dW)."""
    r = _routed_small(400, 128, 256, 5, 2, seed=77, bf16=True, empty=(2,))
    sch = api.moe_build_schedule(dev(r.expert_ids), dev(r.topk_weights), r.E)
    dW0 = torch.full((r.E, r.N, r.K), float("nan"), dtype=torch.bfloat16, device="cuda")
    _, dW, _ = api.moe_fused_bwd(dev(r.dY), dev(r.x), dev(r.W), sch, dx=False, dtopk=False, out_dW=dW0)
    torch.cuda.synchronize()
    got = host(dW)
    assert (got[2] == 0).all() and np.isfinite(got).all()


def test_backward_config2():
    r = WL.config2()
    log(f"fused bwd {r.name}")
    dX, dW, dT = _bwd(r)
    rx, rw, rt = O.moe_backward(r.dY.values, r.x.values, r.W.values, r.expert_ids, r.topk_weights, r.E)
    assert_close(dX, rx, "bf16", "config2 dX")
    assert_close(dW, rw, "bf16", "config2 dW")
    assert_close(dT, rt, "bf16", "config2 d_topk")


@pytest.mark.slow
def test_backward_config3():
    """Full-size config 3 backward: all of dX and d_topk, and the whole weight
    gradient of the hottest expert, of the least-loaded non-empty expert and
    of the empty experts (exact zeros), against the oracle's definitions."""
    r = WL.config3()
    log(f"fused bwd {r.name}")
    dX, dW, dT = _bwd(r)
    counts = np.bincount(r.expert_ids.ravel(), minlength=r.E)
    zero = [int(e) for e in np.nonzero(counts == 0)[0]]
    assert zero, "config 3 has empty experts"
    hot = int(np.argmax(counts))
    small = int(np.argmin(np.where(counts > 0, counts, counts.max() + 1)))
    log(f"  hottest expert {hot} ({counts[hot]} rows), smallest {small} ({counts[small]}), empty {zero}")
    rx, rW, rt = O.moe_backward(r.dY.values, r.x.values, r.W.values, r.expert_ids, r.topk_weights,
                                r.E, dw_experts=[hot, small])
    assert_close(dX, rx, "bf16", "config3 dX")
    assert_close(dT, rt, "bf16", "config3 d_topk")
    assert_close(dW[hot], rW[hot], "bf16", f"config3 dW[{hot}] (hottest)")
    assert_close(dW[small], rW[small], "bf16", f"config3 dW[{small}] (smallest)")
    assert all((dW[e] == 0).all() for e in zero)


def test_unweighted_schedule_equals_unit_weights():
    """A schedule built without routing weights takes the weight gradient's
    instantiation without the per-row multiplications; with every weight 1 the
    products are the same bits, so dW equals, bit for bit, the result of a
    schedule built with explicit unit weights (and dX too: two contributions
    per element add in either order to the same sum)."""
    r = _routed_small(900, 256, 320, 6, 2, seed=77, bf16=True, empty=(2,))
    ids, x, W, dY = dev(r.expert_ids), dev(r.x), dev(r.W), dev(r.dY)
    ones = torch.ones(r.expert_ids.shape, dtype=torch.float32, device="cuda")
    s0 = api.moe_build_schedule(ids, None, r.E)
    s1 = api.moe_build_schedule(ids, ones, r.E)
    assert s0.c.weighted == 0 and s1.c.weighted == 1
    dX0, dW0, dT0 = api.moe_fused_bwd(dY, x, W, s0)
    dX1, dW1, dT1 = api.moe_fused_bwd(dY, x, W, s1)
    torch.cuda.synchronize()
    assert torch.equal(dW0.view(torch.int16), dW1.view(torch.int16)), "dW differs"
    assert torch.equal(dX0, dX1), "dX differs"
    assert_close(host(dT0), host(dT1).astype(np.float64), "f32", "d_topk")


@pytest.mark.parametrize("K,N,E", [
    (384, 520, 9),      # 54 units (expert x 256 x 256 tile): two rounds or fewer, dealt statically
    (1024, 2048, 20),   # 640 units: more than two rounds on 256 compute units, from the queue
])
def test_weight_grad_queue_resets(K, N, E):
    """With more than two rounds of units the weight gradient hands them out
    from a counter pair in the schedule workspace, which the last workgroup of
    each launch sets back to zero: launches in a row on one schedule each see a
    fresh queue and give the same bits; every tile is reduced whole by one
    workgroup, so the order the tiles are taken in does not change a result."""
    r = _routed_small(1500, K, N, E, 2, seed=78, bf16=True, empty=(4,))
    ids, x, W, dY, tw = dev(r.expert_ids), dev(r.x), dev(r.W), dev(r.dY), dev(r.topk_weights)
    sch = api.moe_build_schedule(ids, tw, r.E)
    assert sch.dw_queue.tolist() == [0, 0]
    outs = []
    for _ in range(3):
        _, dW, _ = api.moe_fused_bwd(dY, x, W, sch, dx=False, dtopk=False)
        torch.cuda.synchronize()
        assert sch.dw_queue.tolist() == [0, 0]
        outs.append(dW)
    assert all(torch.equal(o.view(torch.int16), outs[0].view(torch.int16)) for o in outs[1:])
    _, rw, _ = O.moe_backward(r.dY.values, r.x.values, r.W.values, r.expert_ids, r.topk_weights, r.E)
    assert_close(host(outs[0]), rw, "bf16", "dW")


@pytest.mark.parametrize("T,K,N,E,k,masked", [
    (1500, 256, 520, 9, 2, False),
    (333, 128, 264, 5, 1, False),   # k = 1 with the atomic combine forced (the automatic one is ranked)
    (128, 512, 384, 16, 4, True),   # masked, 64-row tiles
])
def test_forward_overwrites_y(T, K, N, E, k, masked):
    """With the atomic combine the library zeroes y before the scattering
    forward adds into it, so a y full of NaN comes back right, and repeated
    launches agree bit for bit (at most two adds per element, which commute)."""
    r = _routed_small(T, K, N, E, k, seed=T + k, bf16=True)
    cap = 64 if masked else 0
    layout = api.MOE_LAYOUT_MASKED if masked else api.MOE_LAYOUT_CONTIGUOUS
    try:
        api.moe_set_combine(api.MOE_COMBINE_ATOMIC)
        sch = api.moe_build_schedule(dev(r.expert_ids), dev(r.topk_weights), E, layout=layout,
                                     capacity=cap)
        outs = []
        for _ in range(3):
            y0 = torch.full((T, N), float("nan"), dtype=torch.float32, device="cuda")
            y = api.moe_fused_fwd(dev(r.x), dev(r.W), sch, y=y0)
            torch.cuda.synchronize()
            outs.append(host(y))
    finally:
        api.moe_set_combine(api.MOE_COMBINE_AUTO)
    if masked:
        ms = O.masked_schedule(r.expert_ids, r.topk_weights, E, cap)
        ref = O.masked_forward(r.x.values, r.W.values, ms, T)
    else:
        ref = O.moe_forward(r.x.values, r.W.values, r.expert_ids, r.topk_weights, E)
    assert_close(outs[0], ref, "bf16", "y")
    if k <= 2:
        assert all(np.array_equal(o.view(np.uint32), outs[0].view(np.uint32)) for o in outs[1:])


def test_weight_grad_config4():
    g = WL.config4()
    r = WL.grouped_as_routed(g)
    log(f"dW {g.name}")
    sch = api.moe_build_schedule(dev(r.expert_ids), None, r.E)
    _, dW, _ = api.moe_fused_bwd(dev(r.dY), dev(r.x), None, sch, dx=False, dtopk=False, N=g.N)
    torch.cuda.synchronize()
    offs = np.cumsum(g.group_sizes).astype(np.int32)
    ref = O.grouped_weight_grad(g.A.values, g.dY.values, offs, g.E)
    got = host(dW)
    assert_close(got, ref, "bf16", "config4 dW")
    assert all((got[e] == 0).all() for e in np.nonzero(g.group_sizes == 0)[0])


# ----------------------------------------------------------------------------
# graph capture: no host sync anywhere in schedule + forward + backward
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("T,K,N,E", [
    (512, 256, 256, 8),
    (1500, 1024, 2048, 20),   # 640 weight-gradient units: the work-queue instantiation
])
def test_graph_capture_layer(T, K, N, E):
    """Build the schedule, run forward and backward inside one captured HIP
    graph ([GG] "What to do next": no device-to-host sync, capture the layer);
    every replay, with eager work in between, equals the eager result (the
    weight gradient's queue counters are reset by the kernel itself, so a
    replay finds them zero)."""
    r = _routed_small(T, K, N, E, 2, seed=12, bf16=True, empty=(5,))
    ids, w, x, W, dY = dev(r.expert_ids), dev(r.topk_weights), dev(r.x), dev(r.W), dev(r.dY)
    E = r.E

    def layer():
        sch = api.moe_build_schedule(ids, w, E, workspace=ws)
        y = api.moe_fused_fwd(x, W, sch, y=y_buf)
        api.moe_fused_bwd(dY, x, W, sch, out_dX=dX_buf, out_dW=dW_buf, out_dtopk=dT_buf)
        return y

    ws = torch.empty(api.moe_schedule_workspace_bytes(r.T, r.k, E), dtype=torch.uint8, device="cuda")
    y_buf = torch.empty((r.T, r.N), dtype=torch.float32, device="cuda")
    dX_buf = torch.empty((r.T, r.K), dtype=torch.float32, device="cuda")
    dW_buf = torch.empty((E, r.N, r.K), dtype=torch.bfloat16, device="cuda")
    dT_buf = torch.empty((r.T, r.k), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = [host(t).copy() for t in (y_buf, dX_buf, dW_buf, dT_buf)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer()
    for rep in range(3):
        for t in (y_buf, dX_buf, dT_buf):
            t.fill_(123.0)
        dW_buf.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [host(t) for t in (y_buf, dX_buf, dW_buf, dT_buf)]
        for a, b, name in zip(got, eager, ("y", "dX", "dW", "d_topk")):
            assert_close(a, b.astype(np.float64), "bf16", f"replay {rep} {name}")
        _ = torch.randn(1000, device="cuda").sum().item()   # eager work between replays
