"""moe_build_schedule_noalloc (the schedule build that allocates nothing and
keeps its block tables in the library's static per-GPU array) against
moe_build_schedule, both called through the C ABI: every array of the schedule
must match bit for bit.  Each case runs two builds in a row, the second on a
smaller input, so the second build works over tables the first one left."""
import ctypes

import numpy as np
import pytest
import torch

from moe_variable_size_amd import _lib
from tests.gpu_util import log

pytestmark = pytest.mark.gpu

CONTIG, MASKED = 0, 1


def _routing(T, k, E, seed, bad=0):
    """Seeded ids (distinct experts per token, skewed) and weights; `bad` ids
    are set out of range."""
    rng = np.random.default_rng(seed)
    p = rng.dirichlet(np.full(E, 0.3))
    ids = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    if bad:
        flat = ids.reshape(-1)
        flat[rng.choice(flat.size, size=bad, replace=False)] = E + 3
    w = rng.random((T, k), dtype=np.float32)
    return torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda()


def _arrays(c: _lib.MoeSchedule):
    """(name, pointer, number of 4-byte words) of every array the build writes."""
    E, R, S, k = c.E, c.R, c.S, c.k
    out = [("counts", c.counts, E), ("offsets", c.offsets, E),
           ("block_start", c.block_start, 4 * (E + 1)), ("expert_order", c.expert_order, E),
           ("row_to_assign", c.row_to_assign, R), ("row_to_token", c.row_to_token, R),
           ("row_weight", c.row_weight, R), ("status", c.status, 2)]
    if c.phases:
        kE = k * E
        out += [("phase_counts", c.phase_counts, kE), ("phase_offsets", c.phase_offsets, kE),
                ("phase_block_start", c.phase_block_start, 4 * (kE + 1)),
                ("phase_row_to_assign", c.phase_row_to_assign, S),
                ("phase_row_to_token", c.phase_row_to_token, S),
                ("phase_row_weight", c.phase_row_weight, S),
                ("phase_sync", c.phase_sync, 8 * 64 + 2)]
    return out


def _words(ws: torch.Tensor, ptr: int, n: int) -> np.ndarray:
    off = ptr - ws.data_ptr()
    assert 0 <= off and off + 4 * n <= ws.numel()
    return ws[off:off + 4 * n].view(torch.int32).cpu().numpy()


def _build(fn, ids, w, E, layout, cap, ws):
    lib = _lib.load()
    c = _lib.MoeSchedule()
    T, k = ids.shape
    st = getattr(lib, fn)(ids.data_ptr(), w.data_ptr(), T, k, E, layout, cap, ws.data_ptr(),
                          ws.numel(), ctypes.byref(c), torch.cuda.current_stream().cuda_stream)
    assert st == 0, f"{fn}: {lib.moe_status_string(st)}"
    return c


@pytest.mark.parametrize("layout,cases", [
    (CONTIG, [(4096, 4, 64, 0, 37), (700, 2, 16, 0, 5)]),      # with the rank-ordered view
    (CONTIG, [(3000, 6, 256, 0, 0), (257, 1, 200, 0, 1)]),     # k*E > 1024: no rank view first
    (MASKED, [(1500, 4, 32, 100, 11), (300, 2, 8, 40, 0)]),
])
def test_noalloc_schedule_matches(layout, cases):
    lib = _lib.load()
    # the ranked setting makes the contiguous builds carry the rank-ordered view too
    lib.moe_set_combine(2)
    try:
        _cases(lib, layout, cases)
    finally:
        lib.moe_set_combine(0)


def _cases(lib, layout, cases):
    for i, (T, k, E, cap, bad) in enumerate(cases):
        log(f"no-alloc schedule layout={layout} call {i}: T={T} k={k} E={E} cap={cap} bad={bad}")
        ids, w = _routing(T, k, E, seed=T + 7 * E + i, bad=bad)
        n = lib.moe_schedule_workspace_bytes(T, k, E, layout, cap)
        assert n > 0
        ws_ref = torch.full((n,), 0xA5, dtype=torch.uint8, device="cuda")
        ws_new = torch.full((n,), 0x5A, dtype=torch.uint8, device="cuda")
        ref = _build("moe_build_schedule", ids, w, E, layout, cap, ws_ref)
        new = _build("moe_build_schedule_noalloc", ids, w, E, layout, cap, ws_new)
        torch.cuda.synchronize()
        assert (new.T, new.S, new.R, new.k, new.E, new.layout, new.capacity, new.phases) == \
               (ref.T, ref.S, ref.R, ref.k, ref.E, ref.layout, ref.capacity, ref.phases)
        for (name, pr, cnt), (_, pn, _) in zip(_arrays(ref), _arrays(new)):
            a, b = _words(ws_ref, pr, cnt), _words(ws_new, pn, cnt)
            bad_at = np.flatnonzero(a != b)
            assert bad_at.size == 0, f"{name} differs at {bad_at[:8]}: {a[bad_at[:8]]} vs {b[bad_at[:8]]}"


def test_noalloc_rejects_small_workspace():
    """Host-side checks: a workspace below the schedule's arrays is refused
    before anything is launched; the full size always suffices."""
    lib = _lib.load()
    ids, w = _routing(64, 2, 8, seed=3)
    n = lib.moe_schedule_workspace_bytes(64, 2, 8, CONTIG, 0)
    small = torch.empty(256, dtype=torch.uint8, device="cuda")
    c = _lib.MoeSchedule()
    st = lib.moe_build_schedule_noalloc(ids.data_ptr(), w.data_ptr(), 64, 2, 8, CONTIG, 0,
                                        small.data_ptr(), small.numel(), ctypes.byref(c),
                                        torch.cuda.current_stream().cuda_stream)
    assert st == 5  # MOE_ERR_WORKSPACE
    full = torch.empty(n, dtype=torch.uint8, device="cuda")
    _build("moe_build_schedule_noalloc", ids, w, 8, CONTIG, 0, full)
    torch.cuda.synchronize()
