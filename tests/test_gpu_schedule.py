"""Schedule builder and tile map on the GPU: bit-exact against the oracle."""
import numpy as np
import pytest
import torch

from moe_variable_size_amd import api
from moe_variable_size_amd import workloads as WL
from oracle import moe_oracle as O
from tests.gpu_util import dev, log

pytestmark = pytest.mark.gpu

BMS = (32, 64, 128, 256)


def _excl_blocks(counts, BM):
    nb = -(-np.asarray(counts, dtype=np.int64) // BM)
    return np.concatenate([[0], np.cumsum(nb)]).astype(np.int64)


def _check_contiguous(ids, w, E, name):
    log(f"schedule contiguous: {name} T={ids.shape[0]} k={ids.shape[1]} E={E}")
    api.moe_set_combine(api.MOE_COMBINE_RANKED)   # so the build also makes the rank-ordered view
    try:
        sch = api.moe_build_schedule(dev(ids), None if w is None else dev(w), E)
    finally:
        api.moe_set_combine(api.MOE_COMBINE_AUTO)
    torch.cuda.synchronize()
    ref = O.routing_schedule(ids, w, E)
    R = ids.size
    nvalid = int(ref.counts.sum())
    assert sch.counts.cpu().numpy().tolist() == ref.counts.tolist()
    assert sch.offsets.cpu().numpy().tolist() == ref.offsets.tolist()
    r2a = sch.row_to_assign.cpu().numpy()
    r2t = sch.row_to_token.cpu().numpy()
    rw = sch.row_weight.cpu().numpy()
    assert r2a[:nvalid].tolist() == ref.perm.tolist()
    assert r2t[:nvalid].tolist() == ref.row_to_token.tolist()
    assert np.array_equal(rw[:nvalid].view(np.uint32), ref.row_weight.astype(np.float32).view(np.uint32))
    assert (r2a[nvalid:R] == -1).all() and (r2t[nvalid:R] == -1).all() and (rw[nvalid:R] == 0).all()
    for BM in BMS:
        assert sch.block_start(BM).cpu().numpy().tolist() == _excl_blocks(ref.counts, BM).tolist()
    order = np.argsort(-ref.counts, kind="stable")
    assert sch.expert_order.cpu().numpy().tolist() == order.tolist()
    assert sch.status.cpu().numpy().tolist() == [ref.n_invalid, 0]
    _check_rank_view(sch, ids, w, E)
    return sch, ref


def _check_rank_view(sch, ids, w, E):
    """The rank-ordered view: built exactly when k <= 8 and k*E <= 1024 (the
    library's limits), and then bit-exact against the oracle's definition."""
    T, k = ids.shape
    if k > 8 or k * E > 1024:
        assert sch.phases == 0
        return
    assert sch.phases == k
    rs = O.rank_schedule(ids, w, E)
    n = int(rs.counts.sum())
    assert sch.phase_counts.cpu().numpy().tolist() == rs.counts.tolist()
    assert sch.phase_offsets.cpu().numpy().tolist() == rs.offsets.tolist()
    for BM in BMS:
        assert sch.phase_block_start(BM).cpu().numpy().tolist() == _excl_blocks(rs.counts, BM).tolist()
    a = sch.phase_row_to_assign.cpu().numpy()
    t = sch.phase_row_to_token.cpu().numpy()
    wt = sch.phase_row_weight.cpu().numpy()
    assert a[:n].tolist() == rs.row_to_assign.tolist()
    assert t[:n].tolist() == rs.row_to_token.tolist()
    assert np.array_equal(wt[:n].view(np.uint32), rs.row_weight.view(np.uint32))
    assert (a[n:] == -1).all() and (t[n:] == -1).all() and (wt[n:] == 0).all()


def test_schedule_page_example():
    ids = np.array([[2], [0], [2], [2], [0], [2], [0], [2]], dtype=np.int32)   # counts [3, 0, 5]
    sch, ref = _check_contiguous(ids, None, 3, "page [3,0,5]")
    assert sch.offsets.cpu().numpy().tolist() == [3, 3, 8]


# the builder cuts the assignments into blocks of 1024 (more when T*k*E is
# large); (700, 2) and (1000, 3) give two and three blocks, where workgroups
# take more than one of the per-expert output jobs
@pytest.mark.parametrize("T,k,E,seed", [(1, 1, 1, 0), (37, 3, 6, 1), (5, 2, 64, 2), (1000, 4, 7, 3),
                                        (4099, 2, 130, 4), (5000, 8, 1000, 5), (333, 1, 1024, 6),
                                        (700, 2, 5, 7), (1000, 3, 9, 8)])
def test_schedule_random(T, k, E, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    _check_contiguous(ids, w, E, f"random seed={seed}")


def test_schedule_out_of_range_ids():
    rng = np.random.default_rng(9)
    ids = rng.integers(-3, 12, size=(300, 3)).astype(np.int32)
    w = rng.random((300, 3)).astype(np.float32)
    _check_contiguous(ids, w, 9, "out-of-range ids")


@pytest.mark.parametrize("cfg", ["c2", "c3", "c5", "c4"])
def test_schedule_workloads(cfg):
    if cfg == "c4":
        g = WL.config4(dense=False)
        r = WL.grouped_as_routed(g)
        _check_contiguous(r.expert_ids, None, r.E, g.name)
        return
    r = {"c2": WL.config2, "c3": WL.config3, "c5": WL.config5}[cfg](dense=False)
    _check_contiguous(r.expert_ids, r.topk_weights, r.E, r.name)


# (cap, seed, T): random ids with k = 4; T = 9000 spans many builder blocks and
# overflows the capacity of most experts
@pytest.mark.parametrize("cap,seed,T", [(64, None, 0), (3, 1, 97), (1, 2, 97), (200, 3, 97),
                                        (500, 4, 9000)])
def test_schedule_masked(cap, seed, T):
    if seed is None:
        r = WL.config5(dense=False)
        ids, w, E = r.expert_ids, r.topk_weights, r.E
    else:
        rng = np.random.default_rng(seed)
        E = 11 if T < 1000 else 70
        ids = rng.integers(-1, E, size=(T, 4)).astype(np.int32)
        w = rng.random((T, 4)).astype(np.float32)
    log(f"schedule masked: cap={cap} E={E} T={ids.shape[0]}")
    sch = api.moe_build_schedule(dev(ids), dev(w), E, layout=api.MOE_LAYOUT_MASKED, capacity=cap)
    torch.cuda.synchronize()
    ref = O.masked_schedule(ids, w, E, cap)
    assert sch.counts.cpu().numpy().tolist() == ref.masked_m.tolist()
    assert sch.offsets.cpu().numpy().tolist() == np.cumsum(ref.masked_m).tolist()
    assert sch.row_to_assign.cpu().numpy().tolist() == ref.slot_assign.reshape(-1).tolist()
    assert sch.row_to_token.cpu().numpy().tolist() == ref.slot_token.reshape(-1).tolist()
    assert np.array_equal(sch.row_weight.cpu().numpy().view(np.uint32),
                          ref.slot_weight.astype(np.float32).reshape(-1).view(np.uint32))
    for BM in BMS:
        expect = (np.arange(E + 1) * -(-cap // BM)).tolist()
        assert sch.block_start(BM).cpu().numpy().tolist() == expect
    assert sch.status.cpu().numpy().tolist() == [ref.n_invalid, ref.n_dropped]
    assert sch.phases == 0   # no rank-ordered view for the masked layout


@pytest.mark.parametrize("N,BM,BN", [(2048, 128, 128), (1408, 256, 256), (7, 32, 16), (130, 64, 64)])
def test_tile_map_bit_exact(N, BM, BN):
    """tile_start, total and the owner of every tile equal the oracle's upper-bound lookup."""
    rng = np.random.default_rng(N)
    counts = np.array([0, 300, 0, 0, 1, 129, 256, 0, 77, 0], dtype=np.int64)
    ids = np.repeat(np.arange(len(counts)), counts)
    rng.shuffle(ids)
    ids = ids.reshape(-1, 1).astype(np.int32)
    log(f"tile map N={N} BM={BM} BN={BN}")
    sch = api.moe_build_schedule(dev(ids), None, len(counts))
    ts, tot, owner = api.moe_tile_map(sch, N, BM, BN)
    torch.cuda.synchronize()
    ref = O.tile_space(counts, N, BM, BN)
    assert ts.cpu().numpy().tolist() == ref.tile_start.tolist()
    assert int(tot.item()) == ref.total
    assert owner.cpu().numpy()[:ref.total].tolist() == O.tile_owner(ref, np.arange(ref.total)).tolist()


def test_worked_example_tile_map():
    """The page's skewed worked example: 2752 tiles at BM = BN = 128, N = 2048."""
    counts = np.array([64] * 32 + [400] * 28 + [784] * 4)
    ids = np.repeat(np.arange(64), counts).reshape(-1, 1).astype(np.int32)
    sch = api.moe_build_schedule(dev(ids), None, 64)
    _, tot, owner = api.moe_tile_map(sch, 2048, 128, 128)
    torch.cuda.synchronize()
    assert int(tot.item()) == 2752
    ref = O.tile_space(counts, 2048, 128, 128)
    assert owner.cpu().numpy()[:2752].tolist() == O.tile_owner(ref, np.arange(2752)).tolist()
