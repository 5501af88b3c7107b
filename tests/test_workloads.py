"""The seeded input generators: deterministic, and the stated properties hold."""
import hashlib

import numpy as np
import pytest

from moe_variable_size_amd import workloads as W


def _h(*arrays):
    m = hashlib.sha256()
    for a in arrays:
        m.update(np.ascontiguousarray(a).tobytes())
    return m.hexdigest()


def test_bf16_rounding_is_nearest_even():
    vals = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9, -2.5], dtype=np.float32)
    bits, out = W.round_to_bf16(vals)
    # ties go to even: 1+2^-8 -> 1.0, 1+3*2^-8 -> 1+2^-6 ... (bf16 has 7 fraction bits)
    assert out.tolist() == [1.0, 1.0, 1.0 + 2.0 ** -6, 1.0, -2.5]
    assert bits.dtype == np.uint16 and bits[0] == 0x3F80


def test_generators_are_deterministic():
    a = W.routed("t", 33, 24, 40, 5, 2, seed=7)
    b = W.routed("t", 33, 24, 40, 5, 2, seed=7)
    assert _h(a.x.bits, a.W.bits, a.expert_ids, a.topk_weights, a.dY.bits) == \
        _h(b.x.bits, b.W.bits, b.expert_ids, b.topk_weights, b.dY.bits)
    c = W.routed("t", 33, 24, 40, 5, 2, seed=8)
    assert _h(a.x.bits) != _h(c.x.bits)
    r = W.routed("t", 33, 24, 40, 5, 2, seed=7, dense=False)
    assert np.array_equal(r.expert_ids, a.expert_ids) and np.array_equal(r.topk_weights, a.topk_weights)


def test_config1_shapes():
    g = W.config1()
    assert g.group_sizes.tolist() == [40, 0, 88, 128]
    assert g.A.shape == (256, 128) and g.W.shape == (4, 128, 128) and g.A.bits is None


def test_config2_routing():
    r = W.config2(dense=False)
    assert r.expert_ids.shape == (4096, 2)
    assert (r.expert_ids[:, 0] != r.expert_ids[:, 1]).all()
    assert r.topk_weights.dtype == np.float32 and (0 <= r.topk_weights).all() and (r.topk_weights < 1).all()
    c = np.bincount(r.expert_ids.reshape(-1), minlength=8)
    assert c.sum() == 8192 and c.min() > 900


def test_config3_routing_is_skewed_with_empties():
    r = W.config3(dense=False)
    ids = r.expert_ids
    assert ids.shape == (8192, 4)
    assert all(len(set(row)) == 4 for row in ids[:500].tolist())
    c = np.bincount(ids.reshape(-1), minlength=64)
    assert (c == 0).sum() == 4 and sorted(np.nonzero(c == 0)[0].tolist()) == r.notes["zero_experts"]
    assert c.max() > 10 * np.median(c[c > 0])
    assert np.allclose(r.topk_weights.sum(axis=1), 1.0, atol=1e-6)


def test_config4_seed_rule():
    g = W.config4(dense=False)
    assert g.group_sizes.sum() == 65536 and len(g.group_sizes) == 128
    assert (g.group_sizes == 0).sum() >= 1 and (g.group_sizes > 4096).sum() >= 2
    assert g.seed >= W.BASE_SEED + 4


def test_config5_fits_capacity():
    r = W.config5(dense=False)
    c = np.bincount(r.expert_ids.reshape(-1), minlength=64)
    assert r.capacity == 64 and c.max() <= 64 and c.min() > 0
    assert all(len(set(row)) == 8 for row in r.expert_ids.tolist())


def test_balanced_routing_and_gated_example():
    """Every expert gets exactly T*k/E assignments, experts are distinct per
    token, and the gated example has the shapes of the page's balanced step."""
    rng = np.random.default_rng(3)
    ids = W.balanced_ids(rng, 96, 8, 3)
    assert (np.bincount(ids.ravel(), minlength=8) == 36).all()
    assert all(len(set(r)) == 3 for r in ids.tolist())
    g = W.gated_page_example(dense=False)
    assert (g.T, g.K, g.F, g.N, g.E, g.k) == (8192, 4096, 2048, 4096, 64, 2)
    assert (np.bincount(g.expert_ids.ravel(), minlength=64) == 256).all()


def test_e4m3_quantization_bounds():
    """Row scales map each row's largest magnitude to 448; every code decodes
    (torch) to within half an E4M3 step of the scaled value."""
    import torch
    rng = np.random.default_rng(4)
    a = rng.standard_normal((5, 64)).astype(np.float32)
    a[2] = 0.0
    q, s = W.quantize_e4m3_rows(a)
    assert q.dtype == np.uint8 and s.shape == (5,) and s[2] == 1.0
    v = torch.from_numpy(q).view(torch.float8_e4m3fn).float().numpy()
    assert np.allclose(np.abs(v).max(axis=1)[[0, 1, 3, 4]], 448.0)
    rel = np.abs(v * s[:, None] - a) / np.maximum(np.abs(a), 2.0 ** -6 * s[:, None])
    assert rel.max() <= 2.0 ** -4 + 1e-6


def test_mx_quantization_bounds():
    """Block scales are powers of two bounding each block by 448; the codes
    times their scale stay within one E4M3 step of the values."""
    import torch
    rng = np.random.default_rng(6)
    a = rng.standard_normal((4, 96)).astype(np.float32) * 10.0 ** rng.integers(-3, 3, (4, 1))
    a[1, 32:64] = 0.0
    q, s = W.quantize_mx_blocks(a)
    assert q.shape == a.shape and s.shape == (4, 3) and s.dtype == np.uint8 and s[1, 1] == 0
    v = torch.from_numpy(q).view(torch.float8_e4m3fn).float().numpy().reshape(4, 3, 32)
    sc = np.exp2(s.astype(np.float64) - 127.0)
    assert (np.abs(v) <= 448.0).all() and np.isfinite(v).all()
    back = (v * sc[..., None]).reshape(4, 96)
    blk_max = np.repeat(np.abs(a.reshape(4, 3, 32)).max(-1), 32, axis=1)
    assert (np.abs(back - a) <= blk_max * 2.0 ** -3 + 1e-30).all()
