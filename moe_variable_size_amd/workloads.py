"""Seeded synthetic inputs for the MoE variable-size grouped GEMM.

This module only draws random inputs: it holds none of the grouped GEMM's
arithmetic (no sorting, no offsets, no products), so that both the HIP path and
the CPU oracle can be fed the very same arrays.

Every array is drawn on the host with numpy's PCG64.  Floating-point values are
drawn in fp32, scaled, and -- where a workload is bf16 -- rounded once to bf16
with round-to-nearest-even.  A bf16 tensor is handed out twice: as its raw
16-bit patterns (``*_bits``, uint16, what the GPU receives) and as the fp32
array holding exactly the same values (what the oracle receives).

Shapes and distributions follow the workloads the pages discuss:
  * tokens x [T, K] and expert weights W [E, N, K] stored like nn.Linear
    ("Grouped GEMM for MoE, in depth" -- "Data layout, offsets and alignment";
    grouped-gemm-moe card -- "Usage");
  * expert_ids [T, k] with k distinct experts per token and routing weights
    [T, k] in fp32 (grouped-gemm-moe card -- "Usage");
  * skewed per-expert loads (Zipf, Dirichlet) standing in for the recorded
    count histograms that "Failure modes" asks to replay, which do not exist
    here.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BASE_SEED = 1000


# ----------------------------------------------------------------------------
# bf16 helpers (input preparation only)
# ----------------------------------------------------------------------------
def round_to_bf16(a: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Round fp32 values to bf16 with round-to-nearest-even.

    Returns (bits uint16, values fp32) where ``values`` holds exactly the bf16
    numbers.  Inputs here are finite normals; NaN/Inf are not produced.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    bits = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    vals = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return bits, vals


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal_blocks(seed_seq: np.random.SeedSequence, nblocks: int, block_shape, scale: float) -> np.ndarray:
    """nblocks independent N(0, scale^2) fp32 blocks, one child stream per block.

    Child streams make the result independent of how many threads draw it.
    """
    children = seed_seq.spawn(nblocks)
    out = np.empty((nblocks,) + tuple(block_shape), dtype=np.float32)

    def draw(i):
        g = np.random.Generator(np.random.PCG64(children[i]))
        blk = g.standard_normal(block_shape, dtype=np.float32)
        if scale != 1.0:
            blk *= np.float32(scale)
        out[i] = blk

    with ThreadPoolExecutor(max_workers=_threads()) as ex:
        list(ex.map(draw, range(nblocks)))
    return out


@dataclass
class Tensor:
    """One input tensor: fp32 values, plus bf16 bit patterns when bf16."""

    values: np.ndarray                 # fp32 (exact bf16 values when bits is set)
    bits: Optional[np.ndarray] = None  # uint16 bf16 patterns, same shape

    @property
    def dtype(self) -> str:
        return "bf16" if self.bits is not None else "f32"

    @property
    def shape(self):
        return self.values.shape


def _make(values: np.ndarray, bf16: bool) -> Tensor:
    if bf16:
        bits, vals = round_to_bf16(values)
        return Tensor(vals, bits)
    return Tensor(np.ascontiguousarray(values, dtype=np.float32))


@dataclass
class Routed:
    """Inputs of the routed (fused) MoE layer."""

    name: str
    T: int
    K: int
    N: int
    E: int
    k: int
    x: Tensor                      # [T, K]
    W: Tensor                      # [E, N, K]
    expert_ids: np.ndarray         # [T, k] int32
    topk_weights: Optional[np.ndarray]  # [T, k] fp32 or None (weight 1)
    dY: Optional[Tensor] = None    # [T, N] incoming gradient
    capacity: int = 0              # > 0: masked fixed-capacity layout
    seed: int = 0
    notes: dict = field(default_factory=dict)

    @property
    def S(self) -> int:
        return self.T * self.k


@dataclass
class Grouped:
    """Inputs of the bare grouped GEMM (rows already grouped by expert)."""

    name: str
    M: int
    K: int
    N: int
    E: int
    group_sizes: np.ndarray        # [E] int64, as drawn / given
    A: Tensor                      # [M, K]
    W: Optional[Tensor]            # [E, N, K] (forward form)
    dY: Optional[Tensor] = None    # [M, N] (weight-gradient form)
    seed: int = 0
    notes: dict = field(default_factory=dict)


# ----------------------------------------------------------------------------
# routing draws
# ----------------------------------------------------------------------------
def distinct_uniform_ids(rng: np.random.Generator, T: int, E: int, k: int) -> np.ndarray:
    """k distinct experts per token, uniformly: the first k entries of a random
    permutation of the E experts (as in the card's usage example)."""
    keys = rng.random((T, E))
    return np.argsort(keys, axis=1, kind="stable")[:, :k].astype(np.int32)


def balanced_ids(rng: np.random.Generator, T: int, E: int, k: int) -> np.ndarray:
    """k distinct experts per token with every expert receiving exactly T*k/E
    assignments (T*k/E and T/E whole): slot 0 is a shuffled list holding each
    expert T/E times, slot j is slot 0 mapped through a random permutation of
    the experts that moves every expert j places along a random cycle."""
    assert T % E == 0 and k <= E
    first = rng.permutation(np.repeat(np.arange(E), T // E))
    cycle = rng.permutation(E)
    pos = np.empty(E, dtype=np.int64)
    pos[cycle] = np.arange(E)
    cols = [cycle[(pos[first] + j) % E] for j in range(k)]
    return np.stack(cols, axis=1).astype(np.int32)


def zipf_gumbel_ids(rng: np.random.Generator, T: int, E: int, k: int, s: float,
                    n_zero: int) -> tuple[np.ndarray, np.ndarray]:
    """k distinct experts per token drawn without replacement with probability
    proportional to rank^-s over a seeded permutation of the experts (Gumbel-top-k).
    The last ``n_zero`` ranks get probability 0, so exactly those experts stay
    empty.  Returns (ids [T,k] int32, expert order by rank)."""
    order = rng.permutation(E)
    rank_of = np.empty(E, dtype=np.int64)
    rank_of[order] = np.arange(E)
    logp = np.full(E, -np.inf)
    live = rank_of < E - n_zero
    logp[live] = -s * np.log(rank_of[live] + 1.0)
    g = rng.gumbel(size=(T, E))
    scores = logp[None, :] + g
    ids = np.argsort(-scores, axis=1, kind="stable")[:, :k].astype(np.int32)
    return ids, order


# ----------------------------------------------------------------------------
# the five workloads
# ----------------------------------------------------------------------------
def config1(seed: int = BASE_SEED + 1) -> Grouped:
    """Bare grouped GEMM in fp32: E=4, K=N=128, group sizes [40, 0, 88, 128]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    E, K, N = 4, 128, 128
    sizes = np.array([40, 0, 88, 128], dtype=np.int64)
    M = int(sizes.sum())
    A = rng.standard_normal((M, K), dtype=np.float32)
    W = rng.standard_normal((E, N, K), dtype=np.float32) * np.float32(1.0 / np.sqrt(K))
    return Grouped("bare_fp32_E4_K128_N128", M, K, N, E, sizes, _make(A, False), _make(W, False), seed=seed)


def routed(name: str, T: int, K: int, N: int, E: int, k: int, *, seed: int, bf16: bool = True,
           routing: str = "uniform", zipf_s: float = 1.2, n_zero: int = 0,
           weights: str = "uniform", with_dy: bool = True, capacity: int = 0,
           dense: bool = True, with_x: bool = True) -> Routed:
    """Generic routed workload.  Draw order: x, W, ids, weights, dY, each from its
    own child stream of ``seed``.  ``dense=False`` skips x, W and dY (routing
    only); ``with_x=False`` skips x alone (for a backward that never reads it);
    the other draws are the same either way."""
    ss = np.random.SeedSequence(seed)
    s_x, s_w, s_r, s_dy = ss.spawn(4)
    x = Wv = None
    if dense:
        if with_x:
            rng_x = np.random.Generator(np.random.PCG64(s_x))
            x = rng_x.standard_normal((T, K), dtype=np.float32)
        Wv = _normal_blocks(s_w, E, (N, K), 1.0 / np.sqrt(K))
    rng = np.random.Generator(np.random.PCG64(s_r))
    notes = {}
    if routing == "uniform":
        ids = distinct_uniform_ids(rng, T, E, k)
    elif routing == "balanced":
        ids = balanced_ids(rng, T, E, k)
    elif routing == "zipf":
        ids, order = zipf_gumbel_ids(rng, T, E, k, zipf_s, n_zero)
        notes["zero_experts"] = sorted(int(e) for e in order[E - n_zero:]) if n_zero else []
    else:
        raise ValueError(routing)
    if weights == "uniform":
        w = rng.random((T, k), dtype=np.float32)
    elif weights == "softmax":
        logits = rng.standard_normal((T, k)).astype(np.float32)
        ex = np.exp(logits - logits.max(axis=1, keepdims=True))
        w = (ex / ex.sum(axis=1, keepdims=True)).astype(np.float32)
    elif weights == "ones":
        w = None
    else:
        raise ValueError(weights)
    dY = None
    if with_dy and dense:
        rng_dy = np.random.Generator(np.random.PCG64(s_dy))
        dY = _make(rng_dy.standard_normal((T, N), dtype=np.float32), bf16)
    return Routed(name, T, K, N, E, k, _make(x, bf16) if x is not None else None,
                  _make(Wv, bf16) if dense else None, ids, w, dY,
                  capacity=capacity, seed=seed, notes=notes)


def config2(seed: int = BASE_SEED + 2, with_dy: bool = True, dense: bool = True) -> Routed:
    """Fused MoE layer, bf16 in / fp32 out: T=4096, K=N=2048, E=8, top-2, uniform
    distinct routing, weights U[0,1), dY ~ N(0,1)."""
    return routed("fused_T4096_K2048_N2048_E8_top2", 4096, 2048, 2048, 8, 2, seed=seed,
                  routing="uniform", weights="uniform", with_dy=with_dy, dense=dense)


def config3(seed: int = BASE_SEED + 3, with_dy: bool = True, dense: bool = True) -> Routed:
    """Fused MoE layer fwd+bwd, bf16: T=8192, E=64, top-4, K=4096, N=1408, Zipf(1.2)
    routing over a seeded expert order with the 4 rarest ranks empty, weights a
    softmax of N(0,1) logits over the chosen 4."""
    return routed("fused_T8192_K4096_N1408_E64_top4_zipf", 8192, 4096, 1408, 64, 4, seed=seed,
                  routing="zipf", zipf_s=1.2, n_zero=4, weights="softmax", with_dy=with_dy,
                  dense=dense)


def config4(base_seed: int = BASE_SEED + 4, dense: bool = True) -> Grouped:
    """Weight-gradient stress, bf16: E=128, K=2048, N=768, 65536 grouped rows with
    sizes ~ Multinomial(65536, Dirichlet(0.3)).  The seed is the first one at or
    above ``base_seed`` whose draw has at least one empty group and at least two
    groups above 4096 rows."""
    E, K, N, S = 128, 2048, 768, 65536
    seed = base_seed
    while True:
        rng = np.random.Generator(np.random.PCG64(seed))
        p = rng.dirichlet(np.full(E, 0.3))
        sizes = rng.multinomial(S, p).astype(np.int64)
        if (sizes == 0).sum() >= 1 and (sizes > 4096).sum() >= 2:
            break
        seed += 1
    A = dY = None
    if dense:
        ss = np.random.SeedSequence(seed)
        s_x, s_dy = ss.spawn(2)
        A = _make(_normal_blocks(s_x, 64, (S // 64, K), 1.0).reshape(S, K), True)
        dY = _make(_normal_blocks(s_dy, 64, (S // 64, N), 1.0).reshape(S, N), True)
    return Grouped("dW_S65536_K2048_N768_E128_dirichlet0.3", S, K, N, E, sizes,
                   A, None, dY, seed=seed)


def config5(seed: int = BASE_SEED + 5, dense: bool = True) -> Routed:
    """Masked decode: E=64, capacity 64, T=128, top-8 uniform distinct, K=7168,
    N=2048, weights U[0,1)."""
    return routed("decode_masked_T128_K7168_N2048_E64_top8_cap64", 128, 7168, 2048, 64, 8,
                  seed=seed, routing="uniform", weights="uniform", with_dy=False, capacity=64,
                  dense=dense)


@dataclass
class Gated:
    """Inputs of the gated expert FFN: the routed layer with a doubled
    up-projection W_gu [E, 2F, K] (gate rows, then up rows) and a down
    projection W_down [E, N, F]."""

    name: str
    T: int
    K: int
    F: int
    N: int
    E: int
    k: int
    x: Optional[Tensor]            # [T, K]
    W_gu: Optional[Tensor]         # [E, 2F, K]
    W_down: Optional[Tensor]       # [E, N, F]
    expert_ids: np.ndarray         # [T, k] int32
    topk_weights: Optional[np.ndarray]
    capacity: int = 0
    seed: int = 0

    @property
    def S(self) -> int:
        return self.T * self.k


def gated(name: str, T: int, K: int, F: int, N: int, E: int, k: int, *, seed: int,
          routing: str = "uniform", weights: str = "uniform", capacity: int = 0,
          dense: bool = True, bf16: bool = True) -> Gated:
    """Gated FFN workload: routing as in ``routed`` (same draws for the same
    seed), x ~ N(0, 1), W_gu ~ N(0, 1/K), W_down ~ N(0, 1/F); bf16 (or fp32
    with ``bf16=False``)."""
    r = routed(name, T, K, 2 * F, E, k, seed=seed, routing=routing, weights=weights,
               with_dy=False, capacity=capacity, dense=dense, bf16=bf16)
    Wd = None
    if dense:
        s_d = np.random.SeedSequence(seed).spawn(5)[4]
        Wd = _make(_normal_blocks(s_d, E, (N, F), 1.0 / np.sqrt(F)), bf16)
    return Gated(name, T, K, F, N, E, k, r.x, r.W, Wd, r.expert_ids, r.topk_weights,
                 capacity=capacity, seed=seed)


def gated_page_example(seed: int = BASE_SEED + 6, dense: bool = True) -> Gated:
    """The balanced step of "Grouped GEMM for MoE, in depth" ("Worked example:
    tile counts under skew"): one up-projection with hidden size 4096 and width
    2048, 8192 tokens, top-2, 64 experts of exactly 256 rows each -- here as a
    gated FFN: gate and up of width F = 2048 each, down projection back to
    4096; weights U[0,1)."""
    return gated("gated_T8192_K4096_F2048_N4096_E64_top2_balanced", 8192, 4096, 2048, 4096, 64,
                 2, seed=seed, routing="balanced", weights="uniform", dense=dense)


@dataclass
class Fp8Routed:
    """Inputs of the 8-bit routed forward: E4M3 codes with a per-token scale
    for x and a per-expert output-channel scale for W."""

    name: str
    T: int
    K: int
    N: int
    E: int
    k: int
    xq: np.ndarray                 # [T, K] uint8 E4M3 codes
    x_scale: np.ndarray            # [T] float32
    Wq: np.ndarray                 # [E, N, K] uint8 E4M3 codes
    w_scale: np.ndarray            # [E, N] float32
    expert_ids: np.ndarray
    topk_weights: Optional[np.ndarray]
    capacity: int = 0


E4M3_MAX = 448.0


def quantize_e4m3_rows(a: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Scale each row of ``a`` (last axis) by max|row| / 448 and round to the
    nearest E4M3 code (torch's float8_e4m3fn conversion).  Returns (codes
    uint8 with the shape of ``a``, scales float32 with one per row; 1 for an
    all-zero row)."""
    import torch
    a = np.asarray(a, dtype=np.float32)
    amax = np.abs(a).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    q = torch.from_numpy(np.ascontiguousarray(a / scale[..., None])).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).numpy(), scale


def fp8_routed(r: Routed) -> Fp8Routed:
    """8-bit version of a routed workload: x and every expert's weight rows
    quantized row by row from the workload's own values."""
    xq, sx = quantize_e4m3_rows(r.x.values)
    Wq, sw = quantize_e4m3_rows(r.W.values)
    return Fp8Routed(r.name + "_e4m3", r.T, r.K, r.N, r.E, r.k, xq, sx, Wq, sw, r.expert_ids,
                     r.topk_weights, capacity=r.capacity)


@dataclass
class MxRouted:
    """Inputs of the 8-bit routed forward with per-32-element block scales."""

    name: str
    T: int
    K: int
    N: int
    E: int
    k: int
    xq: np.ndarray                 # [T, K] uint8 E4M3 codes
    x_bs: np.ndarray               # [T, K/32] uint8 E8M0 codes
    Wq: np.ndarray                 # [E, N, K] uint8 E4M3 codes
    w_bs: np.ndarray               # [E, N, K/32] uint8 E8M0 codes
    expert_ids: np.ndarray
    topk_weights: Optional[np.ndarray]
    capacity: int = 0


def quantize_mx_blocks(a: np.ndarray, block: int = 32) -> tuple[np.ndarray, np.ndarray]:
    """Quantize the last axis of ``a`` in blocks of ``block`` elements: a
    power-of-two scale 2^e per block, e the smallest exponent with
    max|block| / 2^e <= 448 (e = -127 for an all-zero block), stored as the
    E8M0 code 127 + e; codes by torch's float8_e4m3fn conversion of a / 2^e."""
    import torch
    a = np.asarray(a, dtype=np.float32)
    shp = a.shape
    blk = a.reshape(shp[:-1] + (shp[-1] // block, block))
    amax = np.abs(blk).max(axis=-1).astype(np.float64)
    e = np.where(amax > 0, np.ceil(np.log2(np.maximum(amax, 1e-300) / E4M3_MAX)), -127.0)
    e = np.clip(e, -127, 127)
    q = torch.from_numpy(np.ascontiguousarray((blk / np.exp2(e)[..., None]).astype(np.float32)))
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8).numpy().reshape(shp)
    return codes, (e + 127).astype(np.uint8)


def mx_routed(r: Routed) -> MxRouted:
    """Block-scaled 8-bit version of a routed workload (x and W from its values)."""
    xq, xs = quantize_mx_blocks(r.x.values)
    Wq, ws = quantize_mx_blocks(r.W.values)
    return MxRouted(r.name + "_mxfp8", r.T, r.K, r.N, r.E, r.k, xq, xs, Wq, ws, r.expert_ids,
                    r.topk_weights, capacity=r.capacity)


def grouped_as_routed(g: Grouped) -> Routed:
    """The weight-gradient stress case seen as a routed layer with k=1 and rows
    already in expert order (token r belongs to group g(r)), routing weight 1."""
    ids = np.repeat(np.arange(g.E, dtype=np.int32), g.group_sizes).reshape(-1, 1)
    W = None
    return Routed(g.name, g.M, g.K, g.N, g.E, 1, g.A, W, ids, None, g.dY, seed=g.seed)
