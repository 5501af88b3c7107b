"""Python binding of the C ABI (include/moe_vs.h), same names as the C calls.

PyTorch supplies device memory and the current stream; every computation runs
in the HIP library (libmoe_vs.so).  Nothing here falls back to another
implementation: a missing library or a device-side failure raises.

Pages the operations follow:
  [GG]   "Grouped GEMM for MoE, in depth" (aicassindra.com)
  [CARD] "grouped-gemm-moe" (model card of a published grouped GEMM kernel)
  [NOTE] "Grouped GEMM" (scholia-log study notes)
"""
from __future__ import annotations

import contextlib
import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib
from ._lib import MOE_BF16, MOE_F32, MOE_LAYOUT_CONTIGUOUS, MOE_LAYOUT_MASKED, BM_VALUES
from ._lib import MOE_COMBINE_AUTO, MOE_COMBINE_ATOMIC, MOE_COMBINE_RANKED

_DTYPES = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _require(t: torch.Tensor, name: str, dtype=None, ndim=None, contiguous=True) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _require_out(t, name: str, dtype, shape, device) -> None:
    """A caller-supplied output: exactly the dtype, shape and device the call
    writes, dense.  The kernels write every byte of that shape from the
    pointer, so anything smaller would be written past."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != torch.device(device):
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on(stream):
    """Allocation context: buffers the binding allocates for a launch on a
    stream other than the current one come from that stream's pool, so the
    caching allocator never hands them to other work while the launch may
    still use them."""
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")
    return _DTYPES[t.dtype]


@dataclass
class Schedule:
    """A routing schedule built on the device (``moe_build_schedule``).

    ``workspace`` owns every array; ``c`` is the C descriptor that points into
    it.  Views of the arrays are exposed as tensors for inspection.
    """

    c: _lib.MoeSchedule
    workspace: torch.Tensor

    def _view(self, ptr: int, n: int, dtype) -> torch.Tensor:
        base = self.workspace.data_ptr()
        off = ptr - base
        esz = torch.tensor([], dtype=dtype).element_size()
        return self.workspace[off:off + n * esz].view(dtype)

    @property
    def E(self) -> int:
        return self.c.E

    @property
    def counts(self) -> torch.Tensor:
        return self._view(self.c.counts, self.c.E, torch.int32)

    @property
    def offsets(self) -> torch.Tensor:
        return self._view(self.c.offsets, self.c.E, torch.int32)

    def block_start(self, BM: int) -> torch.Tensor:
        i = BM_VALUES.index(BM)
        E = self.c.E
        return self._view(self.c.block_start, 4 * (E + 1), torch.int32)[i * (E + 1):(i + 1) * (E + 1)]

    @property
    def expert_order(self) -> torch.Tensor:
        return self._view(self.c.expert_order, self.c.E, torch.int32)

    @property
    def row_to_assign(self) -> torch.Tensor:
        return self._view(self.c.row_to_assign, self.c.R, torch.int32)

    @property
    def row_to_token(self) -> torch.Tensor:
        return self._view(self.c.row_to_token, self.c.R, torch.int32)

    @property
    def row_weight(self) -> torch.Tensor:
        return self._view(self.c.row_weight, self.c.R, torch.float32)

    @property
    def status(self) -> torch.Tensor:
        return self._view(self.c.status, 2, torch.int32)

    @property
    def dw_queue(self) -> torch.Tensor:
        """The weight-gradient work-queue counters (zero between launches)."""
        return self._view(self.c.dw_queue, 2, torch.int32)

    # rank-ordered view (None when the schedule has none)
    @property
    def phases(self) -> int:
        return self.c.phases

    @property
    def phase_counts(self) -> Optional[torch.Tensor]:
        return self._view(self.c.phase_counts, self.c.k * self.c.E, torch.int32) if self.c.phases else None

    @property
    def phase_offsets(self) -> Optional[torch.Tensor]:
        return self._view(self.c.phase_offsets, self.c.k * self.c.E, torch.int32) if self.c.phases else None

    def phase_block_start(self, BM: int) -> Optional[torch.Tensor]:
        if not self.c.phases:
            return None
        i = BM_VALUES.index(BM)
        n = self.c.k * self.c.E + 1
        return self._view(self.c.phase_block_start, 4 * n, torch.int32)[i * n:(i + 1) * n]

    @property
    def phase_row_to_assign(self) -> Optional[torch.Tensor]:
        return self._view(self.c.phase_row_to_assign, self.c.S, torch.int32) if self.c.phases else None

    @property
    def phase_row_to_token(self) -> Optional[torch.Tensor]:
        return self._view(self.c.phase_row_to_token, self.c.S, torch.int32) if self.c.phases else None

    @property
    def phase_row_weight(self) -> Optional[torch.Tensor]:
        return self._view(self.c.phase_row_weight, self.c.S, torch.float32) if self.c.phases else None

    @property
    def phase_sync(self) -> Optional[torch.Tensor]:
        """Completion counters of the ranked combine ([8, 64] words, then the
        finished-workgroup count and the count of waits that gave up)."""
        return self._view(self.c.phase_sync, 8 * 64 + 2, torch.int32) if self.c.phases else None


def moe_schedule_workspace_bytes(T: int, k: int, E: int, layout: int = MOE_LAYOUT_CONTIGUOUS,
                                 capacity: int = 0) -> int:
    return int(_lib.load().moe_schedule_workspace_bytes(T, k, E, layout, capacity))


def moe_build_schedule(expert_ids: torch.Tensor, topk_weights: Optional[torch.Tensor], E: int, *,
                       layout: int = MOE_LAYOUT_CONTIGUOUS, capacity: int = 0,
                       workspace: Optional[torch.Tensor] = None, stream=None) -> Schedule:
    """Counts, END offsets, tile prefixes and the stable sort by expert, on the
    device ([GG] "Data layout, offsets and alignment"; [CARD] "How it works")."""
    lib = _lib.load()
    _require(expert_ids, "expert_ids", torch.int32, 2)
    T, k = expert_ids.shape
    if topk_weights is not None:
        _require(topk_weights, "topk_weights", torch.float32, 2)
        if tuple(topk_weights.shape) != (T, k):
            raise ValueError("topk_weights must have the shape of expert_ids")
    nbytes = lib.moe_schedule_workspace_bytes(T, k, E, layout, capacity)
    if nbytes == 0:
        raise ValueError(f"invalid schedule sizes T={T} k={k} E={E} layout={layout} capacity={capacity}")
    if workspace is None:
        with _on(stream):
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=expert_ids.device)
    else:
        _require(workspace, "workspace", torch.uint8, 1)
        if workspace.numel() < nbytes:
            raise ValueError(f"workspace holds {workspace.numel()} bytes, the schedule needs {nbytes}")
    c = _lib.MoeSchedule()
    st = lib.moe_build_schedule(_ptr(expert_ids), _ptr(topk_weights), T, k, E, layout, capacity,
                                _ptr(workspace), workspace.numel(), ctypes.byref(c), _stream(stream))
    _lib.check("moe_build_schedule", st)
    return Schedule(c, workspace)


def moe_build_schedule_noalloc(expert_ids: torch.Tensor, topk_weights: Optional[torch.Tensor],
                               E: int, workspace: torch.Tensor, *,
                               layout: int = MOE_LAYOUT_CONTIGUOUS, capacity: int = 0,
                               stream=None) -> Schedule:
    """moe_build_schedule into a caller-given workspace with the build's block
    tables in the library's static per-GPU array: allocates nothing.  Calls
    that overlap in time on one GPU race (they share that array)."""
    lib = _lib.load()
    _require(expert_ids, "expert_ids", torch.int32, 2)
    T, k = expert_ids.shape
    if topk_weights is not None:
        _require(topk_weights, "topk_weights", torch.float32, 2)
        if tuple(topk_weights.shape) != (T, k):
            raise ValueError("topk_weights must have the shape of expert_ids")
    _require(workspace, "workspace", torch.uint8, 1)
    c = _lib.MoeSchedule()
    st = lib.moe_build_schedule_noalloc(_ptr(expert_ids), _ptr(topk_weights), T, k, E, layout,
                                        capacity, _ptr(workspace), workspace.numel(),
                                        ctypes.byref(c), _stream(stream))
    _lib.check("moe_build_schedule_noalloc", st)
    return Schedule(c, workspace)


def grouped_gemm(A: torch.Tensor, W: torch.Tensor, offsets: torch.Tensor, *,
                 out: Optional[torch.Tensor] = None, out_dtype=None, stream=None) -> torch.Tensor:
    """Bare grouped GEMM: C[r] = A[r] @ W[e(r)]^T for rows grouped by END offsets
    ([GG] "Problem descriptors and the tile scheduler")."""
    lib = _lib.load()
    _require(A, "A", None, 2)
    _require(W, "W", A.dtype, 3)
    _require(offsets, "offsets", torch.int32, 1)
    M, K = A.shape
    E, N, K2 = W.shape
    if K2 != K or offsets.numel() != E:
        raise ValueError("shape mismatch: A [M,K], W [E,N,K], offsets [E]")
    if out_dtype is None:
        out_dtype = A.dtype
    if out is None:
        with _on(stream):
            out = torch.zeros((M, N), dtype=out_dtype, device=A.device)
    _require_out(out, "out", out_dtype, (M, N), A.device)
    st = lib.grouped_gemm(_ptr(A), _ptr(W), _ptr(offsets), _ptr(out), M, K, N, E, _dtype_code(A),
                          _DTYPES[out_dtype], _stream(stream))
    _lib.check("grouped_gemm", st)
    return out


def moe_fused_fwd(x: torch.Tensor, W: torch.Tensor, sched: Schedule, *,
                  y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Fused MoE forward: gather on load, weighted atomic scatter-combine on
    store; y [T, N] float32 ([CARD] intro, "How it works")."""
    lib = _lib.load()
    _require(x, "x", None, 2)
    _require(W, "W", x.dtype, 3)
    T, K = x.shape
    E, N, K2 = W.shape
    if K2 != K or T != sched.c.T or E != sched.c.E:
        raise ValueError("shape mismatch between x [T,K], W [E,N,K] and the schedule")
    if y is None:
        with _on(stream):
            y = torch.empty((T, N), dtype=torch.float32, device=x.device)
    _require_out(y, "y", torch.float32, (T, N), x.device)
    st = lib.moe_fused_fwd(_ptr(x), _ptr(W), ctypes.byref(sched.c), _ptr(y), K, N, _dtype_code(x),
                           _stream(stream))
    _lib.check("moe_fused_fwd", st)
    return y


def moe_fused_fwd_fp8(x_q: torch.Tensor, x_scale: torch.Tensor, W_q: torch.Tensor,
                      w_scale: torch.Tensor, sched: Schedule, *, y: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """Fused MoE forward on 8-bit E4M3 operands (uint8 codes or float8_e4m3fn
    tensors) with a per-token scale x_scale [T] and a per-expert output-channel
    scale w_scale [E, N]; y [T, N] float32 ([GG] "Choosing an implementation")."""
    lib = _lib.load()
    f8 = getattr(torch, "float8_e4m3fn", None)
    for t, name in ((x_q, "x_q"), (W_q, "W_q")):
        if t.dtype not in (torch.uint8,) + ((f8,) if f8 is not None else ()):
            raise TypeError(f"{name} must hold E4M3 codes (uint8 or float8_e4m3fn)")
    _require(x_q, "x_q", None, 2)
    _require(W_q, "W_q", None, 3)
    _require(x_scale, "x_scale", torch.float32, 1)
    _require(w_scale, "w_scale", torch.float32, 2)
    T, K = x_q.shape
    E, N, K2 = W_q.shape
    if K2 != K or T != sched.c.T or E != sched.c.E or tuple(x_scale.shape) != (T,) \
            or tuple(w_scale.shape) != (E, N):
        raise ValueError("shape mismatch between x_q [T,K], W_q [E,N,K], the scales and the schedule")
    if y is None:
        with _on(stream):
            y = torch.empty((T, N), dtype=torch.float32, device=x_q.device)
    _require_out(y, "y", torch.float32, (T, N), x_q.device)
    st = lib.moe_fused_fwd_fp8(_ptr(x_q), _ptr(x_scale), _ptr(W_q), _ptr(w_scale),
                               ctypes.byref(sched.c), _ptr(y), K, N, _stream(stream))
    _lib.check("moe_fused_fwd_fp8", st)
    return y


def moe_fused_fwd_mx(x_q: torch.Tensor, x_bs: torch.Tensor, W_q: torch.Tensor, w_bs: torch.Tensor,
                     sched: Schedule, *, y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Fused MoE forward on 8-bit E4M3 operands with a power-of-two (E8M0,
    uint8) scale per 32 reduction elements: x_bs [T, K/32], w_bs [E, N, K/32];
    y [T, N] float32."""
    lib = _lib.load()
    _require(x_q, "x_q", None, 2)
    _require(W_q, "W_q", None, 3)
    _require(x_bs, "x_bs", torch.uint8, 2)
    _require(w_bs, "w_bs", torch.uint8, 3)
    T, K = x_q.shape
    E, N, K2 = W_q.shape
    if K2 != K or T != sched.c.T or E != sched.c.E or tuple(x_bs.shape) != (T, K // 32) \
            or tuple(w_bs.shape) != (E, N, K // 32):
        raise ValueError("shape mismatch between x_q, W_q, their block scales and the schedule")
    if y is None:
        with _on(stream):
            y = torch.empty((T, N), dtype=torch.float32, device=x_q.device)
    _require_out(y, "y", torch.float32, (T, N), x_q.device)
    st = lib.moe_fused_fwd_mx(_ptr(x_q), _ptr(x_bs), _ptr(W_q), _ptr(w_bs), ctypes.byref(sched.c),
                              _ptr(y), K, N, _stream(stream))
    _lib.check("moe_fused_fwd_mx", st)
    return y


def moe_gated_ffn_fwd(x: torch.Tensor, W_gu: torch.Tensor, W_down: torch.Tensor, sched: Schedule, *,
                      h: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                      gu: Optional[torch.Tensor] = None, save_gu: bool = False, stream=None):
    """Gated expert FFN forward: h = silu(x W_gate^T) * (x W_up^T) per schedule
    row from one grouped GEMM over W_gu [E, 2F, K] (gate rows, then up rows),
    then y = the weighted scatter-combine of h W_down^T, W_down [E, N, F]
    ([GG] "Choosing an implementation").  Inputs all bfloat16 or all float32.
    Returns (y [T, N] float32, h [R, F] in the input dtype) and, with
    ``save_gu`` (or ``gu`` given), also the saved gate/up values gu [R, 2F]
    float32 the backward needs."""
    lib = _lib.load()
    _require(x, "x", None, 2)
    if x.dtype not in _DTYPES:
        raise TypeError(f"x must be bfloat16 or float32, got {x.dtype}")
    dt = x.dtype
    _require(W_gu, "W_gu", dt, 3)
    _require(W_down, "W_down", dt, 3)
    T, K = x.shape
    E, F2, K2 = W_gu.shape
    E2, N, F = W_down.shape
    if K2 != K or F2 != 2 * F or E2 != E or T != sched.c.T or E != sched.c.E:
        raise ValueError("shape mismatch between x [T,K], W_gu [E,2F,K], W_down [E,N,F] and the schedule")
    with _on(stream):
        if h is None:
            h = torch.empty((sched.c.R, F), dtype=dt, device=x.device)
        if y is None:
            y = torch.empty((T, N), dtype=torch.float32, device=x.device)
        if gu is None and save_gu:
            gu = torch.empty((sched.c.R, 2 * F), dtype=torch.float32, device=x.device)
    _require_out(h, "h", dt, (sched.c.R, F), x.device)
    _require_out(y, "y", torch.float32, (T, N), x.device)
    if gu is not None:
        _require_out(gu, "gu", torch.float32, (sched.c.R, 2 * F), x.device)
    st = lib.moe_gated_ffn_fwd(_ptr(x), _ptr(W_gu), _ptr(W_down), ctypes.byref(sched.c), _ptr(h),
                               _ptr(gu), _ptr(y), K, F, N, _DTYPES[dt], _stream(stream))
    _lib.check("moe_gated_ffn_fwd", st)
    return (y, h, gu) if gu is not None else (y, h)


def moe_gated_ffn_bwd(dY: torch.Tensor, x: torch.Tensor, W_gu: torch.Tensor, W_down: torch.Tensor,
                      sched: Schedule, gu: torch.Tensor, h: torch.Tensor, *, dx: bool = True,
                      dw_gu: bool = True, dw_down: bool = True, dtopk: bool = True, stream=None):
    """Gated expert FFN backward from the saved gu and h.  Returns (dX [T, K]
    float32 | None, dW_gu [E, 2F, K] | None, dW_down [E, N, F] | None (both in
    the input dtype), d_topk [T, k] float32 | None)."""
    lib = _lib.load()
    if x.dtype not in _DTYPES:
        raise TypeError(f"x must be bfloat16 or float32, got {x.dtype}")
    dt = x.dtype
    for t, name, nd in ((dY, "dY", 2), (x, "x", 2), (W_gu, "W_gu", 3), (W_down, "W_down", 3),
                        (h, "h", 2)):
        _require(t, name, dt, nd)
    _require(gu, "gu", torch.float32, 2)
    T, K = x.shape
    E, F2, _ = W_gu.shape
    F = F2 // 2
    N = W_down.shape[1]
    if tuple(W_down.shape) != (E, N, F) or tuple(dY.shape) != (T, N) or T != sched.c.T \
            or tuple(gu.shape) != (sched.c.R, 2 * F) or tuple(h.shape) != (sched.c.R, F):
        raise ValueError("shape mismatch among dY, x, W_gu, W_down, gu, h and the schedule")
    dev = x.device
    ws_bytes = int(lib.moe_gated_ffn_bwd_workspace_bytes(ctypes.byref(sched.c), F))
    with _on(stream):
        dX = torch.empty((T, K), dtype=torch.float32, device=dev) if dx else None
        dWgu = torch.empty((E, 2 * F, K), dtype=dt, device=dev) if dw_gu else None
        dWd = torch.empty((E, N, F), dtype=dt, device=dev) if dw_down else None
        dT = torch.empty((T, sched.c.k), dtype=torch.float32, device=dev) if dtopk else None
        # dgu workspace: freed into this stream's pool when the call returns, so
        # it is not reused before the launches queued here have run
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    st = lib.moe_gated_ffn_bwd(_ptr(dY), _ptr(x), _ptr(W_gu), _ptr(W_down), ctypes.byref(sched.c),
                               _ptr(gu), _ptr(h), _ptr(dX), _ptr(dWgu), _ptr(dWd), _ptr(dT), K, F, N,
                               _DTYPES[dt], _ptr(ws), ws_bytes, _stream(stream))
    _lib.check("moe_gated_ffn_bwd", st)
    return dX, dWgu, dWd, dT


def moe_fused_bwd_workspace_bytes(sched: Schedule, K: int, N: int, dtype) -> int:
    return int(_lib.load().moe_fused_bwd_workspace_bytes(ctypes.byref(sched.c), K, N, _DTYPES[dtype]))


def moe_fused_bwd(dY: torch.Tensor, x: torch.Tensor, W: Optional[torch.Tensor], sched: Schedule, *,
                  dx: bool = True, dw: bool = True, dtopk: bool = True, N: Optional[int] = None,
                  out_dX=None, out_dW=None, out_dtopk=None, stream=None):
    """Fused MoE backward ([GG] "The backward pass"; [CARD] "How it works").
    Returns (dX [T,K] fp32 | None, dW [E,N,K] in x's dtype | None, d_topk [T,k] fp32 | None)."""
    lib = _lib.load()
    _require(dY, "dY", None, 2)
    _require(x, "x", dY.dtype, 2)
    T, K = x.shape
    N = dY.shape[1] if N is None else N
    E = sched.c.E
    if W is not None:
        _require(W, "W", x.dtype, 3)
        if tuple(W.shape) != (E, N, K):
            raise ValueError("W must be [E, N, K]")
    if dY.shape[0] != T or T != sched.c.T:
        raise ValueError("dY, x and the schedule disagree on T")
    dev = x.device
    code = _dtype_code(x)
    k = sched.c.k
    with _on(stream):
        dX = (out_dX if out_dX is not None else torch.empty((T, K), dtype=torch.float32, device=dev)) if dx else None
        dW = (out_dW if out_dW is not None else torch.empty((E, N, K), dtype=x.dtype, device=dev)) if dw else None
        dT = (out_dtopk if out_dtopk is not None else torch.empty((T, k), dtype=torch.float32, device=dev)) if dtopk else None
        ws_bytes = int(lib.moe_fused_bwd_workspace_bytes(ctypes.byref(sched.c), K, N, code))
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    if dX is not None:
        _require_out(dX, "out_dX", torch.float32, (T, K), dev)
    if dW is not None:
        _require_out(dW, "out_dW", x.dtype, (E, N, K), dev)
    if dT is not None:
        _require_out(dT, "out_dtopk", torch.float32, (T, k), dev)
    st = lib.moe_fused_bwd(_ptr(dY), _ptr(x), _ptr(W), ctypes.byref(sched.c), _ptr(dX), _ptr(dW),
                           _ptr(dT), K, N, code, _ptr(ws), ws_bytes, _stream(stream))
    _lib.check("moe_fused_bwd", st)
    return dX, dW, dT


def moe_tile_map(sched: Schedule, N: int, BM: int, BN: int, owner_capacity: Optional[int] = None,
                 stream=None):
    """Flat tile space of an N-column output with BM x BN tiles: (tile_start [E],
    total [1], owner [owner_capacity]) ([GG] "Problem descriptors and the tile
    scheduler")."""
    lib = _lib.load()
    E = sched.c.E
    tiles_n = -(-N // BN)
    if owner_capacity is None:
        owner_capacity = (sched.c.R // BM + E) * tiles_n + 1
    dev = sched.workspace.device
    with _on(stream):
        tile_start = torch.empty(E, dtype=torch.int32, device=dev)
        total = torch.empty(1, dtype=torch.int32, device=dev)
        owner = torch.full((owner_capacity,), -1, dtype=torch.int32, device=dev)
    st = lib.moe_tile_map(ctypes.byref(sched.c), N, BM, BN, _ptr(tile_start), _ptr(total), _ptr(owner),
                          owner_capacity, _stream(stream))
    _lib.check("moe_tile_map", st)
    return tile_start, total, owner


def moe_set_tile_rows(rows: int) -> None:
    """Tile height of the routed kernels: 0 = chosen on the device per launch
    (default), 128 or 256 = forced for every later launch of this process."""
    _lib.check("moe_set_tile_rows", _lib.load().moe_set_tile_rows(int(rows)))


def moe_set_combine(mode: int) -> None:
    """How the fused forward / input gradient combine a token's k contributions:
    MOE_COMBINE_AUTO (default), MOE_COMBINE_ATOMIC or MOE_COMBINE_RANKED."""
    _lib.check("moe_set_combine", _lib.load().moe_set_combine(int(mode)))


def moe_timing_enable(enable: bool = True) -> None:
    """Start (clearing earlier records) or stop per-kernel event timing."""
    _lib.check("moe_timing_enable", _lib.load().moe_timing_enable(1 if enable else 0))


def moe_timing_read(family: str):
    """(total milliseconds, launches) recorded for a kernel family."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _lib.check("moe_timing_read", _lib.load().moe_timing_read(family.encode(), ctypes.byref(ms),
                                                              ctypes.byref(n)))
    return ms.value, n.value


class MoEFunction(torch.autograd.Function):
    """Differentiable fused MoE layer y = moe(x, W, expert_ids, topk_weights)
    over the C ABI (the card's "Usage": gradients reach the tokens, the expert
    weights and the routing weights)."""

    @staticmethod
    def forward(ctx, x, W, expert_ids, topk_weights):
        sched = moe_build_schedule(expert_ids, topk_weights.detach().float().contiguous(), W.shape[0])
        y = moe_fused_fwd(x.detach().contiguous(), W.detach().contiguous(), sched)
        ctx.save_for_backward(x, W)
        ctx.sched = sched
        ctx.w_dtype = topk_weights.dtype
        return y

    @staticmethod
    def backward(ctx, gy):
        x, W = ctx.saved_tensors
        dY = gy.to(x.dtype).contiguous()
        dX, dW, dT = moe_fused_bwd(dY, x.detach().contiguous(), W.detach().contiguous(), ctx.sched,
                                   dx=ctx.needs_input_grad[0], dw=ctx.needs_input_grad[1],
                                   dtopk=ctx.needs_input_grad[3])
        return (dX.to(x.dtype) if dX is not None else None, dW, None,
                dT.to(ctx.w_dtype) if dT is not None else None)


def moe(x, W, expert_ids, topk_weights):
    return MoEFunction.apply(x, W, expert_ids, topk_weights)


class GatedMoEFunction(torch.autograd.Function):
    """Differentiable gated expert FFN y = gated_moe(x, W_gu, W_down, expert_ids,
    topk_weights) over the C ABI: the forward keeps h and the fp32 gate/up
    values, the backward returns the gradients of x, both weights and the
    routing weights ([GG] "Choosing an implementation", "The backward pass")."""

    @staticmethod
    def forward(ctx, x, W_gu, W_down, expert_ids, topk_weights):
        sched = moe_build_schedule(expert_ids, topk_weights.detach().float().contiguous(),
                                   W_gu.shape[0])
        y, h, gu = moe_gated_ffn_fwd(x.detach().contiguous(), W_gu.detach().contiguous(),
                                     W_down.detach().contiguous(), sched, save_gu=True)
        ctx.save_for_backward(x, W_gu, W_down, h, gu)
        ctx.sched = sched
        ctx.w_dtype = topk_weights.dtype
        return y

    @staticmethod
    def backward(ctx, gy):
        x, W_gu, W_down, h, gu = ctx.saved_tensors
        dY = gy.to(x.dtype).contiguous()
        dX, dWgu, dWd, dT = moe_gated_ffn_bwd(
            dY, x.detach().contiguous(), W_gu.detach().contiguous(), W_down.detach().contiguous(),
            ctx.sched, gu, h, dx=ctx.needs_input_grad[0], dw_gu=ctx.needs_input_grad[1],
            dw_down=ctx.needs_input_grad[2], dtopk=ctx.needs_input_grad[4])
        return (dX.to(x.dtype) if dX is not None else None, dWgu, dWd, None,
                dT.to(ctx.w_dtype) if dT is not None else None)


def gated_moe(x, W_gu, W_down, expert_ids, topk_weights):
    return GatedMoEFunction.apply(x, W_gu, W_down, expert_ids, topk_weights)
