"""Helpers shared by the GPU parity tests: moving seeded inputs to the device
and comparing results with the oracle."""
import sys

import numpy as np
import torch

from moe_variable_size_amd import workloads as WL


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def dev(t: "WL.Tensor | np.ndarray", bf16: bool = None) -> torch.Tensor:
    """Device tensor of a seeded input: bf16 bit patterns as torch.bfloat16,
    otherwise fp32/int as is."""
    if isinstance(t, WL.Tensor):
        if t.bits is not None and bf16 is not False:
            return torch.from_numpy(t.bits.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(t.values)).cuda()
    return torch.from_numpy(np.ascontiguousarray(t)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def max_rel(got: np.ndarray, ref: np.ndarray) -> float:
    """Normwise max relative error: max|g - o| / max|o|."""
    den = float(np.max(np.abs(ref)))
    num = float(np.max(np.abs(got.astype(np.float64) - ref)))
    return num / den if den > 0 else num


def rel_fro(got: np.ndarray, ref: np.ndarray) -> float:
    den = float(np.linalg.norm(ref.ravel()))
    num = float(np.linalg.norm(got.astype(np.float64).ravel() - ref.ravel()))
    return num / den if den > 0 else num


BF16_MAX_REL = 1e-2
BF16_REL_FRO = 3e-3
F32_MAX_REL = 1e-4


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str) -> None:
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    mr = max_rel(got, ref)
    if dtype == "f32":
        assert mr <= F32_MAX_REL, f"{what}: max_rel {mr:.3e} > {F32_MAX_REL}"
    else:
        rf = rel_fro(got, ref)
        assert mr <= BF16_MAX_REL and rf <= BF16_REL_FRO, \
            f"{what}: max_rel {mr:.3e} (<= {BF16_MAX_REL}) rel_fro {rf:.3e} (<= {BF16_REL_FRO})"
