"""The C ABI library: loads, exports every declared symbol, and rejects bad
arguments on the host before any launch (no GPU needed)."""
import ctypes
import os
import re

import pytest

from moe_variable_size_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_vs.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("library not built (run __graft_entry__.build())")
    return _lib.load()


def test_header_declares_the_four_entry_points():
    names = _declared()
    for n in ("moe_build_schedule", "grouped_gemm", "moe_fused_fwd", "moe_fused_bwd"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), f"missing export {n}"
    assert set(names) == set(_lib.SIGNATURES), "binding signatures and header disagree"


def test_status_strings(lib):
    assert lib.moe_status_string(0) == b"ok"
    for code in range(1, 8):
        assert lib.moe_status_string(code) != b"unknown status"
    assert lib.moe_version().startswith(b"moe_vs")


def test_workspace_query(lib):
    b = lib.moe_schedule_workspace_bytes(4096, 2, 8, 0, 0)
    assert b >= 3 * 4 * 8192 and b % 256 == 0
    assert lib.moe_schedule_workspace_bytes(0, 2, 8, 0, 0) == 0
    assert lib.moe_schedule_workspace_bytes(10, 0, 8, 0, 0) == 0
    assert lib.moe_schedule_workspace_bytes(10, 2, 2000, 0, 0) == 0
    assert lib.moe_schedule_workspace_bytes(10, 2, 8, 1, 0) == 0
    assert lib.moe_schedule_workspace_bytes(10, 2, 8, 1, 4) >= 3 * 4 * 32
    assert lib.moe_schedule_workspace_bytes(10, 2, 8, 7, 4) == 0


FAKE = ctypes.c_void_p(1 << 20)   # never dereferenced: validation fails first


def test_build_schedule_rejects_before_launch(lib):
    s = _lib.MoeSchedule()
    ref = ctypes.byref(s)
    assert lib.moe_build_schedule(None, None, 10, 2, 8, 0, 0, FAKE, 1 << 20, ref, None) == 1
    assert lib.moe_build_schedule(FAKE, None, 0, 2, 8, 0, 0, FAKE, 1 << 20, ref, None) == 2
    assert lib.moe_build_schedule(FAKE, None, 10, 2, 2000, 0, 0, FAKE, 1 << 20, ref, None) == 7
    assert lib.moe_build_schedule(FAKE, None, 10, 2, 8, 0, 0, None, 0, ref, None) == 5
    assert lib.moe_build_schedule(FAKE, None, 10, 2, 8, 0, 0, FAKE, 16, ref, None) == 5
    assert lib.moe_build_schedule(ctypes.c_void_p((1 << 20) + 2), None, 10, 2, 8, 0, 0, FAKE,
                                  1 << 20, ref, None) == 4


def test_gemm_entry_points_reject_before_launch(lib):
    P = FAKE
    assert lib.grouped_gemm(P, P, P, P, 10, 0, 8, 2, 1, 0, None) == 2          # K = 0
    assert lib.grouped_gemm(P, P, P, P, 10, 8, 8, 2, 5, 0, None) == 3          # dtype
    assert lib.grouped_gemm(P, P, P, P, 10, 8, 8, 2, 0, 1, None) == 3          # fp32 in, bf16 out
    assert lib.grouped_gemm(None, P, P, P, 10, 8, 8, 2, 1, 0, None) == 1
    assert lib.grouped_gemm(ctypes.c_void_p((1 << 20) + 8), P, P, P, 10, 8, 8, 2, 1, 0, None) == 4
    assert lib.grouped_gemm(P, P, P, P, 1 << 20, 4096, 8, 2, 1, 0, None) == 7  # > 2^31 bytes
    assert lib.grouped_gemm(None, None, None, None, 0, 8, 8, 2, 1, 0, None) == 0  # M = 0: nothing
    s = _lib.MoeSchedule()
    assert lib.moe_fused_fwd(P, P, ctypes.byref(s), P, 8, 8, 1, None) == 1      # empty descriptor
    s.T, s.S, s.R, s.k, s.E = 4, 8, 8, 2, 3
    for f in ("counts", "offsets", "block_start", "expert_order", "row_to_assign", "row_to_token",
              "row_weight", "status", "dw_queue"):
        setattr(s, f, 1 << 20)
    assert lib.moe_fused_fwd(P, P, ctypes.byref(s), P, 8, 8, 9, None) == 3
    assert lib.moe_fused_fwd(None, P, ctypes.byref(s), P, 8, 8, 1, None) == 1
    s.R = 7
    assert lib.moe_fused_fwd(P, P, ctypes.byref(s), P, 8, 8, 1, None) == 2
    s.R = 8
    assert lib.moe_fused_bwd(P, P, None, ctypes.byref(s), P, None, None, 8, 8, 1, None, 0, None) == 1
    assert lib.moe_tile_map(ctypes.byref(s), 8, 48, 16, P, P, P, 4, None) == 2   # BM not in {32..256}
    assert lib.moe_timing_read(b"nope", ctypes.byref(ctypes.c_double()), ctypes.byref(ctypes.c_int64())) == 2


def test_gated_ffn_rejects_before_launch(lib):
    P = FAKE
    s = _lib.MoeSchedule()
    s.T, s.S, s.R, s.k, s.E = 4, 8, 8, 2, 3
    for f in ("counts", "offsets", "block_start", "expert_order", "row_to_assign", "row_to_token",
              "row_weight", "status", "dw_queue"):
        setattr(s, f, 1 << 20)
    r = ctypes.byref(s)
    assert lib.moe_gated_ffn_fwd(P, P, P, r, P, None, P, 16, 16, 16, 5, None) == 3      # dtype code
    assert lib.moe_gated_ffn_fwd(P, P, None, r, P, None, P, 16, 16, 16, 1, None) == 1   # no W_down
    assert lib.moe_gated_ffn_fwd(P, P, P, r, None, None, P, 16, 16, 16, 1, None) == 1   # no h
    assert lib.moe_gated_ffn_fwd(P, P, P, r, P, None, P, 16, 0, 16, 1, None) == 2      # F = 0
    assert lib.moe_gated_ffn_fwd(P, P, P, r, ctypes.c_void_p((1 << 20) + 2), None, P, 16, 16, 16, 1,
                                 None) == 4                                       # h misaligned (16 B)
    # F % 8 != 0 takes the vector-ALU kernels, which need element alignment only
    assert lib.moe_gated_ffn_fwd(P, P, P, r, ctypes.c_void_p((1 << 20) + 1), None, P, 16, 12, 16, 1,
                                 None) == 4                                       # h misaligned (2 B)
    assert lib.moe_gated_ffn_fwd(P, P, P, r, ctypes.c_void_p((1 << 20) + 2), None, P, 16, 12, 16, 0,
                                 None) == 4                                       # fp32 h misaligned (4 B)
    assert lib.moe_gated_ffn_fwd(P, P, P, r, P, None, P, 1 << 16, 1 << 15, 16, 1, None) == 7  # W_gu > 2^31 B


def test_fp8_rejects_before_launch(lib):
    P = FAKE
    s = _lib.MoeSchedule()
    s.T, s.S, s.R, s.k, s.E = 4, 8, 8, 2, 3
    for f in ("counts", "offsets", "block_start", "expert_order", "row_to_assign", "row_to_token",
              "row_weight", "status", "dw_queue"):
        setattr(s, f, 1 << 20)
    r = ctypes.byref(s)
    assert lib.moe_fused_fwd_fp8(P, P, P, P, r, P, 24, 8, None) == 2      # K % 16 != 0
    assert lib.moe_fused_fwd_fp8(P, None, P, P, r, P, 32, 8, None) == 1   # no x_scale
    assert lib.moe_fused_fwd_fp8(ctypes.c_void_p((1 << 20) + 8), P, P, P, r, P, 32, 8, None) == 4
    assert lib.moe_fused_fwd_fp8(P, P, P, P, r, P, 1 << 16, 1 << 15, None) == 7   # W_q >= 2^31 B


def test_gated_backward_rejects_before_launch(lib):
    P = FAKE
    s = _lib.MoeSchedule()
    s.T, s.S, s.R, s.k, s.E = 4, 8, 8, 2, 3
    for f in ("counts", "offsets", "block_start", "expert_order", "row_to_assign", "row_to_token",
              "row_weight", "status", "dw_queue"):
        setattr(s, f, 1 << 20)
    r = ctypes.byref(s)
    assert lib.moe_gated_ffn_bwd_workspace_bytes(r, 16) >= 8 * 32 * 2
    assert lib.moe_gated_ffn_bwd(P, P, P, P, r, None, P, P, P, P, P, 16, 16, 16, 1, P, 1 << 20,
                                 None) == 1                                          # no gu
    assert lib.moe_gated_ffn_bwd(P, P, P, P, r, P, P, P, P, P, P, 16, 16, 16, 1, None, 0,
                                 None) == 5                                          # no workspace
    assert lib.moe_gated_ffn_bwd(P, P, P, P, r, P, P, P, P, P, P, 16, 16, 16, 5, P, 1 << 20,
                                 None) == 3                                          # dtype code
    assert lib.moe_gated_ffn_bwd(P, P, P, P, r, P, P, P, P, P, P, 16, 12, 16, 0, P, 100,
                                 None) == 5                                          # fp32 dgu workspace
    assert lib.moe_gated_ffn_bwd(P, P, P, P, r, P, ctypes.c_void_p((1 << 20) + 2), P, P, P, P, 16, 12,
                                 16, 0, P, 1 << 20, None) == 4                       # fp32 h misaligned


def test_mx_rejects_before_launch(lib):
    P = FAKE
    s = _lib.MoeSchedule()
    s.T, s.S, s.R, s.k, s.E = 4, 8, 8, 2, 3
    for f in ("counts", "offsets", "block_start", "expert_order", "row_to_assign", "row_to_token",
              "row_weight", "status", "dw_queue"):
        setattr(s, f, 1 << 20)
    r = ctypes.byref(s)
    assert lib.moe_fused_fwd_mx(P, P, P, P, r, P, 64, 8, None) == 2        # K % 128 != 0
    assert lib.moe_fused_fwd_mx(P, None, P, P, r, P, 128, 8, None) == 1    # no x block scales
    assert lib.moe_fused_fwd_mx(P, ctypes.c_void_p((1 << 20) + 2), P, P, r, P, 128, 8, None) == 4


def test_tile_rows_setting(lib):
    assert lib.moe_set_tile_rows(100) == 2
    assert lib.moe_set_tile_rows(64 + 1) == 2
    for rows in (128, 256, 0):
        assert lib.moe_set_tile_rows(rows) == 0
