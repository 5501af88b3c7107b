"""Kernel-family attribution of the HBM counter reduction (host logic only)."""
from moe_variable_size_amd import counters as C


def test_families_of_demangled_names():
    ns = "moe::(anonymous namespace)::"
    f = lambda t: C._family(ns + t + "(moe::(anonymous namespace)::FwdArgs)")
    assert f("mfma_fwd_kernel<256, 256, 2, 4, 1, float, false, false>") == "fused_fwd"
    assert f("mfma_fwd_kernel<64, 256, 1, 4, 1, float, false, false>") == "decode_fwd"
    assert f("mfma_fwd_kernel<256, 256, 2, 4, 1, float, true, false>") == "fused_fwd_fp8"
    assert f("mfma_fwd_kernel<64, 256, 1, 4, 1, float, true, false>") == "decode_fwd_fp8"
    assert f("mfma_fwd_kernel<256, 256, 2, 4, 2, float, false, false>") == "gated_up"
    assert f("mfma_fwd_kernel<256, 256, 2, 4, 3, float, false, false>") == "gated_down"
    assert f("mfma_fwd_kernel<256, 256, 2, 4, 0, unsigned short, false, false>") == "grouped_gemm"
    assert f("mfma_fwd_kernel<256, 256, 2, 4, 1, float, true, true>") == "fused_fwd_mx"
    assert f("mfma_fwd_kernel<64, 256, 1, 4, 1, float, true, true>") == "decode_fwd_mx"
    assert C._family(ns + "mfma_dx_kernel<4, false, false>(moe::(anonymous namespace)::DxArgs)") == "bwd_dx"
    assert C._family(ns + "mfma_dx_kernel<4, true, false>(DxArgs)") == "gated_bwd_dh"
    assert C._family(ns + "mfma_dx_kernel<4, false, true>(DxArgs)") == "gated_bwd_dx"
    assert C._family(ns + "mfma_dw_kernel<unsigned short, 8, 0>(DwArgs)") == "bwd_dw"
    assert C._family(ns + "mfma_dw_kernel<unsigned short, 8, 1>(DwArgs)") == "gated_bwd_dw_down"
    assert C._family(ns + "mfma_dw_kernel<unsigned short, 8, 2>(DwArgs)") == "gated_bwd_dw_gu"
    # with the combine-mode parameter the kernels carry now (1 = ranked)
    assert f("mfma_fwd_kernel<256, 256, 2, 4, 1, float, false, false, 0>") == "fused_fwd"
    assert f("mfma_fwd_kernel<256, 256, 2, 4, 1, float, false, false, 1>") == "fused_fwd_ranked"
    assert f("mfma_fwd_kernel<64, 256, 1, 4, 1, float, true, true, 0>") == "decode_fwd_mx"
    assert C._family(ns + "mfma_dx_kernel<4, false, false, 0>(DxArgs)") == "bwd_dx"
    assert C._family(ns + "mfma_dx_kernel<4, false, false, 1>(DxArgs)") == "bwd_dx_ranked"
    assert C._family(ns + "mfma_dx_kernel<4, true, false, 0>(DxArgs)") == "gated_bwd_dh"
    assert C._family(ns + "mfma_dw_kernel<unsigned short, 8, 0, true>(DwArgs)") == "bwd_dw"
    assert C._family(ns + "mfma_dw_kernel<unsigned short, 8, 0, false>(DwArgs)") == "bwd_dw_unweighted"
    assert C._family(ns + "mfma_dw_kernel<unsigned short, 8, 2, false>(DwArgs)") == "gated_bwd_dw_gu"
    # with the work-queue parameter
    assert C._family(ns + "mfma_dw_kernel<unsigned short, 8, 0, true, true>(DwArgs)") == "bwd_dw"
    assert C._family(ns + "mfma_dw_kernel<unsigned short, 8, 0, true, false>(DwArgs)") == "bwd_dw"
    assert C._family(ns + "mfma_dw_kernel<unsigned short, 8, 0, false, true>(DwArgs)") == "bwd_dw_unweighted"
    assert C._family(ns + "mfma_dw_kernel<unsigned short, 8, 1, true, false>(DwArgs)") == "gated_bwd_dw_down"
    assert C._family("__amd_rocclr_copyBuffer") == "copy"
    assert C._family(ns + "sched_hist_kernel(int const*)") is None
