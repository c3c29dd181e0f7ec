"""CPU checks of the C ABI: the library builds, loads and exports every entry
point that include/ptgg.h declares.  No compute call is made (no GPU here)."""
import ctypes
import os
import re

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "ptgg.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pt_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import moe_expert_grouped_gemm_amd as pt
    if not os.path.exists(pt.lib_path()):
        from moe_expert_grouped_gemm_amd import build
        build.build()
    return ctypes.CDLL(pt.lib_path())


def test_header_declares_the_boundary():
    names = declared_functions()
    for fn in ("pt_grouped_gemm_fwd", "pt_grouped_gemm_dgrad", "pt_grouped_gemm_wgrad", "pt_mx_quantize"):
        assert fn in names


def test_library_exports_every_declared_symbol(lib):
    missing = [fn for fn in declared_functions() if not hasattr(lib, fn)]
    assert not missing, missing


def test_binding_lists_every_declared_symbol():
    import moe_expert_grouped_gemm_amd as pt
    assert sorted(pt.EXPORTS) == declared_functions()
    for fn in pt.EXPORTS:
        assert callable(getattr(pt, fn))


def test_status_strings_and_version_host_only():
    import moe_expert_grouped_gemm_amd as pt
    assert pt.pt_status_string(0) == "PT_OK"
    assert pt.pt_status_string(2) == "PT_ERR_UNSUPPORTED"
    assert pt.pt_status_string(99) == "PT_ERR_UNKNOWN"
    assert "gfx950" in pt.pt_version()
    assert pt.pt_grouped_gemm_workspace_size(pt.PT_OP_FWD, 4, 256, 256, 128, pt.PT_BF16) >= 4


def test_enums_match_header():
    import moe_expert_grouped_gemm_amd as pt
    text = open(HEADER).read()
    for name in ("PT_BF16", "PT_MXFP8_E4M3", "PT_MXFP4_E2M1", "PT_EPI_NONE", "PT_EPI_SWIGLU",
                 "PT_EPI_SWIGLU_MXFP4", "PT_OP_FWD", "PT_OP_DGRAD", "PT_OP_WGRAD"):
        m = re.search(r"\b%s\s*=\s*(\d+)" % name, text)
        assert m and int(m.group(1)) == getattr(pt, name), name


def test_package_refuses_to_run_without_gpu():
    import torch
    import moe_expert_grouped_gemm_amd as pt
    if torch.cuda.is_available():
        pytest.skip("GPU present")
    with pytest.raises(RuntimeError):
        pt.load()


def test_new_enums_match_header():
    import moe_expert_grouped_gemm_amd as pt
    text = open(HEADER).read()
    for name in ("PT_FP8_E4M3", "PT_FP8_E4M3_ROWWISE", "PT_OP_DGRAD_SWIGLU"):
        m = re.search(r"\b%s\s*=\s*(\d+)" % name, text)
        assert m and int(m.group(1)) == getattr(pt, name), name
    for name in ("PT_CONFIG_RULES", "PT_CONFIG_TUNE"):
        m = re.search(r"#define\s+%s\s+\((-?\d+)\)" % name, text)
        assert m and int(m.group(1)) == getattr(pt, name), name
    m = re.search(r"#define\s+PT_MAX_GROUPS\s+(\d+)", text)
    assert m and int(m.group(1)) == pt.PT_MAX_GROUPS


def test_workspace_sizes_host_only():
    # closed forms of the scratch each op needs (host arithmetic, no GPU)
    import moe_expert_grouped_gemm_amd as pt
    r256 = lambda x: (x + 255) // 256 * 256
    G, M, N, K = 32, 65536, 5760, 2880
    base = pt.pt_grouped_gemm_workspace_size(pt.PT_OP_FWD, 1, 1, 1, 1, pt.PT_BF16)
    assert base == 1280

    # the weight gradient's split reduction: floor(M / L) fp32 [K, N] slots,
    # L = max(512, ceil(M * tiles / 1024)), tiles = ceil(K/256) * ceil(N/256)
    def split(M, N, K):
        tiles = -(-K // 256) * -(-N // 256)
        L = max(512, -(-M * tiles // 1024))
        return r256((M // L) * K * N * 4)
    assert split(M, N, K) == r256(3 * K * N * 4)            # L = 17664 here: three slots
    assert pt.pt_grouped_gemm_workspace_size(pt.PT_OP_WGRAD, G, M, N, K, pt.PT_BF16) == base + split(M, N, K)
    # MX: the experts' plan (block and stage starts), both gradients' codes
    # transposed to channel rows of `pitch` bytes (every expert padded to
    # whole 32-token blocks), their stage-major scale words (a stage is 128
    # code bytes of a row; each expert adds at most one partial stage), then
    # the split reduction's slots
    for dt, tok_bytes, wpr in ((pt.PT_MXFP8_E4M3, 1.0, 1), (pt.PT_MXFP4_E2M1, 0.5, 2)):
        for g_, m_, n_, k_ in ((G, M, N, K), (3, 40, 64, 136), (5, 0, 64, 64)):
            pitch = -(-int(32 * (m_ // 32 + g_) * tok_bytes) // 128) * 128
            stages = pitch // 128 + g_
            want = (base + r256(8 * g_) + r256(k_ * pitch) + r256(n_ * pitch) + r256(stages * k_ * wpr * 4) +
                    r256(stages * n_ * wpr * 4) + split(m_, n_, k_))
            assert pt.pt_grouped_gemm_workspace_size(pt.PT_OP_WGRAD, g_, m_, n_, k_, dt) == want, (dt, g_, m_)
    # FP8 with one factor per tensor: the plan and both gradients' transposed
    # codes as for MXFP8 (no scale words, no split), then 256 bytes for the
    # amax words and factors of pt_grouped_gemm_wgrad_quantize
    pitch8 = -(-32 * (M // 32 + G) // 128) * 128
    assert (pt.pt_grouped_gemm_workspace_size(pt.PT_OP_WGRAD, G, M, N, K, pt.PT_FP8_E4M3) ==
            base + r256(8 * G) + r256(K * pitch8) + r256(N * pitch8) + 256)
    # one output tile per expert and 14030 rows: 512-token chunks, 27 slots
    assert pt.pt_grouped_gemm_workspace_size(pt.PT_OP_WGRAD, 7, 14030, 256, 256, pt.PT_BF16) == \
        base + 27 * 256 * 256 * 4
    # fewer rows than one chunk: nothing to split
    assert pt.pt_grouped_gemm_workspace_size(pt.PT_OP_WGRAD, 4, 500, 256, 256, pt.PT_BF16) == base
    # the MX forward adds stage-major scale copies: more than the queues alone
    assert pt.pt_grouped_gemm_workspace_size(pt.PT_OP_FWD, G, M, N, K, pt.PT_MXFP8_E4M3) > base


def test_argument_checks_host_only():
    # refusals decided before any device call (no GPU needed)
    import ctypes
    import math
    import moe_expert_grouped_gemm_amd as pt
    L = pt.load(require_gpu=False)
    lens = (ctypes.c_int64 * 4)(1, 2, 3, 4)
    lp = ctypes.cast(lens, ctypes.c_void_p).value
    assert L.pt_grouped_gemm_fwd(None, None, None, None, None, None, lp, None, 0, 10, 64, 64, 0, 0, 0, 0.0,
                                 None, 0, None) == 1                                  # G = 0
    assert L.pt_grouped_gemm_fwd(None, None, None, None, None, None, lp, None, 4, 10, 64, 64, 0, 0, 1, math.nan,
                                 None, 0, None) == 1                                  # NaN limit
    assert L.pt_grouped_gemm_dgrad_swiglu(None, None, None, None, None, None, lp, None, 4, 10, 64, 64, 0, 0,
                                          math.nan, None, 0, None) == 1
    assert L.pt_stack_experts(None, None, 2, 64, 64, 2, None, 0, None) == 1          # layout flag
    assert L.pt_stack_experts(None, None, 2, 60, 64, 0, None, 0, None) == 2          # rows % 8
    assert L.pt_stack_experts(None, None, 0, 64, 64, 0, None, 0, None) == 0          # nothing to do
    assert L.pt_mx_quantize_experts(None, None, None, None, None, 2, 64, 64, 1, None, 0, None) == 1
    assert L.pt_mx_quantize_tokens(None, lp, None, None, None, 4, 10, 64, 0, None, 0, None) == 2   # BF16
    # the MX weight gradient from bf16 gradients: argument refusals, then the
    # dtype (MX formats only), then the 8-column alignment
    mg = (ctypes.c_float * 4)()
    mp = ctypes.cast(mg, ctypes.c_void_p).value
    W = L.pt_grouped_gemm_wgrad_quantize
    assert W(None, None, None, lp, None, 4, 10, 64, 64, 1, 0, 1, None, 0, None) == 1     # no main_grad
    assert W(mp, mp, mp, lp, None, 4, 10, 64, 64, 1, 2, 1, None, 0, None) == 1          # trans_out
    assert W(mp, mp, mp, lp, None, 4, 10, 64, 64, 1, 0, 2, None, 0, None) == 1          # accumulate
    assert W(mp, mp, mp, lp, None, 4, 10, 64, 64, 0, 0, 1, None, 0, None) == 2          # BF16
    assert W(mp, mp, mp, lp, None, 4, 10, 64, 64, 4, 0, 1, None, 0, None) == 2          # FP8 row factors
    assert W(mp, mp, mp, lp, None, 4, 10, 64, 60, 2, 0, 1, None, 0, None) == 2          # K % 8


def test_config_mode_host_only():
    import moe_expert_grouped_gemm_amd as pt
    pt.pt_clear_gemm_tuning()
    try:
        assert pt.pt_set_gemm_config(2) == pt.PT_CONFIG_RULES
        assert pt.pt_set_gemm_config(pt.PT_CONFIG_TUNE) == 2
        with pytest.raises(ValueError):
            pt.pt_set_gemm_config(4)
        assert pt.pt_set_gemm_config(pt.PT_CONFIG_RULES) == pt.PT_CONFIG_TUNE
        for op in (pt.PT_OP_FWD, pt.PT_OP_DGRAD, pt.PT_OP_WGRAD, pt.PT_OP_DGRAD_SWIGLU):
            assert pt.pt_gemm_config_of(op, pt.PT_BF16, 0, 0, 8, 1000, 256, 256) == -1
        assert pt.pt_gemm_config_of(9, pt.PT_BF16, 0, 0, 8, 1000, 256, 256) == -1
    finally:
        pt.pt_set_gemm_config(pt.PT_CONFIG_RULES)
