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
