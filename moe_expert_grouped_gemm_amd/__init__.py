"""MoE expert grouped GEMM for AMD Instinct MI355X (gfx950).

Thin ctypes binding over the C ABI in ``include/ptgg.h`` (``libptgg.so``,
built in-tree by ``build.py``).  Each ``pt_*`` function here has the C
function's name and argument order; it only turns torch tensors into device
pointers, picks the current HIP stream and raises on a non-zero status.
Every step of the computation runs in the library's HIP kernels: there is no
fallback path, and using the package without the built library or without a
GPU raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import build as _build

__all__ = [
    "PT_BF16", "PT_MXFP8_E4M3", "PT_MXFP4_E2M1", "PT_FP8_E4M3", "PT_FP8_E4M3_ROWWISE",
    "PT_EPI_NONE", "PT_EPI_SWIGLU", "PT_EPI_SWIGLU_MXFP4",
    "PT_OP_FWD", "PT_OP_DGRAD", "PT_OP_WGRAD",
    "load", "lib_path", "PtggError",
    "pt_grouped_gemm_fwd", "pt_grouped_gemm_dgrad", "pt_grouped_gemm_dgrad_swiglu",
    "pt_grouped_gemm_wgrad", "pt_grouped_gemm_wgrad_quantize", "pt_grouped_gemm_fwd_swiglu_save",
    "pt_grouped_gemm_fwd_noalloc", "pt_grouped_gemm_fwd_pitched", "pt_mx_quantize", "pt_mx_quantize_pitched",
    "pt_mx_quantize_t", "pt_mx_quantize_tokens", "pt_fp8_quantize", "pt_fp8_quantize_rows",
    "pt_stack_experts", "pt_mx_quantize_experts", "expert_addresses",
    "pt_set_gemm_config", "pt_gemm_config_of", "pt_clear_gemm_tuning", "PT_CONFIG_RULES", "PT_CONFIG_TUNE",
    "PT_OP_DGRAD_SWIGLU", "PT_MAX_GROUPS",
    "pt_grouped_gemm_workspace_size", "pt_read_error_flags", "pt_status_string", "pt_version",
]

PT_BF16, PT_MXFP8_E4M3, PT_MXFP4_E2M1, PT_FP8_E4M3, PT_FP8_E4M3_ROWWISE = 0, 1, 2, 3, 4
PT_EPI_NONE, PT_EPI_SWIGLU, PT_EPI_SWIGLU_MXFP4 = 0, 1, 2
PT_OP_FWD, PT_OP_DGRAD, PT_OP_WGRAD, PT_OP_DGRAD_SWIGLU = 0, 1, 2, 3
PT_CONFIG_RULES, PT_CONFIG_TUNE = -1, -2
PT_MAX_GROUPS = 1024

EXPORTS = (
    "pt_grouped_gemm_fwd", "pt_grouped_gemm_dgrad", "pt_grouped_gemm_dgrad_swiglu", "pt_grouped_gemm_wgrad",
    "pt_grouped_gemm_wgrad_quantize", "pt_grouped_gemm_fwd_swiglu_save", "pt_grouped_gemm_fwd_noalloc",
    "pt_grouped_gemm_fwd_pitched", "pt_mx_quantize", "pt_mx_quantize_pitched", "pt_mx_quantize_t", "pt_mx_quantize_tokens", "pt_fp8_quantize", "pt_fp8_quantize_rows",
    "pt_stack_experts", "pt_mx_quantize_experts",
    "pt_set_gemm_config", "pt_gemm_config_of", "pt_clear_gemm_tuning",
    "pt_grouped_gemm_workspace_size", "pt_read_error_flags", "pt_status_string", "pt_version",
)

_lib = None


class PtggError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {pt_status_string(status)} ({status})")
        self.status = status


def lib_path() -> str:
    return _build.LIB


def load(require_gpu: bool = True):
    """Load libptgg.so (building it first only if it has not been built)."""
    global _lib
    if require_gpu and not torch.cuda.is_available():
        raise RuntimeError("moe_expert_grouped_gemm_amd needs a gfx950 GPU; none is visible")
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB):
        _build.build()
    L = ctypes.CDLL(_build.LIB)
    p, i64, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
    L.pt_grouped_gemm_fwd.restype = i32
    L.pt_grouped_gemm_fwd.argtypes = [p, p, p, p, p, p, p, p, i64, i64, i64, i64, i32, i32, i32, f32, p, sz, p]
    L.pt_grouped_gemm_fwd_noalloc.restype = i32
    L.pt_grouped_gemm_fwd_noalloc.argtypes = [p, p, p, p, p, p, p, p, i64, i64, i64, i64, i32, i32, i32, f32, p]
    L.pt_grouped_gemm_dgrad.restype = i32
    L.pt_grouped_gemm_dgrad.argtypes = [p, p, p, p, p, p, p, i64, i64, i64, i64, i32, i32, p, sz, p]
    L.pt_grouped_gemm_dgrad_swiglu.restype = i32
    L.pt_grouped_gemm_dgrad_swiglu.argtypes = [p, p, p, p, p, p, p, p, i64, i64, i64, i64, i32, i32, f32, p, sz, p]
    L.pt_grouped_gemm_wgrad.restype = i32
    L.pt_grouped_gemm_wgrad.argtypes = [p, p, p, p, p, p, p, i64, i64, i64, i64, i32, i32, i32, p, sz, p]
    L.pt_grouped_gemm_wgrad_quantize.restype = i32
    L.pt_grouped_gemm_wgrad_quantize.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i32, i32, i32, p, sz, p]
    L.pt_mx_quantize.restype = i32
    L.pt_mx_quantize.argtypes = [p, p, p, i64, i64, i32, i32, p]
    L.pt_mx_quantize_pitched.restype = i32
    L.pt_mx_quantize_pitched.argtypes = [p, p, p, i64, i64, i32, i64, p]
    L.pt_grouped_gemm_fwd_pitched.restype = i32
    L.pt_grouped_gemm_fwd_pitched.argtypes = [p, p, p, p, p, p, p, p, i64, i64, i64, i64, i32, i32, f32, i64, p, sz, p]
    L.pt_mx_quantize_t.restype = i32
    L.pt_mx_quantize_t.argtypes = [p, p, p, i64, i64, i64, i32, p]
    L.pt_fp8_quantize.restype = i32
    L.pt_fp8_quantize.argtypes = [p, p, p, p, i64, i64, i64, p]
    L.pt_mx_quantize_tokens.restype = i32
    L.pt_mx_quantize_tokens.argtypes = [p, p, p, p, p, i64, i64, i64, i32, p, sz, p]
    L.pt_fp8_quantize_rows.restype = i32
    L.pt_fp8_quantize_rows.argtypes = [p, p, p, p, i64, i64, p]
    L.pt_grouped_gemm_workspace_size.restype = sz
    L.pt_grouped_gemm_fwd_swiglu_save.restype = i32
    L.pt_grouped_gemm_fwd_swiglu_save.argtypes = [p, p, p, p, p, p, p, p, i64, i64, i64, i64, i32, i32, f32, p, sz, p]
    L.pt_stack_experts.restype = i32
    L.pt_stack_experts.argtypes = [p, p, i64, i64, i64, i32, p, sz, p]
    L.pt_mx_quantize_experts.restype = i32
    L.pt_mx_quantize_experts.argtypes = [p, p, p, p, p, i64, i64, i64, i32, p, sz, p]
    L.pt_set_gemm_config.restype = i32
    L.pt_set_gemm_config.argtypes = [i32]
    L.pt_gemm_config_of.restype = i32
    L.pt_gemm_config_of.argtypes = [i32, i32, i32, i32, i64, i64, i64, i64]
    L.pt_clear_gemm_tuning.restype = None
    L.pt_clear_gemm_tuning.argtypes = []
    L.pt_grouped_gemm_workspace_size.argtypes = [i32, i64, i64, i64, i64, i32]
    L.pt_read_error_flags.restype = i32
    L.pt_read_error_flags.argtypes = [p, p, ctypes.POINTER(ctypes.c_uint32)]
    L.pt_status_string.restype = ctypes.c_char_p
    L.pt_status_string.argtypes = [i32]
    L.pt_version.restype = ctypes.c_char_p
    L.pt_version.argtypes = []
    _lib = L
    return L


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("device tensor expected")
    if not t.is_contiguous():
        raise ValueError("contiguous tensor expected")
    return t.data_ptr()


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn, status):
    if status != 0:
        raise PtggError(fn, status)


def pt_grouped_gemm_fwd(a, a_scale, b, b_scale, out, out_scale, group_lens, group_offs,
                        G, M, N, K, dtype, trans_b, epilogue, workspace=None, stream=None, swiglu_limit=0.0):
    L = load()
    _check("pt_grouped_gemm_fwd", L.pt_grouped_gemm_fwd(
        _ptr(a), _ptr(a_scale), _ptr(b), _ptr(b_scale), _ptr(out), _ptr(out_scale),
        _ptr(group_lens), _ptr(group_offs), G, M, N, K, dtype, trans_b, epilogue, swiglu_limit,
        _ptr(workspace), _nbytes(workspace), _stream(stream)))


def pt_grouped_gemm_fwd_noalloc(a, a_scale, b, b_scale, out, out_scale, group_lens, group_offs,
                                G, M, N, K, dtype, trans_b, epilogue, stream=None, swiglu_limit=0.0):
    L = load()
    _check("pt_grouped_gemm_fwd_noalloc", L.pt_grouped_gemm_fwd_noalloc(
        _ptr(a), _ptr(a_scale), _ptr(b), _ptr(b_scale), _ptr(out), _ptr(out_scale),
        _ptr(group_lens), _ptr(group_offs), G, M, N, K, dtype, trans_b, epilogue, swiglu_limit,
        _stream(stream)))


def pt_grouped_gemm_dgrad(dy, dy_scale, b, b_scale, dx, group_lens, group_offs,
                          G, M, N, K, dtype, trans_b, workspace=None, stream=None):
    L = load()
    _check("pt_grouped_gemm_dgrad", L.pt_grouped_gemm_dgrad(
        _ptr(dy), _ptr(dy_scale), _ptr(b), _ptr(b_scale), _ptr(dx),
        _ptr(group_lens), _ptr(group_offs), G, M, N, K, dtype, trans_b,
        _ptr(workspace), _nbytes(workspace), _stream(stream)))


def pt_grouped_gemm_fwd_swiglu_save(a, a_scale, b, b_scale, h, c, group_lens, group_offs, G, M, N, K, dtype, trans_b,
                                    workspace=None, stream=None, swiglu_limit=0.0):
    L = load()
    _check("pt_grouped_gemm_fwd_swiglu_save", L.pt_grouped_gemm_fwd_swiglu_save(
        _ptr(a), _ptr(a_scale), _ptr(b), _ptr(b_scale), _ptr(h), _ptr(c), _ptr(group_lens), _ptr(group_offs),
        G, M, N, K, dtype, trans_b, swiglu_limit, _ptr(workspace), _nbytes(workspace), _stream(stream)))


def pt_grouped_gemm_dgrad_swiglu(dy, b, c_saved, dc, group_lens, group_offs,
                                 G, M, N, K, trans_b, workspace=None, stream=None, swiglu_limit=0.0,
                                 dtype=PT_BF16, dy_scale=None, b_scale=None):
    L = load()
    _check("pt_grouped_gemm_dgrad_swiglu", L.pt_grouped_gemm_dgrad_swiglu(
        _ptr(dy), _ptr(dy_scale), _ptr(b), _ptr(b_scale), _ptr(c_saved), _ptr(dc), _ptr(group_lens),
        _ptr(group_offs), G, M, N, K, dtype, trans_b, swiglu_limit, _ptr(workspace), _nbytes(workspace),
        _stream(stream)))


def pt_grouped_gemm_wgrad(a, a_scale, dy, dy_scale, main_grad, group_lens, group_offs,
                          G, M, N, K, dtype, trans_out, accumulate, workspace=None, stream=None):
    L = load()
    _check("pt_grouped_gemm_wgrad", L.pt_grouped_gemm_wgrad(
        _ptr(a), _ptr(a_scale), _ptr(dy), _ptr(dy_scale), _ptr(main_grad),
        _ptr(group_lens), _ptr(group_offs), G, M, N, K, dtype, trans_out, accumulate,
        _ptr(workspace), _nbytes(workspace), _stream(stream)))


def pt_grouped_gemm_wgrad_quantize(a, dy, main_grad, group_lens, group_offs, G, M, N, K, dtype, trans_out,
                                   accumulate, workspace=None, stream=None):
    L = load()
    _check("pt_grouped_gemm_wgrad_quantize", L.pt_grouped_gemm_wgrad_quantize(
        _ptr(a), _ptr(dy), _ptr(main_grad), _ptr(group_lens), _ptr(group_offs), G, M, N, K, dtype, trans_out,
        accumulate, _ptr(workspace), _nbytes(workspace), _stream(stream)))


def pt_mx_quantize(x, q, scales, rows, cols, dtype, axis=1, stream=None):
    L = load()
    _check("pt_mx_quantize", L.pt_mx_quantize(
        _ptr(x), _ptr(q), _ptr(scales), rows, cols, dtype, axis, _stream(stream)))


def pt_mx_quantize_pitched(x, q, scales, rows, cols, dtype, q_pitch, stream=None):
    L = load()
    _check("pt_mx_quantize_pitched", L.pt_mx_quantize_pitched(
        _ptr(x), _ptr(q), _ptr(scales), rows, cols, dtype, q_pitch, _stream(stream)))


def pt_grouped_gemm_fwd_pitched(a, a_scale, b, b_scale, out, out_scale, group_lens, group_offs,
                                G, M, N, K, dtype, epilogue, code_pitch, workspace=None, stream=None,
                                swiglu_limit=0.0):
    L = load()
    _check("pt_grouped_gemm_fwd_pitched", L.pt_grouped_gemm_fwd_pitched(
        _ptr(a), _ptr(a_scale), _ptr(b), _ptr(b_scale), _ptr(out), _ptr(out_scale),
        _ptr(group_lens), _ptr(group_offs), G, M, N, K, dtype, epilogue, swiglu_limit, code_pitch,
        _ptr(workspace), _nbytes(workspace), _stream(stream)))


def pt_mx_quantize_t(x, q, scales, batch, rows, cols, dtype, stream=None):
    L = load()
    _check("pt_mx_quantize_t", L.pt_mx_quantize_t(
        _ptr(x), _ptr(q), _ptr(scales), batch, rows, cols, dtype, _stream(stream)))


def pt_fp8_quantize(x, q, amax, dequant, batch, rows, cols, stream=None):
    L = load()
    _check("pt_fp8_quantize", L.pt_fp8_quantize(
        _ptr(x), _ptr(q), _ptr(amax), _ptr(dequant), batch, rows, cols, _stream(stream)))


def pt_mx_quantize_tokens(x, group_lens, group_offs, q, scales, G, M, cols, dtype, workspace=None, stream=None):
    L = load()
    _check("pt_mx_quantize_tokens", L.pt_mx_quantize_tokens(
        _ptr(x), _ptr(group_lens), _ptr(group_offs), _ptr(q), _ptr(scales), G, M, cols, dtype,
        _ptr(workspace), _nbytes(workspace), _stream(stream)))


def pt_fp8_quantize_rows(x, q, amax, dequant, rows, cols, stream=None):
    L = load()
    _check("pt_fp8_quantize_rows", L.pt_fp8_quantize_rows(
        _ptr(x), _ptr(q), _ptr(amax), _ptr(dequant), rows, cols, _stream(stream)))


def expert_addresses(weights, device=None) -> torch.Tensor:
    """The device array of expert weight addresses that pt_stack_experts and
    pt_mx_quantize_experts take, from a list of device tensors (the tensors
    must outlive the calls that use it)."""
    for w in weights:
        _ptr(w)
    dev = device if device is not None else (weights[0].device if len(weights) else "cuda")
    return torch.tensor([w.data_ptr() for w in weights], dtype=torch.int64, device=dev)


def pt_stack_experts(experts, out, G, rows, cols, transpose, workspace=None, stream=None):
    L = load()
    _check("pt_stack_experts", L.pt_stack_experts(
        _ptr(experts), _ptr(out), G, rows, cols, transpose, _ptr(workspace), _nbytes(workspace), _stream(stream)))


def pt_mx_quantize_experts(experts, q, scales, q_t, scales_t, G, rows, cols, dtype, workspace=None, stream=None):
    L = load()
    _check("pt_mx_quantize_experts", L.pt_mx_quantize_experts(
        _ptr(experts), _ptr(q), _ptr(scales), _ptr(q_t), _ptr(scales_t), G, rows, cols, dtype,
        _ptr(workspace), _nbytes(workspace), _stream(stream)))


def pt_set_gemm_config(config) -> int:
    prev = load(require_gpu=False).pt_set_gemm_config(config)
    if prev == -3:
        raise ValueError(f"unknown GEMM configuration mode {config}")
    return int(prev)


def pt_gemm_config_of(op, dtype, epilogue, trans, G, M, N, K) -> int:
    return int(load(require_gpu=False).pt_gemm_config_of(op, dtype, epilogue, trans, G, M, N, K))


def pt_clear_gemm_tuning() -> None:
    load(require_gpu=False).pt_clear_gemm_tuning()


def pt_grouped_gemm_workspace_size(op, G, M, N, K, dtype) -> int:
    return int(load(require_gpu=False).pt_grouped_gemm_workspace_size(op, G, M, N, K, dtype))


def pt_read_error_flags(workspace, stream=None) -> int:
    L = load()
    flags = ctypes.c_uint32(0)
    _check("pt_read_error_flags", L.pt_read_error_flags(_ptr(workspace), _stream(stream), ctypes.byref(flags)))
    return int(flags.value)


def pt_status_string(status: int) -> str:
    return load(require_gpu=False).pt_status_string(int(status)).decode()


def pt_version() -> str:
    return load(require_gpu=False).pt_version().decode()
