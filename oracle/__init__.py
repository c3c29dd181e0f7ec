"""Oracle for the MoE expert grouped GEMM: plain fp64 CPU reference.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the library never
does.  It shares no code with the HIP path and imports nothing from it.

Everything here works on numpy arrays of the raw stored bits:
  * bf16 tensors as ``uint16`` arrays,
  * MXFP8 (E4M3) codes as ``uint8`` [rows, cols],
  * MXFP4 (E2M1) codes as ``uint8`` [rows, cols/2], even column in the low
    nibble (the byte layout of ``float4_e2m1fn_x2`` named in the PR page
    "[Megatron-LM] feat: add grouped gemm fp4 support, ...", section "Changes"),
  * E8M0 scales as ``uint8`` [rows, cols/32], one per 32 consecutive elements.

The arithmetic lives in ``oracle.c`` (binary64 loops over experts, rows and
the reduction index); this module only marshals arrays and composes the
steps in the order the pages give them:

  FC1 -> SwiGLU -> (bf16) -> MXFP4 quantise -> FC2      (blog "Enabling
  DeepSeek-V4-Flash Training on AMD Instinct MI355X GPUs with Primus", section
  "MegaMoE: fusing communication into the grouped GEMM": SwiGLU sits between
  the two grouped GEMMs; the FC1 weight is [experts, 2I, H], gate then up).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

BF16, E4M3, E2M1 = 0, 1, 2          # operand encodings (oracle's own numbering)
EPI_NONE, EPI_SWIGLU, EPI_SWIGLU_MXFP4 = 0, 1, 2

_lib = None


def lib():
    """Load liboracle.so, compiling it first only if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        p, i64, i32, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        L.orc_bf16_value.restype = dbl
        L.orc_bf16_value.argtypes = [ctypes.c_uint16]
        L.orc_e4m3_value.restype = dbl
        L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
        L.orc_e2m1_value.restype = dbl
        L.orc_e2m1_value.argtypes = [ctypes.c_uint8]
        L.orc_e8m0_value.restype = dbl
        L.orc_e8m0_value.argtypes = [ctypes.c_uint8]
        L.orc_round_bf16.restype = ctypes.c_uint16
        L.orc_round_bf16.argtypes = [dbl]
        L.orc_decode.restype = None
        L.orc_decode.argtypes = [i32, p, p, i64, i64, p]
        L.orc_round_bf16_array.restype = None
        L.orc_round_bf16_array.argtypes = [p, i64, p]
        L.orc_round_f32_array.restype = None
        L.orc_round_f32_array.argtypes = [p, i64, p]
        L.orc_mx_quantize.restype = i32
        L.orc_mx_quantize.argtypes = [p, i64, i64, i32, i32, p, p]
        L.orc_fwd_rows.restype = i32
        L.orc_fwd_rows.argtypes = [i32, p, p, p, p, p, i64, i64, i64, i64, i32, p, i64, p]
        L.orc_dgrad_rows.restype = i32
        L.orc_dgrad_rows.argtypes = [p, p, p, i64, i64, i64, i64, i32, p, i64, p]
        L.orc_wgrad_rows.restype = i32
        L.orc_wgrad_rows.argtypes = [p, p, p, i64, i64, i64, i64, p, p, i64, p]
        L.orc_mx_quantize_tokens.restype = i64
        L.orc_mx_quantize_tokens.argtypes = [p, p, i64, i64, i64, ctypes.c_int, p, p]
        L.orc_fp8_quantize.restype = None
        L.orc_fp8_quantize.argtypes = [p, i64, i64, p, p, p]
        L.orc_swiglu.restype = None
        L.orc_swiglu.argtypes = [p, i64, i64, ctypes.c_double, p]
        L.orc_swiglu_bwd.restype = None
        L.orc_swiglu_bwd.argtypes = [p, p, i64, i64, ctypes.c_double, p]
        L.orc_threads.restype = i32
        L.orc_threads.argtypes = []
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def threads() -> int:
    return lib().orc_threads()


# ------------------------------------------------------------------ formats
def bf16_value(bits: int) -> float:
    return lib().orc_bf16_value(int(bits))


def e4m3_value(code: int) -> float:
    return lib().orc_e4m3_value(int(code))


def e2m1_value(nibble: int) -> float:
    return lib().orc_e2m1_value(int(nibble))


def e8m0_value(code: int) -> float:
    return lib().orc_e8m0_value(int(code))


def decode(dtype: int, data: np.ndarray, scale: np.ndarray | None, rows: int, cols: int) -> np.ndarray:
    """Exact binary64 values of a stored [rows, cols] matrix."""
    if dtype == BF16:
        data = _c(data, np.uint16)
    else:
        data = _c(data, np.uint8)
        scale = _c(scale, np.uint8)
    out = np.empty((rows, cols), np.float64)
    lib().orc_decode(dtype, _ptr(data), _ptr(scale), rows, cols, _ptr(out))
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round binary64 values to bf16 bit patterns (nearest, ties to even)."""
    x = _c(x, np.float64)
    out = np.empty(x.shape, np.uint16)
    lib().orc_round_bf16_array(_ptr(x), x.size, _ptr(out))
    return out


def round_f32(x: np.ndarray) -> np.ndarray:
    x = _c(x, np.float64)
    out = np.empty(x.shape, np.float32)
    lib().orc_round_f32_array(_ptr(x), x.size, _ptr(out))
    return out


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    bits = _c(bits, np.uint16)
    return decode(BF16, bits.reshape(1, -1), None, 1, bits.size).reshape(bits.shape)


def mx_quantize(x_bits: np.ndarray, dtype: int, axis: int = 1):
    """OCP-MX quantise a bf16 matrix; returns (codes, scales)."""
    x_bits = _c(x_bits, np.uint16)
    rows, cols = x_bits.shape
    if axis == 1:
        qshape = (rows, cols) if dtype == E4M3 else (rows, cols // 2)
        sshape = (rows, cols // 32)
    else:
        qshape = (rows, cols) if dtype == E4M3 else (rows // 2, cols)
        sshape = (rows // 32, cols)
    q = np.zeros(qshape, np.uint8)
    s = np.zeros(sshape, np.uint8)
    rc = lib().orc_mx_quantize(_ptr(x_bits), rows, cols, dtype, axis, _ptr(q), _ptr(s))
    if rc:
        raise ValueError("orc_mx_quantize: bad arguments")
    return q, s


def stack_experts(weights, transpose: bool) -> np.ndarray:
    """The stacked expert weight ([Primus DeepSeek-V4-Flash blog],
    "Performance optimizations", kernel-fusion table, grouped expert weight
    stack): out[g] = W_g, or W_g^T with transpose.  Pure data movement, so
    the definition is numpy's stack of the (transposed) matrices."""
    return np.stack([np.ascontiguousarray(w.T) if transpose else np.asarray(w) for w in weights])


def mx_quantize_experts(weights, dtype: int):
    """Both MX weight caches per expert: (q, s) = mx_quantize(W_g) along the
    columns, stacked; (qt, st) = mx_quantize(W_g^T) along its columns (the
    rows of W_g), stacked."""
    fw = [mx_quantize(w, dtype, axis=1) for w in weights]
    tr = [mx_quantize(np.ascontiguousarray(np.asarray(w).T), dtype, axis=1) for w in weights]
    return (np.stack([f[0] for f in fw]), np.stack([f[1] for f in fw]),
            np.stack([t[0] for t in tr]), np.stack([t[1] for t in tr]))


def mx_quantize_tokens(x_bits: np.ndarray, group_lens: np.ndarray, dtype: int = E4M3):
    """MX quantisation along tokens within each expert: x_bits [M, cols] bf16
    bits.  Returns (codes: E4M3 [M, cols] / E2M1 [M, cols/2] with the even
    column in the low nibble, scales [M // 32 + G, cols], number of scale
    rows used); unused scale rows are zero."""
    x = _c(x_bits, np.uint16)
    lens = _c(group_lens, np.int64)
    M, cols = x.shape
    q = np.zeros((M, cols if dtype == E4M3 else cols // 2), np.uint8)
    s = np.zeros((M // 32 + lens.size, cols), np.uint8)
    nb = lib().orc_mx_quantize_tokens(_ptr(x), _ptr(lens), lens.size, M, cols, dtype, _ptr(q), _ptr(s))
    if nb < 0:
        raise ValueError("orc_mx_quantize_tokens: bad arguments")
    return q, s, int(nb)


def _element_values(q: np.ndarray, dtype: int) -> np.ndarray:
    """Exact values of E4M3 codes, or of E2M1 nibble pairs unpacked along the
    row (low nibble first)."""
    if dtype == E4M3:
        table = np.array([e4m3_value(c) for c in range(256)], np.float64)
        return table[q]
    table = np.array([e2m1_value(c) for c in range(16)], np.float64)
    out = np.empty((q.shape[0], 2 * q.shape[1]), np.float64)
    out[:, 0::2] = table[q & 0xF]
    out[:, 1::2] = table[q >> 4]
    return out


def mx_dequantize_tokens(q: np.ndarray, s: np.ndarray, group_lens: np.ndarray, dtype: int = E4M3) -> np.ndarray:
    """Exact binary64 values of mx_quantize_tokens' output."""
    lens = np.asarray(group_lens, np.int64)
    vals = _element_values(_c(q, np.uint8), dtype)
    out = np.empty(vals.shape, np.float64)
    off = b = 0
    for g in range(lens.size):
        for j in range((int(lens[g]) + 31) // 32):
            r0, r1 = off + 32 * j, min(off + 32 * j + 32, off + int(lens[g]))
            out[r0:r1] = vals[r0:r1] * np.ldexp(1.0, s[b].astype(np.int64) - 127)[None, :]
            b += 1
        off += int(lens[g])
    return out


def fp8_quantize(x_bits: np.ndarray):
    """FP8 E4M3 with one scale per matrix: x_bits [batch, ...] bf16 bits.
    Returns (codes uint8 of x's shape, amax float32 [batch], dequant float32 [batch]).
    A 2-D [rows, cols] input gives one scale per row (the rowwise recipe)."""
    x = _c(x_bits, np.uint16)
    batch = x.shape[0]
    n = x.size // max(batch, 1)
    q = np.empty(x.shape, np.uint8)
    amax = np.empty(batch, np.float32)
    deq = np.empty(batch, np.float32)
    lib().orc_fp8_quantize(_ptr(x), batch, n, _ptr(q), _ptr(amax), _ptr(deq))
    return q, amax, deq


def mx_dequantize(dtype: int, q: np.ndarray, s: np.ndarray, rows: int, cols: int) -> np.ndarray:
    return decode(dtype, q, s, rows, cols)


def swiglu(c: np.ndarray, limit: float = 0.0) -> np.ndarray:
    """silu(gate) * up over c = [gate | up] ([n, 2I]); with a limit L > 0 the
    clamped SwiGLU (the DeepSeek-V4 blog's swiglu_limit knob): gate clamped to
    at most L, up to [-L, L]."""
    c = _c(c, np.float64)
    n, N = c.shape
    h = np.empty((n, N // 2), np.float64)
    lib().orc_swiglu(_ptr(c), n, N, float(limit), _ptr(h))
    return h


def swiglu_bwd(dh: np.ndarray, c: np.ndarray, limit: float = 0.0) -> np.ndarray:
    """Gradient of c = [gate | up] ([n, 2I]) given dh = d(silu(gate) * up) ([n, I]);
    with a limit, of the clamped SwiGLU (no gradient into a clamped input)."""
    dh, c = _c(dh, np.float64), _c(c, np.float64)
    n, I = dh.shape
    if c.shape != (n, 2 * I):
        raise ValueError("c must be [n, 2I] for dh [n, I]")
    dc = np.empty((n, 2 * I), np.float64)
    lib().orc_swiglu_bwd(_ptr(dh), _ptr(c), n, I, float(limit), _ptr(dc))
    return dc


# ------------------------------------------------------------------ GEMMs
def _operand(dtype, x):
    return _c(x, np.uint16 if dtype == BF16 else np.uint8)


def fwd_rows(dtype, a, a_scale, b, b_scale, group_lens, N, K, trans_b, rows):
    """Unrounded binary64 C[rows, :] = A_g[rows] @ B_g for each row's expert."""
    lens = _c(group_lens, np.int64)
    rows = _c(rows, np.int64)
    a, b = _operand(dtype, a), _operand(dtype, b)
    a_scale, b_scale = _c(a_scale, np.uint8), _c(b_scale, np.uint8)
    out = np.empty((rows.size, N), np.float64)
    M = int(lens.sum())
    rc = lib().orc_fwd_rows(dtype, _ptr(a), _ptr(a_scale), _ptr(b), _ptr(b_scale),
                            _ptr(lens), lens.size, M, N, K, int(trans_b),
                            _ptr(rows), rows.size, _ptr(out))
    if rc:
        raise ValueError("orc_fwd_rows: a requested row belongs to no expert")
    return out


def dgrad_rows(dy, b, group_lens, N, K, trans_b, rows):
    """Unrounded dX[rows, :] = dY[rows] @ B_g^T (bf16 operands)."""
    lens = _c(group_lens, np.int64)
    rows = _c(rows, np.int64)
    dy, b = _c(dy, np.uint16), _c(b, np.uint16)
    out = np.empty((rows.size, K), np.float64)
    rc = lib().orc_dgrad_rows(_ptr(dy), _ptr(b), _ptr(lens), lens.size, int(lens.sum()),
                              N, K, int(trans_b), _ptr(rows), rows.size, _ptr(out))
    if rc:
        raise ValueError("orc_dgrad_rows: a requested row belongs to no expert")
    return out


def wgrad_rows(a, dy, group_lens, N, K, gs, ks):
    """Unrounded D_g[k, :] = sum over expert g's rows of A[r, k] * dY[r, :]."""
    lens = _c(group_lens, np.int64)
    gs, ks = _c(gs, np.int64), _c(ks, np.int64)
    a, dy = _c(a, np.uint16), _c(dy, np.uint16)
    out = np.empty((gs.size, N), np.float64)
    rc = lib().orc_wgrad_rows(_ptr(a), _ptr(dy), _ptr(lens), lens.size, int(lens.sum()),
                              N, K, _ptr(gs), _ptr(ks), gs.size, _ptr(out))
    if rc:
        raise ValueError("orc_wgrad_rows: bad (expert, k) pair")
    return out


def fp8_wgrad_rows(a_q, a_dequant, dy_q, dy_dequant, group_lens, N, K, gs, ks):
    """Unrounded D_g[k, :] for E4M3 codes with one factor per tensor: the
    exact code products summed over expert g's rows (wgrad_rows on the codes'
    values, which every bf16 holds exactly), times a_dequant * dy_dequant."""
    table = np.array([e4m3_value(c) for c in range(256)], np.float64)
    a_bits = round_bf16(table[_c(a_q, np.uint8)])
    dy_bits = round_bf16(table[_c(dy_q, np.uint8)])
    d = wgrad_rows(a_bits, dy_bits, group_lens, N, K, gs, ks)
    return d * (float(np.float64(a_dequant)) * float(np.float64(dy_dequant)))


# ------------------------------------------------------------------ composed ops
def grouped_fwd(dtype, a, a_scale, b, b_scale, group_lens, N, K, trans_b, epilogue, rows, limit=0.0):
    """Forward with its epilogue, for the listed rows.

    Returns a dict:
      "exact": binary64 result before the final rounding ([n, N] or [n, N/2]),
      "bf16":  uint16 bits of the bf16 output (NONE, SWIGLU, and the bf16 SwiGLU
               value that SWIGLU_MXFP4 quantises),
      "q", "s": MXFP4 codes [n, N/4] and scales [n, N/64] (SWIGLU_MXFP4 only).
    """
    c = fwd_rows(dtype, a, a_scale, b, b_scale, group_lens, N, K, trans_b, rows)
    if epilogue == EPI_NONE:
        return {"exact": c, "bf16": round_bf16(c)}
    h = swiglu(c, limit)
    hb = round_bf16(h)
    out = {"exact": h, "bf16": hb}
    if epilogue == EPI_SWIGLU_MXFP4:
        out["q"], out["s"] = mx_quantize(hb, E2M1, axis=1)
    return out


def fp8_fwd_rows(a_q, a_dequant, b_q, b_dequant, group_lens, N, K, rows):
    """Unrounded binary64 C[rows, :] for E4M3 codes with one factor per tensor:
    the code products summed exactly (the MX product with every block scale
    2^0), times a_dequant * b_dequant[g].  a_q [M, K], b_q [G, N, K]."""
    rows = _c(rows, np.int64)
    lens = _c(group_lens, np.int64)
    a_q, b_q = _c(a_q, np.uint8), _c(b_q, np.uint8)
    ones_a = np.full((a_q.shape[0], K // 32), 127, np.uint8)
    ones_b = np.full((b_q.shape[0], N, K // 32), 127, np.uint8)
    c = fwd_rows(E4M3, a_q, ones_a, b_q, ones_b, lens, N, K, 1, rows)
    offs = np.concatenate([[0], np.cumsum(lens)])
    g = np.searchsorted(offs, rows, side="right") - 1
    f = float(np.float64(a_dequant)) * np.asarray(b_dequant, np.float64)[g]
    return c * f[:, None]


def fp8_fwd_rows_rowwise(a_q, a_dequant, b_q, b_dequant, group_lens, N, K, rows):
    """As fp8_fwd_rows with one factor per row of A (a_dequant [M]) and per
    row of each expert's B (b_dequant [G, N]): C[r, n] = (sum of code
    products) * a_dequant[r] * b_dequant[g, n]."""
    rows = _c(rows, np.int64)
    lens = _c(group_lens, np.int64)
    a_q, b_q = _c(a_q, np.uint8), _c(b_q, np.uint8)
    ones_a = np.full((a_q.shape[0], K // 32), 127, np.uint8)
    ones_b = np.full((b_q.shape[0], N, K // 32), 127, np.uint8)
    c = fwd_rows(E4M3, a_q, ones_a, b_q, ones_b, lens, N, K, 1, rows)
    offs = np.concatenate([[0], np.cumsum(lens)])
    g = np.searchsorted(offs, rows, side="right") - 1
    fa = np.asarray(a_dequant, np.float64)[rows]
    fb = np.asarray(b_dequant, np.float64).reshape(-1, N)[g]
    return c * fa[:, None] * fb


def dgrad_swiglu_rows(dy, b, c_saved, group_lens, N, K, trans_b, rows, limit=0.0):
    """FC2's data gradient followed by the SwiGLU backward, for the listed rows.

    dH = dY_g @ B_g^T is rounded to bf16 (what the data gradient stores), then
    the gradient of FC1's output [gate | up] (c_saved, bf16 bits [M, 2K]) is
    formed in binary64.  Returns "dh_bf16" (uint16 [n, K]), "exact" (binary64
    [n, 2K] before the final rounding) and "bf16" (its bf16 bits).
    """
    rows = _c(rows, np.int64)
    dh = dgrad_rows(dy, b, group_lens, N, K, trans_b, rows)
    dhb = round_bf16(dh)
    c = bf16_to_f64(_c(c_saved, np.uint16)[rows])
    dc = swiglu_bwd(bf16_to_f64(dhb), c, limit)
    return {"dh_bf16": dhb, "exact": dc, "bf16": round_bf16(dc)}


def wgrad_accumulate(main_grad_in: np.ndarray, d_exact: np.ndarray, accumulate: bool) -> np.ndarray:
    """fp32 result of main_grad (+)= D, one rounding of the exact sum."""
    base = main_grad_in.astype(np.float64) if accumulate else 0.0
    return round_f32(base + d_exact)


def mlp_mxfp4_rows(x_bits, w1q, w1s, w2q, w2s, group_lens, H, I, rows):
    """Expert MLP FC1 -> SwiGLU -> FC2 in MXFP4 for the listed rows.

    x_bits: bf16 [M, H]; w1q/w1s: FC1 weight [G, 2I, H] as MXFP4 codes/scales;
    w2q/w2s: FC2 weight [G, H, I].  The activations are quantised along H
    (FC1) and along I (FC2) in blocks of 32, from bf16 values.
    Returns dict with "h_q", "h_s" (FC2 input), "exact" (binary64 FC2 output,
    before rounding) and "bf16".
    """
    rows = _c(rows, np.int64)
    xr = np.ascontiguousarray(x_bits[rows])
    xq, xs = mx_quantize(xr, E2M1, axis=1)
    # quantisation is row-local, so quantising only the listed rows is exact;
    # the GEMM helper indexes A by global row, so scatter into a sparse holder
    lens = _c(group_lens, np.int64)
    local_lens, local_rows = _local_groups(lens, rows)
    c1 = fwd_rows(E2M1, xq, xs, w1q, w1s, local_lens, 2 * I, H, 1, local_rows)
    h = swiglu(c1)
    hb = round_bf16(h)
    hq, hs = mx_quantize(hb, E2M1, axis=1)
    c2 = fwd_rows(E2M1, hq, hs, w2q, w2s, local_lens, H, I, 1, local_rows)
    return {"h_bf16": hb, "h_q": hq, "h_s": hs, "exact": c2, "bf16": round_bf16(c2)}


def _local_groups(lens: np.ndarray, rows: np.ndarray):
    """Re-index sorted-by-expert sample rows as a compact ragged batch.

    Row i of the compact batch is global row rows[i]; the compact expert
    lengths count how many sample rows fall in each expert, so the compact
    batch keeps every row's expert.  Requires rows sorted ascending.
    """
    if np.any(np.diff(rows) < 0):
        raise ValueError("rows must be sorted")
    offs = np.concatenate([[0], np.cumsum(lens)])
    g_of = np.searchsorted(offs, rows, side="right") - 1
    if np.any(rows >= offs[-1]) or np.any(rows < 0):
        raise ValueError("row outside every expert")
    local = np.bincount(g_of, minlength=lens.size).astype(np.int64)
    return local, np.arange(rows.size, dtype=np.int64)
