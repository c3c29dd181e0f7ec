"""GPU check of pt_grouped_gemm_fwd_noalloc, the forward that keeps its
scratch (error word and tile-queue counters) in the library's own static
device array instead of a caller's workspace: called through the C ABI, its
outputs equal pt_grouped_gemm_fwd's bit for bit, on two calls in a row, the
second on a smaller problem (the array keeps the first call's counters,
which the second must clear), for BF16 with SwiGLU, MXFP8 and MXFP4."""
import ctypes

import numpy as np
import pytest
import torch

import moe_expert_grouped_gemm_amd as ptm
from moe_expert_grouped_gemm_amd import synth

pytestmark = pytest.mark.gpu


def noalloc_fn():
    L = ptm.load()
    fn = L.pt_grouped_gemm_fwd_noalloc
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p] * 8 + [ctypes.c_int64] * 4 + [ctypes.c_int] * 3 + [ctypes.c_float,
                                                                                        ctypes.c_void_p]
    return fn


def ptr(t):
    return None if t is None else t.data_ptr()


def problem(dev, dtype, lens, K, N, seed):
    M, G = int(lens.sum()), len(lens)
    if dtype == ptm.PT_BF16:
        a = synth.randn_bf16((M, K), seed=seed, std=K ** -0.5, device=dev)
        b = synth.randn_bf16((G, K, N), seed=seed + 1, std=K ** -0.5, device=dev)
        return a, None, b, None, 0
    name = "e4m3" if dtype == ptm.PT_MXFP8_E4M3 else "e2m1"
    aq, as_ = synth.random_mx_codes(M, K, name, seed=seed, device=dev, scale_lo=120, scale_hi=126)
    bq, bs = synth.random_mx_codes(G * N, K, name, seed=seed + 1, device=dev, scale_lo=116, scale_hi=120)
    return aq, as_, bq, bs, 1


CASES = [(ptm.PT_BF16, ptm.PT_EPI_SWIGLU, 256, 512), (ptm.PT_MXFP8_E4M3, ptm.PT_EPI_NONE, 256, 256),
         (ptm.PT_MXFP4_E2M1, ptm.PT_EPI_SWIGLU_MXFP4, 320, 512)]


@pytest.mark.parametrize("dtype,epi,K,N", CASES, ids=["bf16_swiglu", "mxfp8", "mxfp4_k320_mxfp4out"])
def test_noalloc_equals_workspace_forward(dev, dtype, epi, K, N):
    fn = noalloc_fn()
    stream = torch.cuda.current_stream().cuda_stream
    ws = torch.zeros(ptm.pt_grouped_gemm_workspace_size(ptm.PT_OP_FWD, 1, 1, 1, 1, ptm.PT_BF16), dtype=torch.uint8,
                     device=dev)
    # a large ragged problem, then a smaller one
    for lens in (np.array([0, 300, 7, 520, 1, 0, 129, 260], np.int64), np.array([40, 0, 3], np.int64)):
        M, G = int(lens.sum()), len(lens)
        print(f"noalloc dtype={dtype} epi={epi} G={G} M={M} K={K} N={N}", flush=True)
        a, as_, b, bs, trans_b = problem(dev, dtype, lens, K, N, seed=190 + G)
        lens_d = torch.as_tensor(lens, device=dev)
        if epi == ptm.PT_EPI_SWIGLU_MXFP4:
            outs = [torch.full((M, N // 4), 0xEE, dtype=torch.uint8, device=dev) for _ in range(2)]
            oscs = [torch.full((M, N // 64), 0xEE, dtype=torch.uint8, device=dev) for _ in range(2)]
        else:
            cols = N if epi == ptm.PT_EPI_NONE else N // 2
            outs = [torch.full((M, cols), -1, dtype=torch.int16, device=dev).view(torch.bfloat16)
                    for _ in range(2)]
            oscs = [None, None]
        ptm.pt_grouped_gemm_fwd(a, as_, b, bs, outs[0], oscs[0], lens_d, None, G, M, N, K, dtype, trans_b, epi,
                                workspace=ws)
        st = fn(ptr(a), ptr(as_), ptr(b), ptr(bs), ptr(outs[1]), ptr(oscs[1]), ptr(lens_d), None, G, M, N, K, dtype,
                trans_b, epi, 0.0, stream)
        assert st == 0, ptm.pt_status_string(st)
        torch.cuda.synchronize()
        assert torch.equal(outs[0].view(torch.uint8), outs[1].view(torch.uint8))
        if oscs[0] is not None:
            assert torch.equal(oscs[0], oscs[1])


def test_noalloc_argument_errors(dev):
    fn = noalloc_fn()
    lens = torch.as_tensor(np.array([8], np.int64), device=dev)
    a = torch.zeros((8, 64), dtype=torch.bfloat16, device=dev)
    b = torch.zeros((1, 64, 64), dtype=torch.bfloat16, device=dev)
    out = torch.zeros((8, 64), dtype=torch.bfloat16, device=dev)
    st = torch.cuda.current_stream().cuda_stream
    # too many experts, and a NULL operand: refused before any launch
    assert fn(ptr(a), None, ptr(b), None, ptr(out), None, ptr(lens), None, 2000, 8, 64, 64, ptm.PT_BF16, 0,
              ptm.PT_EPI_NONE, 0.0, st) == 2
    assert fn(None, None, ptr(b), None, ptr(out), None, ptr(lens), None, 1, 8, 64, 64, ptm.PT_BF16, 0,
              ptm.PT_EPI_NONE, 0.0, st) == 1
