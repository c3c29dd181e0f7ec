"""GPU check that the SwiGLU -> MXFP4 epilogue is exact: for every operand
dtype (BF16 in both weight layouts, MXFP8, MXFP4, FP8 with tensor and with
row factors), every kernel configuration and the plain and clamped SwiGLU,
the codes and scale bytes it writes equal the oracle's MXFP4 quantisation
of the bf16 SwiGLU values that PT_EPI_SWIGLU writes for the same inputs.

The SwiGLU values themselves are checked against the oracle within the BF16
tolerance by the other forward tests; quantisation of a given bf16 value has
exactly one correct result, so this comparison is bit for bit.  Called
through the C ABI."""
import numpy as np
import pytest
import torch

import moe_expert_grouped_gemm_amd as ptm
from moe_expert_grouped_gemm_amd import synth
from util import bits16, dev_i64, make_ws, u8

pytestmark = pytest.mark.gpu

LENS = np.array([0, 77, 3, 200, 0, 40, 1, 290], np.int64)


def inputs(dev, dtype, M, G, N, K, trans_b):
    """(a, a_scale, b, b_scale) for the dtype; some rows of A are all zero,
    so their SwiGLU blocks are zero (scale byte 0)."""
    zero_rows = torch.as_tensor([5, 6, 100, M - 1], device=dev)
    if dtype == ptm.PT_BF16:
        a = synth.randn_bf16((M, K), seed=170, std=1.0, device=dev, outlier_frac=0.01, outlier_mult=20.0)
        a[zero_rows] = 0
        shape = (G, N, K) if trans_b else (G, K, N)
        b = synth.randn_bf16(shape, seed=171, std=K ** -0.5, device=dev)
        return a, None, b, None
    if dtype in (ptm.PT_MXFP8_E4M3, ptm.PT_MXFP4_E2M1):
        name = "e4m3" if dtype == ptm.PT_MXFP8_E4M3 else "e2m1"
        aq, as_ = synth.random_mx_codes(M, K, name, seed=172, device=dev, scale_lo=118, scale_hi=126)
        bq, bs = synth.random_mx_codes(G * N, K, name, seed=173, device=dev, scale_lo=114, scale_hi=120)
        aq[zero_rows] = 0
        return aq, as_, bq, bs
    x = synth.randn_bf16((M, K), seed=174, device=dev, outlier_frac=0.01, outlier_mult=20.0)
    x[zero_rows] = 0
    w = synth.randn_bf16((G * N, K), seed=175, std=K ** -0.5, device=dev)
    aq = torch.empty((M, K), dtype=torch.uint8, device=dev)
    bq = torch.empty((G * N, K), dtype=torch.uint8, device=dev)
    if dtype == ptm.PT_FP8_E4M3:
        fa = [torch.empty((1,), dtype=torch.float32, device=dev) for _ in range(2)]
        fb = [torch.empty((G,), dtype=torch.float32, device=dev) for _ in range(2)]
        ptm.pt_fp8_quantize(x, aq, fa[0], fa[1], 1, M, K)
        ptm.pt_fp8_quantize(w, bq, fb[0], fb[1], G, N, K)
    else:
        fa = [torch.empty((M,), dtype=torch.float32, device=dev) for _ in range(2)]
        fb = [torch.empty((G * N,), dtype=torch.float32, device=dev) for _ in range(2)]
        ptm.pt_fp8_quantize_rows(x, aq, fa[0], fa[1], M, K)
        ptm.pt_fp8_quantize_rows(w, bq, fb[0], fb[1], G * N, K)
    return aq, fa[1], bq, fb[1]


CASES = [
    ("bf16_kn", ptm.PT_BF16, 0, 256, 512),
    ("bf16_nk", ptm.PT_BF16, 1, 192, 320),
    ("mxfp8", ptm.PT_MXFP8_E4M3, 1, 256, 512),
    ("mxfp8_k288", ptm.PT_MXFP8_E4M3, 1, 288, 320),
    ("mxfp4", ptm.PT_MXFP4_E2M1, 1, 256, 512),
    ("mxfp4_k320", ptm.PT_MXFP4_E2M1, 1, 320, 320),
    ("fp8", ptm.PT_FP8_E4M3, 1, 256, 512),
    ("fp8_rowwise", ptm.PT_FP8_E4M3_ROWWISE, 1, 256, 320),
]


@pytest.fixture
def rules():
    yield
    ptm.pt_set_gemm_config(ptm.PT_CONFIG_RULES)
    ptm.pt_clear_gemm_tuning()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_swiglu_mxfp4_codes_equal_oracle_quantisation_of_swiglu(orc, dev, rules, case):
    name, dtype, trans_b, K, N = case
    M, G, I = int(LENS.sum()), len(LENS), N // 2
    a, as_, b, bs = inputs(dev, dtype, M, G, N, K, trans_b)
    mx = dtype in (ptm.PT_MXFP8_E4M3, ptm.PT_MXFP4_E2M1)
    lens_d = dev_i64(LENS, dev)
    for sched in (["static", "queue", "swz"] if mx else ["static", "queue"]):
        ws = make_ws(dev, sched, G, M, N, K, dtype)
        for cfg in (0, 1, 2, 3):
            ptm.pt_set_gemm_config(cfg)
            for limit in (0.0, 10.0):
                print(f"swiglu->mxfp4 exact {name} sched={sched} cfg={cfg} limit={limit}", flush=True)
                h = torch.empty((M, I), dtype=torch.bfloat16, device=dev)
                q = torch.full((M, I // 2), 0xEE, dtype=torch.uint8, device=dev)
                s = torch.full((M, I // 32), 0xEE, dtype=torch.uint8, device=dev)
                ptm.pt_grouped_gemm_fwd(a, as_, b, bs, h, None, lens_d, None, G, M, N, K, dtype, trans_b,
                                        ptm.PT_EPI_SWIGLU, workspace=ws, swiglu_limit=limit)
                ptm.pt_grouped_gemm_fwd(a, as_, b, bs, q, s, lens_d, None, G, M, N, K, dtype, trans_b,
                                        ptm.PT_EPI_SWIGLU_MXFP4, workspace=ws, swiglu_limit=limit)
                torch.cuda.synchronize()
                rq, rs = orc.mx_quantize(bits16(h), orc.E2M1)
                gq, gs = u8(q), u8(s)
                assert (gs == rs).all(), f"{(gs != rs).sum()} scale bytes differ"
                assert (gq == rq).all(), f"{(gq != rq).sum()} code bytes differ"
                # the inputs reach the interesting parts of the encoding
                if cfg == 0 and limit == 0.0:
                    assert (rs == 0).any()                                # all-zero blocks
                    assert ((rq & 0x7) == 0x7).any()                      # codes at the grid maximum 6
                    assert (((rq >> 4) & 0x7) == 0x1).any() or ((rq & 0x7) == 0x1).any()   # subnormal 0.5
