"""GPU checks of the line-aligned code layout: pt_mx_quantize_pitched writes
each row's codes exactly where pt_mx_quantize writes them, moved to row
r * q_pitch, and leaves the rest of every row alone; pt_grouped_gemm_fwd_pitched
on pitched copies of the same codes gives outputs bit-identical to
pt_grouped_gemm_fwd on the packed ones (MXFP8, MXFP4, FP8 with tensor and
row factors; plain and SwiGLU epilogues; ragged experts that run 256- and
128-row tiles; a partial last reduction stage), and never reads the bytes
past a row's codes: they hold E4M3 NaN codes (0x7F) or E2M1 6.0 codes (0x77),
which would change the results."""
import numpy as np
import pytest
import torch

import moe_expert_grouped_gemm_amd as ptm
from moe_expert_grouped_gemm_amd import synth
from util import bits16, dev_i64, make_ws, u8

pytestmark = pytest.mark.gpu

LENS = np.array([0, 70, 1, 300, 129, 0, 33, 256], np.int64)


def up(x, m):
    return (x + m - 1) // m * m


@pytest.fixture
def rules():
    yield
    ptm.pt_set_gemm_config(ptm.PT_CONFIG_RULES)


@pytest.mark.parametrize("fmt", [ptm.PT_MXFP8_E4M3, ptm.PT_MXFP4_E2M1], ids=["e4m3", "e2m1"])
@pytest.mark.parametrize("rows,cols,extra", [(100, 320, 0), (37, 2880, 128), (64, 4096, 16)],
                         ids=["r100_c320", "r37_c2880", "r64_c4096"])
def test_pitched_quantize_matches_packed(dev, fmt, rows, cols, extra):
    print(f"pitched quantise fmt={fmt} rows={rows} cols={cols}", flush=True)
    kb = cols if fmt == ptm.PT_MXFP8_E4M3 else cols // 2
    pitch = up(kb, 128) + extra
    x = synth.randn_bf16((rows, cols), seed=500 + cols, device=dev, outlier_frac=0.01, outlier_mult=50.0)
    q = torch.zeros((rows, kb), dtype=torch.uint8, device=dev)
    s = torch.zeros((rows, cols // 32), dtype=torch.uint8, device=dev)
    ptm.pt_mx_quantize(x, q, s, rows, cols, fmt, 1)
    qp = torch.full((rows, pitch), 0xEE, dtype=torch.uint8, device=dev)
    sp = torch.zeros_like(s)
    ptm.pt_mx_quantize_pitched(x, qp, sp, rows, cols, fmt, pitch)
    torch.cuda.synchronize()
    assert torch.equal(qp[:, :kb], q)
    assert torch.equal(sp, s)
    assert (qp[:, kb:] == 0xEE).all()


def pitched_copy(q, kb, pitch, fill):
    out = torch.full((q.shape[0], pitch), fill, dtype=torch.uint8, device=q.device)
    out[:, :kb] = q
    return out


DTYPES = [ptm.PT_MXFP8_E4M3, ptm.PT_MXFP4_E2M1, ptm.PT_FP8_E4M3, ptm.PT_FP8_E4M3_ROWWISE]


@pytest.mark.parametrize("dtype", DTYPES, ids=["mxfp8", "mxfp4", "fp8", "fp8_rowwise"])
@pytest.mark.parametrize("epi", [ptm.PT_EPI_NONE, ptm.PT_EPI_SWIGLU], ids=["none", "swiglu"])
@pytest.mark.parametrize("K,extra", [(576, 0), (2880, 256)], ids=["k576", "k2880"])
def test_pitched_fwd_bit_identical(dev, rules, dtype, epi, K, extra):
    M, G, N = int(LENS.sum()), len(LENS), 384
    print(f"pitched fwd dtype={dtype} epi={epi} K={K}", flush=True)
    e2m1 = dtype == ptm.PT_MXFP4_E2M1
    kb = K // 2 if e2m1 else K
    pitch = up(kb, 128) + extra
    fill = 0x77 if e2m1 else 0x7F
    a = synth.randn_bf16((M, K), seed=510, device=dev, outlier_frac=0.01, outlier_mult=50.0)
    w = synth.randn_bf16((G * N, K), seed=511, device=dev, outlier_frac=0.01, outlier_mult=50.0)
    if dtype in (ptm.PT_MXFP8_E4M3, ptm.PT_MXFP4_E2M1):
        aq = torch.empty((M, kb), dtype=torch.uint8, device=dev)
        as_ = torch.empty((M, K // 32), dtype=torch.uint8, device=dev)
        bq = torch.empty((G * N, kb), dtype=torch.uint8, device=dev)
        bs = torch.empty((G * N, K // 32), dtype=torch.uint8, device=dev)
        ptm.pt_mx_quantize(a, aq, as_, M, K, dtype, 1)
        ptm.pt_mx_quantize(w, bq, bs, G * N, K, dtype, 1)
        ap = torch.full((M, pitch), fill, dtype=torch.uint8, device=dev)
        bp = torch.full((G * N, pitch), fill, dtype=torch.uint8, device=dev)
        as2, bs2 = torch.empty_like(as_), torch.empty_like(bs)
        ptm.pt_mx_quantize_pitched(a, ap, as2, M, K, dtype, pitch)
        ptm.pt_mx_quantize_pitched(w, bp, bs2, G * N, K, dtype, pitch)
    else:
        aq = torch.empty((M, K), dtype=torch.uint8, device=dev)
        bq = torch.empty((G * N, K), dtype=torch.uint8, device=dev)
        if dtype == ptm.PT_FP8_E4M3:
            as_, am = torch.empty((1,), device=dev), torch.empty((1,), device=dev)
            bs, bm = torch.empty((G,), device=dev), torch.empty((G,), device=dev)
            ptm.pt_fp8_quantize(a, aq, am, as_, 1, M, K)
            ptm.pt_fp8_quantize(w, bq, bm, bs, G, N, K)
        else:
            as_, am = torch.empty((M,), device=dev), torch.empty((M,), device=dev)
            bs, bm = torch.empty((G * N,), device=dev), torch.empty((G * N,), device=dev)
            ptm.pt_fp8_quantize_rows(a, aq, am, as_, M, K)
            ptm.pt_fp8_quantize_rows(w, bq, bm, bs, G * N, K)
        ap, bp = pitched_copy(aq, kb, pitch, fill), pitched_copy(bq, kb, pitch, fill)
        as2, bs2 = as_, bs
    lens = dev_i64(LENS, dev)
    ws = make_ws(dev, "swz", G, M, N, K, dtype)
    ncol = N if epi == ptm.PT_EPI_NONE else N // 2
    ref = torch.empty((M, ncol), dtype=torch.bfloat16, device=dev)
    out = torch.empty_like(ref)
    ptm.pt_grouped_gemm_fwd(aq, as_, bq, bs, ref, None, lens, None, G, M, N, K, dtype, 1, epi, workspace=ws,
                            swiglu_limit=10.0)
    torch.cuda.synchronize()
    assert torch.isfinite(ref.float()).all()
    for cfg in (ptm.PT_CONFIG_RULES, 0, 1, 3):
        ptm.pt_set_gemm_config(cfg)
        out.fill_(float("nan"))
        ptm.pt_grouped_gemm_fwd_pitched(ap, as2, bp, bs2, out, None, lens, None, G, M, N, K, dtype, epi, pitch,
                                        workspace=ws, swiglu_limit=10.0)
        torch.cuda.synchronize()
        assert (bits16(out) == bits16(ref)).all(), f"configuration {cfg}"


def test_pitched_argument_errors(dev):
    M, G, N, K = 64, 1, 64, 256
    lens = dev_i64(np.array([M], np.int64), dev)
    a = torch.zeros((M, 512), dtype=torch.uint8, device=dev)
    s = torch.zeros((M, K // 32), dtype=torch.uint8, device=dev)
    b = torch.zeros((N, 512), dtype=torch.uint8, device=dev)
    bs = torch.zeros((N, K // 32), dtype=torch.uint8, device=dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    x = torch.zeros((M, K), dtype=torch.bfloat16, device=dev)
    for pitch, status in ((128, 1), (264, 1), (0, 1), (-16, 1)):      # short, not a multiple of 16, none
        with pytest.raises(ptm.PtggError) as e:
            ptm.pt_grouped_gemm_fwd_pitched(a, s, b, bs, out, None, lens, None, G, M, N, K, ptm.PT_MXFP8_E4M3,
                                            ptm.PT_EPI_NONE, pitch)
        assert e.value.status == status
        with pytest.raises(ptm.PtggError) as e:
            ptm.pt_mx_quantize_pitched(x, a, s, M, K, ptm.PT_MXFP8_E4M3, pitch)
        assert e.value.status == status
    with pytest.raises(ptm.PtggError) as e:                             # bf16 has no codes
        ptm.pt_grouped_gemm_fwd_pitched(x, None, x, None, out, None, lens, None, G, M, N, K, ptm.PT_BF16,
                                        ptm.PT_EPI_NONE, 512)
    assert e.value.status == 2
