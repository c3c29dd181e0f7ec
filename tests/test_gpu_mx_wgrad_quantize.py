"""GPU checks of pt_grouped_gemm_wgrad_quantize, the low-precision weight
gradient from bf16 gradients: quantisation fused into the transpose to the
weight gradient's operand layout.  main_grad must come out bit-identical to
pt_mx_quantize_tokens (MXFP8, MXFP4) or pt_fp8_quantize (FP8 with one factor
per tensor, whose amax covers every row) on both gradients followed by
pt_grouped_gemm_wgrad (itself checked against the oracle), in both output layouts,
accumulating and overwriting, with empty, single-row, partial-block and
multi-stage experts, explicit offsets with unowned rows between experts,
the split reduction, and channel counts that leave a partial 128-channel
group.  A workspace filled with 0xA5 beforehand shows that nothing relies on
its previous contents."""
import numpy as np
import pytest
import torch

import moe_expert_grouped_gemm_amd as ptm
from moe_expert_grouped_gemm_amd import synth
from util import dev_i64

pytestmark = pytest.mark.gpu

FMTS = [ptm.PT_MXFP8_E4M3, ptm.PT_MXFP4_E2M1]
FMT_IDS = ["e4m3", "e2m1"]


def main_grad0(dev, G, N, K, trans_out, seed):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    shape = (G, N, K) if trans_out else (G, K, N)
    return (torch.randn(shape, generator=g, device=dev) * 1e-3).float()


def workspace(dev, G, M, N, K, fmt, extra=0):
    n = ptm.pt_grouped_gemm_workspace_size(ptm.PT_OP_WGRAD, G, M, N, K, fmt)
    return torch.full((n + extra,), 0xA5, dtype=torch.uint8, device=dev)


def two_step(dev, a, dy, lens, offs, N, K, fmt, trans_out, accumulate, mg, ws):
    M, G = a.shape[0], len(lens)
    lens_d = dev_i64(lens, dev)
    offs_d = None if offs is None else dev_i64(offs, dev)
    cols = (lambda c: c) if fmt == ptm.PT_MXFP8_E4M3 else (lambda c: c // 2)
    aq = torch.zeros((M, cols(K)), dtype=torch.uint8, device=dev)
    dq = torch.zeros((M, cols(N)), dtype=torch.uint8, device=dev)
    as_ = torch.zeros((M // 32 + G, K), dtype=torch.uint8, device=dev)
    ds = torch.zeros((M // 32 + G, N), dtype=torch.uint8, device=dev)
    ptm.pt_mx_quantize_tokens(a, lens_d, offs_d, aq, as_, G, M, K, fmt)
    ptm.pt_mx_quantize_tokens(dy, lens_d, offs_d, dq, ds, G, M, N, fmt)
    ptm.pt_grouped_gemm_wgrad(aq, as_, dq, ds, mg, lens_d, offs_d, G, M, N, K, fmt, trans_out, accumulate,
                              workspace=ws)
    torch.cuda.synchronize()
    return mg


def fused(dev, a, dy, lens, offs, N, K, fmt, trans_out, accumulate, mg, ws):
    M, G = a.shape[0], len(lens)
    ptm.pt_grouped_gemm_wgrad_quantize(a, dy, mg, dev_i64(lens, dev), None if offs is None else dev_i64(offs, dev),
                                       G, M, N, K, fmt, trans_out, accumulate, workspace=ws)
    torch.cuda.synchronize()
    return mg


CASES = [
    # (name, lens, K, N)
    ("ragged", [0, 70, 1, 0, 300, 129, 0, 33], 264, 136),
    ("multi_stage", [600, 5, 257, 1000], 200, 392),
    ("one_expert", [45], 8, 16),
]


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("trans_out", [0, 1])
@pytest.mark.parametrize("accumulate", [1, 0])
def test_fused_equals_quantize_then_wgrad(dev, fmt, case, trans_out, accumulate):
    name, lens, K, N = case
    lens = np.array(lens, np.int64)
    M, G = int(lens.sum()), len(lens)
    print(f"wgrad_quantize {name} fmt={fmt} trans_out={trans_out} acc={accumulate}", flush=True)
    a = synth.randn_bf16((M, K), seed=400, device=dev, outlier_frac=0.01, outlier_mult=50.0)
    dy = synth.randn_bf16((M, N), seed=401, std=1e-2, device=dev)
    ref = two_step(dev, a, dy, lens, None, N, K, fmt, trans_out, accumulate, main_grad0(dev, G, N, K, trans_out, 402),
                   workspace(dev, G, M, N, K, fmt))
    ws = workspace(dev, G, M, N, K, fmt, extra=4096)
    got = fused(dev, a, dy, lens, None, N, K, fmt, trans_out, accumulate, main_grad0(dev, G, N, K, trans_out, 402),
                ws)
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32))
    n = ws.numel() - 4096
    assert (ws[n:].cpu().numpy() == 0xA5).all(), "write past the workspace"
    # a second call on the same (now dirty) workspace gives the same bits
    again = fused(dev, a, dy, lens, None, N, K, fmt, trans_out, accumulate,
                  main_grad0(dev, G, N, K, trans_out, 402), ws)
    assert torch.equal(again.view(torch.int32), ref.view(torch.int32))


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
def test_fused_with_offsets_and_gaps(dev, fmt):
    # experts at explicit offsets with unowned rows between and after them
    lens = np.array([40, 0, 97, 3], np.int64)
    offs = np.array([2, 50, 50, 160, 170], np.int64)
    M, G, K, N = 180, len(lens), 96, 72
    a = synth.randn_bf16((M, K), seed=410, device=dev)
    dy = synth.randn_bf16((M, N), seed=411, std=1e-2, device=dev)
    ref = two_step(dev, a, dy, lens, offs, N, K, fmt, 0, 1, main_grad0(dev, G, N, K, 0, 412),
                   workspace(dev, G, M, N, K, fmt))
    got = fused(dev, a, dy, lens, offs, N, K, fmt, 0, 1, main_grad0(dev, G, N, K, 0, 412),
                workspace(dev, G, M, N, K, fmt))
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32))


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
def test_fused_split_reduction(dev, fmt):
    # one 12.5k-token expert among short ones, K = N = 256: the split cuts it
    lens = np.array([12500, 480, 0, 350, 499, 1, 200], np.int64)
    M, G, K, N = int(lens.sum()), len(lens), 256, 256
    a = synth.randn_bf16((M, K), seed=420, std=K ** -0.5, device=dev)
    dy = synth.randn_bf16((M, N), seed=421, std=1e-2, device=dev)
    ref = two_step(dev, a, dy, lens, None, N, K, fmt, 0, 1, main_grad0(dev, G, N, K, 0, 422),
                   workspace(dev, G, M, N, K, fmt))
    got = fused(dev, a, dy, lens, None, N, K, fmt, 0, 1, main_grad0(dev, G, N, K, 0, 422),
                workspace(dev, G, M, N, K, fmt))
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32))


def two_step_fp8(dev, a, dy, lens, offs, N, K, trans_out, accumulate, mg, ws):
    M, G = a.shape[0], len(lens)
    aq = torch.zeros((M, K), dtype=torch.uint8, device=dev)
    dq = torch.zeros((M, N), dtype=torch.uint8, device=dev)
    ma, fa, md, fd = (torch.zeros((1,), dtype=torch.float32, device=dev) for _ in range(4))
    ptm.pt_fp8_quantize(a, aq, ma, fa, 1, M, K)
    ptm.pt_fp8_quantize(dy, dq, md, fd, 1, M, N)
    ptm.pt_grouped_gemm_wgrad(aq, fa, dq, fd, mg, dev_i64(lens, dev), None if offs is None else dev_i64(offs, dev),
                              G, M, N, K, ptm.PT_FP8_E4M3, trans_out, accumulate, workspace=ws)
    torch.cuda.synchronize()
    return mg


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("trans_out", [0, 1])
@pytest.mark.parametrize("accumulate", [1, 0])
def test_fused_fp8_equals_quantize_then_wgrad(dev, case, trans_out, accumulate):
    # FP8 with one factor per tensor: amax over the whole tensors, codes
    # straight into the transposed layout
    name, lens, K, N = case
    lens = np.array(lens, np.int64)
    M, G = int(lens.sum()), len(lens)
    fmt = ptm.PT_FP8_E4M3
    print(f"wgrad_quantize fp8 {name} trans_out={trans_out} acc={accumulate}", flush=True)
    a = synth.randn_bf16((M, K), seed=430, device=dev, outlier_frac=0.01, outlier_mult=50.0)
    dy = synth.randn_bf16((M, N), seed=431, std=1e-2, device=dev)
    ref = two_step_fp8(dev, a, dy, lens, None, N, K, trans_out, accumulate, main_grad0(dev, G, N, K, trans_out, 432),
                       workspace(dev, G, M, N, K, fmt))
    ws = workspace(dev, G, M, N, K, fmt, extra=4096)
    got = fused(dev, a, dy, lens, None, N, K, fmt, trans_out, accumulate, main_grad0(dev, G, N, K, trans_out, 432),
                ws)
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32))
    n = ws.numel() - 4096
    assert (ws[n:].cpu().numpy() == 0xA5).all(), "write past the workspace"


def test_fused_fp8_amax_covers_unowned_rows(dev):
    # the tensor factor comes from every row, owned by an expert or not (as
    # pt_fp8_quantize over the whole tensor): a large value in a row between
    # experts changes every code
    lens = np.array([40, 0, 97, 3], np.int64)
    offs = np.array([2, 50, 50, 160, 170], np.int64)
    M, G, K, N = 180, len(lens), 96, 72
    fmt = ptm.PT_FP8_E4M3
    a = synth.randn_bf16((M, K), seed=440, device=dev)
    a[45, 7] = 300.0                                  # row 45 belongs to no expert
    dy = synth.randn_bf16((M, N), seed=441, std=1e-2, device=dev)
    ref = two_step_fp8(dev, a, dy, lens, offs, N, K, 0, 1, main_grad0(dev, G, N, K, 0, 442),
                       workspace(dev, G, M, N, K, fmt))
    got = fused(dev, a, dy, lens, offs, N, K, fmt, 0, 1, main_grad0(dev, G, N, K, 0, 442),
                workspace(dev, G, M, N, K, fmt))
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32))


@pytest.mark.parametrize("fmt", FMTS + [ptm.PT_FP8_E4M3], ids=FMT_IDS + ["fp8"])
def test_fused_no_tokens(dev, fmt):
    # every expert empty (M = 0): main_grad untouched when accumulating,
    # zeroed when not
    G, K, N = 3, 64, 48
    lens = np.zeros(G, np.int64)
    a = torch.empty((0, K), dtype=torch.bfloat16, device=dev)
    dy = torch.empty((0, N), dtype=torch.bfloat16, device=dev)
    ws = workspace(dev, G, 0, N, K, fmt)
    mg = main_grad0(dev, G, N, K, 0, 450)
    before = mg.clone()
    fused(dev, a, dy, lens, None, N, K, fmt, 0, 1, mg, ws)
    assert torch.equal(mg, before)
    fused(dev, a, dy, lens, None, N, K, fmt, 0, 0, mg, ws)
    assert (mg == 0).all()


def test_fused_argument_errors(dev):
    lens = dev_i64([4, 4], dev)
    a = torch.zeros((8, 16), dtype=torch.bfloat16, device=dev)
    dy = torch.zeros((8, 16), dtype=torch.bfloat16, device=dev)
    mg = torch.zeros((2, 16, 16), dtype=torch.float32, device=dev)
    ws = workspace(dev, 2, 8, 16, 16, ptm.PT_MXFP8_E4M3)
    with pytest.raises(ptm.PtggError, match="UNSUPPORTED"):
        ptm.pt_grouped_gemm_wgrad_quantize(a, dy, mg, lens, None, 2, 8, 16, 16, ptm.PT_BF16, 0, 1, workspace=ws)
    with pytest.raises(ptm.PtggError, match="WORKSPACE"):
        ptm.pt_grouped_gemm_wgrad_quantize(a, dy, mg, lens, None, 2, 8, 16, 16, ptm.PT_MXFP8_E4M3, 0, 1,
                                           workspace=ws[:64])


@pytest.mark.parametrize("fmt", [ptm.PT_MXFP8_E4M3, ptm.PT_FP8_E4M3], ids=["e4m3", "fp8"])
def test_fused_full_config3_shape(dev, fmt):
    # the MXFP8 weight-gradient workload at full size (32 experts with Zipf
    # routing, 65536 tokens, K = 2880, N = 5760, accumulating into [G, K, N]),
    # as the benchmark times it: every element of main_grad bit-identical to
    # the two-step path (which the sampled full-size oracle tests pin)
    lens = synth.lens_zipf_distinct(16384, 32, 4, 1.1, seed=3)
    M, G, K, N = int(lens.sum()), len(lens), 2880, 5760
    print(f"wgrad_quantize full config-3 shape fmt={fmt} M={M}", flush=True)
    a = synth.randn_bf16((M, K), seed=104, device=dev, outlier_frac=0.01, outlier_mult=50.0)
    dy = synth.randn_bf16((M, N), seed=106, std=1e-2, device=dev)
    ws = workspace(dev, G, M, N, K, fmt)
    mg_ref = main_grad0(dev, G, N, K, 0, seed=460)
    mg = mg_ref.clone()
    if fmt == ptm.PT_FP8_E4M3:
        two_step_fp8(dev, a, dy, lens, None, N, K, 0, 1, mg_ref, ws)
    else:
        two_step(dev, a, dy, lens, None, N, K, fmt, 0, 1, mg_ref, ws)
    fused(dev, a, dy, lens, None, N, K, fmt, 0, 1, mg, ws)
    assert torch.equal(mg, mg_ref)
