"""GPU checks of the kernel configurations and of tuning, through the C ABI:
every configuration (static or queued tile order, 256 x 256 or 128 x 256
kernel) gives bit-identical outputs for every op and dtype that has it, and
tuning picks one per problem class without changing results, never times a
weight gradient that accumulates, and leaves the rules in place afterwards."""
import numpy as np
import pytest
import torch

import moe_expert_grouped_gemm_amd as ptm
from moe_expert_grouped_gemm_amd import synth
from util import dev_i64, make_ws

pytestmark = pytest.mark.gpu

LENS = np.array([0, 1, 130, 0, 257, 64, 33, 300], np.int64)
CONFIGS = [0, 1, 2, 3]


@pytest.fixture
def rules():
    ptm.pt_clear_gemm_tuning()
    yield
    ptm.pt_set_gemm_config(ptm.PT_CONFIG_RULES)
    ptm.pt_clear_gemm_tuning()


def per_config(fn):
    """fn() -> tensor, once per forced configuration."""
    outs = []
    for c in CONFIGS:
        ptm.pt_set_gemm_config(c)
        outs.append(fn().clone())
        torch.cuda.synchronize()
    ptm.pt_set_gemm_config(ptm.PT_CONFIG_RULES)
    return outs


def assert_identical(outs):
    for c, o in zip(CONFIGS[1:], outs[1:]):
        assert torch.equal(o.view(torch.uint8), outs[0].view(torch.uint8)), f"configuration {c} differs"


@pytest.mark.parametrize("trans_b,epi", [(0, ptm.PT_EPI_SWIGLU), (1, ptm.PT_EPI_NONE), (0, ptm.PT_EPI_SWIGLU_MXFP4),
                                         (1, ptm.PT_EPI_SWIGLU)], ids=["kn_swiglu", "nk_none", "kn_mxfp4", "nk_swiglu"])
def test_bf16_fwd_configs_identical(dev, rules, trans_b, epi):
    M, G, K, N = int(LENS.sum()), len(LENS), 200, 256
    print(f"configs bf16 fwd trans_b={trans_b} epi={epi}", flush=True)
    a = synth.randn_bf16((M, K), seed=120, std=K ** -0.5, device=dev)
    b = synth.randn_bf16((G, N, K) if trans_b else (G, K, N), seed=121, std=K ** -0.5, device=dev)
    ws = make_ws(dev, "queue")
    lens = dev_i64(LENS, dev)
    if epi == ptm.PT_EPI_SWIGLU_MXFP4:
        out = torch.empty((M, N // 4), dtype=torch.uint8, device=dev)
        osc = torch.empty((M, N // 64), dtype=torch.uint8, device=dev)
    else:
        out = torch.empty((M, N if epi == ptm.PT_EPI_NONE else N // 2), dtype=torch.bfloat16, device=dev)
        osc = None

    def fn():
        ptm.pt_grouped_gemm_fwd(a, None, b, None, out, osc, lens, None, G, M, N, K, ptm.PT_BF16, trans_b, epi,
                                workspace=ws)
        return out if osc is None else torch.cat([out.view(-1), osc.view(-1)])
    assert_identical(per_config(fn))


@pytest.mark.parametrize("trans_b", [0, 1])
def test_bf16_dgrad_and_swiglu_bwd_configs_identical(dev, rules, trans_b):
    M, G, K, N = int(LENS.sum()), len(LENS), 136, 264
    dy = synth.randn_bf16((M, N), seed=122, std=1e-2, device=dev)
    b = synth.randn_bf16((G, N, K) if trans_b else (G, K, N), seed=123, std=N ** -0.5, device=dev)
    c = synth.randn_bf16((M, 2 * K), seed=124, std=2.0, device=dev)
    ws = make_ws(dev, "queue")
    lens = dev_i64(LENS, dev)
    dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    dc = torch.empty((M, 2 * K), dtype=torch.bfloat16, device=dev)

    def fn():
        ptm.pt_grouped_gemm_dgrad(dy, None, b, None, dx, lens, None, G, M, N, K, ptm.PT_BF16, trans_b, workspace=ws)
        return dx

    def fn2():
        ptm.pt_grouped_gemm_dgrad_swiglu(dy, b, c, dc, lens, None, G, M, N, K, trans_b, workspace=ws)
        return dc
    assert_identical(per_config(fn))
    assert_identical(per_config(fn2))


@pytest.mark.parametrize("trans_out", [0, 1])
@pytest.mark.parametrize("accumulate", [1, 0])
def test_bf16_wgrad_configs_identical(dev, rules, trans_out, accumulate):
    M, G, K, N = int(LENS.sum()), len(LENS), 200, 136
    a = synth.randn_bf16((M, K), seed=125, std=K ** -0.5, device=dev)
    dy = synth.randn_bf16((M, N), seed=126, std=1e-2, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(127)
    mg0 = torch.randn((G, N, K) if trans_out else (G, K, N), generator=g, device=dev).mul_(1e-3)
    ws = make_ws(dev, "queue")
    lens = dev_i64(LENS, dev)

    def fn():
        mg = mg0.clone()
        ptm.pt_grouped_gemm_wgrad(a, None, dy, None, mg, lens, None, G, M, N, K, ptm.PT_BF16, trans_out, accumulate,
                                  workspace=ws)
        return mg
    assert_identical(per_config(fn))


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
@pytest.mark.parametrize("epi", [ptm.PT_EPI_NONE, ptm.PT_EPI_SWIGLU_MXFP4])
def test_mx_fwd_configs_identical(dev, rules, fmt, epi):
    M, G, K, N = int(LENS.sum()), len(LENS), 320, 256
    dtype = ptm.PT_MXFP8_E4M3 if fmt == "e4m3" else ptm.PT_MXFP4_E2M1
    print(f"configs mx fwd fmt={fmt} epi={epi}", flush=True)
    aq, as_ = synth.random_mx_codes(M, K, fmt, seed=128, device=dev)
    bq, bs = synth.random_mx_codes(G * N, K, fmt, seed=129, device=dev)
    ws = make_ws(dev, "swz", G, M, N, K, dtype)
    lens = dev_i64(LENS, dev)
    if epi == ptm.PT_EPI_SWIGLU_MXFP4:
        out = torch.empty((M, N // 4), dtype=torch.uint8, device=dev)
        osc = torch.empty((M, N // 64), dtype=torch.uint8, device=dev)
    else:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        osc = None

    def fn():
        ptm.pt_grouped_gemm_fwd(aq, as_, bq, bs, out, osc, lens, None, G, M, N, K, dtype, 1, epi, workspace=ws)
        return out if osc is None else torch.cat([out.view(-1), osc.view(-1)])
    assert_identical(per_config(fn))


def test_mx_dgrad_and_fp8_configs_identical(dev, rules):
    M, G, K, N = int(LENS.sum()), len(LENS), 136, 288
    dq, ds = synth.random_mx_codes(M, N, "e4m3", seed=130, device=dev)
    bq, bs = synth.random_mx_codes(G * K, N, "e4m3", seed=131, device=dev)
    ws = torch.zeros((ptm.pt_grouped_gemm_workspace_size(ptm.PT_OP_DGRAD, G, M, N, K, ptm.PT_MXFP8_E4M3),),
                     dtype=torch.uint8, device=dev)
    lens = dev_i64(LENS, dev)
    dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)

    def fn():
        ptm.pt_grouped_gemm_dgrad(dq, ds, bq, bs, dx, lens, None, G, M, N, K, ptm.PT_MXFP8_E4M3, 0, workspace=ws)
        return dx
    assert_identical(per_config(fn))
    # FP8 with tensor factors: only the tile order varies
    fa = torch.tensor([2.0 ** -7], dtype=torch.float32, device=dev)
    fb = torch.tensor(np.linspace(0.001, 0.004, G), dtype=torch.float32, device=dev)
    out = torch.empty((M, K), dtype=torch.bfloat16, device=dev)

    def fn8():
        ptm.pt_grouped_gemm_fwd(dq, fa, bq, fb, out, None, lens, None, G, M, K, N, ptm.PT_FP8_E4M3, 1,
                                ptm.PT_EPI_NONE, workspace=ws)
        return out
    assert_identical(per_config(fn8))


def test_tuning_picks_a_configuration_and_keeps_results(dev, rules):
    M, G, K, N = int(LENS.sum()), len(LENS), 200, 256
    a = synth.randn_bf16((M, K), seed=132, std=K ** -0.5, device=dev)
    b = synth.randn_bf16((G, K, N), seed=133, std=K ** -0.5, device=dev)
    ws = make_ws(dev, "queue")
    lens = dev_i64(LENS, dev)
    out = torch.empty((M, N // 2), dtype=torch.bfloat16, device=dev)
    ptm.pt_grouped_gemm_fwd(a, None, b, None, out, None, lens, None, G, M, N, K, ptm.PT_BF16, 0,
                            ptm.PT_EPI_SWIGLU, workspace=ws)
    ref = out.clone()
    assert ptm.pt_gemm_config_of(ptm.PT_OP_FWD, ptm.PT_BF16, ptm.PT_EPI_SWIGLU, 0, G, M, N, K) == -1
    assert ptm.pt_set_gemm_config(ptm.PT_CONFIG_TUNE) == ptm.PT_CONFIG_RULES
    out.zero_()
    ptm.pt_grouped_gemm_fwd(a, None, b, None, out, None, lens, None, G, M, N, K, ptm.PT_BF16, 0,
                            ptm.PT_EPI_SWIGLU, workspace=ws)
    torch.cuda.synchronize()
    cfg = ptm.pt_gemm_config_of(ptm.PT_OP_FWD, ptm.PT_BF16, ptm.PT_EPI_SWIGLU, 0, G, M, N, K)
    assert cfg in CONFIGS
    assert torch.equal(out, ref)
    # the class covers row counts up to the next power of two
    assert ptm.pt_gemm_config_of(ptm.PT_OP_FWD, ptm.PT_BF16, ptm.PT_EPI_SWIGLU, 0, G, M - 100, N, K) == cfg
    # an accumulating weight gradient is not timed: main_grad grows by one increment
    Nw = 136
    dy = synth.randn_bf16((M, Nw), seed=134, std=1e-2, device=dev)
    mg = torch.ones((G, K, Nw), dtype=torch.float32, device=dev)
    ptm.pt_grouped_gemm_wgrad(a, None, dy, None, mg, lens, None, G, M, Nw, K, ptm.PT_BF16, 0, 1, workspace=ws)
    torch.cuda.synchronize()
    assert ptm.pt_gemm_config_of(ptm.PT_OP_WGRAD, ptm.PT_BF16, 0, 0, G, M, Nw, K) == -1
    ptm.pt_set_gemm_config(ptm.PT_CONFIG_RULES)
    mg_ref = torch.ones((G, K, Nw), dtype=torch.float32, device=dev)
    ptm.pt_grouped_gemm_wgrad(a, None, dy, None, mg_ref, lens, None, G, M, Nw, K, ptm.PT_BF16, 0, 1, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(mg, mg_ref)
    # the same class without accumulation is timed
    ptm.pt_set_gemm_config(ptm.PT_CONFIG_TUNE)
    ptm.pt_grouped_gemm_wgrad(a, None, dy, None, mg, lens, None, G, M, Nw, K, ptm.PT_BF16, 0, 0, workspace=ws)
    torch.cuda.synchronize()
    assert ptm.pt_gemm_config_of(ptm.PT_OP_WGRAD, ptm.PT_BF16, 0, 0, G, M, Nw, K) in CONFIGS
    with pytest.raises(ValueError):
        ptm.pt_set_gemm_config(7)
    ptm.pt_clear_gemm_tuning()
    assert ptm.pt_gemm_config_of(ptm.PT_OP_FWD, ptm.PT_BF16, ptm.PT_EPI_SWIGLU, 0, G, M, N, K) == -1
