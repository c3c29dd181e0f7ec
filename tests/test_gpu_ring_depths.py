"""GPU checks of the BF16 kernel whose operands are both reduction-contiguous
(data gradient with [G,K,N] weights, forward with [G,N,K] weights) at every
stage count of its ring: reduction lengths of 1 to 7 stages of 64 values,
full and partial last stages, on experts whose row blocks run as 128-row
tiles (three ring slots) and as 256-row tiles (two slots), with two column
tiles (the second ragged).  Integer-valued operands keep every sum exact in
fp32, so each output must equal the oracle's exact result rounded once to
bf16, bit for bit, in all four kernel configurations and both tile orders."""
import numpy as np
import pytest
import torch

import moe_expert_grouped_gemm_amd as ptm
from moe_expert_grouped_gemm_amd import synth
from util import bits16, dev_i64, make_ws

pytestmark = pytest.mark.gpu

LENS = np.array([1, 17, 64, 100, 128, 0, 33, 129, 300, 256, 5], np.int64)
REDS = [16, 64, 104, 128, 192, 200, 256, 320, 384, 448]   # multiples of 8 (row alignment)
WIDTH = 264                         # output columns: a full and a ragged column tile
CONFIGS = [0, 1, 2, 3]


@pytest.fixture
def rules():
    yield
    ptm.pt_set_gemm_config(ptm.PT_CONFIG_RULES)


def run_configs(fn, ref_bits):
    for c in CONFIGS:
        ptm.pt_set_gemm_config(c)
        got = fn()
        torch.cuda.synchronize()
        assert (bits16(got) == ref_bits).all(), f"configuration {c}"


@pytest.mark.parametrize("red", REDS)
def test_dgrad_every_stage_count_bit_exact(orc, dev, rules, red):
    M, G, K, N = int(LENS.sum()), len(LENS), WIDTH, red
    print(f"ring depths dgrad N={N}", flush=True)
    dy = synth.integer_bf16((M, N), seed=300 + red, device=dev)
    b = synth.integer_bf16((G, K, N), seed=301 + red, device=dev)
    lens = dev_i64(LENS, dev)
    ws = make_ws(dev, "queue")
    dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    ref = orc.round_bf16(orc.dgrad_rows(bits16(dy), bits16(b), LENS, N, K, 0, np.arange(M)))

    def fn():
        dx.fill_(float("nan"))
        ptm.pt_grouped_gemm_dgrad(dy, None, b, None, dx, lens, None, G, M, N, K, ptm.PT_BF16, 0, workspace=ws)
        return dx
    run_configs(fn, ref)


@pytest.mark.parametrize("red", REDS)
def test_fwd_nk_weights_every_stage_count_bit_exact(orc, dev, rules, red):
    M, G, K, N = int(LENS.sum()), len(LENS), red, WIDTH
    print(f"ring depths fwd [G,N,K] K={K}", flush=True)
    a = synth.integer_bf16((M, K), seed=310 + red, device=dev)
    b = synth.integer_bf16((G, N, K), seed=311 + red, device=dev)
    lens = dev_i64(LENS, dev)
    ws = make_ws(dev, "queue")
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ref = orc.round_bf16(orc.fwd_rows(orc.BF16, bits16(a), None, bits16(b), None, LENS, N, K, 1, np.arange(M)))

    def fn():
        out.fill_(float("nan"))
        ptm.pt_grouped_gemm_fwd(a, None, b, None, out, None, lens, None, G, M, N, K, ptm.PT_BF16, 1,
                                ptm.PT_EPI_NONE, workspace=ws)
        return out
    run_configs(fn, ref)
