"""GPU parity of the FP8 weight gradient with one factor per tensor
(pt_grouped_gemm_wgrad, PT_FP8_E4M3) against the oracle, through the C ABI:
A and dY quantised by pt_fp8_quantize, accumulating into and overwriting a
seeded fp32 main_grad in both layouts, empty experts, refusals, and sampled
rows at the GPT-OSS-20B-like MoE shape."""
import numpy as np
import pytest
import torch

import moe_expert_grouped_gemm_amd as ptm
from moe_expert_grouped_gemm_amd import synth
from util import BF16_TOL, dev_i64, floored_rel_err, u8

pytestmark = pytest.mark.gpu


def quantize(dev, x):
    q = torch.empty(x.shape, dtype=torch.uint8, device=dev)
    amax = torch.empty((1,), dtype=torch.float32, device=dev)
    deq = torch.empty((1,), dtype=torch.float32, device=dev)
    ptm.pt_fp8_quantize(x, q, amax, deq, 1, x.shape[0], x.shape[1])
    return q, deq


def run(dev, aq, ad, dq, dd, lens, N, K, trans_out, accumulate, seed_mg=103):
    M, G = aq.shape[0], len(lens)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed_mg)
    mg = torch.randn((G, N, K) if trans_out else (G, K, N), generator=gen, device=dev).mul_(1e-3)
    before = mg.clone()
    ws = torch.zeros((ptm.pt_grouped_gemm_workspace_size(ptm.PT_OP_WGRAD, G, M, N, K, ptm.PT_FP8_E4M3),),
                     dtype=torch.uint8, device=dev)
    ptm.pt_grouped_gemm_wgrad(aq, ad, dq, dd, mg, dev_i64(lens, dev), None, G, M, N, K, ptm.PT_FP8_E4M3,
                              trans_out, accumulate, workspace=ws)
    torch.cuda.synchronize()
    return before.cpu().numpy(), mg.cpu().numpy()


@pytest.mark.parametrize("trans_out", [0, 1])
@pytest.mark.parametrize("accumulate", [1, 0])
def test_fp8_wgrad_vs_oracle(orc, dev, trans_out, accumulate):
    lens = np.array([0, 70, 1, 0, 300, 129, 0], np.int64)
    K, N = 200, 136
    M, G = int(lens.sum()), len(lens)
    print(f"fp8 wgrad trans_out={trans_out} acc={accumulate}", flush=True)
    a = synth.randn_bf16((M, K), seed=101, device=dev, outlier_frac=0.01, outlier_mult=50.0)
    dy = synth.randn_bf16((M, N), seed=102, std=1e-2, device=dev)
    aq, ad = quantize(dev, a)
    dq, dd = quantize(dev, dy)
    before, after = run(dev, aq, ad, dq, dd, lens, N, K, trans_out, accumulate)
    gs, ks = np.repeat(np.arange(G), K), np.tile(np.arange(K), G)
    D = orc.fp8_wgrad_rows(u8(aq), ad.cpu().numpy()[0], u8(dq), dd.cpu().numpy()[0], lens, N, K, gs, ks)
    D = D.reshape(G, K, N)
    if trans_out:
        D = D.transpose(0, 2, 1)
    for g in range(G):
        if lens[g] == 0:
            if accumulate:
                assert np.array_equal(after[g].view(np.uint32), before[g].view(np.uint32)), "empty expert touched"
            else:
                assert (after[g] == 0).all()
            continue
        inc = after[g].astype(np.float64) - (before[g] if accumulate else 0.0)
        assert floored_rel_err(inc, D[g]) <= BF16_TOL, g


def test_fp8_wgrad_empty_batch_and_refusals(dev):
    G, N, K = 3, 64, 64
    lens = dev_i64(np.zeros(G, np.int64), dev)
    mg = torch.ones((G, K, N), dtype=torch.float32, device=dev)
    ptm.pt_grouped_gemm_wgrad(None, None, None, None, mg, lens, None, G, 0, N, K, ptm.PT_FP8_E4M3, 0, 1)
    torch.cuda.synchronize()
    assert (mg == 1).all()
    ptm.pt_grouped_gemm_wgrad(None, None, None, None, mg, lens, None, G, 0, N, K, ptm.PT_FP8_E4M3, 0, 0)
    torch.cuda.synchronize()
    assert (mg == 0).all()
    L = ptm.load()
    st = torch.cuda.current_stream().cuda_stream
    lens1 = dev_i64(np.array([40], np.int64), dev)
    q = torch.zeros((40, 64), dtype=torch.uint8, device=dev)
    f = torch.ones((1,), dtype=torch.float32, device=dev)
    mg1 = torch.zeros((1, 64, 64), dtype=torch.float32, device=dev)
    small = torch.zeros((4096,), dtype=torch.uint8, device=dev)
    args = (q.data_ptr(), f.data_ptr(), q.data_ptr(), f.data_ptr(), mg1.data_ptr(), lens1.data_ptr(), None,
            1, 40, 64, 64)
    assert L.pt_grouped_gemm_wgrad(*args, ptm.PT_FP8_E4M3, 0, 1, small.data_ptr(), 4096, st) == 4
    assert L.pt_grouped_gemm_wgrad(*args, ptm.PT_FP8_E4M3_ROWWISE, 0, 1, None, 0, st) == 2
    assert L.pt_grouped_gemm_wgrad(q.data_ptr(), None, q.data_ptr(), f.data_ptr(), mg1.data_ptr(), lens1.data_ptr(),
                                   None, 1, 40, 64, 64, ptm.PT_FP8_E4M3, 0, 1, None, 0, st) == 1


def test_fp8_wgrad_mxfp8_shape_sampled(orc, dev):
    # G = 32 (Zipf 1.1), M = 65536, K = 2880, N = 5760, accumulated into a
    # seeded main_grad [32, 2880, 5760]; sampled (expert, k) rows
    lens = synth.lens_zipf_distinct(16384, 32, 4, 1.1, seed=3)
    G, M, K, N = 32, int(lens.sum()), 2880, 5760
    a = synth.randn_bf16((M, K), seed=104, device=dev, outlier_frac=0.01, outlier_mult=50.0)
    dy = synth.randn_bf16((M, N), seed=106, std=1e-2, device=dev)
    aq, ad = quantize(dev, a)
    dq, dd = quantize(dev, dy)
    del a, dy
    gen = torch.Generator(device=dev)
    gen.manual_seed(103)
    mg = torch.randn((G, K, N), generator=gen, device=dev).mul_(1e-3)
    rng = np.random.default_rng(17)
    gs = np.concatenate([rng.choice(G, size=6, replace=False), [int(np.argmax(lens))]])
    ks = rng.integers(0, K, size=gs.size)
    gi, ki = torch.as_tensor(gs, device=dev), torch.as_tensor(ks, device=dev)
    before = mg[gi, ki].cpu().numpy()
    ws = torch.zeros((ptm.pt_grouped_gemm_workspace_size(ptm.PT_OP_WGRAD, G, M, N, K, ptm.PT_FP8_E4M3),),
                     dtype=torch.uint8, device=dev)
    ptm.pt_grouped_gemm_wgrad(aq, ad, dq, dd, mg, dev_i64(lens, dev), None, G, M, N, K, ptm.PT_FP8_E4M3, 0, 1,
                              workspace=ws)
    torch.cuda.synchronize()
    after = mg[gi, ki].cpu().numpy()
    del mg, ws
    D = orc.fp8_wgrad_rows(u8(aq), ad.cpu().numpy()[0], u8(dq), dd.cpu().numpy()[0], lens, N, K, gs, ks)
    for i in range(gs.size):
        assert floored_rel_err(after[i].astype(np.float64) - before[i], D[i]) <= BF16_TOL, (gs[i], ks[i])
