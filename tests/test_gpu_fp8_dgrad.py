"""GPU parity of the FP8 data gradient (current scaling, one factor per
tensor or per row) against the oracle, through the C ABI: dY quantised by
pt_fp8_quantize / pt_fp8_quantize_rows, the forward weight [G, N, K]
transposed per expert by pt_stack_experts and quantised as the [G, K, N]
cache, then pt_grouped_gemm_dgrad with PT_FP8_E4M3 / PT_FP8_E4M3_ROWWISE.
Ragged sizes spanning several tiles with a partial last reduction stage,
both tile orders, and sampled rows at the GPT-OSS-20B-like MoE shape."""
import numpy as np
import pytest
import torch

import moe_expert_grouped_gemm_amd as ptm
from moe_expert_grouped_gemm_amd import synth
from util import (BF16_TOL, MX_TOL, SCHEDS, bf16_values, bits16, dev_i64, floored_rel_err, group_of_rows, make_ws,
                  norm_err, per_group_max, u8)

pytestmark = pytest.mark.gpu

CASES = [
    # (name, lens, K = dX columns, N = reduction)
    ("ragged", [0, 1, 130, 0, 257, 64, 33], 200, 256),
    ("ntail", [200, 0, 56], 192, 288),
    ("one", [129], 128, 64),
]


def quantize(dev, x, batch, rowwise):
    """FP8 codes of x and its factors: one per matrix of the batch, or one per row."""
    rows, cols = x.numel() // x.shape[-1], x.shape[-1]
    q = torch.full(x.shape, 0xEE, dtype=torch.uint8, device=dev)
    n = rows if rowwise else batch
    amax = torch.empty((n,), dtype=torch.float32, device=dev)
    deq = torch.empty((n,), dtype=torch.float32, device=dev)
    if rowwise:
        ptm.pt_fp8_quantize_rows(x, q, amax, deq, rows, cols)
    else:
        ptm.pt_fp8_quantize(x, q, amax, deq, batch, rows // batch, cols)
    return q, deq


def transposed_weight(dev, w, G, N, K):
    """[G, K, N] bf16 from the stacked forward weight [G, N, K], one pass."""
    addr = torch.tensor([w.data_ptr() + g * N * K * 2 for g in range(G)], dtype=torch.int64, device=dev)
    wt = torch.empty((G, K, N), dtype=torch.bfloat16, device=dev)
    ptm.pt_stack_experts(addr, wt, G, N, K, 1)
    return wt


def run(dev, dy, w, lens, N, K, rowwise, ws=None):
    M, G = dy.shape[0], len(lens)
    dq, dd = quantize(dev, dy, 1, rowwise)
    wt = transposed_weight(dev, w, G, N, K)
    wq, wd = quantize(dev, wt, G, rowwise)
    dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    ptm.pt_grouped_gemm_dgrad(dq, dd, wq, wd, dx, dev_i64(lens, dev), None, G, M, N, K,
                              ptm.PT_FP8_E4M3_ROWWISE if rowwise else ptm.PT_FP8_E4M3, 0, workspace=ws)
    torch.cuda.synchronize()
    return dq, dd, wq, wd, dx


def oracle_rows(orc, dq, dd, wq, wd, lens, N, K, rows, rowwise):
    G = len(lens)
    if rowwise:
        return orc.fp8_fwd_rows_rowwise(u8(dq), dd.cpu().numpy(), u8(wq).reshape(G, K, N),
                                        wd.cpu().numpy().reshape(G, K), lens, K, N, rows)
    return orc.fp8_fwd_rows(u8(dq), dd.cpu().numpy()[0], u8(wq).reshape(G, K, N), wd.cpu().numpy(), lens, K, N,
                            rows)


@pytest.mark.parametrize("rowwise", [0, 1], ids=["tensor", "rowwise"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("sched", SCHEDS)
def test_fp8_dgrad_vs_oracle(orc, dev, case, sched, rowwise):
    name, lens, K, N = case
    lens = np.array(lens, np.int64)
    M, G = int(lens.sum()), len(lens)
    print(f"fp8 dgrad case={name} sched={sched} rowwise={rowwise} M={M} K={K} N={N}", flush=True)
    dy = synth.randn_bf16((M, N), seed=95, std=1e-2, device=dev, outlier_frac=0.01, outlier_mult=50.0)
    w = synth.randn_bf16((G, N, K), seed=96, std=K ** -0.5, device=dev)
    dq, dd, wq, wd, dx = run(dev, dy, w, lens, N, K, rowwise, ws=make_ws(dev, sched))
    rows = np.arange(M)
    ref = oracle_rows(orc, dq, dd, wq, wd, lens, N, K, rows, rowwise)
    got = bf16_values(bits16(dx))
    grp = group_of_rows(lens, rows)
    assert per_group_max(floored_rel_err, got, ref, grp) <= BF16_TOL
    assert per_group_max(norm_err, got, ref, grp) <= MX_TOL


def test_fp8_transposed_cache_keeps_the_forward_factor(orc, dev):
    # the transpose has the forward weight's amax, so its per-expert factor
    # (and every code, transposed) is the forward weight's
    G, N, K = 3, 96, 64
    w = synth.randn_bf16((G, N, K), seed=97, std=0.1, device=dev, outlier_frac=0.01, outlier_mult=50.0)
    fq, fd = quantize(dev, w, G, 0)
    tq, td = quantize(dev, transposed_weight(dev, w, G, N, K), G, 0)
    torch.cuda.synchronize()
    assert torch.equal(fd, td)
    assert torch.equal(fq.transpose(1, 2).contiguous(), tq)


def test_fp8_dgrad_refusals(dev):
    L = ptm.load()
    st = torch.cuda.current_stream().cuda_stream
    lens = dev_i64(np.array([64], np.int64), dev)
    q = torch.zeros((64, 64), dtype=torch.uint8, device=dev)
    f = torch.ones((64,), dtype=torch.float32, device=dev)
    dx = torch.zeros((64, 64), dtype=torch.bfloat16, device=dev)
    args = (q.data_ptr(), f.data_ptr(), q.data_ptr(), f.data_ptr(), dx.data_ptr(), lens.data_ptr(), None, 1, 64)
    assert L.pt_grouped_gemm_dgrad(*args, 64, 64, ptm.PT_FP8_E4M3, 1, None, 0, st) == 2      # [G,N,K] weight
    assert L.pt_grouped_gemm_dgrad(*args, 48, 64, ptm.PT_FP8_E4M3, 0, None, 0, st) == 2      # N % 32
    assert L.pt_grouped_gemm_dgrad(q.data_ptr(), None, q.data_ptr(), f.data_ptr(), dx.data_ptr(), lens.data_ptr(),
                                   None, 1, 64, 64, 64, ptm.PT_FP8_E4M3, 0, None, 0, st) == 1  # missing factor


@pytest.mark.parametrize("rowwise", [0, 1], ids=["tensor", "rowwise"])
def test_fp8_dgrad_mxfp8_shape_sampled(orc, dev, rowwise):
    # the GPT-OSS-20B-like shape: 32 experts (Zipf 1.1), 65536 rows,
    # dY [65536, 5760] -> dX [65536, 2880]; sampled rows of every expert
    lens = synth.lens_zipf_distinct(16384, 32, 4, 1.1, seed=3)
    G, M, K, N = 32, int(lens.sum()), 2880, 5760
    dy = synth.randn_bf16((M, N), seed=106, std=1e-2, device=dev, outlier_frac=0.01, outlier_mult=50.0)
    w = synth.randn_bf16((G, N, K), seed=1104, device=dev, outlier_frac=0.01, outlier_mult=50.0)
    dq, dd, wq, wd, dx = run(dev, dy, w, lens, N, K, rowwise, ws=make_ws(dev, "queue"))
    del dy, w
    offs = synth.offsets(lens)
    rng = np.random.default_rng(13)
    rows = np.unique(np.concatenate([[offs[g], offs[g + 1] - 1, rng.integers(offs[g], offs[g + 1])]
                                     for g in range(G) if lens[g] > 0]))
    ref = oracle_rows(orc, dq, dd, wq, wd, lens, N, K, rows, rowwise)
    got = bf16_values(bits16(dx[torch.as_tensor(rows, device=dev)]))
    assert floored_rel_err(got, ref) <= BF16_TOL
