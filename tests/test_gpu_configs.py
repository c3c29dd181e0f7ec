"""Parity at the full workload sizes, in the launch configuration bench.py
times.  The GPU computes the whole problem; the oracle recomputes sampled
outputs one by one: the first, last and a few random rows of a seeded subset
of experts (a compact sub-batch with the same expert weights, so every
sampled row keeps its expert), sampled (expert, k) rows of main_grad, and
whole tensors for the quantiser (bit-exact).

Workloads:
  fc1    DeepSeek-V4-Flash-like FC1: 256 experts, 8192 tokens top-6 = 49152
         rows (imbalanced routing with empty experts), K = N = 4096, weights
         [G, K, N], fused SwiGLU -> [49152, 2048] bf16.
  bwd    dgrad and wgrad at the same shape; wgrad accumulates into a seeded
         fp32 main_grad [256, 4096, 4096].
  mxfp8  GPT-OSS-20B-like: 32 experts, 16384 tokens top-4 = 65536 rows with
         Zipf(1.1) routing, K = 2880, N = 5760, operands quantised from bf16
         N(0,1) with 1% outliers x50.
  mxfp4  expert MLP: quantise -> FC1 + SwiGLU + MXFP4 -> FC2, 256 experts,
         H = 4096, I = 2048, 49152 rows.
"""
import numpy as np
import pytest
import torch

import moe_expert_grouped_gemm_amd as ptm
from moe_expert_grouped_gemm_amd import synth
from util import (BF16_TOL, MX_TOL, bits16, bf16_values, floored_rel_err, make_ws, norm_err, u8)

pytestmark = pytest.mark.gpu

N_EXPERTS_SAMPLED = 12
ROWS_PER_EXPERT = 3


def sample_plan(lens, seed, n_experts=N_EXPERTS_SAMPLED, per=ROWS_PER_EXPERT):
    """Seeded subset of non-empty experts (always including the smallest and
    largest) and, per expert, its first, last and `per` random rows."""
    rng = np.random.default_rng(seed)
    offs = synth.offsets(lens)
    nz = np.nonzero(lens)[0]
    pick = set(rng.choice(nz, size=min(n_experts, nz.size), replace=False).tolist())
    pick.add(int(nz[np.argmin(lens[nz])]))
    pick.add(int(nz[np.argmax(lens[nz])]))
    experts = sorted(pick)
    rows, local_lens = [], []
    for g in experts:
        a, b = int(offs[g]), int(offs[g + 1])
        r = np.unique(np.concatenate([[a, b - 1], rng.integers(a, b, size=min(per, b - a))]))
        rows.append(r)
        local_lens.append(r.size)
    return np.array(experts), rows, np.array(local_lens, np.int64)


def take_rows(t, rows):
    return t[torch.as_tensor(np.concatenate(rows), device=t.device)]


@pytest.fixture(scope="module")
def fc1(dev):
    lens = synth.lens_topk_gaussian(8192, 256, 6, seed=1)
    G, M, K, N = 256, int(lens.sum()), 4096, 4096
    a = synth.randn_bf16((M, K), seed=101, std=K ** -0.5, device=dev)
    b = synth.randn_bf16((G, K, N), seed=1101, std=K ** -0.5, device=dev)
    yield dict(lens=lens, G=G, M=M, K=K, N=N, a=a, b=b)
    del a, b
    torch.cuda.empty_cache()


def test_fc1_routing_shape(fc1):
    lens = fc1["lens"]
    assert lens.sum() == 49152 and lens.size == 256
    assert (lens == 0).sum() >= 4 and lens.max() > 4 * np.median(lens)


def test_fc1_bf16_swiglu_sampled(orc, dev, fc1):
    lens, G, M, K, N, a, b = (fc1[k] for k in ("lens", "G", "M", "K", "N", "a", "b"))
    out = torch.empty((M + 2, N // 2), dtype=torch.bfloat16, device=dev)
    out.view(torch.int16).fill_(0x7FC1)
    ptm.pt_grouped_gemm_fwd(a, None, b, None, out[1:M + 1], None, torch.as_tensor(lens, device=dev), None,
                            G, M, N, K, ptm.PT_BF16, 0, ptm.PT_EPI_SWIGLU, workspace=make_ws(dev, "queue"))
    torch.cuda.synchronize()
    assert (bits16(out[0]) == 0x7FC1).all() and (bits16(out[M + 1]) == 0x7FC1).all()
    experts, rows, local = sample_plan(lens, seed=1)
    print(f"fc1: {local.sum()} rows of experts {experts.tolist()}", flush=True)
    ref = orc.grouped_fwd(orc.BF16, bits16(take_rows(a, rows)), None, bits16(b[torch.as_tensor(experts, device=dev)]),
                          None, local, N, K, 0, orc.EPI_SWIGLU, np.arange(local.sum()))["exact"]
    got = bf16_values(bits16(take_rows(out[1:M + 1], rows)))
    start = 0
    for g, r in zip(experts, rows):
        sl = slice(start, start + r.size)
        assert floored_rel_err(got[sl], ref[sl]) <= BF16_TOL, g
        start += r.size
    assert floored_rel_err(got, ref) <= BF16_TOL


def test_bwd_dgrad_sampled(orc, dev, fc1):
    lens, G, M, K, N, b = (fc1[k] for k in ("lens", "G", "M", "K", "N", "b"))
    dy = synth.randn_bf16((M, N), seed=102, std=1e-2, device=dev)
    dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    ptm.pt_grouped_gemm_dgrad(dy, None, b, None, dx, torch.as_tensor(lens, device=dev), None,
                              G, M, N, K, ptm.PT_BF16, 0, workspace=make_ws(dev, "queue"))
    torch.cuda.synchronize()
    experts, rows, local = sample_plan(lens, seed=2)
    ref = orc.dgrad_rows(bits16(take_rows(dy, rows)), bits16(b[torch.as_tensor(experts, device=dev)]),
                         local, N, K, 0, np.arange(local.sum()))
    got = bf16_values(bits16(take_rows(dx, rows)))
    start = 0
    for g, r in zip(experts, rows):
        sl = slice(start, start + r.size)
        assert floored_rel_err(got[sl], ref[sl]) <= BF16_TOL, g
        start += r.size


def test_bwd_wgrad_sampled_and_empty_experts_untouched(orc, dev, fc1):
    lens, G, M, K, N, a = (fc1[k] for k in ("lens", "G", "M", "K", "N", "a"))
    dy = synth.randn_bf16((M, N), seed=102, std=1e-2, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(103)
    mg = torch.randn((G, K, N), generator=gen, device=dev, dtype=torch.float32).mul_(1e-3)
    rng = np.random.default_rng(3)
    nz = np.nonzero(lens)[0]
    gs = np.concatenate([rng.choice(nz, size=10, replace=False), [nz[np.argmax(lens[nz])]]])
    ks = rng.integers(0, K, size=gs.size)
    ks[:3] = [0, K - 1, 2048]
    empty = np.nonzero(lens == 0)[0]
    before_rows = mg[torch.as_tensor(gs, device=dev), torch.as_tensor(ks, device=dev)].cpu().numpy()
    before_empty = mg[torch.as_tensor(empty, device=dev)].clone()
    ptm.pt_grouped_gemm_wgrad(a, None, dy, None, mg, torch.as_tensor(lens, device=dev), None,
                              G, M, N, K, ptm.PT_BF16, 0, 1, workspace=make_ws(dev, "queue"))
    torch.cuda.synchronize()
    assert torch.equal(mg[torch.as_tensor(empty, device=dev)], before_empty)
    after = mg[torch.as_tensor(gs, device=dev), torch.as_tensor(ks, device=dev)].cpu().numpy()
    offs = synth.offsets(lens)
    for i, (g, k) in enumerate(zip(gs, ks)):
        r0, r1 = int(offs[g]), int(offs[g + 1])
        d = orc.wgrad_rows(bits16(a[r0:r1]), bits16(dy[r0:r1]), np.array([r1 - r0]), N, K,
                           np.array([0]), np.array([k]))[0]
        inc = after[i].astype(np.float64) - before_rows[i]
        assert floored_rel_err(inc, d) <= BF16_TOL, (g, k)
    del mg, before_empty
    torch.cuda.empty_cache()


def test_mxfp8_quantize_and_fwd(orc, dev):
    lens = synth.lens_zipf_distinct(16384, 32, 4, 1.1, seed=3)
    assert lens.sum() == 65536 and lens.max() <= 16384
    G, M, K, N = 32, int(lens.sum()), 2880, 5760
    x = synth.randn_bf16((M, K), seed=104, device=dev, outlier_frac=0.01, outlier_mult=50.0)
    w = synth.randn_bf16((G * N, K), seed=1104, device=dev, outlier_frac=0.01, outlier_mult=50.0)
    aq = torch.empty((M, K), dtype=torch.uint8, device=dev)
    as_ = torch.empty((M, K // 32), dtype=torch.uint8, device=dev)
    bq = torch.empty((G * N, K), dtype=torch.uint8, device=dev)
    bs = torch.empty((G * N, K // 32), dtype=torch.uint8, device=dev)
    ptm.pt_mx_quantize(x, aq, as_, M, K, ptm.PT_MXFP8_E4M3, 1)
    ptm.pt_mx_quantize(w, bq, bs, G * N, K, ptm.PT_MXFP8_E4M3, 1)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ptm.pt_grouped_gemm_fwd(aq, as_, bq, bs, out, None, torch.as_tensor(lens, device=dev), None,
                            G, M, N, K, ptm.PT_MXFP8_E4M3, 1, ptm.PT_EPI_NONE,
                            workspace=make_ws(dev, "swz", G, M, N, K, ptm.PT_MXFP8_E4M3))
    torch.cuda.synchronize()
    # quantiser: whole tensors, bit-exact, against the oracle's own quantiser
    rxq, rxs = orc.mx_quantize(bits16(x), orc.E4M3)
    assert (u8(as_) == rxs).all() and (u8(aq) == rxq).all()
    rwq, rws = orc.mx_quantize(bits16(w), orc.E4M3)
    assert (u8(bs) == rws).all() and (u8(bq) == rwq).all()
    # GEMM on sampled rows, oracle fed its own quantised operands
    experts, rows, local = sample_plan(lens, seed=4, n_experts=8)
    allrows = np.concatenate(rows)
    wq3, ws3 = rwq.reshape(G, N, K), rws.reshape(G, N, K // 32)
    ref = orc.fwd_rows(orc.E4M3, rxq[allrows], rxs[allrows], wq3[experts], ws3[experts],
                       local, N, K, 1, np.arange(allrows.size))
    got = bf16_values(bits16(take_rows(out, rows)))
    start = 0
    for g, r in zip(experts, rows):
        sl = slice(start, start + r.size)
        assert norm_err(got[sl], ref[sl]) <= MX_TOL, g
        start += r.size
    assert floored_rel_err(got, ref) <= BF16_TOL


def test_mxfp4_mlp_chain(orc, dev):
    lens = synth.lens_topk_gaussian(8192, 256, 6, seed=1)
    G, M, H, I = 256, int(lens.sum()), 4096, 2048
    x = synth.randn_bf16((M, H), seed=105, device=dev)
    w1 = synth.randn_bf16((G * 2 * I, H), seed=1105, device=dev)
    w2 = synth.randn_bf16((G * H, I), seed=2105, device=dev)
    w1q = torch.empty((G * 2 * I, H // 2), dtype=torch.uint8, device=dev)
    w1s = torch.empty((G * 2 * I, H // 32), dtype=torch.uint8, device=dev)
    w2q = torch.empty((G * H, I // 2), dtype=torch.uint8, device=dev)
    w2s = torch.empty((G * H, I // 32), dtype=torch.uint8, device=dev)
    ptm.pt_mx_quantize(w1, w1q, w1s, G * 2 * I, H, ptm.PT_MXFP4_E2M1, 1)
    ptm.pt_mx_quantize(w2, w2q, w2s, G * H, I, ptm.PT_MXFP4_E2M1, 1)
    xq = torch.empty((M, H // 2), dtype=torch.uint8, device=dev)
    xs = torch.empty((M, H // 32), dtype=torch.uint8, device=dev)
    hq = torch.empty((M, I // 2), dtype=torch.uint8, device=dev)
    hs = torch.empty((M, I // 32), dtype=torch.uint8, device=dev)
    out = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    lens_d = torch.as_tensor(lens, device=dev)
    ptm.pt_mx_quantize(x, xq, xs, M, H, ptm.PT_MXFP4_E2M1, 1)
    ws = make_ws(dev, "swz", G, M, 2 * I, H, ptm.PT_MXFP4_E2M1)     # the larger of the two calls
    ptm.pt_grouped_gemm_fwd(xq, xs, w1q, w1s, hq, hs, lens_d, None, G, M, 2 * I, H,
                            ptm.PT_MXFP4_E2M1, 1, ptm.PT_EPI_SWIGLU_MXFP4, workspace=ws)
    ptm.pt_grouped_gemm_fwd(hq, hs, w2q, w2s, out, None, lens_d, None, G, M, H, I,
                            ptm.PT_MXFP4_E2M1, 1, ptm.PT_EPI_NONE, workspace=ws)
    torch.cuda.synchronize()
    experts, rows, local = sample_plan(lens, seed=5, n_experts=8)
    e_d = torch.as_tensor(experts, device=dev)
    # the oracle quantises the sampled experts' bf16 weights itself; the
    # GPU's weights for those experts must match bit for bit
    w1e = bits16(w1.view(G, 2 * I, H)[e_d]).reshape(-1, H)
    w2e = bits16(w2.view(G, H, I)[e_d]).reshape(-1, I)
    r1q, r1s = orc.mx_quantize(w1e, orc.E2M1)
    r2q, r2s = orc.mx_quantize(w2e, orc.E2M1)
    assert (u8(w1q.view(G, 2 * I, -1)[e_d]).reshape(r1q.shape) == r1q).all()
    assert (u8(w1s.view(G, 2 * I, -1)[e_d]).reshape(r1s.shape) == r1s).all()
    assert (u8(w2q.view(G, H, -1)[e_d]).reshape(r2q.shape) == r2q).all()
    assert (u8(w2s.view(G, H, -1)[e_d]).reshape(r2s.shape) == r2s).all()
    ne = len(experts)
    ref = orc.mlp_mxfp4_rows(bits16(take_rows(x, rows)),
                             r1q.reshape(ne, 2 * I, H // 2), r1s.reshape(ne, 2 * I, H // 32),
                             r2q.reshape(ne, H, I // 2), r2s.reshape(ne, H, I // 32),
                             local, H, I, np.arange(local.sum()))
    allrows = np.concatenate(rows)
    # activation quantisation of the sampled rows is bit-exact
    rxq, rxs = orc.mx_quantize(bits16(take_rows(x, rows)), orc.E2M1)
    assert (u8(xq)[allrows] == rxq).all() and (u8(xs)[allrows] == rxs).all()
    # FC1 -> SwiGLU -> MXFP4 intermediate, compared dequantised
    got_h = orc.mx_dequantize(orc.E2M1, u8(hq)[allrows], u8(hs)[allrows], allrows.size, I)
    want_h = orc.mx_dequantize(orc.E2M1, ref["h_q"], ref["h_s"], allrows.size, I)
    got = bf16_values(bits16(take_rows(out, rows)))
    start = 0
    for g, r in zip(experts, rows):
        sl = slice(start, start + r.size)
        assert norm_err(got_h[sl], want_h[sl]) <= MX_TOL, ("h", g)
        assert norm_err(got[sl], ref["exact"][sl]) <= MX_TOL, ("out", g)
        start += r.size
