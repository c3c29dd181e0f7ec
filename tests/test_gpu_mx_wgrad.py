"""GPU parity of the MX weight gradient (MXFP8 and MXFP4):
pt_mx_quantize_tokens bit-exact against the oracle (blocks of 32 tokens
inside each expert, the last one partial), and pt_grouped_gemm_wgrad on those
codes against the oracle's sum of exact products, accumulating into and
overwriting main_grad, in both output layouts, through the C ABI."""
import numpy as np
import pytest
import torch

import moe_expert_grouped_gemm_amd as ptm
from moe_expert_grouped_gemm_amd import synth
from util import BF16_TOL, bits16, dev_i64, floored_rel_err, u8

pytestmark = pytest.mark.gpu


FMTS = [ptm.PT_MXFP8_E4M3, ptm.PT_MXFP4_E2M1]
FMT_IDS = ["e4m3", "e2m1"]


def quantize_tokens(dev, x, lens, fmt=ptm.PT_MXFP8_E4M3):
    M, C = x.shape
    G = len(lens)
    q = torch.full((M, C if fmt == ptm.PT_MXFP8_E4M3 else C // 2), 0xEE, dtype=torch.uint8, device=dev)
    s = torch.zeros((M // 32 + G, C), dtype=torch.uint8, device=dev)
    ptm.pt_mx_quantize_tokens(x, dev_i64(lens, dev), None, q, s, G, M, C, fmt)
    torch.cuda.synchronize()
    return q, s


# the oracle numbers its encodings as the library does (1 = E4M3, 2 = E2M1)
@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("lens,C", [([0, 70, 1, 0, 300, 129, 0], 136), ([32, 64, 33], 48), ([5], 8)],
                         ids=["ragged", "aligned_and_one_over", "tiny"])
def test_quantize_tokens_bit_exact(orc, dev, lens, C, fmt):
    lens = np.array(lens, np.int64)
    M = int(lens.sum())
    x = synth.randn_bf16((M, C), seed=100, device=dev, outlier_frac=0.01, outlier_mult=50.0)
    q, s = quantize_tokens(dev, x, lens, fmt)
    rq, rs, nb = orc.mx_quantize_tokens(bits16(x), lens, fmt)
    assert (u8(q) == rq).all()
    assert (u8(s)[:nb] == rs[:nb]).all()


def wgrad_mx(dev, aq, as_, dq, ds, lens, N, K, trans_out, accumulate, fmt=ptm.PT_MXFP8_E4M3, seed_mg=103):
    M, G = aq.shape[0], len(lens)
    shape = (G, N, K) if trans_out else (G, K, N)
    g = torch.Generator(device=dev)
    g.manual_seed(seed_mg)
    mg = (torch.randn(shape, generator=g, device=dev) * 1e-3).float()
    before = mg.clone()
    ws = torch.zeros((ptm.pt_grouped_gemm_workspace_size(ptm.PT_OP_WGRAD, G, M, N, K, fmt),),
                     dtype=torch.uint8, device=dev)
    ptm.pt_grouped_gemm_wgrad(aq, as_, dq, ds, mg, dev_i64(lens, dev), None, G, M, N, K, fmt,
                              trans_out, accumulate, workspace=ws)
    torch.cuda.synchronize()
    return before.cpu().numpy(), mg.cpu().numpy()


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("trans_out", [0, 1])
@pytest.mark.parametrize("accumulate", [1, 0])
def test_mx_wgrad_vs_oracle(orc, dev, trans_out, accumulate, fmt):
    lens = np.array([0, 70, 1, 0, 300, 129, 0], np.int64)
    K, N = 200, 136
    M, G = int(lens.sum()), len(lens)
    print(f"mx wgrad fmt={fmt} trans_out={trans_out} acc={accumulate}", flush=True)
    a = synth.randn_bf16((M, K), seed=101, std=K ** -0.5, device=dev)
    dy = synth.randn_bf16((M, N), seed=102, std=1e-2, device=dev)
    aq, as_ = quantize_tokens(dev, a, lens, fmt)
    dq, ds = quantize_tokens(dev, dy, lens, fmt)
    raq, ras, _ = orc.mx_quantize_tokens(bits16(a), lens, fmt)
    rdq, rds, nb = orc.mx_quantize_tokens(bits16(dy), lens, fmt)
    assert (u8(aq) == raq).all() and (u8(dq) == rdq).all()
    before, after = wgrad_mx(dev, aq, as_, dq, ds, lens, N, K, trans_out, accumulate, fmt)
    av = orc.mx_dequantize_tokens(raq, ras, lens, fmt)
    dv = orc.mx_dequantize_tokens(rdq, rds, lens, fmt)
    offs = synth.offsets(lens)
    for g in range(G):
        if lens[g] == 0:
            if accumulate:
                assert (after[g] == before[g]).all(), "empty expert touched"
            else:
                assert (after[g] == 0).all()
            continue
        D = av[offs[g]:offs[g + 1]].T @ dv[offs[g]:offs[g + 1]]          # [K, N], binary64
        if trans_out:
            D = D.T
        inc = after[g].astype(np.float64) - (before[g] if accumulate else 0.0)
        assert floored_rel_err(inc, D) <= BF16_TOL, g


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("trans_out", [0, 1])
def test_mx_wgrad_multi_tile_both_orders(orc, dev, trans_out, fmt):
    # several output tiles with ragged edges (K = 520, N = 264), an expert
    # over five 128-byte stages and experts ending inside a stage, block and
    # tile; the queued and the static tile order give the same bits
    lens = np.array([700, 0, 33, 260, 1, 64], np.int64)
    K, N = 520, 264
    M, G = int(lens.sum()), len(lens)
    a = synth.randn_bf16((M, K), seed=111, std=K ** -0.5, device=dev)
    dy = synth.randn_bf16((M, N), seed=112, std=1e-2, device=dev)
    aq, as_ = quantize_tokens(dev, a, lens, fmt)
    dq, ds = quantize_tokens(dev, dy, lens, fmt)
    raq, ras, _ = orc.mx_quantize_tokens(bits16(a), lens, fmt)
    rdq, rds, _ = orc.mx_quantize_tokens(bits16(dy), lens, fmt)
    av = orc.mx_dequantize_tokens(raq, ras, lens, fmt)
    dv = orc.mx_dequantize_tokens(rdq, rds, lens, fmt)
    offs = synth.offsets(lens)
    runs = []
    try:
        for cfg in (ptm.PT_CONFIG_RULES, 1):
            ptm.pt_set_gemm_config(cfg)
            print(f"mx wgrad multi-tile fmt={fmt} trans_out={trans_out} cfg={cfg}", flush=True)
            runs.append(wgrad_mx(dev, aq, as_, dq, ds, lens, N, K, trans_out, 1, fmt))
    finally:
        ptm.pt_set_gemm_config(ptm.PT_CONFIG_RULES)
    before, after = runs[0]
    assert (runs[1][0] == before).all() and (runs[1][1] == after).all(), "tile orders disagree"
    for g in range(G):
        if lens[g] == 0:
            assert (after[g] == before[g]).all()
            continue
        D = av[offs[g]:offs[g + 1]].T @ dv[offs[g]:offs[g + 1]]
        inc = after[g].astype(np.float64) - before[g]
        assert floored_rel_err(inc, D.T if trans_out else D) <= BF16_TOL, g


def test_mx_wgrad_needs_its_workspace(dev):
    lens = dev_i64(np.array([40], np.int64), dev)
    q = torch.zeros((40, 64), dtype=torch.uint8, device=dev)
    s = torch.zeros((3, 64), dtype=torch.uint8, device=dev)
    mg = torch.zeros((1, 64, 64), dtype=torch.float32, device=dev)
    L = ptm.load()
    st = torch.cuda.current_stream().cuda_stream
    small = torch.zeros((4096,), dtype=torch.uint8, device=dev)
    args = (q.data_ptr(), s.data_ptr(), q.data_ptr(), s.data_ptr(), mg.data_ptr(), lens.data_ptr(), None,
            1, 40, 64, 64, ptm.PT_MXFP8_E4M3, 0, 1)
    assert L.pt_grouped_gemm_wgrad(*args, None, 0, st) == 4
    assert L.pt_grouped_gemm_wgrad(*args, small.data_ptr(), 4096, st) == 4
    assert L.pt_grouped_gemm_wgrad(q.data_ptr(), s.data_ptr(), q.data_ptr(), s.data_ptr(), mg.data_ptr(),
                                   lens.data_ptr(), None, 1, 40, 64, 64, ptm.PT_MXFP4_E2M1, 0, 1, None, 0, st) == 4
    # FP8 with row factors has no weight gradient
    assert L.pt_grouped_gemm_wgrad(q.data_ptr(), s.data_ptr(), q.data_ptr(), s.data_ptr(), mg.data_ptr(),
                                   lens.data_ptr(), None, 1, 40, 64, 64, ptm.PT_FP8_E4M3_ROWWISE, 0, 1, None, 0,
                                   st) == 2


def element_values(orc, codes, fmt):
    # exact values of a [rows, cols] (E4M3) or [rows, cols/2] (E2M1) code array
    if fmt == ptm.PT_MXFP8_E4M3:
        return np.array([orc.e4m3_value(c) for c in range(256)], np.float64)[codes]
    table = np.array([orc.e2m1_value(c) for c in range(16)], np.float64)
    out = np.empty(codes.shape[:-1] + (2 * codes.shape[-1],), np.float64)
    out[..., 0::2], out[..., 1::2] = table[codes & 0xF], table[codes >> 4]
    return out


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
def test_mx_wgrad_full_shape_sampled(orc, dev, fmt):
    # The weight gradient at the headline's shape: 256 experts, 49152 tokens,
    # K = N = 4096, accumulated into a seeded fp32 main_grad; sampled
    # (expert, k) rows of the increment against the oracle.
    lens = synth.lens_topk_gaussian(8192, 256, 6, seed=1)
    G, M, K, N = 256, int(lens.sum()), 4096, 4096
    offs = synth.offsets(lens)
    a = synth.randn_bf16((M, K), seed=101, std=K ** -0.5, device=dev)
    dy = synth.randn_bf16((M, N), seed=102, std=1e-2, device=dev)
    aq, as_ = quantize_tokens(dev, a, lens, fmt)
    dq, ds = quantize_tokens(dev, dy, lens, fmt)
    del a, dy
    gen = torch.Generator(device=dev)
    gen.manual_seed(103)
    mg = torch.randn((G, K, N), generator=gen, device=dev, dtype=torch.float32).mul_(1e-3)
    rng = np.random.default_rng(11)
    nz = np.nonzero(lens)[0]
    gs = np.concatenate([rng.choice(nz, size=8, replace=False), [nz[np.argmax(lens[nz])]]])
    ks = rng.integers(0, K, size=gs.size)
    gi, ki = torch.as_tensor(gs, device=dev), torch.as_tensor(ks, device=dev)
    before = mg[gi, ki].cpu().numpy()
    ws = torch.zeros((ptm.pt_grouped_gemm_workspace_size(ptm.PT_OP_WGRAD, G, M, N, K, fmt),),
                     dtype=torch.uint8, device=dev)
    ptm.pt_grouped_gemm_wgrad(aq, as_, dq, ds, mg, dev_i64(lens, dev), None, G, M, N, K, fmt, 0, 1,
                              workspace=ws)
    torch.cuda.synchronize()
    after = mg[gi, ki].cpu().numpy()
    del mg, ws
    aqn, asn, dqn, dsn = u8(aq), u8(as_), u8(dq), u8(ds)
    for i, (g, k) in enumerate(zip(gs, ks)):
        r0, r1 = offs[g], offs[g + 1]
        b0 = int(sum((int(l) + 31) // 32 for l in lens[:g]))
        blk = b0 + (np.arange(r1 - r0) // 32)
        av = element_values(orc, aqn[r0:r1], fmt)[:, k] * np.ldexp(1.0, asn[blk, k].astype(np.int64) - 127)
        dv = element_values(orc, dqn[r0:r1], fmt) * np.ldexp(1.0, dsn[blk].astype(np.int64) - 127)
        D = av @ dv                                                     # [N], binary64
        assert floored_rel_err(after[i].astype(np.float64) - before[i], D) <= BF16_TOL, (g, k)


@pytest.mark.parametrize("fmt", FMTS + [ptm.PT_FP8_E4M3], ids=FMT_IDS + ["fp8"])
def test_wgrad_with_offsets_and_gaps(orc, dev, fmt):
    # experts at explicit offsets with unowned rows between them: the token
    # quantiser leaves those rows alone, and the weight gradients read only
    # each expert's own rows
    lens = np.array([40, 0, 70, 33], np.int64)
    offs = np.array([5, 60, 60, 140, 173], np.int64)      # rows 0-4, 45-59, 130-139 unowned
    M, G, K, N = 180, len(lens), 64, 48
    a = synth.randn_bf16((M, K), seed=150, std=K ** -0.5, device=dev)
    dy = synth.randn_bf16((M, N), seed=151, std=1e-2, device=dev)
    owned = np.concatenate([np.arange(offs[g], offs[g] + lens[g]) for g in range(G)])
    lens_d, offs_d = dev_i64(lens, dev), dev_i64(offs, dev)
    ws = torch.zeros((ptm.pt_grouped_gemm_workspace_size(ptm.PT_OP_WGRAD, G, M, N, K, fmt),), dtype=torch.uint8,
                     device=dev)
    if fmt == ptm.PT_FP8_E4M3:
        aq = torch.empty((M, K), dtype=torch.uint8, device=dev)
        dq = torch.empty((M, N), dtype=torch.uint8, device=dev)
        f = [torch.empty((1,), dtype=torch.float32, device=dev) for _ in range(4)]
        ptm.pt_fp8_quantize(a, aq, f[0], f[1], 1, M, K)
        ptm.pt_fp8_quantize(dy, dq, f[2], f[3], 1, M, N)
        as_, ds = f[1], f[3]
    else:
        cols = lambda c: c if fmt == ptm.PT_MXFP8_E4M3 else c // 2
        aq = torch.full((M, cols(K)), 0xEE, dtype=torch.uint8, device=dev)
        dq = torch.full((M, cols(N)), 0xEE, dtype=torch.uint8, device=dev)
        as_ = torch.zeros((M // 32 + G, K), dtype=torch.uint8, device=dev)
        ds = torch.zeros((M // 32 + G, N), dtype=torch.uint8, device=dev)
        ptm.pt_mx_quantize_tokens(a, lens_d, offs_d, aq, as_, G, M, K, fmt, workspace=ws)
        ptm.pt_mx_quantize_tokens(dy, lens_d, offs_d, dq, ds, G, M, N, fmt, workspace=ws)
        torch.cuda.synchronize()
        unowned = np.setdiff1d(np.arange(M), owned)
        assert (u8(aq)[unowned] == 0xEE).all() and (u8(dq)[unowned] == 0xEE).all()
        # the owned rows equal the quantisation of the compacted batch
        raq, ras, _ = orc.mx_quantize_tokens(bits16(a)[owned], lens, fmt)
        assert (u8(aq)[owned] == raq).all()
    mg = torch.full((G, K, N), 0.25, dtype=torch.float32, device=dev)
    ptm.pt_grouped_gemm_wgrad(aq, as_, dq, ds, mg, lens_d, offs_d, G, M, N, K, fmt, 0, 1, workspace=ws)
    # rows between the experts' ranges are valid input: no error bit
    assert ptm.pt_read_error_flags(ws) == 0
    got = mg.cpu().numpy().astype(np.float64) - 0.25
    gs, ks = np.repeat(np.arange(G), K), np.tile(np.arange(K), G)
    if fmt == ptm.PT_FP8_E4M3:
        D = orc.fp8_wgrad_rows(u8(aq)[owned], as_.cpu().numpy()[0], u8(dq)[owned], ds.cpu().numpy()[0], lens, N, K,
                               gs, ks).reshape(G, K, N)
    else:
        raq, ras, _ = orc.mx_quantize_tokens(bits16(a)[owned], lens, fmt)
        rdq, rds, _ = orc.mx_quantize_tokens(bits16(dy)[owned], lens, fmt)
        av = orc.mx_dequantize_tokens(raq, ras, lens, fmt)
        dv = orc.mx_dequantize_tokens(rdq, rds, lens, fmt)
        co = np.concatenate([[0], np.cumsum(lens)])
        D = np.stack([av[co[g]:co[g + 1]].T @ dv[co[g]:co[g + 1]] for g in range(G)])
    for g in range(G):
        if lens[g] == 0:
            assert (got[g] == 0).all()
        else:
            assert floored_rel_err(got[g], D[g]) <= BF16_TOL, g
