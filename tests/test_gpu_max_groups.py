"""GPU parity at the largest expert count the library accepts (PT_MAX_GROUPS =
1024), through the C ABI.  At this count the group table takes 12 KiB of LDS
next to each kernel's operand ring, so every kernel family is run: the BF16
forward (both weight layouts, plain and SwiGLU epilogues, every kernel
configuration and both tile orders), the dgrad, the weight gradient (with
and without the split-reduction workspace), and the MXFP8 / MXFP4 forward
and weight gradient (also from bf16 with the fused quantisation).
The routing mixes empty experts, single rows, experts under one tile and a
few over two tiles."""
import numpy as np
import pytest
import torch

import moe_expert_grouped_gemm_amd as ptm
from moe_expert_grouped_gemm_amd import synth
from util import (BF16_TOL, MX_TOL, bits16, bf16_values, dev_i64, floored_rel_err, group_of_rows, make_ws,
                  norm_err, per_group_max, u8)

pytestmark = pytest.mark.gpu

G = ptm.PT_MAX_GROUPS


def routing() -> np.ndarray:
    rng = np.random.default_rng(1024)
    lens = rng.integers(1, 40, size=G)
    lens[rng.random(G) < 0.3] = 0
    lens[[3, 511, 1023]] = [600, 257, 300]
    lens[[0, 1022]] = [0, 1]
    return lens.astype(np.int64)


LENS = routing()
M = int(LENS.sum())


@pytest.fixture
def rules():
    yield
    ptm.pt_set_gemm_config(ptm.PT_CONFIG_RULES)


def test_routing_shape():
    assert len(LENS) == 1024 and (LENS == 0).sum() > 200 and LENS.max() > 512


@pytest.mark.parametrize("trans_b", [0, 1])
@pytest.mark.parametrize("epi", [ptm.PT_EPI_NONE, ptm.PT_EPI_SWIGLU])
def test_bf16_fwd_max_groups(orc, dev, rules, trans_b, epi):
    K, N = 64, 96
    a = synth.randn_bf16((M, K), seed=300, std=K ** -0.5, device=dev)
    b = synth.randn_bf16((G, K, N), seed=301, std=K ** -0.5, device=dev)
    bb = b.transpose(1, 2).contiguous() if trans_b else b
    rows = np.arange(M)
    ref = orc.grouped_fwd(orc.BF16, bits16(a), None, bits16(bb), None, LENS, N, K, trans_b, epi, rows)["exact"]
    lens_d = dev_i64(LENS, dev)
    first = None
    for cfg in (0, 1, 2, 3):
        ptm.pt_set_gemm_config(cfg)
        for sched in ("static", "queue"):
            print(f"G=1024 bf16 fwd trans_b={trans_b} epi={epi} cfg={cfg} sched={sched} M={M}", flush=True)
            out = torch.full((M, N if epi == ptm.PT_EPI_NONE else N // 2), float("nan"), dtype=torch.bfloat16,
                             device=dev)
            ptm.pt_grouped_gemm_fwd(a, None, bb, None, out, None, lens_d, None, G, M, N, K, ptm.PT_BF16, trans_b,
                                    epi, workspace=make_ws(dev, sched))
            torch.cuda.synchronize()
            got = bits16(out)
            err = per_group_max(floored_rel_err, bf16_values(got), ref, group_of_rows(LENS, rows))
            assert err <= BF16_TOL, (cfg, sched, err)
            if first is None:
                first = got
            assert (got == first).all(), "configurations or tile orders disagree"


@pytest.mark.parametrize("trans_b", [0, 1])
def test_bf16_dgrad_max_groups(orc, dev, trans_b):
    K, N = 80, 64
    dy = synth.randn_bf16((M, N), seed=302, std=1e-2, device=dev)
    b = synth.randn_bf16((G, K, N), seed=303, std=K ** -0.5, device=dev)
    bb = b.transpose(1, 2).contiguous() if trans_b else b
    rows = np.arange(M)
    ref = orc.dgrad_rows(bits16(dy), bits16(bb), LENS, N, K, trans_b, rows)
    for sched in ("static", "queue"):
        print(f"G=1024 bf16 dgrad trans_b={trans_b} sched={sched}", flush=True)
        dx = torch.full((M, K), float("nan"), dtype=torch.bfloat16, device=dev)
        ptm.pt_grouped_gemm_dgrad(dy, None, bb, None, dx, dev_i64(LENS, dev), None, G, M, N, K, ptm.PT_BF16,
                                  trans_b, workspace=make_ws(dev, sched))
        torch.cuda.synchronize()
        err = per_group_max(floored_rel_err, bf16_values(bits16(dx)), ref, group_of_rows(LENS, rows))
        assert err <= BF16_TOL, (sched, err)


@pytest.mark.parametrize("ws_kind", ["none", "queue", "full"])
def test_bf16_wgrad_max_groups(orc, dev, ws_kind):
    K, N = 64, 48
    a = synth.randn_bf16((M, K), seed=304, std=K ** -0.5, device=dev)
    dy = synth.randn_bf16((M, N), seed=305, std=1e-2, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(306)
    mg = (torch.randn((G, K, N), generator=g, device=dev) * 1e-3).float()
    before = mg.cpu().numpy()
    if ws_kind == "none":
        ws = None
    elif ws_kind == "queue":
        ws = make_ws(dev, "queue")
        ws[:4] = 0                              # the error word is the caller's to clear
    else:
        n = ptm.pt_grouped_gemm_workspace_size(ptm.PT_OP_WGRAD, G, M, N, K, ptm.PT_BF16)
        ws = torch.zeros((n,), dtype=torch.uint8, device=dev)
    print(f"G=1024 bf16 wgrad ws={ws_kind}", flush=True)
    ptm.pt_grouped_gemm_wgrad(a, None, dy, None, mg, dev_i64(LENS, dev), None, G, M, N, K, ptm.PT_BF16, 0, 1,
                              workspace=ws)
    torch.cuda.synchronize()
    after = mg.cpu().numpy()
    if ws is not None:
        assert ptm.pt_read_error_flags(ws) == 0
    gs, ks = np.repeat(np.arange(G), K), np.tile(np.arange(K), G)
    D = orc.wgrad_rows(bits16(a), bits16(dy), LENS, N, K, gs, ks).reshape(G, K, N)
    for e in range(G):
        if LENS[e] == 0:
            assert (after[e] == before[e]).all(), f"empty expert {e} touched"
        else:
            assert floored_rel_err(after[e].astype(np.float64) - before[e], D[e]) <= BF16_TOL, e


FMTS = [(ptm.PT_MXFP8_E4M3, "e4m3"), (ptm.PT_MXFP4_E2M1, "e2m1")]


@pytest.mark.parametrize("fmt,name", FMTS, ids=[f[1] for f in FMTS])
@pytest.mark.parametrize("epi", [ptm.PT_EPI_NONE, ptm.PT_EPI_SWIGLU])
def test_mx_fwd_max_groups(orc, dev, rules, fmt, name, epi):
    K, N = 128, 128
    ofmt = orc.E4M3 if fmt == ptm.PT_MXFP8_E4M3 else orc.E2M1
    aq, as_ = synth.random_mx_codes(M, K, name, seed=307, device=dev)
    bq, bs = synth.random_mx_codes(G * N, K, name, seed=308, device=dev)
    rows = np.arange(M)
    ref = orc.grouped_fwd(ofmt, u8(aq), u8(as_), u8(bq).reshape(G, N, -1), u8(bs).reshape(G, N, -1), LENS, N, K,
                          1, epi, rows)["exact"]
    lens_d = dev_i64(LENS, dev)
    first = None
    for cfg in (0, 1, 2, 3):
        ptm.pt_set_gemm_config(cfg)
        for sched in ("static", "queue", "swz"):
            print(f"G=1024 {name} fwd epi={epi} cfg={cfg} sched={sched}", flush=True)
            out = torch.full((M, N if epi == ptm.PT_EPI_NONE else N // 2), float("nan"), dtype=torch.bfloat16,
                             device=dev)
            ptm.pt_grouped_gemm_fwd(aq, as_, bq, bs, out, None, lens_d, None, G, M, N, K, fmt, 1, epi,
                                    workspace=make_ws(dev, sched, G, M, N, K, fmt))
            torch.cuda.synchronize()
            got = bits16(out)
            err = per_group_max(norm_err, bf16_values(got), ref, group_of_rows(LENS, rows))
            assert err <= MX_TOL, (cfg, sched, err)
            if first is None:
                first = got
            assert (got == first).all(), "configurations or tile orders disagree"


@pytest.mark.parametrize("fmt,name", FMTS, ids=[f[1] for f in FMTS])
def test_mx_wgrad_max_groups(orc, dev, fmt, name):
    # the MX weight gradient's transposer and kernel at 1024 experts (most of
    # them far shorter than one 32-token block, one over five stages)
    K, N = 64, 96
    ofmt = orc.E4M3 if fmt == ptm.PT_MXFP8_E4M3 else orc.E2M1
    a = synth.randn_bf16((M, K), seed=309, std=K ** -0.5, device=dev)
    dy = synth.randn_bf16((M, N), seed=310, std=1e-2, device=dev)
    lens_d = dev_i64(LENS, dev)
    cols = (lambda c: c) if fmt == ptm.PT_MXFP8_E4M3 else (lambda c: c // 2)
    aq = torch.empty((M, cols(K)), dtype=torch.uint8, device=dev)
    dq = torch.empty((M, cols(N)), dtype=torch.uint8, device=dev)
    as_ = torch.zeros((M // 32 + G, K), dtype=torch.uint8, device=dev)
    ds = torch.zeros((M // 32 + G, N), dtype=torch.uint8, device=dev)
    ptm.pt_mx_quantize_tokens(a, lens_d, None, aq, as_, G, M, K, fmt)
    ptm.pt_mx_quantize_tokens(dy, lens_d, None, dq, ds, G, M, N, fmt)
    g = torch.Generator(device=dev)
    g.manual_seed(311)
    mg = (torch.randn((G, K, N), generator=g, device=dev) * 1e-3).float()
    before = mg.cpu().numpy()
    n = ptm.pt_grouped_gemm_workspace_size(ptm.PT_OP_WGRAD, G, M, N, K, fmt)
    ws = torch.zeros((n,), dtype=torch.uint8, device=dev)
    print(f"G=1024 {name} wgrad M={M}", flush=True)
    ptm.pt_grouped_gemm_wgrad(aq, as_, dq, ds, mg, lens_d, None, G, M, N, K, fmt, 0, 1, workspace=ws)
    torch.cuda.synchronize()
    after = mg.cpu().numpy()
    assert ptm.pt_read_error_flags(ws) == 0
    raq, ras, _ = orc.mx_quantize_tokens(bits16(a), LENS, ofmt)
    rdq, rds, _ = orc.mx_quantize_tokens(bits16(dy), LENS, ofmt)
    assert (u8(aq) == raq).all() and (u8(dq) == rdq).all()
    av = orc.mx_dequantize_tokens(raq, ras, LENS, ofmt)
    dv = orc.mx_dequantize_tokens(rdq, rds, LENS, ofmt)
    offs = np.concatenate([[0], np.cumsum(LENS)])
    for e in range(G):
        if LENS[e] == 0:
            assert (after[e] == before[e]).all(), f"empty expert {e} touched"
            continue
        D = av[offs[e]:offs[e + 1]].T @ dv[offs[e]:offs[e + 1]]
        assert floored_rel_err(after[e].astype(np.float64) - before[e], D) <= BF16_TOL, e
    # the same from bf16 in one call (quantisation fused into the transpose):
    # bit-identical
    mg2 = torch.as_tensor(before, device=dev)
    ptm.pt_grouped_gemm_wgrad_quantize(a, dy, mg2, lens_d, None, G, M, N, K, fmt, 0, 1, workspace=ws)
    torch.cuda.synchronize()
    assert (mg2.cpu().numpy().view(np.int32) == after.view(np.int32)).all()
