"""GPU parity of the weight gradient's split reduction, through the C ABI.

With a workspace of pt_grouped_gemm_workspace_size(PT_OP_WGRAD, ...) bytes,
an expert with more tokens than the chunk length is cut into token chunks
whose fp32 partial sums are added into main_grad in chunk order.  At a shape
with one output tile per expert (K = N = 256, chunk length 512 tokens) a
12.5k-token expert among experts of at most 500 tokens is cut into 25
chunks.  Checked: the increment against the oracle's A_g^T dY_g (BF16
tolerance), zero-token experts untouched when accumulating and zeroed when
not, bit-identical reruns, both output layouts, the static and queued tile
orders, the MXFP8 / MXFP4 weight gradient's own split (whole 256-token
stages per chunk), and that malformed (overlapping) ranges never write past
the partial slots."""
import numpy as np
import pytest
import torch

import moe_expert_grouped_gemm_amd as ptm
from moe_expert_grouped_gemm_amd import synth
from util import BF16_TOL, bits16, dev_i64, floored_rel_err, u8

pytestmark = pytest.mark.gpu

LENS = np.array([12500, 480, 0, 350, 499, 1, 200], np.int64)
K, N = 256, 256


def ws_full(dev, G, M, dtype=ptm.PT_BF16, tail=0):
    n = ptm.pt_grouped_gemm_workspace_size(ptm.PT_OP_WGRAD, G, M, N, K, dtype)
    buf = torch.full((n + tail,), 0xA5, dtype=torch.uint8, device=dev)
    return buf, n


def run(dev, a, dy, lens, trans_out, accumulate, ws, nbytes, dtype=ptm.PT_BF16, a_s=None, d_s=None, offs=None):
    G, M = len(lens), a.shape[0]
    shape = (G, N, K) if trans_out else (G, K, N)
    g = torch.Generator(device=dev)
    g.manual_seed(203)
    mg = (torch.randn(shape, generator=g, device=dev) * 1e-3).float()
    before = mg.cpu().numpy()
    L = ptm.load()
    st = L.pt_grouped_gemm_wgrad(a.data_ptr(), None if a_s is None else a_s.data_ptr(), dy.data_ptr(),
                                 None if d_s is None else d_s.data_ptr(), mg.data_ptr(),
                                 dev_i64(lens, dev).data_ptr(), None if offs is None else offs.data_ptr(),
                                 G, M, N, K, dtype, trans_out, accumulate, ws.data_ptr(), nbytes,
                                 torch.cuda.current_stream().cuda_stream)
    assert st == 0, ptm.pt_status_string(st)
    torch.cuda.synchronize()
    return before, mg.cpu().numpy()


def oracle_D(orc, a_bits, dy_bits, lens):
    G = len(lens)
    gs, ks = np.repeat(np.arange(G), K), np.tile(np.arange(K), G)
    return orc.wgrad_rows(a_bits, dy_bits, lens, N, K, gs, ks).reshape(G, K, N)


def check(before, after, D, lens, trans_out, accumulate):
    for g in range(len(lens)):
        want = D[g].T if trans_out else D[g]
        if lens[g] == 0:
            assert (after[g] == (before[g] if accumulate else 0)).all(), g
            continue
        inc = after[g].astype(np.float64) - (before[g] if accumulate else 0)
        assert floored_rel_err(inc, want) <= BF16_TOL, g


@pytest.fixture(scope="module")
def data(orc, dev):
    M = int(LENS.sum())
    a = synth.randn_bf16((M, K), seed=210, std=K ** -0.5, device=dev)
    dy = synth.randn_bf16((M, N), seed=211, std=1e-2, device=dev)
    return a, dy, oracle_D(orc, bits16(a), bits16(dy), LENS)


def test_split_engages_at_this_shape(dev):
    M, G = int(LENS.sum()), len(LENS)
    small = ptm.pt_grouped_gemm_workspace_size(ptm.PT_OP_FWD, 1, 1, 1, 1, ptm.PT_BF16)
    # chunk length max(512, ceil(M * tiles / 1024)) = 512 tokens, M // 512 partial slots of K x N fp32
    assert ptm.pt_grouped_gemm_workspace_size(ptm.PT_OP_WGRAD, G, M, N, K, ptm.PT_BF16) >= \
        small + (M // 512) * K * N * 4


@pytest.mark.parametrize("trans_out", [0, 1])
@pytest.mark.parametrize("accumulate", [1, 0])
def test_split_wgrad_vs_oracle_and_deterministic(dev, data, trans_out, accumulate):
    a, dy, D = data
    M, G = a.shape[0], len(LENS)
    print(f"split wgrad trans_out={trans_out} accumulate={accumulate} M={M}", flush=True)
    ws, n = ws_full(dev, G, M, tail=4096)
    before, after = run(dev, a, dy, LENS, trans_out, accumulate, ws, n)
    check(before, after, D, LENS, trans_out, accumulate)
    assert (u8(ws[n:]) == 0xA5).all(), "write past the workspace"
    _, again = run(dev, a, dy, LENS, trans_out, accumulate, ws, n)
    assert (again == after).all(), "split reduction not deterministic"
    # the static tile order gives the same bits
    ptm.pt_set_gemm_config(1)
    try:
        _, st = run(dev, a, dy, LENS, trans_out, accumulate, ws, n)
    finally:
        ptm.pt_set_gemm_config(ptm.PT_CONFIG_RULES)
    assert (st == after).all()


def test_split_close_to_unsplit(dev, data):
    # the same sums in another order: within fp32 rounding of the unsplit kernel
    a, dy, D = data
    M, G = a.shape[0], len(LENS)
    ws, n = ws_full(dev, G, M)
    _, split = run(dev, a, dy, LENS, 0, 0, ws, n)
    small = torch.zeros(ptm.pt_grouped_gemm_workspace_size(ptm.PT_OP_FWD, 1, 1, 1, 1, ptm.PT_BF16),
                       dtype=torch.uint8, device=dev)
    _, whole = run(dev, a, dy, LENS, 0, 0, small, small.numel())
    assert floored_rel_err(split, whole) <= 1e-4


@pytest.mark.parametrize("fmt", [ptm.PT_MXFP8_E4M3, ptm.PT_MXFP4_E2M1], ids=["e4m3", "e2m1"])
def test_split_mx_wgrad_vs_oracle_and_deterministic(orc, dev, data, fmt):
    # the MX weight gradient cuts the long expert the same way (chunks of
    # 512 tokens, whole 256-token stages): against the oracle on the same
    # codes, bit-identical on a rerun and within fp32 rounding of the uncut
    # sum (a workspace one byte short of the full size has no slots)
    a, dy, _ = data
    M, G = a.shape[0], len(LENS)
    lens_d = dev_i64(LENS, dev)
    cols = (lambda c: c) if fmt == ptm.PT_MXFP8_E4M3 else (lambda c: c // 2)
    aq = torch.empty((M, cols(K)), dtype=torch.uint8, device=dev)
    dq = torch.empty((M, cols(N)), dtype=torch.uint8, device=dev)
    as_ = torch.zeros((M // 32 + G, K), dtype=torch.uint8, device=dev)
    ds = torch.zeros((M // 32 + G, N), dtype=torch.uint8, device=dev)
    ptm.pt_mx_quantize_tokens(a, lens_d, None, aq, as_, G, M, K, fmt)
    ptm.pt_mx_quantize_tokens(dy, lens_d, None, dq, ds, G, M, N, fmt)
    ws, n = ws_full(dev, G, M, fmt, tail=4096)
    print(f"split mx wgrad fmt={fmt}", flush=True)
    before, after = run(dev, aq, dy=dq, lens=LENS, trans_out=0, accumulate=1, ws=ws, nbytes=n,
                        dtype=fmt, a_s=as_, d_s=ds)
    assert (u8(ws[n:]) == 0xA5).all()
    ofmt = orc.E4M3 if fmt == ptm.PT_MXFP8_E4M3 else orc.E2M1
    raq, ras, _ = orc.mx_quantize_tokens(bits16(a), LENS, ofmt)
    rdq, rds, _ = orc.mx_quantize_tokens(bits16(dy), LENS, ofmt)
    assert (u8(aq) == raq).all() and (u8(dq) == rdq).all()
    av = orc.mx_dequantize_tokens(raq, ras, LENS, ofmt)
    dv = orc.mx_dequantize_tokens(rdq, rds, LENS, ofmt)
    co = np.concatenate([[0], np.cumsum(LENS)])
    D = np.stack([av[co[g]:co[g + 1]].T @ dv[co[g]:co[g + 1]] for g in range(G)])
    check(before, after, D, LENS, 0, 1)
    _, again = run(dev, aq, dy=dq, lens=LENS, trans_out=0, accumulate=1, ws=ws, nbytes=n, dtype=fmt, a_s=as_,
                   d_s=ds)
    assert (again == after).all(), "split reduction not deterministic"
    _, whole = run(dev, aq, dy=dq, lens=LENS, trans_out=0, accumulate=1, ws=ws, nbytes=n - 1, dtype=fmt, a_s=as_,
                   d_s=ds)
    assert not (whole == after).all(), "the short workspace should run uncut"
    assert floored_rel_err(after, whole) <= 1e-4


def test_split_overlapping_ranges_stay_in_bounds(dev, data):
    # overlapping explicit ranges (flagged in the error word) cut more chunks
    # than the workspace has slots: the extra partial sums are dropped, never
    # written past the workspace
    a, dy, _ = data
    M = a.shape[0]
    lens = np.array([M, M], np.int64)
    offs = dev_i64([0, 0, M], dev)
    ws, n = ws_full(dev, 2, M, tail=1 << 20)
    ws[:4] = 0
    run(dev, a, dy, lens, 0, 1, ws, n, offs=offs)
    assert (u8(ws[n:]) == 0xA5).all(), "write past the workspace"
    assert ptm.pt_read_error_flags(ws) & 4
