"""GPU parity of the MX data gradient and its transposed weight cache:
pt_mx_quantize_t bit-exact against the oracle's quantiser applied to each
matrix's transpose, and pt_grouped_gemm_dgrad in MXFP8 / MXFP4 against the
oracle on the same MX bytes (tolerance on random codes, bit-exact on codes
whose products and sums are exact), through the C ABI."""
import numpy as np
import pytest
import torch

import moe_expert_grouped_gemm_amd as ptm
from moe_expert_grouped_gemm_amd import synth
from util import BF16_TOL, MX_TOL, bits16, bf16_values, dev_i64, floored_rel_err, group_of_rows, norm_err, \
    per_group_max, u8

pytestmark = pytest.mark.gpu

FMTS = [(ptm.PT_MXFP8_E4M3, 1, "e4m3"), (ptm.PT_MXFP4_E2M1, 2, "e2m1")]


def quantize_t(dev, x, fmt):
    batch, rows, cols = x.shape
    q = torch.full((batch, cols, rows if fmt == ptm.PT_MXFP8_E4M3 else rows // 2), 0xEE, dtype=torch.uint8,
                   device=dev)
    s = torch.full((batch, cols, rows // 32), 0xEE, dtype=torch.uint8, device=dev)
    ptm.pt_mx_quantize_t(x, q, s, batch, rows, cols, fmt)
    torch.cuda.synchronize()
    return q, s


@pytest.mark.parametrize("fmt,ofmt,name", FMTS, ids=[f[2] for f in FMTS])
@pytest.mark.parametrize("shape", [(3, 96, 72), (2, 160, 200), (1, 64, 64), (1, 32, 8)],
                         ids=lambda s: "x".join(map(str, s)))
def test_quantize_t_bit_exact(orc, dev, fmt, ofmt, name, shape):
    batch, rows, cols = shape
    x = synth.randn_bf16((batch, rows, cols), seed=60, device=dev, outlier_frac=0.01, outlier_mult=50.0)
    x[0, :32, :1] = 0                                   # an all-zero block
    if rows >= 64:
        x[-1, 32:64, -1] = synth.randn_bf16((32,), seed=61, std=1e-38, device=dev)   # subnormals
    q, s = quantize_t(dev, x, fmt)
    xb = bits16(x)
    for b in range(batch):
        rq, rs = orc.mx_quantize(np.ascontiguousarray(xb[b].T), ofmt, axis=1)
        assert (u8(s[b]) == rs).all(), b
        assert (u8(q[b]) == rq).all(), b


def mx_dgrad(dev, dq, ds, bq, bs, lens, N, K, fmt, ws_kind="static"):
    M, G = dq.shape[0], len(lens)
    ws = None
    if ws_kind == "queue":
        ws = torch.full((ptm.pt_grouped_gemm_workspace_size(ptm.PT_OP_DGRAD, 1, 1, 1, 1, ptm.PT_BF16),), 0xFF,
                        dtype=torch.uint8, device=dev)
    elif ws_kind == "swz":
        n = ptm.pt_grouped_gemm_workspace_size(ptm.PT_OP_DGRAD, G, M, N, K, fmt)
        assert n > 1280
        ws = torch.full((n,), 0xFF, dtype=torch.uint8, device=dev)
    buf = torch.empty((M + 6, K), dtype=torch.bfloat16, device=dev)
    buf.view(torch.int16).fill_(0x7FC1)
    dx = buf[3:3 + M]
    ptm.pt_grouped_gemm_dgrad(dq, ds, bq, bs, dx, dev_i64(lens, dev), None, G, M, N, K, fmt, 0, workspace=ws)
    torch.cuda.synchronize()
    assert (bits16(buf[:3]) == 0x7FC1).all() and (bits16(buf[3 + M:]) == 0x7FC1).all(), "guard rows written"
    return dx


CASES = [
    # (name, lens, N = reduction, K = outputs)
    ("ragged", [0, 1, 130, 0, 257, 64, 33], 320, 264),
    ("ntail", [200, 0, 56], 288, 192),            # N = 288: partial stages
    ("one", [129], 64, 136),
]


@pytest.mark.parametrize("fmt,ofmt,name", FMTS, ids=[f[2] for f in FMTS])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("ws_kind", ["static", "queue", "swz"])
def test_mx_dgrad_random_codes_vs_oracle(orc, dev, fmt, ofmt, name, case, ws_kind):
    _, lens, N, K = case
    lens = np.array(lens, np.int64)
    M, G = int(lens.sum()), len(lens)
    print(f"mx dgrad {name} case={case[0]} ws={ws_kind} M={M} N={N} K={K}", flush=True)
    dq, ds = synth.random_mx_codes(M, N, name, seed=62, device=dev)
    bq, bs = synth.random_mx_codes(G * K, N, name, seed=63, device=dev)     # [G, K, N] along N
    dx = mx_dgrad(dev, dq, ds, bq, bs, lens, N, K, fmt, ws_kind)
    rows = np.arange(M)
    ref = orc.fwd_rows(ofmt, u8(dq), u8(ds), u8(bq).reshape(G, K, -1), u8(bs).reshape(G, K, -1),
                       lens, K, N, 1, rows)
    got = bf16_values(bits16(dx))
    grp = group_of_rows(lens, rows)
    assert per_group_max(norm_err, got, ref, grp) <= MX_TOL
    assert per_group_max(floored_rel_err, got, ref, grp) <= BF16_TOL


def grid_codes(rows, cols, name, seed, dev):
    """Values in {0, +-1, +-1.5, +-2} x 2^(E-127), E in {126, 127, 128}: every
    product and partial sum of a short reduction is exact in fp32."""
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    if name == "e4m3":
        table = torch.tensor([0x00, 0x38, 0x3C, 0x40, 0xB8, 0xBC, 0xC0], dtype=torch.uint8, device=dev)
        q = table[torch.randint(0, 7, (rows, cols), generator=g, device=dev)]
    else:
        table = torch.tensor([0x0, 0x2, 0x3, 0x4, 0xA, 0xB, 0xC], dtype=torch.uint8, device=dev)
        nib = table[torch.randint(0, 7, (rows, cols), generator=g, device=dev)]
        q = (nib[:, 0::2] | (nib[:, 1::2] << 4)).contiguous()
    s = torch.randint(126, 129, (rows, cols // 32), generator=g, device=dev, dtype=torch.int32).to(torch.uint8)
    return q, s


@pytest.mark.parametrize("fmt,ofmt,name", FMTS, ids=[f[2] for f in FMTS])
def test_mx_dgrad_exact_codes_bit_exact(orc, dev, fmt, ofmt, name):
    lens = np.array([33, 0, 128, 1, 70], np.int64)
    N, K = 256, 200
    M, G = int(lens.sum()), len(lens)
    dq, ds = grid_codes(M, N, name, 64, dev)
    bq, bs = grid_codes(G * K, N, name, 65, dev)
    dx = mx_dgrad(dev, dq, ds, bq, bs, lens, N, K, fmt, "swz")
    ref = orc.fwd_rows(ofmt, u8(dq), u8(ds), u8(bq).reshape(G, K, -1), u8(bs).reshape(G, K, -1),
                       lens, K, N, 1, np.arange(M))
    assert (bits16(dx) == orc.round_bf16(ref)).all()


@pytest.mark.parametrize("fmt,ofmt,name", FMTS, ids=[f[2] for f in FMTS])
def test_mx_dgrad_from_bf16_weight_chain(orc, dev, fmt, ofmt, name):
    # bf16 dY and a forward weight [G, N, K] -> pt_mx_quantize (dY along N)
    # and pt_mx_quantize_t (the weight's transposed cache along N) -> the MX
    # data gradient.  The GPU's bytes are first checked bit-exact against the
    # oracle's quantiser; the oracle then runs on its own bytes.
    lens = np.array([70, 0, 300, 45], np.int64)
    N, K = 256, 160
    M, G = int(lens.sum()), len(lens)
    dy = synth.randn_bf16((M, N), seed=66, std=1e-2, device=dev)
    w = synth.randn_bf16((G, N, K), seed=67, std=N ** -0.5, device=dev)
    dq = torch.empty((M, N if fmt == ptm.PT_MXFP8_E4M3 else N // 2), dtype=torch.uint8, device=dev)
    ds = torch.empty((M, N // 32), dtype=torch.uint8, device=dev)
    ptm.pt_mx_quantize(dy, dq, ds, M, N, fmt, 1)
    wq, ws_ = quantize_t(dev, w, fmt)
    rdq, rds = orc.mx_quantize(bits16(dy), ofmt, axis=1)
    wb = bits16(w)
    rw = [orc.mx_quantize(np.ascontiguousarray(wb[g].T), ofmt, axis=1) for g in range(G)]
    rwq, rws = np.stack([r[0] for r in rw]), np.stack([r[1] for r in rw])
    assert (u8(dq) == rdq).all() and (u8(ds) == rds).all()
    assert (u8(wq) == rwq).all() and (u8(ws_) == rws).all()
    dx = mx_dgrad(dev, dq, ds, wq.reshape(G * K, -1), ws_.reshape(G * K, -1), lens, N, K, fmt, "swz")
    rows = np.arange(M)
    ref = orc.fwd_rows(ofmt, rdq, rds, rwq, rws, lens, K, N, 1, rows)
    got = bf16_values(bits16(dx))
    grp = group_of_rows(lens, rows)
    assert per_group_max(norm_err, got, ref, grp) <= MX_TOL
    assert per_group_max(floored_rel_err, got, ref, grp) <= BF16_TOL


def test_mx_dgrad_and_quantize_t_refusals(dev):
    L = ptm.load()
    st = torch.cuda.current_stream().cuda_stream
    lens = dev_i64(np.array([8], np.int64), dev)
    t = torch.zeros((8, 64), dtype=torch.uint8, device=dev)
    sc = torch.zeros((8, 2), dtype=torch.uint8, device=dev)
    w = torch.zeros((64, 64), dtype=torch.uint8, device=dev)
    ws = torch.zeros((64, 2), dtype=torch.uint8, device=dev)
    dx = torch.zeros((8, 64), dtype=torch.bfloat16, device=dev)
    f = lambda N, K, tb, s1=sc.data_ptr(): L.pt_grouped_gemm_dgrad(
        t.data_ptr(), s1, w.data_ptr(), ws.data_ptr(), dx.data_ptr(), lens.data_ptr(), None, 1, 8, N, K,
        ptm.PT_MXFP8_E4M3, tb, None, 0, st)
    assert f(64, 64, 1) == 2          # MX takes the transposed cache: trans_b = 0 only
    assert f(48, 64, 0) == 2          # the reduction N must be a multiple of 32
    assert f(64, 64, 0, None) == 1    # scales are required
    x = torch.zeros((2, 64, 64), dtype=torch.bfloat16, device=dev)
    q = torch.zeros((2, 64, 64), dtype=torch.uint8, device=dev)
    s = torch.zeros((2, 64, 2), dtype=torch.uint8, device=dev)
    g = lambda b, r, c, d=ptm.PT_MXFP8_E4M3: L.pt_mx_quantize_t(x.data_ptr(), q.data_ptr(), s.data_ptr(), b, r, c,
                                                                   d, st)
    assert g(2, 48, 64) == 2          # rows % 32
    assert g(2, 64, 60) == 2          # cols % 8
    assert g(2, 64, 64, ptm.PT_BF16) == 2
    assert g(-1, 64, 64) == 1
    assert g(0, 64, 64) == 0


def test_mx_dgrad_mxfp8_full_shape_sampled(orc, dev):
    # The MXFP8 workload's data gradient: 32 experts (Zipf 1.1 routing),
    # 65536 rows, reduction N = 5760, K = 2880 outputs; sampled rows of every
    # expert against the oracle on a compact sub-batch.
    lens = synth.lens_zipf_distinct(16384, 32, 4, 1.1, seed=3)
    G, M, N, K = 32, int(lens.sum()), 5760, 2880
    offs = synth.offsets(lens)
    dq, ds = synth.random_mx_codes(M, N, "e4m3", seed=70, device=dev)
    bq, bs = synth.random_mx_codes(G * K, N, "e4m3", seed=71, device=dev)
    dx = mx_dgrad(dev, dq, ds, bq, bs, lens, N, K, ptm.PT_MXFP8_E4M3, "swz")
    rng = np.random.default_rng(7)
    experts = [g for g in range(G) if lens[g] > 0]
    rows = [np.unique(np.concatenate([[offs[g], offs[g + 1] - 1], rng.integers(offs[g], offs[g + 1], size=2)]))
            for g in experts]
    local = np.array([r.size for r in rows], np.int64)
    allr = torch.as_tensor(np.concatenate(rows), device=dev)
    ref = orc.fwd_rows(1, u8(dq[allr]), u8(ds[allr]), u8(bq).reshape(G, K, -1)[experts],
                       u8(bs).reshape(G, K, -1)[experts], local, K, N, 1, np.arange(local.sum()))
    got = bf16_values(bits16(dx[allr]))
    start = 0
    for g, r in zip(experts, rows):
        sl = slice(start, start + r.size)
        assert norm_err(got[sl], ref[sl]) <= MX_TOL, g
        start += r.size
