"""GPU parity of the MX path: the quantise kernel (bit-exact against the
oracle, including an exhaustive probe of every finite bf16 pattern under
every block exponent) and the MXFP8 / MXFP4 grouped GEMM with its epilogues
(tolerance against the oracle on the same MX bytes; bit-exact on inputs whose
products and sums are exact)."""
import numpy as np
import pytest
import torch

import moe_expert_grouped_gemm_amd as ptm
from moe_expert_grouped_gemm_amd import synth
from util import (BF16_TOL, MX_SCHEDS, MX_TOL, bits16, bf16_values, dev_i64, floored_rel_err, group_of_rows,
                  make_ws, norm_err, per_group_max, u8)

pytestmark = pytest.mark.gpu

FMTS = [(ptm.PT_MXFP8_E4M3, 1, "e4m3"), (ptm.PT_MXFP4_E2M1, 2, "e2m1")]


def quantize(dev, x, fmt):
    rows, cols = x.shape
    q = torch.empty((rows, cols if fmt == ptm.PT_MXFP8_E4M3 else cols // 2), dtype=torch.uint8, device=dev)
    s = torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev)
    ptm.pt_mx_quantize(x, q, s, rows, cols, fmt, 1)
    torch.cuda.synchronize()
    return u8(q), u8(s)


# ------------------------------------------------------------------ quantise
@pytest.mark.parametrize("fmt,ofmt,name", FMTS, ids=[f[2] for f in FMTS])
def test_quantize_random_bit_exact(orc, dev, fmt, ofmt, name):
    parts = [
        synth.randn_bf16((96, 2880), seed=30, device=dev),
        synth.randn_bf16((64, 2880), seed=31, device=dev, outlier_frac=0.01, outlier_mult=50.0),
        synth.randn_bf16((32, 2880), seed=32, std=1e-38, device=dev),      # bf16 subnormals
        torch.zeros((8, 2880), dtype=torch.bfloat16, device=dev),
        -synth.randn_bf16((8, 2880), seed=33, std=3e37, device=dev),       # near the top
    ]
    x = torch.cat(parts)
    q, s = quantize(dev, x, fmt)
    rq, rs = orc.mx_quantize(bits16(x), ofmt, axis=1)
    assert (s == rs).all()
    assert (q == rq).all()


@pytest.mark.parametrize("fmt,ofmt,name", FMTS, ids=[f[2] for f in FMTS])
@pytest.mark.parametrize("rows,cols", [(32, 8), (96, 2880), (2048, 264)], ids=["one_block", "wide", "tall"])
def test_quantize_axis0_bit_exact(orc, dev, fmt, ofmt, name, rows, cols):
    # blocks of 32 consecutive rows of a column (pt_mx_quantize axis 0)
    x = synth.randn_bf16((rows, cols), seed=34, device=dev, outlier_frac=0.01, outlier_mult=50.0)
    if rows >= 96:
        x[32:64] = synth.randn_bf16((32, cols), seed=35, std=1e-38, device=dev)    # bf16 subnormal blocks
        x[64:96, : cols // 2] = 0                                                   # all-zero blocks
        x[64:96, cols // 2:] = -synth.randn_bf16((32, cols - cols // 2), seed=36, std=3e37, device=dev)
    q = torch.full((rows if fmt == ptm.PT_MXFP8_E4M3 else rows // 2, cols), 0xEE, dtype=torch.uint8, device=dev)
    s = torch.full((rows // 32, cols), 0xEE, dtype=torch.uint8, device=dev)
    ptm.pt_mx_quantize(x, q, s, rows, cols, fmt, 0)
    torch.cuda.synchronize()
    rq, rs = orc.mx_quantize(bits16(x), ofmt, axis=0)
    assert (u8(s) == rs).all()
    assert (u8(q) == rq).all()


def test_quantize_axis_refusals(dev):
    x = torch.zeros((64, 64), dtype=torch.bfloat16, device=dev)
    q = torch.zeros((64, 64), dtype=torch.uint8, device=dev)
    s = torch.zeros((64, 64), dtype=torch.uint8, device=dev)
    for rows, cols, axis, want in [(64, 64, 2, 1), (48, 64, 0, 2), (64, 60, 0, 2), (64, 48, 1, 2)]:
        with pytest.raises(ptm.PtggError) as e:
            ptm.pt_mx_quantize(x, q, s, rows, cols, ptm.PT_MXFP8_E4M3, axis)
        assert e.value.status == want, (rows, cols, axis)


@pytest.mark.parametrize("fmt,ofmt,name", FMTS, ids=[f[2] for f in FMTS])
def test_quantize_exhaustive_patterns(orc, dev, fmt, ofmt, name):
    # For every block exponent byte e (amax = m * 2^(e-127), two mantissas),
    # every finite bf16 pattern of magnitude <= amax appears as an element.
    blocks = []
    pats = np.arange(0x8000, dtype=np.uint32)              # non-negative patterns
    for e in range(1, 255):
        for top in (0x00, 0x7F):
            amax = (e << 7) | top
            probe = pats[pats <= amax]
            probe = np.concatenate([probe, probe | 0x8000]).astype(np.uint16)
            n = (len(probe) + 30) // 31
            pad = np.zeros(n * 31, np.uint16)
            pad[:len(probe)] = probe
            blk = np.empty((n, 32), np.uint16)
            blk[:, 0] = amax
            blk[:, 1:] = pad.reshape(n, 31)
            blocks.append(blk)
    # plus subnormal-only and zero blocks
    sub = np.arange(0x80, dtype=np.uint16)
    blk = np.zeros((8, 32), np.uint16)
    blk.reshape(-1)[:256] = np.concatenate([sub, sub | 0x8000])
    blocks.append(blk)
    allb = np.concatenate(blocks)
    nb = (allb.shape[0] + 7) // 8 * 8               # 8 blocks per row, zero-padded
    padded = np.zeros((nb, 32), np.uint16)
    padded[:allb.shape[0]] = allb
    mat = padded.reshape(-1, 32 * 8)
    x = torch.from_numpy(mat.view(np.int16)).to(dev).view(torch.bfloat16)
    print(f"exhaustive {name}: {mat.size} elements", flush=True)
    q, s = quantize(dev, x, fmt)
    rq, rs = orc.mx_quantize(mat, ofmt, axis=1)
    assert (s == rs).all()
    assert (q == rq).all()


def test_quantize_host_errors(dev):
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device=dev)
    q = torch.empty((4, 64), dtype=torch.uint8, device=dev)
    s = torch.empty((4, 2), dtype=torch.uint8, device=dev)
    L = ptm.load()
    st = torch.cuda.current_stream().cuda_stream
    assert L.pt_mx_quantize(x.data_ptr(), q.data_ptr(), s.data_ptr(), 4, 48, 1, 1, st) == 2
    assert L.pt_mx_quantize(x.data_ptr(), q.data_ptr(), s.data_ptr(), 4, 64, 0, 1, st) == 2
    assert L.pt_mx_quantize(x.data_ptr(), q.data_ptr(), s.data_ptr(), 4, 64, 1, 0, st) == 2
    assert L.pt_mx_quantize(None, q.data_ptr(), s.data_ptr(), 4, 64, 1, 1, st) == 1
    assert L.pt_mx_quantize(x.data_ptr(), q.data_ptr(), s.data_ptr(), 0, 64, 1, 1, st) == 0


# ------------------------------------------------------------------ MX GEMM
def mx_fwd(dev, aq, as_, bq, bs, lens, N, K, fmt, epi, ws=None, sched=None):
    M, G = aq.shape[0], len(lens)
    if sched is not None:
        ws = make_ws(dev, sched, G, M, N, K, fmt)
    lens_d = dev_i64(lens, dev)
    if epi == ptm.PT_EPI_SWIGLU_MXFP4:
        out = torch.full((M, N // 4), 0xEE, dtype=torch.uint8, device=dev)
        osc = torch.full((M, N // 64), 0xEE, dtype=torch.uint8, device=dev)
    else:
        out = torch.empty((M, N if epi == ptm.PT_EPI_NONE else N // 2), dtype=torch.bfloat16, device=dev)
        osc = None
    ptm.pt_grouped_gemm_fwd(aq, as_, bq, bs, out, osc, lens_d, None, G, M, N, K, fmt, 1, epi, workspace=ws)
    torch.cuda.synchronize()
    return out, osc


MX_CASES = [
    ("ragged", [0, 1, 130, 0, 257, 64, 33], 320, 256),
    ("ktail", [200, 0, 56], 2880 // 10, 192),           # K = 288: partial k-steps
    ("one", [129], 64, 128),
]


@pytest.mark.parametrize("fmt,ofmt,name", FMTS, ids=[f[2] for f in FMTS])
@pytest.mark.parametrize("case", MX_CASES, ids=[c[0] for c in MX_CASES])
@pytest.mark.parametrize("sched", MX_SCHEDS)
def test_mx_fwd_random_codes_vs_oracle(orc, dev, fmt, ofmt, name, case, sched):
    _, lens, K, N = case
    lens = np.array(lens, np.int64)
    M, G = int(lens.sum()), len(lens)
    print(f"mx fwd {name} case={case[0]} sched={sched} M={M} K={K} N={N}", flush=True)
    aq, as_ = synth.random_mx_codes(M, K, name, seed=40, device=dev)
    bq, bs = synth.random_mx_codes(G * N, K, name, seed=41, device=dev)
    out, _ = mx_fwd(dev, aq, as_, bq, bs, lens, N, K, fmt, ptm.PT_EPI_NONE, sched=sched)
    rows = np.arange(M)
    ref = orc.fwd_rows(ofmt, u8(aq), u8(as_), u8(bq).reshape(G, N, -1), u8(bs).reshape(G, N, -1),
                       lens, N, K, 1, rows)
    got = bf16_values(bits16(out))
    err = per_group_max(norm_err, got, ref, group_of_rows(lens, rows))
    assert err <= MX_TOL, err
    # and elementwise with the BF16 floor (the products are exact, only the
    # fp32 sum order and the final bf16 rounding differ)
    assert per_group_max(floored_rel_err, got, ref, group_of_rows(lens, rows)) <= BF16_TOL


def grid_codes(rows, cols, name, seed, dev):
    """MX operand whose values are in {0, +-1, +-1.5, +-2} x 2^(E-127) with
    E in {126, 127, 128}: every product and every partial sum of a short
    reduction is exact in fp32."""
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    if name == "e4m3":
        table = torch.tensor([0x00, 0x38, 0x3C, 0x40, 0xB8, 0xBC, 0xC0], dtype=torch.uint8, device=dev)
        q = table[torch.randint(0, 7, (rows, cols), generator=g, device=dev)]
    else:
        table = torch.tensor([0x0, 0x2, 0x3, 0x4, 0xA, 0xB, 0xC], dtype=torch.uint8, device=dev)
        idx = torch.randint(0, 7, (rows, cols), generator=g, device=dev)
        nib = table[idx]
        q = (nib[:, 0::2] | (nib[:, 1::2] << 4)).contiguous()
    s = torch.randint(126, 129, (rows, cols // 32), generator=g, device=dev, dtype=torch.int32).to(torch.uint8)
    return q, s


@pytest.mark.parametrize("fmt,ofmt,name", FMTS, ids=[f[2] for f in FMTS])
@pytest.mark.parametrize("sched", ["static", "swz"])
def test_mx_fwd_exact_inputs_bit_exact_and_scale_doubling(orc, dev, fmt, ofmt, name, sched):
    lens = np.array([33, 0, 128, 1, 70], np.int64)
    K, N = 256, 256
    M, G = int(lens.sum()), len(lens)
    aq, as_ = grid_codes(M, K, name, 50, dev)
    bq, bs = grid_codes(G * N, K, name, 51, dev)
    out, _ = mx_fwd(dev, aq, as_, bq, bs, lens, N, K, fmt, ptm.PT_EPI_NONE, sched=sched)
    ref = orc.fwd_rows(ofmt, u8(aq), u8(as_), u8(bq).reshape(G, N, -1), u8(bs).reshape(G, N, -1),
                       lens, N, K, 1, np.arange(M))
    assert (bits16(out) == orc.round_bf16(ref)).all()
    # raising every A scale byte by one doubles every output exactly
    out2, _ = mx_fwd(dev, aq, as_ + 1, bq, bs, lens, N, K, fmt, ptm.PT_EPI_NONE, sched=sched)
    assert (bf16_values(bits16(out2)) == 2.0 * bf16_values(bits16(out))).all()
    # raising only block 3 of B changes exactly the products of that block
    bs3 = bs.clone()
    bs3[:, 3] += 1
    out3, _ = mx_fwd(dev, aq, as_, bq, bs3, lens, N, K, fmt, ptm.PT_EPI_NONE, sched=sched)
    ref3 = orc.fwd_rows(ofmt, u8(aq), u8(as_), u8(bq).reshape(G, N, -1), u8(bs3).reshape(G, N, -1),
                        lens, N, K, 1, np.arange(M))
    assert (bits16(out3) == orc.round_bf16(ref3)).all()


@pytest.mark.parametrize("fmt,ofmt,name", FMTS, ids=[f[2] for f in FMTS])
@pytest.mark.parametrize("sched", ["static", "swz"])
def test_mx_fwd_swiglu_vs_oracle(orc, dev, fmt, ofmt, name, sched):
    lens = np.array([5, 0, 140, 31, 0, 64], np.int64)
    K, N = 256, 384
    M, G = int(lens.sum()), len(lens)
    aq, as_ = synth.random_mx_codes(M, K, name, seed=60, device=dev)
    bq, bs = synth.random_mx_codes(G * N, K, name, seed=61, device=dev)
    out, _ = mx_fwd(dev, aq, as_, bq, bs, lens, N, K, fmt, ptm.PT_EPI_SWIGLU, sched=sched)
    rows = np.arange(M)
    ref = orc.grouped_fwd(ofmt, u8(aq), u8(as_), u8(bq).reshape(G, N, -1), u8(bs).reshape(G, N, -1),
                          lens, N, K, 1, orc.EPI_SWIGLU, rows)["exact"]
    got = bf16_values(bits16(out))
    assert per_group_max(norm_err, got, ref, group_of_rows(lens, rows)) <= MX_TOL


@pytest.mark.parametrize("fmt,ofmt,name", FMTS + [(ptm.PT_BF16, 0, "bf16")], ids=[f[2] for f in FMTS] + ["bf16"])
@pytest.mark.parametrize("sched", ["static", "swz"])
def test_swiglu_mxfp4_epilogue_vs_oracle(orc, dev, fmt, ofmt, name, sched):
    lens = np.array([0, 77, 3, 200, 0, 40], np.int64)
    K, N = 256, 512
    M, G = int(lens.sum()), len(lens)
    if fmt == ptm.PT_BF16:
        a = synth.randn_bf16((M, K), seed=70, std=K ** -0.5, device=dev)
        b = synth.randn_bf16((G, N, K), seed=71, std=K ** -0.5, device=dev)
        aq, as_, bq, bs = a, None, b, None
        ref = orc.grouped_fwd(orc.BF16, bits16(a), None, bits16(b), None, lens, N, K, 1,
                              orc.EPI_SWIGLU_MXFP4, np.arange(M))
    else:
        aq, as_ = synth.random_mx_codes(M, K, name, seed=72, device=dev)
        bq, bs = synth.random_mx_codes(G * N, K, name, seed=73, device=dev)
        ref = orc.grouped_fwd(ofmt, u8(aq), u8(as_), u8(bq).reshape(G, N, -1), u8(bs).reshape(G, N, -1),
                              lens, N, K, 1, orc.EPI_SWIGLU_MXFP4, np.arange(M))
    out, osc = mx_fwd(dev, aq, as_, bq, bs, lens, N, K, fmt, ptm.PT_EPI_SWIGLU_MXFP4, sched=sched)
    q, s = u8(out), u8(osc)
    I = N // 2
    got = orc.mx_dequantize(orc.E2M1, q, s, M, I)
    want = orc.mx_dequantize(orc.E2M1, ref["q"], ref["s"], M, I)
    rows = np.arange(M)
    # end to end against the oracle's chain (its bf16 SwiGLU value may differ
    # from the GPU's in the last bit, which can move a code) ...
    assert per_group_max(norm_err, got, want, group_of_rows(lens, rows)) <= MX_TOL
    # ... and exactly: the codes and scale bytes are the oracle's quantisation
    # of the bf16 SwiGLU values the GPU computes for the same inputs
    h, _ = mx_fwd(dev, aq, as_, bq, bs, lens, N, K, fmt, ptm.PT_EPI_SWIGLU, sched=sched)
    rq, rs = orc.mx_quantize(bits16(h), orc.E2M1)
    assert (s == rs).all()
    assert (q == rq).all()
