"""GPU parity of FP8 E4M3 with one scale per tensor (current scaling):
pt_fp8_quantize bit-exact against the oracle (codes, amax and the
dequantisation factor), and the grouped GEMM on its codes (dtype
PT_FP8_E4M3) against the oracle on the same bytes, with every epilogue,
through the C ABI."""
import numpy as np
import pytest
import torch

import moe_expert_grouped_gemm_amd as ptm
from moe_expert_grouped_gemm_amd import synth
from util import (BF16_TOL, MX_TOL, bits16, bf16_values, dev_i64, floored_rel_err, group_of_rows, make_ws,
                  norm_err, per_group_max, u8)

pytestmark = pytest.mark.gpu


def fp8_quantize(dev, x):
    batch = x.shape[0]
    n = x.numel() // batch
    cols = x.shape[-1]
    q = torch.full(x.shape, 0xEE, dtype=torch.uint8, device=dev)
    amax = torch.full((batch,), -1.0, dtype=torch.float32, device=dev)
    deq = torch.full((batch,), -1.0, dtype=torch.float32, device=dev)
    ptm.pt_fp8_quantize(x, q, amax, deq, batch, n // cols, cols)
    torch.cuda.synchronize()
    return q, amax, deq


@pytest.mark.parametrize("shape,std", [((1, 65536, 64), 1.0), ((5, 96, 200), 0.03), ((3, 1, 8), 7.0),
                                       ((2, 257, 136), 1e-30), ((2, 64, 64), 1e-37)],
                         ids=["one_big", "five", "tiny", "small_values", "scale_overflow"])
def test_fp8_quantize_bit_exact(orc, dev, shape, std):
    x = synth.randn_bf16(shape, seed=80, std=std, device=dev, outlier_frac=0.01, outlier_mult=50.0)
    q, amax, deq = fp8_quantize(dev, x)
    rq, ra, rd = orc.fp8_quantize(bits16(x).reshape(shape[0], -1))
    assert (amax.cpu().numpy() == ra).all()
    assert (deq.cpu().numpy() == rd).all()
    assert (u8(q).reshape(shape[0], -1) == rq).all()


# The tensor amax pass: threads take 16-byte chunks a grid apart, four at a
# time then one at a time, and a workgroup's four waves meet in LDS before one
# atomic.  A single spike in batch 1 at positions that land in each of those
# places (another wave of workgroup 0, the fourth load of a group, the
# one-at-a-time tail, the last element) must come out as that batch's amax;
# the other batches keep their own.
S = 2048 * 256                       # chunks per grid pass (8 workgroups per CU, 256 CUs)


@pytest.mark.parametrize("pos", [0, 512 + 3, 3 * 512 + 5, (3 * S + 100) * 8 + 1, (4 * S + 700) * 8 + 7, -1],
                         ids=["first", "wave1", "wave3", "fourth_load", "tail", "last"])
@pytest.mark.parametrize("sign", [1.0, -1.0], ids=["pos", "neg"])
def test_fp8_amax_spike_positions(dev, pos, sign):
    print(f"fp8 amax spike pos={pos} sign={sign}", flush=True)
    x = synth.randn_bf16((3, 8192, 2880), seed=92, device=dev)
    flat = x[1].reshape(-1)
    flat[pos] = sign * 768.0                           # exact in bf16, far above any N(0, 1) draw
    q, amax, deq = fp8_quantize(dev, x)
    assert amax[1].item() == 768.0
    for b in (0, 2):
        assert amax[b].item() == x[b].abs().max().float().item()


def test_fp8_quantize_zero_matrix_and_repeat(orc, dev):
    x = torch.zeros((2, 64, 64), dtype=torch.bfloat16, device=dev)
    x[1] = synth.randn_bf16((64, 64), seed=81, device=dev)
    q, amax, deq = fp8_quantize(dev, x)
    assert amax[0].item() == 0.0 and deq[0].item() == 1.0 and (u8(q[0]) == 0).all()
    # a second call into the same buffers gives the same bytes (amax restarts from zero)
    q2, amax2, deq2 = fp8_quantize(dev, x)
    assert torch.equal(q, q2) and torch.equal(amax, amax2) and torch.equal(deq, deq2)


def fp8_fwd(dev, aq, ad, bq, bd, lens, N, K, epi, ws=None):
    M, G = aq.shape[0], len(lens)
    if epi == ptm.PT_EPI_SWIGLU_MXFP4:
        out = torch.full((M, N // 4), 0xEE, dtype=torch.uint8, device=dev)
        osc = torch.full((M, N // 64), 0xEE, dtype=torch.uint8, device=dev)
    else:
        out = torch.empty((M, N if epi == ptm.PT_EPI_NONE else N // 2), dtype=torch.bfloat16, device=dev)
        osc = None
    ptm.pt_grouped_gemm_fwd(aq, ad, bq, bd, out, osc, dev_i64(lens, dev), None, G, M, N, K, ptm.PT_FP8_E4M3, 1,
                            epi, workspace=ws)
    torch.cuda.synchronize()
    return out, osc


def random_codes(rows, cols, seed, dev):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    q = torch.randint(0, 256, (rows, cols), generator=g, device=dev, dtype=torch.int32)
    return torch.where((q & 0x7F) == 0x7F, q - 1, q).to(torch.uint8)      # no NaN codes


CASES = [
    ("ragged", [0, 1, 130, 0, 257, 64, 33], 320, 256),
    ("ktail", [200, 0, 56], 288, 192),
    ("one", [129], 64, 128),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("sched", ["static", "queue"])
def test_fp8_fwd_random_codes_vs_oracle(orc, dev, case, sched):
    _, lens, K, N = case
    lens = np.array(lens, np.int64)
    M, G = int(lens.sum()), len(lens)
    print(f"fp8 fwd case={case[0]} sched={sched} M={M} K={K} N={N}", flush=True)
    aq = random_codes(M, K, 82, dev)
    bq = random_codes(G * N, K, 83, dev)
    ad = torch.tensor([2.0 ** -7], dtype=torch.float32, device=dev)
    bd = torch.tensor(np.linspace(0.001, 0.004, G), dtype=torch.float32, device=dev)
    out, _ = fp8_fwd(dev, aq, ad, bq, bd, lens, N, K, ptm.PT_EPI_NONE, ws=make_ws(dev, sched))
    rows = np.arange(M)
    ref = orc.fp8_fwd_rows(u8(aq), ad.cpu().numpy()[0], u8(bq).reshape(G, N, -1), bd.cpu().numpy(), lens, N, K, rows)
    got = bf16_values(bits16(out))
    grp = group_of_rows(lens, rows)
    assert per_group_max(norm_err, got, ref, grp) <= MX_TOL
    assert per_group_max(floored_rel_err, got, ref, grp) <= BF16_TOL


def test_fp8_fwd_from_bf16_with_epilogues(orc, dev):
    # bf16 activations and weights -> pt_fp8_quantize (one factor for A, one
    # per expert for B) -> the grouped GEMM with SwiGLU and SwiGLU -> MXFP4.
    lens = np.array([70, 0, 300, 45], np.int64)
    K, N = 256, 384
    M, G = int(lens.sum()), len(lens)
    a = synth.randn_bf16((1, M, K), seed=84, device=dev)
    w = synth.randn_bf16((G, N, K), seed=85, std=K ** -0.5, device=dev)
    aq, aa, ad = fp8_quantize(dev, a)
    bq, ba, bd = fp8_quantize(dev, w)
    rq, _, rad = orc.fp8_quantize(bits16(a).reshape(1, -1))
    rbq, _, rbd = orc.fp8_quantize(bits16(w).reshape(G, -1))
    assert (u8(aq).reshape(1, -1) == rq).all() and (u8(bq).reshape(G, -1) == rbq).all()
    rows = np.arange(M)
    c = orc.fp8_fwd_rows(rq.reshape(M, K), rad[0], rbq.reshape(G, N, K), rbd, lens, N, K, rows)
    grp = group_of_rows(lens, rows)
    out, _ = fp8_fwd(dev, aq.reshape(M, K), ad, bq.reshape(G * N, K), bd, lens, N, K, ptm.PT_EPI_NONE)
    assert per_group_max(floored_rel_err, bf16_values(bits16(out)), c, grp) <= BF16_TOL
    out, _ = fp8_fwd(dev, aq.reshape(M, K), ad, bq.reshape(G * N, K), bd, lens, N, K, ptm.PT_EPI_SWIGLU)
    h = orc.swiglu(c)
    assert per_group_max(floored_rel_err, bf16_values(bits16(out)), h, grp) <= BF16_TOL
    q4, s4 = fp8_fwd(dev, aq.reshape(M, K), ad, bq.reshape(G * N, K), bd, lens, N, K, ptm.PT_EPI_SWIGLU_MXFP4)
    # exactly the oracle's MXFP4 quantisation of the SwiGLU values just written
    rq4, rs4 = orc.mx_quantize(bits16(out), orc.E2M1)
    assert (u8(s4) == rs4).all() and (u8(q4) == rq4).all()


def test_fp8_refusals(dev):
    L = ptm.load()
    st = torch.cuda.current_stream().cuda_stream
    lens = dev_i64(np.array([8], np.int64), dev)
    a = torch.zeros((8, 64), dtype=torch.uint8, device=dev)
    b = torch.zeros((64, 64), dtype=torch.uint8, device=dev)
    f = torch.ones((1,), dtype=torch.float32, device=dev)
    out = torch.zeros((8, 64), dtype=torch.bfloat16, device=dev)
    g = lambda tb, K, sa=f.data_ptr(): L.pt_grouped_gemm_fwd(a.data_ptr(), sa, b.data_ptr(), f.data_ptr(),
                                                            out.data_ptr(), None, lens.data_ptr(), None, 1, 8, 64,
                                                            K, ptm.PT_FP8_E4M3, tb, 0, 0.0, None, 0, st)
    assert g(0, 64) == 2            # codes must be K-contiguous ([G, N, K])
    assert g(1, 48) == 2            # K % 32
    assert g(1, 64, None) == 1      # factors required
    x = torch.zeros((2, 8, 60), dtype=torch.bfloat16, device=dev)
    assert L.pt_fp8_quantize(x.data_ptr(), a.data_ptr(), f.data_ptr(), f.data_ptr(), 2, 8, 60, st) == 2


def test_fp8_fwd_mxfp8_shape_sampled(orc, dev):
    # The MXFP8 workload's shapes in FP8 with current scaling: 32 experts
    # (Zipf 1.1), 65536 rows, K = 2880, N = 5760; sampled rows of every expert.
    lens = synth.lens_zipf_distinct(16384, 32, 4, 1.1, seed=3)
    G, M, K, N = 32, int(lens.sum()), 2880, 5760
    offs = synth.offsets(lens)
    a = synth.randn_bf16((1, M, K), seed=104, device=dev, outlier_frac=0.01, outlier_mult=50.0)
    w = synth.randn_bf16((G, N, K), seed=1104, device=dev, outlier_frac=0.01, outlier_mult=50.0)
    aq, _, ad = fp8_quantize(dev, a)
    bq, _, bd = fp8_quantize(dev, w)
    del a, w
    out, _ = fp8_fwd(dev, aq.reshape(M, K), ad, bq.reshape(G * N, K), bd, lens, N, K, ptm.PT_EPI_NONE,
                     ws=make_ws(dev, "queue"))
    rng = np.random.default_rng(9)
    experts = [g for g in range(G) if lens[g] > 0]
    rows = [np.unique(np.concatenate([[offs[g], offs[g + 1] - 1], rng.integers(offs[g], offs[g + 1], size=2)]))
            for g in experts]
    local = np.array([r.size for r in rows], np.int64)
    allr = torch.as_tensor(np.concatenate(rows), device=dev)
    ref = orc.fp8_fwd_rows(u8(aq.reshape(M, K)[allr]), ad.cpu().numpy()[0], u8(bq)[experts],
                           bd.cpu().numpy()[experts], local, N, K, np.arange(local.sum()))
    got = bf16_values(bits16(out[allr]))
    start = 0
    for g, r in zip(experts, rows):
        sl = slice(start, start + r.size)
        assert floored_rel_err(got[sl], ref[sl]) <= BF16_TOL, g
        start += r.size


# ------------------------------------------------------------------ rowwise
def fp8_quantize_rows(dev, x2d):
    rows, cols = x2d.shape
    q = torch.full((rows, cols), 0xEE, dtype=torch.uint8, device=dev)
    amax = torch.full((rows,), -1.0, dtype=torch.float32, device=dev)
    deq = torch.full((rows,), -1.0, dtype=torch.float32, device=dev)
    ptm.pt_fp8_quantize_rows(x2d, q, amax, deq, rows, cols)
    torch.cuda.synchronize()
    return q, amax, deq


# widths for each register-held row length (up to 2048, 4096, 6144 and 8192
# values) and past them (the two-pass kernel), each with a partial last chunk
@pytest.mark.parametrize("rows,cols", [(1000, 2880), (7, 8), (3, 600), (9, 2048), (5, 5760), (6, 8192), (5, 8200),
                                       (3, 12296)],
                         ids=["rows1000", "tiny", "odd512", "w2048", "w5760", "w8192", "w8200", "w12296"])
def test_fp8_quantize_rows_bit_exact(orc, dev, rows, cols):
    x = synth.randn_bf16((rows, cols), seed=90, device=dev, outlier_frac=0.01, outlier_mult=50.0)
    x[0] = 0                                                   # an all-zero row
    if rows > 2:
        x[2] *= 1e-36                                           # a row whose scale overflows fp32
    q, amax, deq = fp8_quantize_rows(dev, x)
    rq, ra, rd = orc.fp8_quantize(bits16(x))
    assert (amax.cpu().numpy() == ra).all()
    assert (deq.cpu().numpy() == rd).all()
    assert (u8(q) == rq).all()


@pytest.mark.parametrize("epi", [ptm.PT_EPI_NONE, ptm.PT_EPI_SWIGLU])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fp8_rowwise_fwd_vs_oracle(orc, dev, case, epi):
    _, lens, K, N = case
    lens = np.array(lens, np.int64)
    M, G = int(lens.sum()), len(lens)
    a = synth.randn_bf16((M, K), seed=91, device=dev)
    w = synth.randn_bf16((G * N, K), seed=92, std=K ** -0.5, device=dev)
    aq, _, ad = fp8_quantize_rows(dev, a)
    bq, _, bd = fp8_quantize_rows(dev, w)
    M_out = N if epi == ptm.PT_EPI_NONE else N // 2
    out = torch.empty((M, M_out), dtype=torch.bfloat16, device=dev)
    ptm.pt_grouped_gemm_fwd(aq, ad, bq, bd, out, None, dev_i64(lens, dev), None, G, M, N, K,
                            ptm.PT_FP8_E4M3_ROWWISE, 1, epi)
    torch.cuda.synchronize()
    rows = np.arange(M)
    c = orc.fp8_fwd_rows_rowwise(u8(aq), ad.cpu().numpy(), u8(bq).reshape(G, N, K), bd.cpu().numpy().reshape(G, N),
                                 lens, N, K, rows)
    ref = c if epi == ptm.PT_EPI_NONE else orc.swiglu(c)
    grp = group_of_rows(lens, rows)
    assert per_group_max(floored_rel_err, bf16_values(bits16(out)), ref, grp) <= BF16_TOL
