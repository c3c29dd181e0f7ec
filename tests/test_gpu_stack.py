"""GPU parity of the expert weight stack (pt_stack_experts) and of the
one-pass MX weight caches (pt_mx_quantize_experts) against the oracle,
through the C ABI: separately allocated experts of ragged sizes, both
layouts, both MX formats, bad expert addresses, argument errors, and the
expert-MLP shape (256 experts of [4096, 4096])."""
import numpy as np
import pytest
import torch

import moe_expert_grouped_gemm_amd as ptm
from moe_expert_grouped_gemm_amd import synth
from util import bits16, u8

pytestmark = pytest.mark.gpu

GUARD_BYTES = 16    # keeps the outputs 16-byte aligned
SENTINEL = 0x7FC1


def experts(dev, G, R, C, seed, **kw):
    return [synth.randn_bf16((R, C), seed=seed + g, device=dev, **kw) for g in range(G)]


def guard_of(dtype):
    return GUARD_BYTES // torch.empty((), dtype=dtype).element_size()


def guarded(dev, shape, dtype=torch.bfloat16):
    n, GUARD = int(np.prod(shape)), guard_of(dtype)
    buf = torch.empty((n + 2 * GUARD,), dtype=dtype, device=dev)
    if dtype == torch.bfloat16:
        buf.view(torch.int16).fill_(SENTINEL)
    else:
        buf.fill_(0xEE)
    return buf, buf[GUARD:GUARD + n].view(shape)


def guards_intact(buf, n, dtype=torch.bfloat16):
    GUARD = guard_of(dtype)
    want = SENTINEL if dtype == torch.bfloat16 else 0xEE
    raw = bits16(buf) if dtype == torch.bfloat16 else u8(buf)
    return (raw[:GUARD] == want).all() and (raw[GUARD + n:] == want).all()


@pytest.mark.parametrize("R,C", [(200, 136), (64, 64), (8, 8), (136, 520)])
@pytest.mark.parametrize("transpose", [0, 1])
def test_stack_bit_exact(orc, dev, R, C, transpose):
    G = 5
    print(f"stack R={R} C={C} transpose={transpose}", flush=True)
    ws = experts(dev, G, R, C, seed=200)
    addr = ptm.expert_addresses(ws)
    buf, out = guarded(dev, (G, C, R) if transpose else (G, R, C))
    ptm.pt_stack_experts(addr, out, G, R, C, transpose)
    torch.cuda.synchronize()
    assert guards_intact(buf, G * R * C), "wrote outside the output"
    assert (bits16(out) == orc.stack_experts([bits16(w) for w in ws], bool(transpose))).all()


def test_stack_bad_addresses_read_as_zero(orc, dev):
    G, R, C = 4, 72, 40
    ws = experts(dev, G, R, C, seed=210)
    raw = [w.data_ptr() for w in ws]
    raw[1] = 0                       # NULL
    raw[3] = ws[3].data_ptr() + 2    # not 16-byte aligned (still inside the tensor)
    addr = torch.tensor(raw, dtype=torch.int64, device=dev)
    for transpose in (0, 1):
        ws_err = torch.zeros((64,), dtype=torch.uint8, device=dev)
        out = torch.empty((G, C, R) if transpose else (G, R, C), dtype=torch.bfloat16, device=dev)
        ptm.pt_stack_experts(addr, out, G, R, C, transpose, workspace=ws_err)
        assert ptm.pt_read_error_flags(ws_err) & 8
        ref = orc.stack_experts([bits16(w) for w in ws], bool(transpose))
        got = bits16(out)
        for g in (0, 2):
            assert (got[g] == ref[g]).all()
        for g in (1, 3):
            assert (got[g] == 0).all()
    ok_err = torch.zeros((64,), dtype=torch.uint8, device=dev)
    ptm.pt_stack_experts(ptm.expert_addresses(ws), out, G, R, C, 1, workspace=ok_err)
    assert ptm.pt_read_error_flags(ok_err) == 0


@pytest.mark.parametrize("fmt", [ptm.PT_MXFP8_E4M3, ptm.PT_MXFP4_E2M1], ids=["e4m3", "e2m1"])
@pytest.mark.parametrize("R,C", [(96, 160), (64, 64), (224, 96)])
def test_mx_caches_bit_exact(orc, dev, fmt, R, C):
    G = 3
    print(f"mx caches fmt={fmt} R={R} C={C}", flush=True)
    ws = experts(dev, G, R, C, seed=220, outlier_frac=0.01, outlier_mult=50.0)
    addr = ptm.expert_addresses(ws)
    half = fmt == ptm.PT_MXFP4_E2M1
    qb, q = guarded(dev, (G, R, C // 2 if half else C), torch.uint8)
    sb, s = guarded(dev, (G, R, C // 32), torch.uint8)
    qtb, qt = guarded(dev, (G, C, R // 2 if half else R), torch.uint8)
    stb, st = guarded(dev, (G, C, R // 32), torch.uint8)
    ptm.pt_mx_quantize_experts(addr, q, s, qt, st, G, R, C, fmt)
    torch.cuda.synchronize()
    for b, t in ((qb, q), (sb, s), (qtb, qt), (stb, st)):
        assert guards_intact(b, t.numel(), torch.uint8)
    rq, rs, rqt, rst = orc.mx_quantize_experts([bits16(w) for w in ws], 1 if fmt == ptm.PT_MXFP8_E4M3 else 2)
    assert (u8(q) == rq).all() and (u8(s) == rs).all()
    assert (u8(qt) == rqt).all() and (u8(st) == rst).all()
    # and the same bytes as the library's contiguous quantisers on the stack
    stacked = torch.stack(ws)
    q2, s2 = torch.empty_like(q), torch.empty_like(s)
    ptm.pt_mx_quantize(stacked, q2, s2, G * R, C, fmt, 1)
    qt2, st2 = torch.empty_like(qt), torch.empty_like(st)
    ptm.pt_mx_quantize_t(stacked, qt2, st2, G, R, C, fmt)
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(s, s2) and torch.equal(qt, qt2) and torch.equal(st, st2)


def test_mx_caches_one_pair_only(orc, dev):
    # only the forward cache (R need not be a multiple of 32), then only the
    # transposed one (C need not be): the other pair is left alone
    G = 2
    for R, C, fwd in ((40, 64, True), (64, 40, False)):
        ws = experts(dev, G, R, C, seed=230)
        addr = ptm.expert_addresses(ws)
        rq = [orc.mx_quantize(bits16(w), 1, axis=1) if fwd else
              orc.mx_quantize(np.ascontiguousarray(bits16(w).T), 1, axis=1) for w in ws]
        shape_q = (G, R, C) if fwd else (G, C, R)
        shape_s = (G, R, C // 32) if fwd else (G, C, R // 32)
        q = torch.full(shape_q, 0xEE, dtype=torch.uint8, device=dev)
        s = torch.full(shape_s, 0xEE, dtype=torch.uint8, device=dev)
        if fwd:
            ptm.pt_mx_quantize_experts(addr, q, s, None, None, G, R, C, ptm.PT_MXFP8_E4M3)
        else:
            ptm.pt_mx_quantize_experts(addr, None, None, q, s, G, R, C, ptm.PT_MXFP8_E4M3)
        torch.cuda.synchronize()
        for g in range(G):
            assert (u8(q)[g] == rq[g][0]).all() and (u8(s)[g] == rq[g][1]).all()


def test_stack_argument_errors(dev):
    L = ptm.load()
    st = torch.cuda.current_stream().cuda_stream
    w = torch.zeros((64, 64), dtype=torch.bfloat16, device=dev)
    addr = ptm.expert_addresses([w])
    out = torch.zeros((1, 64, 64), dtype=torch.bfloat16, device=dev)
    q = torch.zeros((1, 64, 64), dtype=torch.uint8, device=dev)
    s = torch.zeros((1, 64, 2), dtype=torch.uint8, device=dev)
    a, o = addr.data_ptr(), out.data_ptr()
    assert L.pt_stack_experts(a, o, 1, 64, 64, 2, None, 0, st) == 1          # bad layout flag
    assert L.pt_stack_experts(a, o, 1, 60, 64, 0, None, 0, st) == 2          # rows % 8
    assert L.pt_stack_experts(None, o, 1, 64, 64, 0, None, 0, st) == 1
    assert L.pt_stack_experts(a, o + 8, 1, 64, 64, 0, None, 0, st) == 3      # misaligned output
    assert L.pt_stack_experts(a, o, 0, 64, 64, 0, None, 0, st) == 0          # nothing to do
    qp, sp = q.data_ptr(), s.data_ptr()
    assert L.pt_mx_quantize_experts(a, None, None, None, None, 1, 64, 64, 1, None, 0, st) == 1
    assert L.pt_mx_quantize_experts(a, qp, None, None, None, 1, 64, 64, 1, None, 0, st) == 1
    assert L.pt_mx_quantize_experts(a, qp, sp, None, None, 1, 64, 48, 1, None, 0, st) == 2   # cols % 32
    assert L.pt_mx_quantize_experts(a, None, None, qp, sp, 1, 48, 64, 1, None, 0, st) == 2   # rows % 32
    assert L.pt_mx_quantize_experts(a, qp, sp, None, None, 1, 64, 64, 0, None, 0, st) == 2   # BF16 is no MX
    torch.cuda.synchronize()


def test_stack_and_caches_mlp_shape_sampled(orc, dev):
    # 256 separately allocated experts of [4096, 4096] (FC1's [2I, H]): the
    # transposed stack and both MXFP8 caches, whole experts compared for a
    # seeded sample
    G, R, C = 256, 4096, 4096
    ws = [synth.randn_bf16((R, C), seed=300 + g, std=R ** -0.5, device=dev) for g in range(G)]
    addr = ptm.expert_addresses(ws)
    out = torch.empty((G, C, R), dtype=torch.bfloat16, device=dev)
    ptm.pt_stack_experts(addr, out, G, R, C, 1)
    q = torch.empty((G, R, C), dtype=torch.uint8, device=dev)
    s = torch.empty((G, R, C // 32), dtype=torch.uint8, device=dev)
    qt = torch.empty((G, C, R), dtype=torch.uint8, device=dev)
    st = torch.empty((G, C, R // 32), dtype=torch.uint8, device=dev)
    ptm.pt_mx_quantize_experts(addr, q, s, qt, st, G, R, C, ptm.PT_MXFP8_E4M3)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    for g in sorted(set(rng.choice(G, size=3, replace=False).tolist()) | {0, G - 1}):
        wb = bits16(ws[g])
        assert (bits16(out[g]) == wb.T).all(), g
        rq, rs, rqt, rst = orc.mx_quantize_experts([wb], 1)
        assert (u8(q[g]) == rq[0]).all() and (u8(s[g]) == rs[0]).all(), g
        assert (u8(qt[g]) == rqt[0]).all() and (u8(st[g]) == rst[0]).all(), g
