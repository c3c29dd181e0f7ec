"""Pins for the oracle: every check here compares it with something other than
itself -- a library routine (torch's float8 decoders and fp32->fp8/bf16
conversions, numpy's dense matmul and integer matmul), closed forms of the OCP
element formats, exact arithmetic on integer or power-of-two inputs,
invariants of the grouped GEMM, and hand-worked quantisation fixtures under
tests/golden/.  CPU only.
"""
import math
import os

import numpy as np
import pytest
import torch

from conftest import GOLDEN

BF16, E4M3, E2M1 = 0, 1, 2


def bf16_of(x):
    """Exact bf16 bits of float values that are representable in bf16."""
    t = torch.tensor(np.asarray(x, np.float32))
    b = t.to(torch.bfloat16)
    assert torch.equal(b.float(), t), "value not representable in bf16"
    return b.view(torch.int16).numpy().view(np.uint16)


def rand_bf16(shape, seed, std=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * std).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------------ decoding
def test_bf16_decode_all_patterns(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = orc.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    same = (mine == ref) | (np.isnan(mine) & np.isnan(ref))
    assert same.all()
    assert (np.signbit(mine) == np.signbit(ref)).all()


def test_e4m3_decode_matches_torch(orc):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    mine = np.array([orc.e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert (np.isnan(mine) == nan).all()
    assert (mine[~nan] == ref[~nan]).all()
    assert (np.signbit(mine[~nan]) == np.signbit(ref[~nan])).all()
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]


def test_e8m0_decode_matches_torch(orc):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    mine = np.array([orc.e8m0_value(c) for c in range(256)])
    assert np.isnan(mine[255]) and np.isnan(ref[255])
    assert (mine[:255] == ref[:255]).all()


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                c, v = line.split()
                rows.append((int(c, 16), float(v)))
    return rows


def test_e2m1_decode_golden(orc):
    rows = _read_table("e2m1_values.txt")
    assert len(rows) == 16
    for code, val in rows:
        got = orc.e2m1_value(code)
        assert got == val and math.copysign(1, got) == math.copysign(1, val), (code, got, val)


def test_e4m3_decode_golden(orc):
    for code, val in _read_table("e4m3_selected.txt"):
        got = orc.e4m3_value(code)
        if math.isnan(val):
            assert math.isnan(got)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), (code, got, val)


# ------------------------------------------------------------------ rounding
def test_round_bf16_matches_torch_on_fp32_inputs(orc):
    g = torch.Generator().manual_seed(7)
    x = torch.randn(200000, generator=g) * torch.exp2(torch.randint(-140, 120, (200000,), generator=g).float())
    x = torch.cat([x, torch.tensor([0.0, -0.0, 3.4e38, -3.4e38, 1e-45, 2.0 ** -133, 2.0 ** -134])])
    ref = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    mine = orc.round_bf16(x.double().numpy())
    assert (mine == ref).all()


def test_round_bf16_ties_and_single_rounding(orc):
    one_ulp = 2.0 ** -7
    # exact midpoints round to the even neighbour
    assert orc.round_bf16(np.array([1.0 + one_ulp / 2]))[0] == 0x3F80          # -> 1.0
    assert orc.round_bf16(np.array([1.0 + 3 * one_ulp / 2]))[0] == 0x3F82      # -> 1+2ulp
    # just above a midpoint by less than an fp32 ulp: a double rounding through
    # fp32 would land on the midpoint and then go to even; one rounding goes up
    x = 1.0 + one_ulp / 2 + 2.0 ** -40
    assert orc.round_bf16(np.array([x]))[0] == 0x3F81
    # overflow and signed zero
    assert orc.round_bf16(np.array([1e39]))[0] == 0x7F80
    assert orc.round_bf16(np.array([-0.0]))[0] == 0x8000


# ------------------------------------------------------------------ quantiser
def _golden_quant_cases():
    cases = []
    with open(os.path.join(GOLDEN, "quantize_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            fmt, vals, e, codes = [p.strip() for p in line.split("|")]
            cases.append((fmt, [float(v) for v in vals.split()], int(e),
                          [int(c, 16) for c in codes.split()]))
    return cases


@pytest.mark.parametrize("case", _golden_quant_cases(), ids=lambda c: c[0] + "_" + str(c[2]))
def test_quantize_golden_cases(orc, case):
    fmt, vals, E, codes = case
    assert len(vals) == 32 and len(codes) == 32
    x = bf16_of(vals).reshape(1, 32)
    dt = E4M3 if fmt == "e4m3" else E2M1
    q, s = orc.mx_quantize(x, dt, axis=1)
    assert s[0, 0] == E
    if dt == E4M3:
        assert list(q[0]) == codes
    else:
        unpacked = [(int(q[0, i // 2]) >> (4 * (i & 1))) & 15 for i in range(32)]
        assert unpacked == codes


def _scale_exponent(vals):
    """Block scale from the closed form, floor(log2 amax) via exact frexp."""
    amax = np.abs(vals).max(axis=-1)
    _, e = np.frexp(amax)
    return e - 1


def test_quantize_e4m3_elements_match_torch(orc):
    # torch's fp32 -> float8_e4m3fn conversion rounds to nearest-even and does
    # not saturate, so clamp to +-448 before handing it the scaled values
    x = rand_bf16((256, 256), seed=11)
    xv = orc.bf16_to_f64(x)
    # outliers and tiny values to reach saturation and subnormals
    x2 = rand_bf16((64, 256), seed=12, std=1e-3)
    x = np.concatenate([x, x2], axis=0)
    xv = orc.bf16_to_f64(x)
    q, s = orc.mx_quantize(x, E4M3, axis=1)
    blocks = xv.reshape(-1, 32)
    scale = np.exp2(s.reshape(-1).astype(np.float64) - 127.0)
    scaled = np.clip(blocks / scale[:, None], -448.0, 448.0)
    ref = torch.from_numpy(scaled.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (q.reshape(-1, 32) == ref).all()
    # the scale: floor(log2 amax) - 8 + 127, from numpy's frexp
    assert (s.reshape(-1) == np.clip(_scale_exponent(blocks) - 8 + 127, 0, 254)).all()


def test_quantize_roundtrip_exact_on_representable(orc):
    # blocks whose elements are grid values times 2^k and whose largest
    # magnitude is the grid maximum's exponent: dequant(quant(v)) == v
    rng = np.random.default_rng(5)
    for dt, grid, top in ((E4M3, [orc.e4m3_value(c) for c in range(0x7F)], 1.75 * 256),
                          (E2M1, [orc.e2m1_value(c) for c in range(8)], 6.0)):
        grid = np.array(grid)
        rows = []
        for k in range(-20, 21, 4):
            v = rng.choice(grid[grid >= 0.015625 if dt == E4M3 else grid >= 0], size=32)
            v *= rng.choice([-1.0, 1.0], size=32)
            v[rng.integers(32)] = top
            rows.append(v * 2.0 ** k)
        vals = np.array(rows)
        x = bf16_of(vals)
        q, s = orc.mx_quantize(x, dt, axis=1)
        back = orc.mx_dequantize(dt, q, s, *vals.shape)
        assert (back == vals).all()


def test_quantize_axis0_equals_axis1_of_transpose(orc):
    x = rand_bf16((64, 96), seed=3)
    for dt in (E4M3, E2M1):
        q0, s0 = orc.mx_quantize(x, dt, axis=0)
        q1, s1 = orc.mx_quantize(np.ascontiguousarray(x.T), dt, axis=1)
        assert (s0 == s1.T).all()
        if dt == E4M3:
            assert (q0 == q1.T).all()
        else:
            lo0, hi0 = q0 & 15, q0 >> 4          # rows 2i, 2i+1
            lo1, hi1 = q1 & 15, q1 >> 4          # cols 2i, 2i+1
            assert (lo0 == lo1.T).all() and (hi0 == hi1.T).all()


def test_quantize_scale_power_of_two_invariance(orc):
    # multiplying a block by 2^j shifts its scale byte by j and keeps its codes
    x = rand_bf16((32, 64), seed=9)
    xv = orc.bf16_to_f64(x)
    for dt in (E4M3, E2M1):
        q, s = orc.mx_quantize(x, dt)
        q3, s3 = orc.mx_quantize(bf16_of(xv * 8.0), dt)
        assert (q3 == q).all() and (s3.astype(int) == s.astype(int) + 3).all()


def test_e2m1_packing_low_nibble_is_even_column(orc):
    vals = np.zeros(32)
    vals[0], vals[1] = 1.0, 6.0          # scale 2^0 (amax 6): codes 2 and 7
    q, s = orc.mx_quantize(bf16_of(vals).reshape(1, 32), E2M1)
    assert s[0, 0] == 127 and q[0, 0] == 0x72


# ------------------------------------------------------------------ SwiGLU
def test_swiglu_closed_forms(orc):
    c = np.array([[0.0, 1.0, 40.0, -40.0, 2.0, 3.0, 1.0, 0.5]])
    h = orc.swiglu(c)
    assert h.shape == (1, 4)
    assert h[0, 0] == 0.0                                    # silu(0) = 0
    assert h[0, 1] == pytest.approx(3.0 / (1 + math.exp(-1.0)), rel=1e-15)  # gate first
    assert h[0, 2] == pytest.approx(40.0, rel=1e-15)         # silu(x) -> x
    assert abs(h[0, 3]) < 1e-15                              # silu(-x) -> 0
    # swapping the halves changes the result: gate/up order matters
    assert orc.swiglu(c[:, [4, 5, 6, 7, 0, 1, 2, 3]])[0, 1] != h[0, 1]



def test_swiglu_bwd_matches_central_differences_of_forward(orc):
    # The backward is pinned to the (separately pinned) forward: d/dg and d/du
    # of silu(g) * u by central differences in binary64.
    rng = np.random.default_rng(21)
    n, I = 6, 40
    g = rng.uniform(-8.0, 8.0, size=(n, I))
    u = rng.uniform(-4.0, 4.0, size=(n, I))
    dh = rng.uniform(-2.0, 2.0, size=(n, I))
    dc = orc.swiglu_bwd(dh, np.concatenate([g, u], axis=1))
    eps = 1e-5
    h = lambda gg, uu: orc.swiglu(np.concatenate([gg, uu], axis=1))
    dg_fd = dh * (h(g + eps, u) - h(g - eps, u)) / (2 * eps)
    du_fd = dh * (h(g, u + eps) - h(g, u - eps)) / (2 * eps)
    assert np.allclose(dc[:, :I], dg_fd, rtol=1e-8, atol=1e-9)
    assert np.allclose(dc[:, I:], du_fd, rtol=1e-8, atol=1e-9)


def test_swiglu_bwd_closed_forms(orc):
    # g = 0: silu'(0) = 1/2 and silu(0) = 0.  g -> +inf: silu' -> 1, silu -> g.
    # g -> -inf: both -> 0.  Layout: [d gate | d up], gate half first.
    c = np.array([[0.0, 40.0, -40.0, 3.0, 5.0, 7.0]])
    dh = np.array([[2.0, 0.5, 1.0]])
    dc = orc.swiglu_bwd(dh, c)
    assert dc[0, 0] == 2.0 * 3.0 * 0.5 and dc[0, 3] == 0.0
    assert dc[0, 1] == pytest.approx(0.5 * 5.0, rel=1e-15) and dc[0, 4] == pytest.approx(0.5 * 40.0, rel=1e-15)
    assert abs(dc[0, 2]) < 1e-14 and abs(dc[0, 5]) < 1e-14
    with pytest.raises(ValueError):
        orc.swiglu_bwd(dh, c[:, :4])


def test_swiglu_clamp_closed_forms(orc):
    # L = 10: a gate above L becomes L, an up value outside [-L, L] becomes
    # +-L; a gate far below -L is left alone (the gate clamp is one-sided)
    c = np.array([[20.0, 1.0, 0.5, -30.0, 3.0, -20.0, 30.0, 2.0]])
    h = orc.swiglu(c, 10.0)
    silu = lambda x: x / (1 + math.exp(-x))
    assert h[0, 0] == pytest.approx(silu(10.0) * 3.0, rel=1e-15)
    assert h[0, 1] == pytest.approx(silu(1.0) * -10.0, rel=1e-15)
    assert h[0, 2] == pytest.approx(silu(0.5) * 10.0, rel=1e-15)
    assert h[0, 3] == pytest.approx(silu(-30.0) * 2.0, rel=1e-15)
    # a limit at or above every input changes nothing; 0 and inf mean "off"
    rng = np.random.default_rng(22)
    c2 = rng.uniform(-5.0, 5.0, size=(4, 16))
    for lim in (5.0, 0.0, math.inf):
        assert np.array_equal(orc.swiglu(c2, lim), orc.swiglu(c2))


def test_swiglu_clamp_bwd_matches_central_differences(orc):
    # away from the kinks the clamped backward is the derivative of the
    # clamped forward: zero into a clamped input, the plain one elsewhere
    rng = np.random.default_rng(23)
    n, I, lim = 6, 40, 2.5
    g = rng.uniform(-6.0, 6.0, size=(n, I))
    u = rng.uniform(-6.0, 6.0, size=(n, I))
    g[np.abs(g - lim) < 1e-3] += 0.01
    u[np.abs(np.abs(u) - lim) < 1e-3] += 0.01
    dh = rng.uniform(-2.0, 2.0, size=(n, I))
    dc = orc.swiglu_bwd(dh, np.concatenate([g, u], axis=1), lim)
    eps = 1e-6
    h = lambda gg, uu: orc.swiglu(np.concatenate([gg, uu], axis=1), lim)
    dg_fd = dh * (h(g + eps, u) - h(g - eps, u)) / (2 * eps)
    du_fd = dh * (h(g, u + eps) - h(g, u - eps)) / (2 * eps)
    assert np.allclose(dc[:, :I], dg_fd, rtol=1e-7, atol=1e-8)
    assert np.allclose(dc[:, I:], du_fd, rtol=1e-7, atol=1e-8)
    assert (dc[:, :I][g > lim] == 0).all() and (dc[:, I:][np.abs(u) > lim] == 0).all()
    assert (dc[:, :I][g < lim] != 0).any()


def test_dgrad_swiglu_rows_composition(orc):
    # Integer operands keep dH exact; the composed op must equal the pinned
    # backward applied to bf16(dH) from a numpy per-expert matmul, row by row,
    # for a sampled, unordered row list.
    lens = np.array([5, 0, 7, 4])
    G, K, N = 4, 24, 16
    offs = np.concatenate([[0], np.cumsum(lens)])
    M = int(lens.sum())
    rng = np.random.default_rng(22)
    dyv = rng.integers(-3, 4, size=(M, N)).astype(np.float64)
    bv = rng.integers(-3, 4, size=(G, K, N)).astype(np.float64)
    cv = rng.integers(-6, 7, size=(M, 2 * K)).astype(np.float64) / 4.0
    dy, b, c = bf16_of(dyv), bf16_of(bv), bf16_of(cv)
    rows = np.array([15, 0, 9, 4, 5, 11])
    for trans_b in (0, 1):
        bb = np.ascontiguousarray(b.transpose(0, 2, 1)) if trans_b else b
        got = orc.dgrad_swiglu_rows(dy, bb, c, lens, N, K, trans_b, rows)
        g_of = np.searchsorted(offs, rows, side="right") - 1
        dh = np.stack([dyv[r] @ bv[g].T for r, g in zip(rows, g_of)])
        assert np.array_equal(orc.bf16_to_f64(got["dh_bf16"]), dh)      # small integers: exact
        ref = orc.swiglu_bwd(dh, cv[rows])
        assert np.array_equal(got["exact"], ref)
        assert np.array_equal(got["bf16"], orc.round_bf16(ref))


def _torch_e4m3(v32):
    """torch's float32 -> float8_e4m3fn cast (nearest, ties to even) as codes."""
    return torch.tensor(np.asarray(v32, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_fp8_quantize_unit_scale_matches_torch_cast(orc):
    # amax = 448 gives s = 1: every code is the plain E4M3 cast of the value
    v = rand_bf16((4, 256), seed=70, std=60.0)
    vf = orc.bf16_to_f64(v)
    vf = np.clip(vf, -448, 448)
    vf[:, 0] = 448.0                                   # pin amax of each matrix to 448
    x = bf16_of(vf)
    q, amax, deq = orc.fp8_quantize(x)
    assert (amax == 448.0).all() and (deq == 1.0).all()
    assert (q == _torch_e4m3(orc.bf16_to_f64(x))).all()


def test_fp8_quantize_general_scale_matches_fp32_product_then_cast(orc):
    x = rand_bf16((3, 512), seed=71, std=0.37)
    q, amax, deq = orc.fp8_quantize(x)
    xf = orc.bf16_to_f64(x).astype(np.float32)
    for b in range(3):
        m = np.float32(np.abs(xf[b]).max())
        assert amax[b] == m
        s = np.float32(448.0) / m                       # one IEEE fp32 division
        assert deq[b] == np.float32(1.0) / s
        y = np.clip(xf[b] * s, np.float32(-448), np.float32(448))   # fp32 product
        assert (q[b] == _torch_e4m3(y)).all(), b


def test_fp8_quantize_power_of_two_invariance_and_zero(orc):
    x = rand_bf16((2, 128), seed=72, std=3.0)
    q, amax, deq = orc.fp8_quantize(x)
    x8 = bf16_of(orc.bf16_to_f64(x) * 8.0)              # exact in bf16
    q8, amax8, deq8 = orc.fp8_quantize(x8)
    assert (q8 == q).all() and (amax8 == 8 * amax).all() and (deq8 == 8 * deq).all()
    z = np.zeros((1, 64), np.uint16)
    qz, az, dz = orc.fp8_quantize(z)
    assert (qz == 0).all() and az[0] == 0 and dz[0] == 1.0


def test_fp8_fwd_rows_matches_dense_on_decoded_codes(orc):
    lens = np.array([5, 0, 9, 3])
    G, K, N = 4, 64, 40
    M = int(lens.sum())
    rng = np.random.default_rng(73)
    aq = rng.integers(0, 0x7E, size=(M, K)).astype(np.uint8) | (rng.integers(0, 2, size=(M, K)) << 7).astype(np.uint8)
    bq = rng.integers(0, 0x7E, size=(G, N, K)).astype(np.uint8)
    ad, bd = np.float32(0.03125), np.array([1.5, 2.0, 0.25, 3.0], np.float32)
    rows = np.array([0, 4, 13, 16, 7])
    got = orc.fp8_fwd_rows(aq, ad, bq, bd, lens, N, K, rows)
    dec = lambda c: torch.tensor(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    offs = np.concatenate([[0], np.cumsum(lens)])
    for i, r in enumerate(rows):
        g = np.searchsorted(offs, r, side="right") - 1
        ref = dec(aq[r]) @ dec(bq[g]).T * (float(ad) * float(bd[g]))
        assert np.allclose(got[i], ref, rtol=1e-14, atol=0), r


def test_fp8_wgrad_rows_matches_dense_on_torch_decoded_codes(orc):
    # per expert: factors times (decoded A_g)^T (decoded dY_g), the codes
    # decoded by torch's float8_e4m3fn, the product by numpy
    lens = np.array([5, 0, 40, 17])
    M, K, N = int(lens.sum()), 24, 16
    rng = np.random.default_rng(70)
    aq = rng.integers(0, 256, size=(M, K)).astype(np.uint8)
    dq = rng.integers(0, 256, size=(M, N)).astype(np.uint8)
    aq[(aq & 0x7F) == 0x7F] = 0x38
    dq[(dq & 0x7F) == 0x7F] = 0xB8
    da, dd = np.float32(0.0123), np.float32(3.5e-4)
    G = lens.size
    gs, ks = np.repeat(np.arange(G), K), np.tile(np.arange(K), G)
    got = orc.fp8_wgrad_rows(aq, da, dq, dd, lens, N, K, gs, ks).reshape(G, K, N)
    av = torch.from_numpy(aq).view(torch.float8_e4m3fn).double().numpy()
    dv = torch.from_numpy(dq).view(torch.float8_e4m3fn).double().numpy()
    offs = np.concatenate([[0], np.cumsum(lens)])
    for g in range(G):
        want = (av[offs[g]:offs[g + 1]].T @ dv[offs[g]:offs[g + 1]]) * (float(da) * float(dd))
        assert np.allclose(got[g], want, rtol=1e-13, atol=0), g


def test_fp8_rowwise_scales_each_row_on_its_own(orc):
    # rows of very different magnitude: each row's codes are torch's cast of
    # fp32(x * 448 / amax_row), independent of the other rows
    x = np.concatenate([rand_bf16((1, 96), seed=74, std=s) for s in (1e-3, 1.0, 300.0)])
    q, amax, deq = orc.fp8_quantize(x)
    xf = orc.bf16_to_f64(x).astype(np.float32)
    for r in range(3):
        s = np.float32(448.0) / np.float32(np.abs(xf[r]).max())
        assert deq[r] == np.float32(1.0) / s
        assert (q[r] == _torch_e4m3(np.clip(xf[r] * s, -448, 448))).all(), r


def test_fp8_fwd_rows_rowwise_matches_dense(orc):
    lens = np.array([4, 6, 0, 2])
    G, K, N = 4, 32, 24
    M = int(lens.sum())
    rng = np.random.default_rng(75)
    aq = rng.integers(0, 0x7E, size=(M, K)).astype(np.uint8)
    bq = (rng.integers(0, 0x7E, size=(G, N, K)) | (rng.integers(0, 2, size=(G, N, K)) << 7)).astype(np.uint8)
    ad = rng.uniform(0.5, 2.0, size=M).astype(np.float32)
    bd = rng.uniform(0.01, 0.1, size=(G, N)).astype(np.float32)
    rows = np.array([1, 9, 11, 4])
    got = orc.fp8_fwd_rows_rowwise(aq, ad, bq, bd, lens, N, K, rows)
    dec = lambda c: torch.tensor(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    offs = np.concatenate([[0], np.cumsum(lens)])
    for i, r in enumerate(rows):
        g = np.searchsorted(offs, r, side="right") - 1
        ref = (dec(aq[r]) @ dec(bq[g]).T) * float(ad[r]) * bd[g].astype(np.float64)
        assert np.allclose(got[i], ref, rtol=1e-14, atol=0), r


def _codes_axis0(q, fmt):
    # per-element codes of the axis-0 quantiser (E2M1 packs rows 2i, 2i+1)
    if fmt == E4M3:
        return q
    out = np.empty((2 * q.shape[0], q.shape[1]), np.uint8)
    out[0::2], out[1::2] = q & 0xF, q >> 4
    return out


def _codes_tokens(q, fmt):
    # per-element codes along tokens (E2M1 packs columns 2c, 2c+1)
    if fmt == E4M3:
        return q
    out = np.empty((q.shape[0], 2 * q.shape[1]), np.uint8)
    out[:, 0::2], out[:, 1::2] = q & 0xF, q >> 4
    return out


@pytest.mark.parametrize("fmt", [E4M3, E2M1], ids=["e4m3", "e2m1"])
def test_mx_quantize_tokens_full_blocks_equal_axis0(orc, fmt):
    # experts whose lengths are multiples of 32 reduce to the plain column-block
    # quantiser (axis 0) on each expert's rows
    lens = np.array([64, 0, 32, 96])
    x = rand_bf16((int(lens.sum()), 48), seed=76, std=2.0)
    q, s, nb = orc.mx_quantize_tokens(x, lens, fmt)
    assert nb == 6
    codes = _codes_tokens(q, fmt)
    offs = np.concatenate([[0], np.cumsum(lens)])
    b = 0
    for g in range(lens.size):
        if lens[g] == 0:
            continue
        rq, rs = orc.mx_quantize(x[offs[g]:offs[g + 1]], fmt, axis=0)
        assert (codes[offs[g]:offs[g + 1]] == _codes_axis0(rq, fmt)).all(), g
        assert (s[b:b + lens[g] // 32] == rs).all(), g
        b += lens[g] // 32


@pytest.mark.parametrize("fmt", [E4M3, E2M1], ids=["e4m3", "e2m1"])
def test_mx_quantize_tokens_partial_block_equals_zero_padding(orc, fmt):
    # a partial last block behaves as if padded with zero rows (zeros change
    # neither the amax nor the other codes), and it never mixes two experts
    lens = np.array([45, 7, 33])
    M = int(lens.sum())
    x = rand_bf16((M, 32), seed=77, std=1.0)
    q, s, nb = orc.mx_quantize_tokens(x, lens, fmt)
    assert nb == 2 + 1 + 2
    codes = _codes_tokens(q, fmt)
    offs = np.concatenate([[0], np.cumsum(lens)])
    b = 0
    for g in range(lens.size):
        n = int(lens[g])
        pad = np.zeros((((n + 31) // 32) * 32, 32), np.uint16)
        pad[:n] = x[offs[g]:offs[g + 1]]
        rq, rs = orc.mx_quantize(pad, fmt, axis=0)
        assert (codes[offs[g]:offs[g + 1]] == _codes_axis0(rq, fmt)[:n]).all(), g
        assert (s[b:b + (n + 31) // 32] == rs).all(), g
        b += (n + 31) // 32
    # the dequantised values are the codes times their block's scale
    v = orc.mx_dequantize_tokens(q, s, lens, fmt)
    tol = 2 ** -3 if fmt == E4M3 else 2 ** -1
    assert np.abs(v - orc.bf16_to_f64(x)).max() <= np.abs(orc.bf16_to_f64(x)).max() * tol


def _token_block_scales(s, lens):
    blk = np.concatenate([b0 + np.arange(n) // 32 for b0, n in
                          zip(np.concatenate([[0], np.cumsum((lens + 31) // 32)[:-1]]), lens)])
    return torch.from_numpy(np.ascontiguousarray(s[blk])).view(torch.float8_e8m0fnu).double().numpy()


def test_mx_dequantize_tokens_matches_torch_decode(orc):
    # every finite E4M3 code, decoded by torch's float8_e4m3fn and scaled by
    # its own block's E8M0 byte (decoded by torch's float8_e8m0fnu): a wrong
    # block index (expert start, short last block) moves some row's scale
    lens = np.array([0, 40, 1, 31, 0, 70])
    M, C = int(lens.sum()), 24
    rng = np.random.default_rng(78)
    q = rng.integers(0, 256, size=(M, C)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x3C
    nb = int(sum((n + 31) // 32 for n in lens))
    s = np.zeros((M // 32 + lens.size, C), np.uint8)
    s[:nb] = rng.integers(110, 145, size=(nb, C))
    got = orc.mx_dequantize_tokens(q, s, lens)
    vals = torch.from_numpy(q).view(torch.float8_e4m3fn).double().numpy()
    assert (got == vals * _token_block_scales(s, lens)).all()


def test_mx_dequantize_tokens_e2m1_matches_golden_table(orc):
    # E2M1 nibbles decoded from the OCP table in tests/golden (low nibble =
    # even column), times torch's decoding of the row's block scale
    table = dict(_read_table("e2m1_values.txt"))
    assert len(table) == 16
    lens = np.array([33, 0, 64, 5])
    M, C = int(lens.sum()), 16
    rng = np.random.default_rng(79)
    q = rng.integers(0, 256, size=(M, C // 2)).astype(np.uint8)
    nb = int(sum((n + 31) // 32 for n in lens))
    s = np.zeros((M // 32 + lens.size, C), np.uint8)
    s[:nb] = rng.integers(110, 145, size=(nb, C))
    got = orc.mx_dequantize_tokens(q, s, lens, E2M1)
    vals = np.empty((M, C))
    for r in range(M):
        for c in range(C):
            nib = (q[r, c // 2] >> (4 * (c & 1))) & 0xF
            vals[r, c] = table[int(nib)]
    assert (got == vals * _token_block_scales(s, lens)).all()


def test_stack_experts_by_index(orc):
    # element by element on tiny experts: out[g, i, j] = W_g[i, j], or W_g[j, i]
    ws = [rand_bf16((3, 5), seed=80 + g) for g in range(4)]
    for transpose in (False, True):
        out = orc.stack_experts(ws, transpose)
        assert out.shape == ((4, 5, 3) if transpose else (4, 3, 5))
        for g in range(4):
            for i in range(3):
                for j in range(5):
                    assert (out[g, j, i] if transpose else out[g, i, j]) == ws[g][i, j]


def test_mx_quantize_experts_caches(orc):
    # the forward cache is the row quantiser on each expert; the transposed
    # cache equals the column-block (axis 0) quantiser's codes and scales,
    # transposed -- an independent route through the C oracle
    ws = [rand_bf16((64, 96), seed=90 + g, std=3.0) for g in range(3)]
    for fmt in (E4M3, E2M1):
        q, s, qt, st = orc.mx_quantize_experts(ws, fmt)
        for g, w in enumerate(ws):
            rq, rs = orc.mx_quantize(w, fmt, axis=1)
            assert (q[g] == rq).all() and (s[g] == rs).all()
            aq, as_ = orc.mx_quantize(w, fmt, axis=0)
            # (for E2M1 axis 0 packs rows 2i, 2i+1 of a column into one byte,
            # the same pair the transpose packs along its row)
            assert (st[g] == as_.T).all() and (qt[g] == aq.T).all()


# ------------------------------------------------------------------ GEMMs
def _setup(G, lens, K, N, seed, trans_b=0, integer=False):
    M = int(sum(lens))
    if integer:
        rng = np.random.default_rng(seed)
        av = rng.integers(-4, 5, size=(M, K)).astype(np.float64)
        bv = rng.integers(-4, 5, size=(G, K, N)).astype(np.float64)
        a, b = bf16_of(av), bf16_of(bv)
    else:
        a = rand_bf16((M, K), seed)
        b = rand_bf16((G, K, N), seed + 1)
    if trans_b:
        b = np.ascontiguousarray(b.transpose(0, 2, 1))
    return M, a, b


def test_fwd_single_expert_equals_dense_numpy(orc):
    lens = np.array([37])
    M, a, b = _setup(1, lens, 48, 20, seed=1)
    got = orc.fwd_rows(BF16, a, None, b, None, lens, 20, 48, 0, np.arange(M))
    ref = orc.bf16_to_f64(a) @ orc.bf16_to_f64(b)[0]
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("trans_b", [0, 1])
def test_fwd_integer_inputs_exact(orc, trans_b):
    lens = np.array([5, 0, 7, 1, 0, 3])
    G, K, N = 6, 32, 12
    M, a, b = _setup(G, lens, K, N, seed=2, trans_b=trans_b, integer=True)
    got = orc.fwd_rows(BF16, a, None, b, None, lens, N, K, trans_b, np.arange(M))
    ai = orc.bf16_to_f64(a).astype(np.int64)
    bi = orc.bf16_to_f64(b).astype(np.int64)
    if trans_b:
        bi = bi.transpose(0, 2, 1)
    offs = np.concatenate([[0], np.cumsum(lens)])
    for g in range(G):
        ref = ai[offs[g]:offs[g + 1]] @ bi[g]
        assert (got[offs[g]:offs[g + 1]] == ref).all()


def test_fwd_scaled_identity_maps_rows_to_experts(orc):
    # B_g = 2^(g+1) I: every output row is its A row times its expert's factor,
    # so any wrong row -> expert assignment shows up exactly
    lens = np.array([3, 0, 4, 2])
    G, K = 4, 16
    M = int(lens.sum())
    a = rand_bf16((M, K), seed=4)
    bv = np.stack([np.eye(K) * 2.0 ** (g + 1) for g in range(G)])
    got = orc.fwd_rows(BF16, a, None, bf16_of(bv), None, lens, K, K, 0, np.arange(M))
    expert = np.repeat(np.arange(G), lens)
    assert (got == orc.bf16_to_f64(a) * (2.0 ** (expert + 1))[:, None]).all()


def test_fwd_row_sampling_and_rejects_uncovered_rows(orc):
    lens = np.array([4, 0, 5])
    M, a, b = _setup(3, lens, 32, 8, seed=6)
    full = orc.fwd_rows(BF16, a, None, b, None, lens, 8, 32, 0, np.arange(M))
    some = orc.fwd_rows(BF16, a, None, b, None, lens, 8, 32, 0, np.array([8, 0, 4]))
    assert (some == full[[8, 0, 4]]).all()
    with pytest.raises(ValueError):
        orc.fwd_rows(BF16, a, None, b, None, lens, 8, 32, 0, np.array([M]))


def test_adjoint_identity_fwd_dgrad_wgrad(orc):
    # <dY, A B> = <dY B^T, A> = <A^T dY, B> summed over experts
    lens = np.array([6, 0, 9, 3])
    G, K, N = 4, 32, 24
    M, a, b = _setup(G, lens, K, N, seed=8)
    dy = rand_bf16((M, N), seed=10)
    rows = np.arange(M)
    av, bv, dyv = orc.bf16_to_f64(a), orc.bf16_to_f64(b), orc.bf16_to_f64(dy)
    c = orc.fwd_rows(BF16, a, None, b, None, lens, N, K, 0, rows)
    dx = orc.dgrad_rows(dy, b, lens, N, K, 0, rows)
    gs = np.repeat(np.arange(G), K)
    ks = np.tile(np.arange(K), G)
    dw = orc.wgrad_rows(a, dy, lens, N, K, gs, ks).reshape(G, K, N)
    t1 = (dyv * c).sum()
    t2 = (dx * av).sum()
    t3 = (dw * bv).sum()
    assert t1 == pytest.approx(t2, rel=1e-12) and t1 == pytest.approx(t3, rel=1e-12)
    assert (dw[1] == 0).all()                        # empty expert


def test_dgrad_layouts_agree_and_match_numpy(orc):
    lens = np.array([7, 2, 0, 5])
    G, K, N = 4, 40, 16
    M, a, b = _setup(G, lens, K, N, seed=12)
    dy = rand_bf16((M, N), seed=13)
    rows = np.arange(M)
    d0 = orc.dgrad_rows(dy, b, lens, N, K, 0, rows)
    d1 = orc.dgrad_rows(dy, np.ascontiguousarray(b.transpose(0, 2, 1)), lens, N, K, 1, rows)
    assert np.allclose(d0, d1, rtol=1e-13, atol=1e-14)
    offs = np.concatenate([[0], np.cumsum(lens)])
    bv, dyv = orc.bf16_to_f64(b), orc.bf16_to_f64(dy)
    for g in range(G):
        ref = dyv[offs[g]:offs[g + 1]] @ bv[g].T
        assert np.allclose(d0[offs[g]:offs[g + 1]], ref, rtol=1e-13, atol=1e-14)


def test_wgrad_sum_over_experts_is_dense_atdy(orc):
    lens = np.array([5, 0, 11, 1])
    G, K, N = 4, 24, 20
    M, a, _ = _setup(G, lens, K, N, seed=14)
    dy = rand_bf16((M, N), seed=15)
    gs = np.repeat(np.arange(G), K)
    ks = np.tile(np.arange(K), G)
    dw = orc.wgrad_rows(a, dy, lens, N, K, gs, ks).reshape(G, K, N)
    ref = orc.bf16_to_f64(a).T @ orc.bf16_to_f64(dy)
    assert np.allclose(dw.sum(0), ref, rtol=1e-12, atol=1e-13)
    offs = np.concatenate([[0], np.cumsum(lens)])
    g = 2
    refg = orc.bf16_to_f64(a)[offs[g]:offs[g + 1]].T @ orc.bf16_to_f64(dy)[offs[g]:offs[g + 1]]
    assert np.allclose(dw[g], refg, rtol=1e-12, atol=1e-13)


def test_wgrad_accumulate_rounds_once(orc):
    base = np.array([1.0, 1.0, -2.0], np.float32)
    d = np.array([2.0 ** -24, 2.0 ** -24 + 2.0 ** -50, 0.0])
    out = orc.wgrad_accumulate(base, d, accumulate=True)
    # 1 + 2^-24 is an exact fp32 midpoint -> even (1.0); a hair above -> up
    assert out[0] == np.float32(1.0)
    assert out[1] == np.nextafter(np.float32(1.0), np.float32(2.0))
    assert out[2] == np.float32(-2.0)
    assert (orc.wgrad_accumulate(base, d, accumulate=False) == d.astype(np.float32)).all()


@pytest.mark.parametrize("fmt", [E4M3, E2M1])
def test_mx_fwd_matches_dense_on_decoded_values(orc, fmt):
    rng = np.random.default_rng(21 + fmt)
    lens = np.array([9, 0, 4])
    G, K, N = 3, 64, 16
    M = int(lens.sum())
    cols = K if fmt == E4M3 else K // 2
    a = rng.integers(0, 256, size=(M, cols), dtype=np.uint8)
    b = rng.integers(0, 256, size=(G, N, cols), dtype=np.uint8)
    if fmt == E4M3:                                  # avoid the NaN codes
        a[(a & 0x7F) == 0x7F] -= 1
        b[(b & 0x7F) == 0x7F] -= 1
    as_ = rng.integers(120, 135, size=(M, K // 32), dtype=np.uint8)
    bs = rng.integers(120, 135, size=(G, N, K // 32), dtype=np.uint8)
    got = orc.fwd_rows(fmt, a, as_, b, bs, lens, N, K, 1, np.arange(M))
    # independent decode: per-code tables (pinned above) times 2^(E-127)
    if fmt == E4M3:
        tab = np.array([orc.e4m3_value(c) for c in range(256)])
        av, bvv = tab[a], tab[b]
    else:
        tab = np.array([orc.e2m1_value(c) for c in range(16)])
        av = np.stack([tab[a & 15], tab[a >> 4]], axis=-1).reshape(M, K)
        bvv = np.stack([tab[b & 15], tab[b >> 4]], axis=-1).reshape(G, N, K)
    av = av * np.repeat(np.exp2(as_.astype(float) - 127), 32, axis=1)
    bvv = bvv * np.repeat(np.exp2(bs.astype(float) - 127), 32, axis=2)
    offs = np.concatenate([[0], np.cumsum(lens)])
    for g in range(G):
        ref = av[offs[g]:offs[g + 1]] @ bvv[g].T
        assert np.allclose(got[offs[g]:offs[g + 1]], ref, rtol=1e-13, atol=0)
    # one scale byte up doubles exactly the products that use that block
    as2 = as_.copy()
    as2[:, 1] += 1
    got2 = orc.fwd_rows(fmt, a, as2, b, bs, lens, N, K, 1, np.arange(M))
    half = av.copy()
    half[:, 32:] *= 2
    for g in range(G):
        ref = half[offs[g]:offs[g + 1]] @ bvv[g].T
        assert np.allclose(got2[offs[g]:offs[g + 1]], ref, rtol=1e-13, atol=0)


def test_epilogue_composition(orc):
    lens = np.array([3, 4])
    G, K, N = 2, 32, 64
    M, a, b = _setup(G, lens, K, N, seed=30)
    rows = np.arange(M)
    r = orc.grouped_fwd(BF16, a, None, b, None, lens, N, K, 0, orc.EPI_SWIGLU_MXFP4, rows)
    c = orc.fwd_rows(BF16, a, None, b, None, lens, N, K, 0, rows)
    g, u = c[:, :N // 2], c[:, N // 2:]
    assert np.allclose(r["exact"], g / (1 + np.exp(-g)) * u, rtol=1e-14, atol=0)
    assert r["q"].shape == (M, N // 4) and r["s"].shape == (M, N // 64)


def test_mlp_row_sampling_matches_full(orc):
    rng = np.random.default_rng(40)
    lens = np.array([5, 0, 6, 3])
    G, H, I = 4, 64, 32
    M = int(lens.sum())
    x = rand_bf16((M, H), seed=41)
    w1 = rand_bf16((G * 2 * I, H), seed=42)
    w2 = rand_bf16((G * H, I), seed=43)
    w1q, w1s = orc.mx_quantize(w1, E2M1)
    w2q, w2s = orc.mx_quantize(w2, E2M1)
    w1q, w1s = w1q.reshape(G, 2 * I, H // 2), w1s.reshape(G, 2 * I, H // 32)
    w2q, w2s = w2q.reshape(G, H, I // 2), w2s.reshape(G, H, I // 32)
    full = orc.mlp_mxfp4_rows(x, w1q, w1s, w2q, w2s, lens, H, I, np.arange(M))
    pick = np.sort(rng.choice(M, size=6, replace=False))
    some = orc.mlp_mxfp4_rows(x, w1q, w1s, w2q, w2s, lens, H, I, pick)
    assert (some["exact"] == full["exact"][pick]).all()
    # and it equals the step-by-step chain over all rows
    xq, xs = orc.mx_quantize(x, E2M1)
    c1 = orc.fwd_rows(E2M1, xq, xs, w1q, w1s, lens, 2 * I, H, 1, np.arange(M))
    hq, hs = orc.mx_quantize(orc.round_bf16(orc.swiglu(c1)), E2M1)
    c2 = orc.fwd_rows(E2M1, hq, hs, w2q, w2s, lens, H, I, 1, np.arange(M))
    assert (c2 == full["exact"]).all()
