"""GPU parity of FC2's data gradient with the fused SwiGLU backward for the
low-precision operands (pt_grouped_gemm_dgrad_swiglu with MXFP8, MXFP4, FP8
with tensor factors and FP8 with row factors), through the C ABI.

For each dtype, tile order and clamp: (1) the output equals the oracle's
SwiGLU backward applied to the bf16 dH that pt_grouped_gemm_dgrad writes for
the same operands (the fused epilogue starts from that dH), within the BF16
tolerance; (2) for the MX formats, end to end against the oracle's dH on the
same MX bytes (exactly dequantised, rounded to bf16), within the MX
tolerance per expert.  Rows outside every expert stay unwritten."""
import numpy as np
import pytest
import torch

import moe_expert_grouped_gemm_amd as ptm
from moe_expert_grouped_gemm_amd import synth
from util import (BF16_TOL, MX_TOL, bits16, bf16_values, dev_i64, floored_rel_err, group_of_rows, norm_err,
                  per_group_max, u8)

pytestmark = pytest.mark.gpu

LENS = np.array([0, 1, 130, 0, 257, 64, 33], np.int64)
GUARD, NAN16 = 3, 0x7FC1
DTYPES = [(ptm.PT_MXFP8_E4M3, "e4m3", 1), (ptm.PT_MXFP4_E2M1, "e2m1", 2), (ptm.PT_FP8_E4M3, "fp8", None),
          (ptm.PT_FP8_E4M3_ROWWISE, "fp8rows", None)]


def operands(dev, dtype, name, M, G, N, K):
    """dY [M, N] and the transposed weight cache [G, K, N], both along N."""
    if name in ("e4m3", "e2m1"):
        dq, ds = synth.random_mx_codes(M, N, name, seed=230, device=dev, scale_lo=118, scale_hi=124)
        bq, bs = synth.random_mx_codes(G * K, N, name, seed=231, device=dev, scale_lo=118, scale_hi=124)
        return dq, ds, bq, bs
    dy = synth.randn_bf16((M, N), seed=232, std=1e-2, device=dev)
    wt = synth.randn_bf16((G * K, N), seed=233, std=N ** -0.5, device=dev)
    dq = torch.empty((M, N), dtype=torch.uint8, device=dev)
    bq = torch.empty((G * K, N), dtype=torch.uint8, device=dev)
    if dtype == ptm.PT_FP8_E4M3:
        f = [torch.empty((1,), dtype=torch.float32, device=dev) for _ in range(2)] + \
            [torch.empty((G,), dtype=torch.float32, device=dev) for _ in range(2)]
        ptm.pt_fp8_quantize(dy, dq, f[0], f[1], 1, M, N)
        ptm.pt_fp8_quantize(wt, bq, f[2], f[3], G, K, N)
    else:
        f = [torch.empty((M,), dtype=torch.float32, device=dev) for _ in range(2)] + \
            [torch.empty((G * K,), dtype=torch.float32, device=dev) for _ in range(2)]
        ptm.pt_fp8_quantize_rows(dy, dq, f[0], f[1], M, N)
        ptm.pt_fp8_quantize_rows(wt, bq, f[2], f[3], G * K, N)
    return dq, f[1], bq, f[3]


def workspace(dev, kind, op, G, M, N, K, dtype):
    if kind == "static":
        return None
    mx = dtype in (ptm.PT_MXFP8_E4M3, ptm.PT_MXFP4_E2M1)
    n = ptm.pt_grouped_gemm_workspace_size(op, G, M, N, K, dtype if (kind == "swz" and mx) else ptm.PT_BF16)
    return torch.full((n,), 0xFF, dtype=torch.uint8, device=dev)


@pytest.mark.parametrize("dtype,name,ofmt", DTYPES, ids=[d[1] for d in DTYPES])
@pytest.mark.parametrize("N", [320, 256])
@pytest.mark.parametrize("kind", ["static", "queue", "swz"])
@pytest.mark.parametrize("limit", [0.0, 10.0])
def test_lowp_dgrad_swiglu(orc, dev, dtype, name, ofmt, N, kind, limit):
    K = 264                                   # outputs per half: a partial 256-column tile
    M, G = int(LENS.sum()), len(LENS)
    print(f"lowp dgrad_swiglu {name} N={N} ws={kind} limit={limit}", flush=True)
    dq, ds, bq, bs = operands(dev, dtype, name, M, G, N, K)
    c = synth.randn_bf16((M, 2 * K), seed=234, std=4.0, device=dev)     # gates and ups across the clamp
    lens_d = dev_i64(LENS, dev)
    ws = workspace(dev, kind, ptm.PT_OP_DGRAD_SWIGLU, G, M, N, K, dtype)
    buf = torch.empty((M + 2 * GUARD, 2 * K), dtype=torch.bfloat16, device=dev)
    buf.view(torch.int16).fill_(NAN16)
    dc = buf[GUARD:GUARD + M]
    call = lambda: ptm.pt_grouped_gemm_dgrad_swiglu(dq, bq, c, dc, lens_d, None, G, M, N, K, 0, workspace=ws,
                                                    swiglu_limit=limit, dtype=dtype, dy_scale=ds, b_scale=bs)
    if dtype == ptm.PT_MXFP4_E2M1 and N % 256 and kind != "swz":
        with pytest.raises(ptm.PtggError) as e:          # the 256 x 256 kernel needs the scale copies here
            call()
        assert e.value.status == 2
        return
    call()
    dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    ptm.pt_grouped_gemm_dgrad(dq, ds, bq, bs, dx, lens_d, None, G, M, N, K, dtype, 0,
                              workspace=workspace(dev, kind, ptm.PT_OP_DGRAD, G, M, N, K, dtype))
    torch.cuda.synchronize()
    assert (bits16(buf[:GUARD]) == NAN16).all() and (bits16(buf[GUARD + M:]) == NAN16).all()
    got = bf16_values(bits16(dc))
    cv = bf16_values(bits16(c))
    rows = np.arange(M)
    grp = group_of_rows(LENS, rows)
    ref = orc.swiglu_bwd(bf16_values(bits16(dx)), cv, limit)
    for half in (slice(0, K), slice(K, 2 * K)):
        assert per_group_max(floored_rel_err, got[:, half], ref[:, half], grp) <= BF16_TOL, half
    if ofmt is not None:
        dh = orc.fwd_rows(ofmt, u8(dq), u8(ds), u8(bq).reshape(G, K, -1), u8(bs).reshape(G, K, -1), LENS, K, N, 1,
                          rows)
        ref2 = orc.swiglu_bwd(bf16_values(orc.round_bf16(dh)), cv, limit)
        for half in (slice(0, K), slice(K, 2 * K)):
            assert per_group_max(norm_err, got[:, half], ref2[:, half], grp) <= MX_TOL, half
