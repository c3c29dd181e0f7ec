"""GPU checks of FC1 with the SwiGLU epilogue that also keeps FC1's output
(pt_grouped_gemm_fwd_swiglu_save), through the C ABI: both outputs
bit-identical to the single-epilogue calls (PT_EPI_NONE and PT_EPI_SWIGLU,
which the other tests hold to the oracle), both weight layouts and tile
orders, with and without the clamp, guard rows, refusals, and the oracle at
the expert-MLP shape on sampled rows."""
import numpy as np
import pytest
import torch

import moe_expert_grouped_gemm_amd as ptm
from moe_expert_grouped_gemm_amd import synth
from util import BF16_TOL, SCHEDS, bf16_values, bits16, dev_i64, floored_rel_err, make_ws

pytestmark = pytest.mark.gpu

GUARD = 8
NAN16 = 0x7FC1


def guarded(dev, rows, cols):
    buf = torch.empty((rows + 2 * GUARD, cols), dtype=torch.bfloat16, device=dev)
    buf.view(torch.int16).fill_(NAN16)
    return buf, buf[GUARD:GUARD + rows]


@pytest.mark.parametrize("limit", [0.0, 1.5], ids=["plain", "clamped"])
@pytest.mark.parametrize("trans_b", [0, 1])
@pytest.mark.parametrize("sched", SCHEDS)
def test_save_equals_single_epilogues(dev, trans_b, sched, limit):
    lens = np.array([0, 1, 130, 0, 257, 64, 33], np.int64)
    M, G, K, N = int(lens.sum()), len(lens), 200, 512
    print(f"swiglu save trans_b={trans_b} sched={sched} limit={limit}", flush=True)
    a = synth.randn_bf16((M, K), seed=160, device=dev)
    b = synth.randn_bf16((G, N, K) if trans_b else (G, K, N), seed=161, std=2.0 * K ** -0.5, device=dev)
    lens_d = dev_i64(lens, dev)
    ws = make_ws(dev, sched)
    hb, h = guarded(dev, M, N // 2)
    cb, c = guarded(dev, M, N)
    ptm.pt_grouped_gemm_fwd_swiglu_save(a, None, b, None, h, c, lens_d, None, G, M, N, K, ptm.PT_BF16, trans_b,
                                        workspace=ws, swiglu_limit=limit)
    c_ref = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    h_ref = torch.empty((M, N // 2), dtype=torch.bfloat16, device=dev)
    ptm.pt_grouped_gemm_fwd(a, None, b, None, c_ref, None, lens_d, None, G, M, N, K, ptm.PT_BF16, trans_b,
                            ptm.PT_EPI_NONE, workspace=ws)
    ptm.pt_grouped_gemm_fwd(a, None, b, None, h_ref, None, lens_d, None, G, M, N, K, ptm.PT_BF16, trans_b,
                            ptm.PT_EPI_SWIGLU, workspace=ws, swiglu_limit=limit)
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int16), c_ref.view(torch.int16))
    assert torch.equal(h.view(torch.int16), h_ref.view(torch.int16))
    for buf in (hb, cb):
        raw = bits16(buf)
        assert (raw[:GUARD] == NAN16).all() and (raw[GUARD + M:] == NAN16).all(), "guard rows written"


def test_save_refusals_and_empty_batch(dev):
    L = ptm.load()
    st = torch.cuda.current_stream().cuda_stream
    lens = dev_i64(np.array([8], np.int64), dev)
    a = torch.zeros((8, 64), dtype=torch.bfloat16, device=dev)
    b = torch.zeros((1, 64, 64), dtype=torch.bfloat16, device=dev)
    h = torch.zeros((8, 32), dtype=torch.bfloat16, device=dev)
    c = torch.zeros((8, 64), dtype=torch.bfloat16, device=dev)
    args = lambda N=64, tb=0, cc=c.data_ptr(), dt=ptm.PT_BF16: (a.data_ptr(), None, b.data_ptr(), None, h.data_ptr(),
                                                                cc, lens.data_ptr(), None, 1, 8, N, 64, dt, tb, 0.0,
                                                                None, 0, st)
    assert L.pt_grouped_gemm_fwd_swiglu_save(*args(cc=None)) == 1            # no place for FC1's output
    assert L.pt_grouped_gemm_fwd_swiglu_save(*args(N=56)) == 2               # N % 16
    assert L.pt_grouped_gemm_fwd_swiglu_save(*args(tb=2)) == 1
    assert L.pt_grouped_gemm_fwd_swiglu_save(*args(cc=c.data_ptr() + 2)) == 3
    assert L.pt_grouped_gemm_fwd_swiglu_save(*args(dt=ptm.PT_MXFP8_E4M3, tb=0)) == 2      # MX codes need [G, N, K]
    assert L.pt_grouped_gemm_fwd_swiglu_save(*args(dt=9)) == 2
    zl = dev_i64(np.zeros(3, np.int64), dev)
    ptm.pt_grouped_gemm_fwd_swiglu_save(a[:0], None, b, None, h[:0], c[:0], zl, None, 3, 0, 64, 64, ptm.PT_BF16, 0)
    torch.cuda.synchronize()


def test_save_mlp_shape_sampled(orc, dev):
    # FC1 at the expert-MLP shape (256 experts, 49152 rows, H = 4096,
    # 2I = 4096): sampled rows of both outputs against the oracle
    lens = synth.lens_topk_gaussian(8192, 256, 6, seed=1)
    G, M, K, N = 256, int(lens.sum()), 4096, 4096
    a = synth.randn_bf16((M, K), seed=101, std=K ** -0.5, device=dev)
    b = synth.randn_bf16((G, K, N), seed=1101, std=K ** -0.5, device=dev)
    h = torch.empty((M, N // 2), dtype=torch.bfloat16, device=dev)
    c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ptm.pt_grouped_gemm_fwd_swiglu_save(a, None, b, None, h, c, dev_i64(lens, dev), None, G, M, N, K, ptm.PT_BF16, 0,
                                        workspace=make_ws(dev, "queue"))
    torch.cuda.synchronize()
    offs = synth.offsets(lens)
    rng = np.random.default_rng(19)
    nz = np.nonzero(lens)[0]
    experts = sorted(set(rng.choice(nz, size=6, replace=False).tolist()) | {int(nz[np.argmax(lens[nz])])})
    rows = np.unique(np.concatenate([[offs[g], offs[g + 1] - 1, rng.integers(offs[g], offs[g + 1])] for g in experts]))
    ra = bits16(a[torch.as_tensor(rows, device=dev)])
    local = np.array([np.sum((rows >= offs[g]) & (rows < offs[g + 1])) for g in experts], np.int64)
    bsub = bits16(b[torch.as_tensor(experts, device=dev)])
    ref = orc.grouped_fwd(orc.BF16, ra, None, bsub, None, local, N, K, 0, orc.EPI_NONE, np.arange(rows.size))
    refh = orc.grouped_fwd(orc.BF16, ra, None, bsub, None, local, N, K, 0, orc.EPI_SWIGLU, np.arange(rows.size))
    idx = torch.as_tensor(rows, device=dev)
    assert floored_rel_err(bf16_values(bits16(c[idx])), ref["exact"]) <= BF16_TOL
    assert floored_rel_err(bf16_values(bits16(h[idx])), refh["exact"]) <= BF16_TOL



@pytest.mark.parametrize("dtype,name", [(ptm.PT_MXFP8_E4M3, "e4m3"), (ptm.PT_MXFP4_E2M1, "e2m1"),
                                        (ptm.PT_FP8_E4M3, "fp8"), (ptm.PT_FP8_E4M3_ROWWISE, "fp8rows")],
                         ids=["mxfp8", "mxfp4", "fp8", "fp8_rowwise"])
@pytest.mark.parametrize("sched", ["static", "swz"])
@pytest.mark.parametrize("K", [512, 320])
def test_save_low_precision_equals_single_epilogues(dev, dtype, name, sched, K):
    # K = 320 leaves a partial 256-deep MXFP4 step, which the save epilogue
    # serves only through the swizzled-scale kernel; every kernel
    # configuration is forced in turn (the save falls back to the
    # configurations it has)
    lens = np.array([0, 1, 130, 0, 257, 64, 33], np.int64)
    M, G, N = int(lens.sum()), len(lens), 256
    if dtype in (ptm.PT_MXFP8_E4M3, ptm.PT_MXFP4_E2M1):
        aq, as_ = synth.random_mx_codes(M, K, name, seed=162, device=dev, scale_lo=122, scale_hi=125)
        bq, bs = synth.random_mx_codes(G * N, K, name, seed=163, device=dev, scale_lo=116, scale_hi=119)
    else:
        g = torch.Generator(device=dev)
        g.manual_seed(164)
        aq = torch.randint(0, 126, (M, K), generator=g, device=dev, dtype=torch.int32).to(torch.uint8)
        bq = torch.randint(0, 126, (G * N, K), generator=g, device=dev, dtype=torch.int32).to(torch.uint8)
        rows_a, rows_b = (M, G * N) if dtype == ptm.PT_FP8_E4M3_ROWWISE else (1, G)
        as_ = torch.rand((rows_a,), generator=g, device=dev).mul_(1e-2).add_(1e-3)
        bs = torch.rand((rows_b,), generator=g, device=dev).mul_(1e-2).add_(1e-3)
    ws = make_ws(dev, sched, G, M, N, K, dtype if dtype in (ptm.PT_MXFP8_E4M3, ptm.PT_MXFP4_E2M1) else ptm.PT_BF16)
    lens_d = dev_i64(lens, dev)
    try:
        for cfg in (ptm.PT_CONFIG_RULES, 0, 1, 2, 3):
            ptm.pt_set_gemm_config(cfg)
            print(f"swiglu save dtype={name} sched={sched} K={K} cfg={cfg}", flush=True)
            h = torch.empty((M, N // 2), dtype=torch.bfloat16, device=dev)
            c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            if dtype == ptm.PT_MXFP4_E2M1 and K % 256 and ws is None:
                with pytest.raises(ptm.PtggError) as e:
                    ptm.pt_grouped_gemm_fwd_swiglu_save(aq, as_, bq, bs, h, c, lens_d, None, G, M, N, K, dtype, 1,
                                                        workspace=ws, swiglu_limit=4.0)
                assert e.value.status == 2          # PT_ERR_UNSUPPORTED
                continue
            ptm.pt_grouped_gemm_fwd_swiglu_save(aq, as_, bq, bs, h, c, lens_d, None, G, M, N, K, dtype, 1,
                                                workspace=ws, swiglu_limit=4.0)
            c_ref = torch.empty_like(c)
            h_ref = torch.empty_like(h)
            ptm.pt_grouped_gemm_fwd(aq, as_, bq, bs, c_ref, None, lens_d, None, G, M, N, K, dtype, 1,
                                    ptm.PT_EPI_NONE, workspace=ws)
            ptm.pt_grouped_gemm_fwd(aq, as_, bq, bs, h_ref, None, lens_d, None, G, M, N, K, dtype, 1,
                                    ptm.PT_EPI_SWIGLU, workspace=ws, swiglu_limit=4.0)
            torch.cuda.synchronize()
            assert torch.equal(c.view(torch.int16), c_ref.view(torch.int16))
            assert torch.equal(h.view(torch.int16), h_ref.view(torch.int16))
    finally:
        ptm.pt_set_gemm_config(ptm.PT_CONFIG_RULES)
