"""Regression test of the MX grouped GEMM forward on experts small enough to
run as 128-row tiles (three-slot ring, per-lane scale loads): every output
element against the oracle on the same MX bytes, and bit-identical results
over repeated calls, in every tile order and scale layout.

The k-loop's waits count its vector-memory operations exactly; a scale load
the MFMAs never read (a 128-row tile uses one A row per lane) used to be
dropped by the compiler, so a stage could be read while its last direct load
was still landing.  That showed as groups of 8 output columns of a 128-row
tile taking wrong values in some calls and not in others.  The element-wise
check (the BF16 tolerance: operands are exact, only fp32 sums and the bf16
output round) and the repeat check both catch it."""
import numpy as np
import pytest
import torch

import moe_expert_grouped_gemm_amd as ptm
from moe_expert_grouped_gemm_amd import synth
from util import BF16_TOL, MX_SCHEDS, bf16_values, bits16, dev_i64, floored_rel_err, make_ws, u8

pytestmark = pytest.mark.gpu

FMTS = [(ptm.PT_MXFP8_E4M3, 1, "e4m3"), (ptm.PT_MXFP4_E2M1, 2, "e2m1")]
# mostly experts of at most 128 rows (128-row tiles), a few longer ones whose
# last row block is short, and empty ones
LENS = np.array([5, 128, 0, 33, 1, 64, 100, 17, 290, 77, 0, 127, 3, 129, 60, 45, 256, 9, 120, 31], np.int64)
K, N = 2048, 512


@pytest.fixture(scope="module", params=FMTS, ids=[f[2] for f in FMTS])
def case(request, orc, dev):
    fmt, ofmt, name = request.param
    G, M = len(LENS), int(LENS.sum())
    aq, as_ = synth.random_mx_codes(M, K, name, seed=301, device=dev)
    bq, bs = synth.random_mx_codes(G * N, K, name, seed=302, device=dev)
    refs = {}
    for epi, oepi in ((ptm.PT_EPI_NONE, orc.EPI_NONE), (ptm.PT_EPI_SWIGLU, orc.EPI_SWIGLU)):
        refs[epi] = orc.grouped_fwd(ofmt, u8(aq), u8(as_), u8(bq).reshape(G, N, -1), u8(bs).reshape(G, N, -1),
                                    LENS, N, K, 1, oepi, np.arange(M))["exact"]
    return fmt, name, aq, as_, bq, bs, refs


@pytest.mark.parametrize("sched", MX_SCHEDS)
@pytest.mark.parametrize("epi", [ptm.PT_EPI_NONE, ptm.PT_EPI_SWIGLU], ids=["none", "swiglu"])
def test_small_experts_every_element_and_repeatable(dev, case, sched, epi):
    fmt, name, aq, as_, bq, bs, refs = case
    G, M = len(LENS), int(LENS.sum())
    nout = N if epi == ptm.PT_EPI_NONE else N // 2
    print(f"mx small experts {name} sched={sched} epi={epi}", flush=True)
    ws = make_ws(dev, sched, G, M, N, K, fmt)
    lens = dev_i64(LENS, dev)
    outs = []
    for _ in range(4):
        out = torch.full((M, nout), float("nan"), dtype=torch.bfloat16, device=dev)
        ptm.pt_grouped_gemm_fwd(aq, as_, bq, bs, out, None, lens, None, G, M, N, K, fmt, 1, epi, workspace=ws)
        torch.cuda.synchronize()
        outs.append(bits16(out))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0]), "results differ between identical calls"
    got = bf16_values(outs[0])
    ref = refs[epi]
    offs = synth.offsets(LENS)
    for g in range(G):
        r0, r1 = int(offs[g]), int(offs[g + 1])
        if r1 > r0:
            assert floored_rel_err(got[r0:r1], ref[r0:r1]) <= BF16_TOL, g
