"""GPU parity of FC2's data gradient with the fused SwiGLU backward
(pt_grouped_gemm_dgrad_swiglu) against the oracle, through the C ABI:
ragged sizes spanning several tiles, both weight layouts, both tile orders,
an exact case, the empty batch, and sampled rows at the expert-MLP shape
(256 experts, 49152 rows, I = 2048, H = 4096)."""
import numpy as np
import pytest
import torch

import moe_expert_grouped_gemm_amd as ptm
from moe_expert_grouped_gemm_amd import synth
from util import (BF16_TOL, SCHEDS, bits16, bf16_values, dev_i64, floored_rel_err, group_of_rows,
                  make_ws, per_group_max)

pytestmark = pytest.mark.gpu

GUARD = 3
NAN16 = 0x7FC1

CASES = [
    # (name, lens, K = I, N = H)
    ("tiny", [91, 73, 92, 0], 128, 256),
    ("ragged", [0, 1, 130, 0, 257, 64, 33], 200, 208),
    ("one_expert", [300], 264, 144),
    ("many_small", [3, 0, 0, 5, 1, 2, 0, 7, 129, 4, 0, 1], 96, 80),
]


def run(dev, dy, b, c, lens, N, K, trans_b, ws=None):
    M, G = dy.shape[0], len(lens)
    buf = torch.empty((M + 2 * GUARD, 2 * K), dtype=torch.bfloat16, device=dev)
    buf.view(torch.int16).fill_(NAN16)
    dc = buf[GUARD:GUARD + M]
    ptm.pt_grouped_gemm_dgrad_swiglu(dy, b, c, dc, dev_i64(lens, dev), None, G, M, N, K, trans_b, workspace=ws)
    torch.cuda.synchronize()
    assert (bits16(buf[:GUARD]) == NAN16).all() and (bits16(buf[GUARD + M:]) == NAN16).all(), "guard rows written"
    return bits16(dc)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("trans_b", [0, 1])
@pytest.mark.parametrize("sched", SCHEDS)
def test_dgrad_swiglu_random_vs_oracle(orc, dev, case, trans_b, sched):
    name, lens, K, N = case
    lens = np.array(lens, np.int64)
    M, G = int(lens.sum()), len(lens)
    print(f"dgrad_swiglu case={name} trans_b={trans_b} sched={sched} M={M} K={K} N={N}", flush=True)
    dy = synth.randn_bf16((M, N), seed=102, std=1e-2, device=dev)
    b = synth.randn_bf16((G, K, N), seed=103, std=N ** -0.5, device=dev)
    c = synth.randn_bf16((M, 2 * K), seed=104, std=2.0, device=dev)      # gates across silu's range
    bb = b.transpose(1, 2).contiguous() if trans_b else b
    got = run(dev, dy, bb, c, lens, N, K, trans_b, ws=make_ws(dev, sched))
    rows = np.arange(M)
    ref = orc.dgrad_swiglu_rows(bits16(dy), bits16(bb), bits16(c), lens, N, K, trans_b, rows)
    grp = group_of_rows(lens, rows)
    for half in (slice(0, K), slice(K, 2 * K)):                          # d gate, d up
        err = per_group_max(floored_rel_err, bf16_values(got[:, half]), ref["exact"][:, half], grp)
        assert err <= BF16_TOL, (half, err)


def test_dgrad_swiglu_zero_gates_bit_exact(orc, dev):
    # Integer dY and B make dH exact; with every gate 0, s = 1/2 exactly, so
    # d gate = bf16(dH * u / 2) and d up = 0 leave no rounding to the exp.
    lens = np.array([0, 33, 1, 200], np.int64)
    K, N = 120, 144
    M, G = int(lens.sum()), len(lens)
    dy = synth.integer_bf16((M, N), seed=14, device=dev)
    b = synth.integer_bf16((G, K, N), seed=15, device=dev)
    c = synth.randn_bf16((M, 2 * K), seed=16, std=1.0, device=dev)
    c[:, :K] = 0
    for trans_b in (0, 1):
        bb = b.transpose(1, 2).contiguous() if trans_b else b
        got = run(dev, dy, bb, c, lens, N, K, trans_b)
        ref = orc.dgrad_swiglu_rows(bits16(dy), bits16(bb), bits16(c), lens, N, K, trans_b, np.arange(M))
        assert (got == ref["bf16"]).all()
        assert (bf16_values(got[:, K:]) == 0).all()


def test_dgrad_swiglu_matches_dgrad_then_oracle_backward(orc, dev):
    # The fused epilogue starts from the same bf16 dH that pt_grouped_gemm_dgrad
    # stores: feeding that dH to the oracle's backward must agree to rounding.
    lens = np.array([40, 0, 300, 17], np.int64)
    K, N = 256, 192
    M, G = int(lens.sum()), len(lens)
    dy = synth.randn_bf16((M, N), seed=21, std=1e-2, device=dev)
    b = synth.randn_bf16((G, K, N), seed=22, std=N ** -0.5, device=dev)
    c = synth.randn_bf16((M, 2 * K), seed=23, std=2.0, device=dev)
    dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    ptm.pt_grouped_gemm_dgrad(dy, None, b, None, dx, dev_i64(lens, dev), None, G, M, N, K, ptm.PT_BF16, 0)
    got = run(dev, dy, b, c, lens, N, K, 0)
    ref = orc.swiglu_bwd(bf16_values(bits16(dx)), bf16_values(bits16(c)))
    assert floored_rel_err(bf16_values(got), ref) <= BF16_TOL


def test_dgrad_swiglu_empty_batch_and_errors(dev):
    lens = np.zeros(3, np.int64)
    dy = torch.empty((0, 64), dtype=torch.bfloat16, device=dev)
    b = torch.empty((3, 64, 64), dtype=torch.bfloat16, device=dev)
    c = torch.empty((0, 128), dtype=torch.bfloat16, device=dev)
    dc = torch.empty((0, 128), dtype=torch.bfloat16, device=dev)
    ptm.pt_grouped_gemm_dgrad_swiglu(dy, b, c, dc, dev_i64(lens, dev), None, 3, 0, 64, 64, 0)
    torch.cuda.synchronize()
    L = ptm.load()
    lens1 = dev_i64(np.array([8], np.int64), dev)
    t = torch.zeros((8, 64), dtype=torch.bfloat16, device=dev)
    w = torch.zeros((1, 64, 64), dtype=torch.bfloat16, device=dev)
    cc = torch.zeros((8, 128), dtype=torch.bfloat16, device=dev)
    st = torch.cuda.current_stream().cuda_stream
    # a missing saved FC1 output, an odd K, and a bad layout flag are refused
    assert L.pt_grouped_gemm_dgrad_swiglu(t.data_ptr(), None, w.data_ptr(), None, None, cc.data_ptr(),
                                          lens1.data_ptr(), None, 1, 8, 64, 64, ptm.PT_BF16, 0, 0.0, None, 0, st) == 1
    assert L.pt_grouped_gemm_dgrad_swiglu(t.data_ptr(), None, w.data_ptr(), None, cc.data_ptr(), cc.data_ptr(),
                                          lens1.data_ptr(), None, 1, 8, 64, 60, ptm.PT_BF16, 0, 0.0, None, 0, st) == 2
    assert L.pt_grouped_gemm_dgrad_swiglu(t.data_ptr(), None, w.data_ptr(), None, cc.data_ptr(), cc.data_ptr(),
                                          lens1.data_ptr(), None, 1, 8, 64, 64, ptm.PT_BF16, 2, 0.0, None, 0, st) == 1
    # BF16 takes no scales; the low-precision dtypes need the [G, K, N] cache (trans_b = 0)
    assert L.pt_grouped_gemm_dgrad_swiglu(t.data_ptr(), t.data_ptr(), w.data_ptr(), None, cc.data_ptr(),
                                          cc.data_ptr(), lens1.data_ptr(), None, 1, 8, 64, 64, ptm.PT_BF16, 0, 0.0,
                                          None, 0, st) == 1
    assert L.pt_grouped_gemm_dgrad_swiglu(t.data_ptr(), t.data_ptr(), w.data_ptr(), t.data_ptr(), cc.data_ptr(),
                                          cc.data_ptr(), lens1.data_ptr(), None, 1, 8, 64, 64, ptm.PT_MXFP8_E4M3, 1,
                                          0.0, None, 0, st) == 2


def test_dgrad_swiglu_mlp_shape_sampled(orc, dev):
    # FC2's backward at the expert-MLP shape: 256 experts, 49152 rows,
    # I = 2048 (K here), H = 4096 (N), weights [G, I, H]; sampled rows of a
    # seeded subset of experts against the oracle on a compact sub-batch.
    lens = synth.lens_topk_gaussian(8192, 256, 6, seed=1)
    G, M, K, N = 256, int(lens.sum()), 2048, 4096
    offs = synth.offsets(lens)
    dy = synth.randn_bf16((M, N), seed=111, std=1e-2, device=dev)
    b = synth.randn_bf16((G, K, N), seed=112, std=N ** -0.5, device=dev)
    c = synth.randn_bf16((M, 2 * K), seed=113, std=2.0, device=dev)
    dc = torch.empty((M, 2 * K), dtype=torch.bfloat16, device=dev)
    ptm.pt_grouped_gemm_dgrad_swiglu(dy, b, c, dc, dev_i64(lens, dev), None, G, M, N, K, 0,
                                     workspace=make_ws(dev, "queue"))
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    nz = np.nonzero(lens)[0]
    experts = sorted(set(rng.choice(nz, size=10, replace=False).tolist()) | {int(nz[np.argmax(lens[nz])])})
    rows = [np.unique(np.concatenate([[offs[g], offs[g + 1] - 1], rng.integers(offs[g], offs[g + 1], size=3)]))
            for g in experts]
    local = np.array([r.size for r in rows], np.int64)
    allr = torch.as_tensor(np.concatenate(rows), device=dev)
    ref = orc.dgrad_swiglu_rows(bits16(dy[allr]), bits16(b[torch.as_tensor(experts, device=dev)]),
                                bits16(c[allr]), local, N, K, 0, np.arange(local.sum()))
    got = bf16_values(bits16(dc[allr]))
    start = 0
    for g, r in zip(experts, rows):
        sl = slice(start, start + r.size)
        assert floored_rel_err(got[sl, :K], ref["exact"][sl, :K]) <= BF16_TOL, g
        assert floored_rel_err(got[sl, K:], ref["exact"][sl, K:]) <= BF16_TOL, g
        start += r.size
