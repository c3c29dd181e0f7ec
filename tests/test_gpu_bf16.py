"""GPU parity of the BF16 grouped GEMM (forward, SwiGLU epilogue, dgrad,
wgrad) against the oracle, through the C ABI.  Sizes span several tiles,
ragged tails in every dimension and empty experts."""
import numpy as np
import pytest
import torch

import moe_expert_grouped_gemm_amd as ptm
from moe_expert_grouped_gemm_amd import synth
from util import (BF16_TOL, SCHEDS, bits16, bf16_values, dev_i64, floored_rel_err, group_of_rows,
                  make_ws, per_group_max)

pytestmark = pytest.mark.gpu

GUARD = 3            # guard rows on each side of every output
NAN16 = 0x7FC1       # bf16 NaN pattern the kernels never write


CASES = [
    # (name, lens, K, N)
    ("tiny_4_experts", None, 128, 256),
    ("ragged", [0, 1, 130, 0, 257, 64, 33], 200, 208),
    ("one_expert", [300], 64, 144),
    ("many_small", [3, 0, 0, 5, 1, 2, 0, 7, 129, 4, 0, 1], 96, 80),
]


def lens_of(case):
    name, lens, K, N = case
    if lens is None:
        return synth.lens_multinomial(256, 4, seed=0, n_empty=1)
    return np.array(lens, np.int64)


def guarded(rows, cols, dtype, dev, fill):
    buf = torch.empty((rows + 2 * GUARD, cols), dtype=dtype, device=dev)
    buf.view(torch.int16 if dtype == torch.bfloat16 else dtype).fill_(fill)
    return buf, buf[GUARD:GUARD + rows]


def check_guards(buf, rows, fill_bits):
    head = bits16(buf[:GUARD]) if buf.dtype == torch.bfloat16 else None
    tail = bits16(buf[GUARD + rows:]) if buf.dtype == torch.bfloat16 else None
    assert (head == fill_bits).all() and (tail == fill_bits).all(), "guard rows overwritten"


def fwd(dev, a, b, lens, N, K, trans_b, epi, offs=None, ws=None):
    M, G = a.shape[0], len(lens)
    cols = N if epi == ptm.PT_EPI_NONE else N // 2
    buf, out = guarded(M, cols, torch.bfloat16, dev, NAN16)
    lens_d = dev_i64(lens, dev)
    offs_d = None if offs is None else dev_i64(offs, dev)
    ptm.pt_grouped_gemm_fwd(a, None, b, None, out, None, lens_d, offs_d, G, M, N, K,
                            ptm.PT_BF16, trans_b, epi, workspace=ws)
    torch.cuda.synchronize()
    check_guards(buf, M, NAN16)
    return bits16(out)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("trans_b", [0, 1])
@pytest.mark.parametrize("epi", [ptm.PT_EPI_NONE, ptm.PT_EPI_SWIGLU])
@pytest.mark.parametrize("sched", SCHEDS)
def test_fwd_random_vs_oracle(orc, dev, case, trans_b, epi, sched):
    lens = lens_of(case)
    _, _, K, N = case
    M, G = int(lens.sum()), len(lens)
    print(f"fwd case={case[0]} trans_b={trans_b} epi={epi} sched={sched} M={M} G={G} K={K} N={N}", flush=True)
    a = synth.randn_bf16((M, K), seed=100, std=K ** -0.5, device=dev)
    b = synth.randn_bf16((G, K, N), seed=101, std=K ** -0.5, device=dev)
    bb = b.transpose(1, 2).contiguous() if trans_b else b
    got = bf16_values(fwd(dev, a, bb, lens, N, K, trans_b, epi, ws=make_ws(dev, sched)))
    rows = np.arange(M)
    ref = orc.grouped_fwd(orc.BF16, bits16(a), None, bits16(bb), None, lens, N, K, trans_b,
                          epi, rows)["exact"]
    err = per_group_max(floored_rel_err, got, ref, group_of_rows(lens, rows))
    assert err <= BF16_TOL, err


@pytest.mark.parametrize("trans_b", [0, 1])
def test_fwd_integer_inputs_bit_exact(orc, dev, trans_b):
    lens = np.array([17, 0, 140, 3, 0, 99], np.int64)
    K, N = 136, 200
    M, G = int(lens.sum()), len(lens)
    a = synth.integer_bf16((M, K), seed=5, device=dev)
    b = synth.integer_bf16((G, K, N), seed=6, device=dev)
    bb = b.transpose(1, 2).contiguous() if trans_b else b
    got = fwd(dev, a, bb, lens, N, K, trans_b, ptm.PT_EPI_NONE)
    ref = orc.grouped_fwd(orc.BF16, bits16(a), None, bits16(bb), None, lens, N, K, trans_b,
                          orc.EPI_NONE, np.arange(M))["bf16"]
    assert (got == ref).all()


def test_fwd_scaled_identity_maps_rows_to_experts(orc, dev):
    # B_g = 2^(g-3) I makes every output row its A row times its expert's factor
    lens = np.array([40, 0, 129, 1, 77, 0, 256, 5], np.int64)
    K = N = 128
    M, G = int(lens.sum()), len(lens)
    a = synth.randn_bf16((M, K), seed=7, device=dev)
    eye = torch.eye(K, device=dev, dtype=torch.float32)
    b = torch.stack([eye * 2.0 ** (g - 3) for g in range(G)]).to(torch.bfloat16)
    for trans_b in (0, 1):
        got = bf16_values(fwd(dev, a, b, lens, N, K, trans_b, ptm.PT_EPI_NONE))
        expert = np.repeat(np.arange(G), lens)
        want = bf16_values(bits16(a)) * (2.0 ** (expert - 3))[:, None]
        assert (got == want).all()


def test_fwd_explicit_offsets_equal_derived(orc, dev):
    lens = np.array([5, 0, 300, 2, 0, 61], np.int64)
    K, N = 64, 128
    M, G = int(lens.sum()), len(lens)
    a = synth.randn_bf16((M, K), seed=8, device=dev)
    b = synth.randn_bf16((G, K, N), seed=9, device=dev)
    offs = synth.offsets(lens)
    x = fwd(dev, a, b, lens, N, K, 0, ptm.PT_EPI_NONE)
    y = fwd(dev, a, b, lens, N, K, 0, ptm.PT_EPI_NONE, offs=offs)
    assert (x == y).all()


def test_fwd_deterministic(dev):
    lens = synth.lens_topk_gaussian(512, 16, 4, seed=11)
    K, N = 256, 384
    M, G = int(lens.sum()), len(lens)
    a = synth.randn_bf16((M, K), seed=12, device=dev)
    b = synth.randn_bf16((G, K, N), seed=13, device=dev)
    x = fwd(dev, a, b, lens, N, K, 0, ptm.PT_EPI_SWIGLU)
    y = fwd(dev, a, b, lens, N, K, 0, ptm.PT_EPI_SWIGLU)
    assert (x == y).all()


# ------------------------------------------------------------------ dgrad
@pytest.mark.parametrize("trans_b", [0, 1])
@pytest.mark.parametrize("case", CASES[:3], ids=[c[0] for c in CASES[:3]])
@pytest.mark.parametrize("sched", SCHEDS)
def test_dgrad_random_vs_oracle(orc, dev, case, trans_b, sched):
    lens = lens_of(case)
    _, _, K, N = case
    M, G = int(lens.sum()), len(lens)
    print(f"dgrad case={case[0]} trans_b={trans_b} sched={sched} M={M} K={K} N={N}", flush=True)
    dy = synth.randn_bf16((M, N), seed=102, std=1e-2, device=dev)
    b = synth.randn_bf16((G, K, N), seed=103, std=K ** -0.5, device=dev)
    bb = b.transpose(1, 2).contiguous() if trans_b else b
    buf, dx = guarded(M, K, torch.bfloat16, dev, NAN16)
    ptm.pt_grouped_gemm_dgrad(dy, None, bb, None, dx, dev_i64(lens, dev), None, G, M, N, K,
                              ptm.PT_BF16, trans_b, workspace=make_ws(dev, sched))
    torch.cuda.synchronize()
    check_guards(buf, M, NAN16)
    rows = np.arange(M)
    ref = orc.dgrad_rows(bits16(dy), bits16(bb), lens, N, K, trans_b, rows)
    err = per_group_max(floored_rel_err, bf16_values(bits16(dx)), ref, group_of_rows(lens, rows))
    assert err <= BF16_TOL, err


def test_dgrad_integer_bit_exact(orc, dev):
    lens = np.array([0, 33, 1, 200], np.int64)
    K, N = 120, 144
    M, G = int(lens.sum()), len(lens)
    dy = synth.integer_bf16((M, N), seed=14, device=dev)
    b = synth.integer_bf16((G, K, N), seed=15, device=dev)
    for trans_b in (0, 1):
        bb = b.transpose(1, 2).contiguous() if trans_b else b
        dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        ptm.pt_grouped_gemm_dgrad(dy, None, bb, None, dx, dev_i64(lens, dev), None, G, M, N, K,
                                  ptm.PT_BF16, trans_b)
        torch.cuda.synchronize()
        ref = orc.round_bf16(orc.dgrad_rows(bits16(dy), bits16(bb), lens, N, K, trans_b, np.arange(M)))
        assert (bits16(dx) == ref).all()


# ------------------------------------------------------------------ wgrad
def wgrad_run(dev, a, dy, lens, N, K, trans_out, accumulate, seed_mg=103, ws=None):
    M, G = a.shape[0], len(lens)
    shape = (G, N, K) if trans_out else (G, K, N)
    g = torch.Generator(device=dev)
    g.manual_seed(seed_mg)
    mg = (torch.randn(shape, generator=g, device=dev) * 1e-3).float()
    before = mg.clone()
    ptm.pt_grouped_gemm_wgrad(a, None, dy, None, mg, dev_i64(lens, dev), None, G, M, N, K,
                              ptm.PT_BF16, trans_out, accumulate, workspace=ws)
    torch.cuda.synchronize()
    return before.cpu().numpy(), mg.cpu().numpy()


@pytest.mark.parametrize("trans_out", [0, 1])
@pytest.mark.parametrize("accumulate", [1, 0])
@pytest.mark.parametrize("sched", SCHEDS)
def test_wgrad_vs_oracle(orc, dev, trans_out, accumulate, sched):
    lens = np.array([0, 70, 1, 0, 300, 129, 0], np.int64)
    K, N = 200, 136
    M, G = int(lens.sum()), len(lens)
    print(f"wgrad trans_out={trans_out} acc={accumulate} sched={sched}", flush=True)
    a = synth.randn_bf16((M, K), seed=101, std=K ** -0.5, device=dev)
    dy = synth.randn_bf16((M, N), seed=102, std=1e-2, device=dev)
    before, after = wgrad_run(dev, a, dy, lens, N, K, trans_out, accumulate, ws=make_ws(dev, sched))
    gs = np.repeat(np.arange(G), K)
    ks = np.tile(np.arange(K), G)
    D = orc.wgrad_rows(bits16(a), bits16(dy), lens, N, K, gs, ks).reshape(G, K, N)
    if trans_out:
        D = D.transpose(0, 2, 1)
    for g in range(G):
        if lens[g] == 0:
            if accumulate:
                assert (after[g] == before[g]).all(), "empty expert touched"
            else:
                assert (after[g] == 0).all()
            continue
        inc = after[g].astype(np.float64) - (before[g] if accumulate else 0.0)
        assert floored_rel_err(inc, D[g]) <= BF16_TOL, g


def test_wgrad_integer_bit_exact(orc, dev):
    lens = np.array([9, 0, 150, 64], np.int64)
    K, N = 72, 136
    M, G = int(lens.sum()), len(lens)
    a = synth.integer_bf16((M, K), seed=16, device=dev)
    dy = synth.integer_bf16((M, N), seed=17, device=dev)
    mg = synth.integer_bf16((G, K, N), seed=18, lo=-100, hi=100, device=dev).float()
    before = mg.cpu().numpy()
    ptm.pt_grouped_gemm_wgrad(a, None, dy, None, mg, dev_i64(lens, dev), None, G, M, N, K,
                              ptm.PT_BF16, 0, 1)
    torch.cuda.synchronize()
    gs = np.repeat(np.arange(G), K)
    ks = np.tile(np.arange(K), G)
    D = orc.wgrad_rows(bits16(a), bits16(dy), lens, N, K, gs, ks).reshape(G, K, N)
    want = orc.wgrad_accumulate(before, D, accumulate=True)
    for g in range(G):
        if lens[g] == 0:
            want[g] = before[g]
    assert (mg.cpu().numpy() == want).all()


def test_wgrad_deterministic(dev):
    lens = np.array([0, 700, 3, 1500], np.int64)
    K, N = 128, 256
    M = int(lens.sum())
    a = synth.randn_bf16((M, K), seed=19, device=dev)
    dy = synth.randn_bf16((M, N), seed=20, device=dev)
    _, x = wgrad_run(dev, a, dy, lens, N, K, 0, 1)
    _, y = wgrad_run(dev, a, dy, lens, N, K, 0, 1)
    assert (x == y).all()


# ------------------------------------------------------------------ contract
def test_device_error_word_and_clamping(dev):
    # negative and oversized lengths are clamped on the device (no write
    # outside [0, M)) and reported in the workspace's error word
    K, N, M = 64, 128, 200
    a = synth.randn_bf16((M, K), seed=21, device=dev)
    b = synth.randn_bf16((3, K, N), seed=22, device=dev)
    ws = torch.zeros(64, dtype=torch.int32, device=dev)
    buf, out = guarded(M, N, torch.bfloat16, dev, NAN16)
    lens = dev_i64([100, -5, 400], dev)          # sums past M
    ptm.pt_grouped_gemm_fwd(a, None, b, None, out, None, lens, None, 3, M, N, K,
                            ptm.PT_BF16, 0, ptm.PT_EPI_NONE, workspace=ws)
    flags = ptm.pt_read_error_flags(ws)
    check_guards(buf, M, NAN16)
    assert flags & 1 and flags & 2
    ws.zero_()
    good = dev_i64([100, 0, 100], dev)
    ptm.pt_grouped_gemm_fwd(a, None, b, None, out, None, good, None, 3, M, N, K,
                            ptm.PT_BF16, 0, ptm.PT_EPI_NONE, workspace=ws)
    assert ptm.pt_read_error_flags(ws) == 0


def test_explicit_offsets_gaps_legal_overlaps_flagged(orc, dev):
    # explicit offsets with rows no expert owns: those rows stay unwritten and
    # no error bit is set; overlapping or out-of-order ranges, or offs[G] past
    # M, set bit 2
    K, N, M = 64, 128, 200
    a = synth.randn_bf16((M, K), seed=25, std=K ** -0.5, device=dev)
    b = synth.randn_bf16((3, K, N), seed=26, std=K ** -0.5, device=dev)
    lens = np.array([50, 0, 90], np.int64)
    offs = np.array([10, 70, 70, 190], np.int64)        # rows 0-9, 60-69 and 160-199 unowned
    ws = torch.zeros(64, dtype=torch.int32, device=dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    out.view(torch.int16).fill_(NAN16)
    ptm.pt_grouped_gemm_fwd(a, None, b, None, out, None, dev_i64(lens, dev), dev_i64(offs, dev), 3, M, N, K,
                            ptm.PT_BF16, 0, ptm.PT_EPI_NONE, workspace=ws)
    assert ptm.pt_read_error_flags(ws) == 0
    got = bits16(out)
    owned = np.concatenate([np.arange(offs[g], offs[g] + lens[g]) for g in range(3)])
    unowned = np.setdiff1d(np.arange(M), owned)
    assert (got[unowned] == NAN16).all()
    ref = orc.fwd_rows(orc.BF16, bits16(a)[owned], None, bits16(b), None, lens, N, K, 0, np.arange(owned.size))
    assert floored_rel_err(bf16_values(got[owned]), ref) <= BF16_TOL
    for bad_offs in ([10, 50, 70, 190], [70, 10, 10, 100], [10, 70, 70, 201]):
        ws.zero_()
        ptm.pt_grouped_gemm_fwd(a, None, b, None, out, None, dev_i64(lens, dev), dev_i64(bad_offs, dev), 3, M, N,
                                K, ptm.PT_BF16, 0, ptm.PT_EPI_NONE, workspace=ws)
        assert ptm.pt_read_error_flags(ws) & 4, bad_offs


def test_host_argument_errors(dev):
    K, N, M = 64, 128, 64
    a = synth.randn_bf16((M, K), seed=23, device=dev)
    b = synth.randn_bf16((2, K, N), seed=24, device=dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    lens = dev_i64([32, 32], dev)
    L = ptm.load()
    s = torch.cuda.current_stream().cuda_stream

    def call(**kw):
        args = dict(a=a.data_ptr(), a_scale=None, b=b.data_ptr(), b_scale=None, out=out.data_ptr(),
                    out_scale=None, lens=lens.data_ptr(), offs=None, G=2, M=M, N=N, K=K,
                    dtype=ptm.PT_BF16, trans_b=0, epi=ptm.PT_EPI_NONE)
        args.update(kw)
        return L.pt_grouped_gemm_fwd(args["a"], args["a_scale"], args["b"], args["b_scale"],
                                     args["out"], args["out_scale"], args["lens"], args["offs"],
                                     args["G"], args["M"], args["N"], args["K"], args["dtype"],
                                     args["trans_b"], args["epi"], 0.0, None, 0, s)

    assert call() == 0
    assert call(a=None) == 1
    assert call(lens=None) == 1
    assert call(G=0) == 1
    assert call(K=60) == 2                    # K % 8
    assert call(dtype=7) == 2
    assert call(epi=ptm.PT_EPI_SWIGLU_MXFP4) == 1   # no out_scale
    assert call(dtype=ptm.PT_MXFP8_E4M3, trans_b=0) == 2   # MX needs [G, N, K]
    assert call(a=a.data_ptr() + 2) == 3
    assert call(G=5000) == 2
    torch.cuda.synchronize()


# ------------------------------------------------------------------ tile queues
def test_queue_order_matches_static_many_tiles(dev):
    # ~1.2k forward tiles and 1k wgrad tiles over the persistent grid: every
    # workgroup takes several ids, every queue several chunks, and the queues
    # drain each other at the end.  Each tile is computed identically in either
    # order, so the results are bit-identical; a tile taken twice would
    # double-accumulate into main_grad, one never taken would keep its guard.
    lens = synth.lens_topk_gaussian(2400, 24, 6, seed=31)
    K, N = 64, 4096
    M, G = int(lens.sum()), len(lens)
    print(f"queue fwd M={M} G={G}", flush=True)
    a = synth.randn_bf16((M, K), seed=32, std=K ** -0.5, device=dev)
    b = synth.randn_bf16((G, K, N), seed=33, std=K ** -0.5, device=dev)
    ws = make_ws(dev, "queue")
    x = fwd(dev, a, b, lens, N, K, 0, ptm.PT_EPI_SWIGLU)
    y = fwd(dev, a, b, lens, N, K, 0, ptm.PT_EPI_SWIGLU, ws=ws)
    z = fwd(dev, a, b, lens, N, K, 0, ptm.PT_EPI_SWIGLU, ws=ws)      # same workspace again
    assert (x == y).all() and (x == z).all()
    # a smaller problem through the same workspace right after
    small = np.array([3, 0, 77], np.int64)
    a2 = a[:80].contiguous()
    x2 = fwd(dev, a2, b[:3].contiguous(), small, N, K, 1, ptm.PT_EPI_NONE)
    y2 = fwd(dev, a2, b[:3].contiguous(), small, N, K, 1, ptm.PT_EPI_NONE, ws=ws)
    assert (x2 == y2).all()

    wl = np.full(64, 40, np.int64)
    wl[[3, 17]] = 0
    Kw, Nw = 1024, 768
    Mw = int(wl.sum())
    print(f"queue wgrad M={Mw} G={len(wl)}", flush=True)
    aw = synth.randn_bf16((Mw, Kw), seed=34, std=Kw ** -0.5, device=dev)
    dyw = synth.randn_bf16((Mw, Nw), seed=35, std=1e-2, device=dev)
    _, p = wgrad_run(dev, aw, dyw, wl, Nw, Kw, 0, 1)
    _, q = wgrad_run(dev, aw, dyw, wl, Nw, Kw, 0, 1, ws=ws)
    assert (p == q).all()
