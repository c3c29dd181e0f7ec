"""Benchmark of the MoE expert grouped GEMM on one MI355X.

Headline (the JSON line's `value`): BF16 grouped GEMM forward of a
DeepSeek-V4-Flash-like MoE FC1 layer -- 256 experts, 8192 tokens routed top-6
(49152 rows, imbalanced seeded routing with empty and tiny experts),
hidden K = 4096, N = 4096 ([gate | up] for intermediate 2048), weights
[experts, K, N], fused SwiGLU epilogue to [49152, 2048] -- in TFLOP/s of
useful FLOPs (2 * sum(group_lens) * K * N per step).  A step is one call of
pt_grouped_gemm_fwd with inputs resident in HBM.

Every `per_config` launch is timed after a 512 MiB write that flushes the
MALL (outside the launch's event pair); the headline is timed back to back
and reported flushed as well (`kernel_ms_median_cache_flushed`).

`per_config` adds the other workloads (measured the same way, not part of
`value`): the tiny 4-expert case, BF16 dgrad and wgrad into an fp32
main_grad at the same shape, MXFP8 forward and its quantise kernel at a
GPT-OSS-20B-like shape, and the MXFP4 expert MLP (quantise -> FC1 + SwiGLU +
MXFP4 epilogue -> FC2).

`cpu_baseline` times the oracle (fp64 CPU reference) on a bounded sample of
the headline workload's rows on this host; its outputs also give a parity
check of the same GPU output.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import moe_expert_grouped_gemm_amd as ptm  # noqa: E402
from moe_expert_grouped_gemm_amd import synth  # noqa: E402

PEAK_TFLOPS = {"bf16": 2516.6, "mxfp8": 5033.2, "fp8": 5033.2, "mxfp4": 10066.3}   # dense MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "grouped-GEMM TFLOP/s (useful FLOPs) + % of dtype MFMA peak, BF16/MXFP8/MXFP4"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "moe_expert_grouped_gemm_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernels changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(kernel_key)
    if not ent or ent.get("src_hash") != kernel_source_hash():
        return None
    return ent.get("bytes_per_launch")


FLUSH_BYTES = 512 << 20       # twice the 256 MB MALL (the last-level cache in front of HBM)
FLUSH = [None]


# per_config rows -> the profiled kernels whose HBM bytes per launch (from the
# counter summaries in profiles/) make up that row's `traffic`
TRAFFIC_KEYS = {
    "cfg2_bf16_dgrad": ["cfg2_bf16_dgrad"],
    "cfg2_bf16_wgrad": ["cfg2_bf16_wgrad"],
    "cfg3_mxfp8_fwd": ["cfg3_mxfp8_fwd"],
    "cfg3_mxfp8_quantize_A": ["cfg3_mx_quantize_e4m3_A"],
    "cfg3_mxfp8_fwd_line_aligned": ["cfg3_mxfp8_fwd_line_aligned"],
    # A and dY each quantised along tokens and transposed (per-launch means), then the weight gradient
    "cfg3_mxfp8_wgrad": ["cfg3_mx_tokens_quant", "cfg3_mx_tokens_quant", "cfg3_mx_wgrad_transpose",
                         "cfg3_mx_wgrad_transpose", "cfg3_mxfp8_wgrad"],
    # the two-pass tensor quantise of A and dY, their transposes, the weight gradient
    "cfg3_fp8_tensor_wgrad": ["cfg3_fp8_wgrad_amax", "cfg3_fp8_wgrad_amax", "cfg3_fp8_wgrad_encode",
                              "cfg3_fp8_wgrad_encode", "cfg3_mx_wgrad_transpose", "cfg3_mx_wgrad_transpose",
                              "cfg3_fp8_tensor_wgrad_gemm"],
    "cfg4_mxfp4_mlp": ["cfg4_mx_quantize_e2m1_X", "cfg4_mxfp4_fc1_swiglu_mxfp4", "cfg4_mxfp4_fc2"],
    "fc2_bf16_dgrad_swiglu_bwd": ["fc2_bf16_dgrad_swiglu_bwd"],
    "fc2_mxfp8_dgrad_swiglu_bwd": ["fc2_mxfp8_dgrad_swiglu_bwd"],
    "fc2_mxfp4_dgrad_swiglu_bwd": ["fc2_mxfp4_dgrad_swiglu_bwd"],
    "fc1_bf16_swiglu_clamped": ["fc1_bf16_swiglu_clamped"],
    "fc1_bf16_swiglu_save": ["fc1_bf16_swiglu_save"],
    "ep8_share_bf16_fc1_swiglu": ["ep8_share_bf16_fc1_swiglu"],
    # the activation's (or output gradient's) quantise passes, then the GEMM
    "cfg3_fp8_tensor_fwd": ["cfg3_fp8_amax_A", "cfg3_fp8_encode_A", "cfg3_fp8_tensor_fwd_gemm"],
    "cfg3_fp8_rowwise_fwd": ["cfg3_fp8_rows_A", "cfg3_fp8_rowwise_fwd_gemm"],
    "cfg3_fp8_tensor_dgrad": ["cfg3_fp8_amax_dY", "cfg3_fp8_encode_dY", "cfg3_fp8_tensor_dgrad_gemm"],
    "cfg3_fp8_rowwise_dgrad": ["cfg3_fp8_rows_dY", "cfg3_fp8_rowwise_dgrad_gemm"],
    "cfg3_mxfp8_dgrad": ["cfg3_mx_quantize_e4m3_dY", "cfg3_mxfp8_dgrad_gemm"],
    "stack_experts_transpose": ["stack_experts_transpose"],
    "stack_experts_mxfp8_caches": ["stack_experts_mxfp8_caches"],
}


def attach_traffic(per):
    for row, keys in TRAFFIC_KEYS.items():
        if row in per:
            vals = [measured_traffic(k) for k in keys]
            per[row]["roofline"]["traffic"] = None if any(v is None for v in vals) else int(sum(vals))


def time_launches(fn, steps, warmup, stream, flush=True, settle_ms=30.0):
    """Warm up, then time exactly `steps` calls: wall clock between two
    device synchronisations, and each launch between HIP events on the
    stream the kernels run on.  With `flush`, a 512 MiB buffer is written on
    that stream before every timed call, outside its event pair, so each
    call starts with caches holding none of its operands (the wall clock
    then includes the flushes).  After the `warmup` calls, untimed calls
    continue until `settle_ms` of them have run: the engine clock ramps for
    some tens of milliseconds after the GPU idles (measured on the headline:
    its first dozen launches after a 1 s pause take 2.2-3.1 ms against 2.17
    once settled).  The headline's own timing passes 0 and keeps exactly
    the requested warm-up steps."""
    for _ in range(warmup):
        fn()
    if settle_ms > 0:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < settle_ms:
            fn()
            torch.cuda.synchronize()
    if flush and FLUSH[0] is None:
        FLUSH[0] = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=stream.device)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for i, (s, e) in enumerate(evs):
            if flush:
                FLUSH[0].fill_(i & 0xFF)
            s.record(stream)
            fn()
            e.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    per = np.array([s.elapsed_time(e) for s, e in evs])
    return wall_ms / steps, per


def roofline(flops, nbytes, seconds, dtype):
    t_mfma = flops / (PEAK_TFLOPS[dtype] * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    if t_hbm >= t_mfma:
        ach = nbytes / seconds / 1e9
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4)}
    ach = flops / seconds / 1e12
    return {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_TFLOPS[dtype], "unit": "TFLOP/s",
            "frac": round(ach / PEAK_TFLOPS[dtype], 4)}


def summary(name, dtype, flops, nbytes, per_ms, extra=None):
    sec = float(np.median(per_ms)) * 1e-3
    d = {"workload": name, "dtype": dtype,
         "ms_median": round(float(np.median(per_ms)), 4),
         "ms_p10": round(float(np.percentile(per_ms, 10)), 4),
         "ms_p90": round(float(np.percentile(per_ms, 90)), 4),
         "useful_tflops": round(flops / sec / 1e12, 2) if flops else None,
         "pct_mfma_peak": round(100 * flops / sec / 1e12 / PEAK_TFLOPS[dtype], 2) if flops else None,
         "algorithmic_gbs": round(nbytes / sec / 1e9, 1),
         "roofline": roofline(flops, nbytes, sec, dtype) if flops else
         {"bound": "hbm", "achieved": round(nbytes / sec / 1e9, 1), "peak": PEAK_HBM_GBS,
          "unit": "GB/s", "frac": round(nbytes / sec / 1e9 / PEAK_HBM_GBS, 4)}}
    if extra:
        d.update(extra)
    return d


# ------------------------------------------------------------------ workloads
# One workspace for every GEMM call (calls on one stream run one after
# another, so they can share it): the error word, the tile queues and, for the
# MX forwards, stage-major copies of the scales; sized for the largest call.
WS = [None]


def make_workspace(dev):
    sizes = [ptm.pt_grouped_gemm_workspace_size(ptm.PT_OP_FWD, 1, 1, 1, 1, ptm.PT_BF16),
             ptm.pt_grouped_gemm_workspace_size(ptm.PT_OP_FWD, 32, 65536, 5760, 2880, ptm.PT_MXFP8_E4M3),
             ptm.pt_grouped_gemm_workspace_size(ptm.PT_OP_FWD, 256, 49152, 4096, 4096, ptm.PT_MXFP4_E2M1),
             ptm.pt_grouped_gemm_workspace_size(ptm.PT_OP_FWD, 256, 49152, 4096, 2048, ptm.PT_MXFP4_E2M1),
             ptm.pt_grouped_gemm_workspace_size(ptm.PT_OP_DGRAD, 32, 65536, 5760, 2880, ptm.PT_MXFP8_E4M3),
             ptm.pt_grouped_gemm_workspace_size(ptm.PT_OP_DGRAD_SWIGLU, 256, 49152, 4096, 2048, ptm.PT_MXFP8_E4M3),
             ptm.pt_grouped_gemm_workspace_size(ptm.PT_OP_DGRAD_SWIGLU, 256, 49152, 4096, 2048, ptm.PT_MXFP4_E2M1)]
    WS[0] = torch.zeros(max(sizes), dtype=torch.uint8, device=dev)


def fc1_inputs(dev):
    lens = synth.lens_topk_gaussian(8192, 256, 6, seed=1)
    G, M, K, N = 256, int(lens.sum()), 4096, 4096
    a = synth.randn_bf16((M, K), seed=101, std=K ** -0.5, device=dev)
    b = synth.randn_bf16((G, K, N), seed=101 + 1000, std=K ** -0.5, device=dev)
    return lens, G, M, K, N, a, b


def up(x, m):
    return (x + m - 1) // m * m


def bytes_weights(lens, per_expert):
    return int((lens > 0).sum()) * per_expert


def cpu_baseline(lens, a, b, out, K, N, min_s=10.0, max_s=30.0):
    """Oracle (fp64) over whole experts' rows of the headline workload until
    about min_s seconds of CPU work; returns the baseline record and the
    parity of the GPU output on those rows."""
    import oracle
    offs = synth.offsets(lens)
    rng = np.random.default_rng(7)
    order = [g for g in rng.permutation(len(lens)) if lens[g] > 0]
    done_flops, t_used, errs, rows_done, experts = 0.0, 0.0, [], 0, 0
    for g in order:
        r0, r1 = int(offs[g]), int(offs[g + 1])
        rows = np.arange(r0, r1)
        if rows.size > 64:
            rows = np.sort(rng.choice(rows, size=64, replace=False))
        a_rows = synth.bf16_bits(a[torch.as_tensor(rows, device=a.device)])
        bg = synth.bf16_bits(b[g:g + 1])
        t0 = time.perf_counter()
        res = oracle.grouped_fwd(oracle.BF16, a_rows, None, bg, None, np.array([rows.size]), N, K, 0,
                                 oracle.EPI_SWIGLU, np.arange(rows.size))
        t_used += time.perf_counter() - t0
        done_flops += 2.0 * rows.size * K * N
        rows_done += rows.size
        experts += 1
        got = (out[torch.as_tensor(rows, device=out.device)].view(torch.int16).cpu().numpy()
               .view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        ref = res["exact"]
        floor = float(np.sqrt(np.mean(ref * ref)))
        errs.append(float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), floor))))
        if t_used >= min_s or t_used >= max_s:
            break
    rec = {"value": round(done_flops / t_used / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.threads(),
           "kind": "oracle",
           "sample": f"{rows_done} rows (<=64 per expert) of {experts} experts of the headline "
                     f"workload, fwd + SwiGLU in fp64, {t_used:.1f} s"}
    return rec, max(errs)


def bench_fc1(dev, stream, steps, warmup):
    lens, G, M, K, N, a, b = fc1_inputs(dev)
    out = torch.empty((M, N // 2), dtype=torch.bfloat16, device=dev)
    lens_d = torch.as_tensor(lens, device=dev)

    def step():
        ptm.pt_grouped_gemm_fwd(a, None, b, None, out, None, lens_d, None, G, M, N, K,
                                ptm.PT_BF16, 0, ptm.PT_EPI_SWIGLU, workspace=WS[0], stream=stream)

    # back to back, as a training step issues them (the 8.5 GB of weights
    # dwarf every cache, so warm and cold launches time alike: see per_flush)
    ms_step, per = time_launches(step, steps, warmup, stream, flush=False, settle_ms=0.0)
    _, per_flush = time_launches(step, max(5, min(steps, 20)), 1, stream, flush=True)
    flops = 2.0 * M * K * N
    nbytes = bytes_weights(lens, K * N * 2) + M * K * 2 + M * (N // 2) * 2
    return dict(lens=lens, G=G, M=M, K=K, N=N, a=a, b=b, out=out, lens_d=lens_d,
                ms_step=ms_step, per=per, per_flush=per_flush, flops=flops, nbytes=nbytes)


def bench_cfg0(dev, stream, iters):
    lens = synth.lens_multinomial(256, 4, seed=0, n_empty=1)
    G, M, K, N = 4, int(lens.sum()), 128, 256
    a = synth.randn_bf16((M, K), seed=100, std=K ** -0.5, device=dev)
    b = synth.randn_bf16((G, K, N), seed=101, std=K ** -0.5, device=dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    lens_d = torch.as_tensor(lens, device=dev)
    _, per = time_launches(lambda: ptm.pt_grouped_gemm_fwd(
        a, None, b, None, out, None, lens_d, None, G, M, N, K, ptm.PT_BF16, 0, ptm.PT_EPI_NONE,
        workspace=WS[0], stream=stream), iters, 10, stream)
    _, per_warm = time_launches(lambda: ptm.pt_grouped_gemm_fwd(
        a, None, b, None, out, None, lens_d, None, G, M, N, K, ptm.PT_BF16, 0, ptm.PT_EPI_NONE,
        workspace=WS[0], stream=stream), iters, 10, stream, flush=False)
    # with tuning on: the first call times the configurations, the rest use the choice
    ptm.pt_clear_gemm_tuning()
    ptm.pt_set_gemm_config(ptm.PT_CONFIG_TUNE)
    try:
        _, per_t = time_launches(lambda: ptm.pt_grouped_gemm_fwd(
            a, None, b, None, out, None, lens_d, None, G, M, N, K, ptm.PT_BF16, 0, ptm.PT_EPI_NONE,
            workspace=WS[0], stream=stream), iters, 10, stream)
        chosen = ptm.pt_gemm_config_of(ptm.PT_OP_FWD, ptm.PT_BF16, ptm.PT_EPI_NONE, 0, G, M, N, K)
    finally:
        ptm.pt_set_gemm_config(ptm.PT_CONFIG_RULES)
        ptm.pt_clear_gemm_tuning()
    flops = 2.0 * M * K * N
    nbytes = bytes_weights(lens, K * N * 2) + M * K * 2 + M * N * 2
    return summary("tiny BF16 fwd, 4 experts, M=256, K=128, N=256", "bf16", flops, nbytes, per,
                   {"tuned_config": chosen, "tuned_ms_median": round(float(np.median(per_t)), 4),
                    "warm_ms_median": round(float(np.median(per_warm)), 4)})


def bench_ep_share(dev, stream, iters):
    """One GPU's share under 8-way expert parallelism at the training shape
    of the headline (4096 tokens per GPU, top-6 over 256 experts): its 32
    local experts receive 8 * 4096 * 6 / 8 = 24576 rows, 768 per expert on
    average, so the kernel is MFMA-bound here where the headline streams
    weights.  The rows are spread over the 32 experts by the headline's
    imbalanced routing recipe (4096 tokens, top-6 over 32 experts, no
    masked experts)."""
    lens = synth.lens_topk_gaussian(4096, 32, 6, seed=7, n_masked=0)
    G, M, K, N = 32, int(lens.sum()), 4096, 4096
    a = synth.randn_bf16((M, K), seed=107, std=K ** -0.5, device=dev)
    b = synth.randn_bf16((G, K, N), seed=108, std=K ** -0.5, device=dev)
    out = torch.empty((M, N // 2), dtype=torch.bfloat16, device=dev)
    lens_d = torch.as_tensor(lens, device=dev)
    _, per = time_launches(lambda: ptm.pt_grouped_gemm_fwd(
        a, None, b, None, out, None, lens_d, None, G, M, N, K, ptm.PT_BF16, 0, ptm.PT_EPI_SWIGLU,
        workspace=WS[0], stream=stream), iters, 3, stream)
    flops = 2.0 * M * K * N
    nbytes = bytes_weights(lens, K * N * 2) + M * K * 2 + M * (N // 2) * 2
    return summary(f"one GPU's share of 8-way expert parallelism: BF16 FC1 + SwiGLU, 32 experts, M={M}, "
                   "K=N=4096, [G,K,N] weights", "bf16", flops, nbytes, per,
                   {"group_lens_min_median_max": [int(lens.min()), int(np.median(lens)), int(lens.max())]})


def bench_cfg2(dev, stream, iters, fc1):
    lens, G, M, K, N, a, b = fc1["lens"], fc1["G"], fc1["M"], fc1["K"], fc1["N"], fc1["a"], fc1["b"]
    lens_d = fc1["lens_d"]
    dy = synth.randn_bf16((M, N), seed=102, std=1e-2, device=dev)
    dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    _, per_d = time_launches(lambda: ptm.pt_grouped_gemm_dgrad(
        dy, None, b, None, dx, lens_d, None, G, M, N, K, ptm.PT_BF16, 0, workspace=WS[0], stream=stream), iters, 2, stream)
    flops = 2.0 * M * K * N
    d = summary("BF16 dgrad, 256 experts, M=49152, K=N=4096", "bf16", flops,
                bytes_weights(lens, K * N * 2) + M * N * 2 + M * K * 2, per_d)
    del dx
    g = torch.Generator(device=dev)
    g.manual_seed(103)
    mg = torch.randn((G, K, N), generator=g, device=dev, dtype=torch.float32).mul_(1e-3)
    _, per_w = time_launches(lambda: ptm.pt_grouped_gemm_wgrad(
        a, None, dy, None, mg, lens_d, None, G, M, N, K, ptm.PT_BF16, 0, 1, workspace=WS[0], stream=stream), iters, 2, stream)
    w = summary("BF16 wgrad accumulated into fp32 main_grad [256, 4096, 4096]", "bf16", flops,
                bytes_weights(lens, K * N * 4 * 2) + M * K * 2 + M * N * 2, per_w)
    del mg, dy
    torch.cuda.empty_cache()
    return d, w


def bench_cfg3(dev, stream, iters):
    lens = synth.lens_zipf_distinct(16384, 32, 4, 1.1, seed=3)
    G, M, K, N = 32, int(lens.sum()), 2880, 5760
    x = synth.randn_bf16((M, K), seed=104, device=dev, outlier_frac=0.01, outlier_mult=50.0)
    w = synth.randn_bf16((G * N, K), seed=104 + 1000, device=dev, outlier_frac=0.01, outlier_mult=50.0)
    aq = torch.empty((M, K), dtype=torch.uint8, device=dev)
    as_ = torch.empty((M, K // 32), dtype=torch.uint8, device=dev)
    bq = torch.empty((G * N, K), dtype=torch.uint8, device=dev)
    bs = torch.empty((G * N, K // 32), dtype=torch.uint8, device=dev)
    ptm.pt_mx_quantize(w, bq, bs, G * N, K, ptm.PT_MXFP8_E4M3, 1, stream=stream)
    del w
    _, per_q = time_launches(lambda: ptm.pt_mx_quantize(x, aq, as_, M, K, ptm.PT_MXFP8_E4M3, 1, stream=stream),
                             iters, 3, stream)
    q = summary("MXFP8 quantise of A [65536, 2880]", "mxfp8", 0, M * K * 2 + M * K + M * K // 32, per_q)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    lens_d = torch.as_tensor(lens, device=dev)
    _, per = time_launches(lambda: ptm.pt_grouped_gemm_fwd(
        aq, as_, bq, bs, out, None, lens_d, None, G, M, N, K, ptm.PT_MXFP8_E4M3, 1, ptm.PT_EPI_NONE,
        workspace=WS[0], stream=stream), iters, 3, stream)
    flops = 2.0 * M * K * N
    nbytes = bytes_weights(lens, N * K + N * K // 32) + M * K + M * K // 32 + M * N * 2
    f = summary("MXFP8 fwd, 32 experts (Zipf 1.1), M=65536, K=2880, N=5760", "mxfp8", flops, nbytes, per,
                {"group_lens_min_median_max": [int(lens.min()), int(np.median(lens)), int(lens.max())]})
    return f, q


def bench_cfg3_aligned(dev, stream, iters):
    """The MXFP8 forward of the same workload on line-aligned codes: A and
    the weights quantised by pt_mx_quantize_pitched with rows 2944 bytes
    apart (each row starting on a 128-byte line), then
    pt_grouped_gemm_fwd_pitched; timed as the packed line (GEMM with its
    scale pre-pass), the pitched quantise of A beside it."""
    lens = synth.lens_zipf_distinct(16384, 32, 4, 1.1, seed=3)
    G, M, K, N = 32, int(lens.sum()), 2880, 5760
    P = up(K, 128)
    x = synth.randn_bf16((M, K), seed=104, device=dev, outlier_frac=0.01, outlier_mult=50.0)
    w = synth.randn_bf16((G * N, K), seed=104 + 1000, device=dev, outlier_frac=0.01, outlier_mult=50.0)
    ap = torch.empty((M, P), dtype=torch.uint8, device=dev)
    as_ = torch.empty((M, K // 32), dtype=torch.uint8, device=dev)
    bp = torch.empty((G * N, P), dtype=torch.uint8, device=dev)
    bs = torch.empty((G * N, K // 32), dtype=torch.uint8, device=dev)
    ptm.pt_mx_quantize_pitched(w, bp, bs, G * N, K, ptm.PT_MXFP8_E4M3, P, stream=stream)
    del w
    _, per_q = time_launches(lambda: ptm.pt_mx_quantize_pitched(x, ap, as_, M, K, ptm.PT_MXFP8_E4M3, P,
                                                                stream=stream), iters, 3, stream)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    lens_d = torch.as_tensor(lens, device=dev)
    _, per = time_launches(lambda: ptm.pt_grouped_gemm_fwd_pitched(
        ap, as_, bp, bs, out, None, lens_d, None, G, M, N, K, ptm.PT_MXFP8_E4M3, ptm.PT_EPI_NONE, P,
        workspace=WS[0], stream=stream), iters, 3, stream)
    flops = 2.0 * M * K * N
    nbytes = bytes_weights(lens, N * K + N * K // 32) + M * K + M * K // 32 + M * N * 2
    return summary(f"MXFP8 fwd on line-aligned codes (row pitch {P} bytes), 32 experts (Zipf 1.1), M=65536, "
                   "K=2880, N=5760", "mxfp8", flops, nbytes, per,
                   {"code_pitch": P, "quantise_A_pitched_ms_median": round(float(np.median(per_q)), 4)})


def bench_cfg3_dgrad(dev, stream, iters):
    """The MXFP8 workload's data gradient: dY [65536, 5760] quantised along N,
    then the MX grouped GEMM against the weight's transposed cache (the
    forward weight [32, 5760, 2880] quantised along N by pt_mx_quantize_t,
    once, outside the step, like the forward's weight quantisation)."""
    lens = synth.lens_zipf_distinct(16384, 32, 4, 1.1, seed=3)
    G, M, K, N = 32, int(lens.sum()), 2880, 5760
    lens_d = torch.as_tensor(lens, device=dev)
    w = synth.randn_bf16((G, N, K), seed=104 + 1000, device=dev, outlier_frac=0.01, outlier_mult=50.0)
    wq = torch.empty((G, K, N), dtype=torch.uint8, device=dev)
    wsc = torch.empty((G, K, N // 32), dtype=torch.uint8, device=dev)
    _, per_t = time_launches(lambda: ptm.pt_mx_quantize_t(w, wq, wsc, G, N, K, ptm.PT_MXFP8_E4M3, stream=stream),
                             max(3, iters // 4), 1, stream)
    del w
    dy = synth.randn_bf16((M, N), seed=106, std=1e-2, device=dev)
    dq = torch.empty((M, N), dtype=torch.uint8, device=dev)
    ds = torch.empty((M, N // 32), dtype=torch.uint8, device=dev)
    dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)

    def step():
        ptm.pt_mx_quantize(dy, dq, ds, M, N, ptm.PT_MXFP8_E4M3, 1, stream=stream)
        ptm.pt_grouped_gemm_dgrad(dq, ds, wq, wsc, dx, lens_d, None, G, M, N, K, ptm.PT_MXFP8_E4M3, 0,
                                  workspace=WS[0], stream=stream)
    _, per = time_launches(step, iters, 3, stream)
    _, per_g = time_launches(lambda: ptm.pt_grouped_gemm_dgrad(
        dq, ds, wq, wsc, dx, lens_d, None, G, M, N, K, ptm.PT_MXFP8_E4M3, 0, workspace=WS[0], stream=stream),
        iters, 3, stream)
    flops = 2.0 * M * K * N
    nbytes = (bytes_weights(lens, N * K + N * K // 32) + M * N * 2 + 2 * (M * N + M * N // 32) + M * K * 2)
    d = summary("MXFP8 dgrad (dY quantise + grouped GEMM on the transposed weight cache), 32 experts, "
                "M=65536, N=5760 -> K=2880", "mxfp8", flops, nbytes, per,
                {"gemm_only_ms_median": round(float(np.median(per_g)), 4),
                 "weight_transposed_cache_ms": round(float(np.median(per_t)), 4)})
    del dy, dq, ds, dx, wq, wsc
    torch.cuda.empty_cache()
    return d


def bench_cfg3_fp8(dev, stream, iters):
    """The MXFP8 workload's shapes in FP8 with one scale per tensor (current
    scaling): the activations are quantised inside the step (two passes:
    amax, then codes), the weights once outside it."""
    lens = synth.lens_zipf_distinct(16384, 32, 4, 1.1, seed=3)
    G, M, K, N = 32, int(lens.sum()), 2880, 5760
    lens_d = torch.as_tensor(lens, device=dev)
    w = synth.randn_bf16((G, N, K), seed=104 + 1000, device=dev, outlier_frac=0.01, outlier_mult=50.0)
    bq = torch.empty((G, N, K), dtype=torch.uint8, device=dev)
    bamax = torch.empty((G,), dtype=torch.float32, device=dev)
    bd = torch.empty((G,), dtype=torch.float32, device=dev)
    ptm.pt_fp8_quantize(w, bq, bamax, bd, G, N, K, stream=stream)
    del w
    x = synth.randn_bf16((M, K), seed=104, device=dev, outlier_frac=0.01, outlier_mult=50.0)
    aq = torch.empty((M, K), dtype=torch.uint8, device=dev)
    aamax = torch.empty((1,), dtype=torch.float32, device=dev)
    ad = torch.empty((1,), dtype=torch.float32, device=dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def step():
        ptm.pt_fp8_quantize(x, aq, aamax, ad, 1, M, K, stream=stream)
        ptm.pt_grouped_gemm_fwd(aq, ad, bq, bd, out, None, lens_d, None, G, M, N, K, ptm.PT_FP8_E4M3, 1,
                                ptm.PT_EPI_NONE, workspace=WS[0], stream=stream)
    _, per = time_launches(step, iters, 3, stream)
    _, per_g = time_launches(lambda: ptm.pt_grouped_gemm_fwd(
        aq, ad, bq, bd, out, None, lens_d, None, G, M, N, K, ptm.PT_FP8_E4M3, 1, ptm.PT_EPI_NONE,
        workspace=WS[0], stream=stream), iters, 3, stream)
    flops = 2.0 * M * K * N
    nbytes = bytes_weights(lens, N * K) + M * K * 2 * 2 + M * K + M * K + M * N * 2
    d = summary("FP8 E4M3 with one scale per tensor (activation quantise + grouped GEMM), 32 experts, "
                "M=65536, K=2880, N=5760", "fp8", flops, nbytes, per,
                {"gemm_only_ms_median": round(float(np.median(per_g)), 4)})
    # rowwise: one scale per activation row and per weight row (output column)
    bamax_r = torch.empty((G * N,), dtype=torch.float32, device=dev)
    bd_r = torch.empty((G * N,), dtype=torch.float32, device=dev)
    w = synth.randn_bf16((G * N, K), seed=104 + 1000, device=dev, outlier_frac=0.01, outlier_mult=50.0)
    ptm.pt_fp8_quantize_rows(w, bq, bamax_r, bd_r, G * N, K, stream=stream)
    del w
    aamax_r = torch.empty((M,), dtype=torch.float32, device=dev)
    ad_r = torch.empty((M,), dtype=torch.float32, device=dev)

    def step_rows():
        ptm.pt_fp8_quantize_rows(x, aq, aamax_r, ad_r, M, K, stream=stream)
        ptm.pt_grouped_gemm_fwd(aq, ad_r, bq, bd_r, out, None, lens_d, None, G, M, N, K, ptm.PT_FP8_E4M3_ROWWISE, 1,
                                ptm.PT_EPI_NONE, workspace=WS[0], stream=stream)
    _, per_r = time_launches(step_rows, iters, 3, stream)
    r = summary("FP8 E4M3 rowwise (one scale per row of A and of B; activation quantise + grouped GEMM), "
                "32 experts, M=65536, K=2880, N=5760", "fp8", flops, nbytes - M * K * 2, per_r)
    del x, aq, out, bq
    torch.cuda.empty_cache()
    return d, r


def bench_cfg3_fp8_dgrad(dev, stream, iters):
    """The MXFP8 workload's data gradient in FP8 with tensor factors and with
    row factors: dY [65536, 5760] quantised inside the step, the transposed
    weight cache [32, 2880, 5760] (pt_stack_experts, then the FP8 quantiser)
    built once outside it."""
    lens = synth.lens_zipf_distinct(16384, 32, 4, 1.1, seed=3)
    G, M, K, N = 32, int(lens.sum()), 2880, 5760
    lens_d = torch.as_tensor(lens, device=dev)
    w = synth.randn_bf16((G, N, K), seed=104 + 1000, device=dev, outlier_frac=0.01, outlier_mult=50.0)
    addr = torch.tensor([w.data_ptr() + g * N * K * 2 for g in range(G)], dtype=torch.int64, device=dev)
    wt = torch.empty((G, K, N), dtype=torch.bfloat16, device=dev)
    ptm.pt_stack_experts(addr, wt, G, N, K, 1, stream=stream)
    del w
    wq = torch.empty((G, K, N), dtype=torch.uint8, device=dev)
    wamax, wd = torch.empty((G,), dtype=torch.float32, device=dev), torch.empty((G,), dtype=torch.float32, device=dev)
    ptm.pt_fp8_quantize(wt, wq, wamax, wd, G, K, N, stream=stream)
    wq_r = torch.empty((G, K, N), dtype=torch.uint8, device=dev)
    wamax_r = torch.empty((G * K,), dtype=torch.float32, device=dev)
    wd_r = torch.empty((G * K,), dtype=torch.float32, device=dev)
    ptm.pt_fp8_quantize_rows(wt, wq_r, wamax_r, wd_r, G * K, N, stream=stream)
    del wt
    dy = synth.randn_bf16((M, N), seed=106, std=1e-2, device=dev)
    dq = torch.empty((M, N), dtype=torch.uint8, device=dev)
    damax, dd = torch.empty((1,), dtype=torch.float32, device=dev), torch.empty((1,), dtype=torch.float32, device=dev)
    damax_r, dd_r = (torch.empty((M,), dtype=torch.float32, device=dev),
                     torch.empty((M,), dtype=torch.float32, device=dev))
    dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)

    def step():
        ptm.pt_fp8_quantize(dy, dq, damax, dd, 1, M, N, stream=stream)
        ptm.pt_grouped_gemm_dgrad(dq, dd, wq, wd, dx, lens_d, None, G, M, N, K, ptm.PT_FP8_E4M3, 0,
                                  workspace=WS[0], stream=stream)

    def step_rows():
        ptm.pt_fp8_quantize_rows(dy, dq, damax_r, dd_r, M, N, stream=stream)
        ptm.pt_grouped_gemm_dgrad(dq, dd_r, wq_r, wd_r, dx, lens_d, None, G, M, N, K, ptm.PT_FP8_E4M3_ROWWISE, 0,
                                  workspace=WS[0], stream=stream)
    _, per = time_launches(step, iters, 3, stream)
    _, per_r = time_launches(step_rows, iters, 3, stream)
    flops = 2.0 * M * K * N
    nbytes = bytes_weights(lens, N * K) + M * N * 2 * 2 + M * N * 2 + M * K * 2
    d = summary("FP8 dgrad with tensor factors (two-pass dY quantise + grouped GEMM on the transposed FP8 weight "
                "cache), 32 experts, M=65536, N=5760 -> K=2880", "fp8", flops, nbytes, per)
    r = summary("FP8 dgrad with row factors (one-pass dY quantise + grouped GEMM), 32 experts, M=65536, "
                "N=5760 -> K=2880", "fp8", flops, nbytes - M * N * 2, per_r)
    del dy, dq, dx, wq, wq_r
    torch.cuda.empty_cache()
    return d, r


def bench_cfg4(dev, stream, iters, lens):
    G, M, H, I = 256, int(lens.sum()), 4096, 2048
    x = synth.randn_bf16((M, H), seed=105, device=dev)
    w1q = torch.empty((G * 2 * I, H // 2), dtype=torch.uint8, device=dev)
    w1s = torch.empty((G * 2 * I, H // 32), dtype=torch.uint8, device=dev)
    w2q = torch.empty((G * H, I // 2), dtype=torch.uint8, device=dev)
    w2s = torch.empty((G * H, I // 32), dtype=torch.uint8, device=dev)
    for rows, cols, q, s, seed in ((G * 2 * I, H, w1q, w1s, 1105), (G * H, I, w2q, w2s, 2105)):
        wb = synth.randn_bf16((rows, cols), seed=seed, device=dev)
        ptm.pt_mx_quantize(wb, q, s, rows, cols, ptm.PT_MXFP4_E2M1, 1, stream=stream)
        del wb
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    xq = torch.empty((M, H // 2), dtype=torch.uint8, device=dev)
    xs = torch.empty((M, H // 32), dtype=torch.uint8, device=dev)
    hq = torch.empty((M, I // 2), dtype=torch.uint8, device=dev)
    hs = torch.empty((M, I // 32), dtype=torch.uint8, device=dev)
    out = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    lens_d = torch.as_tensor(lens, device=dev)

    def mlp():
        ptm.pt_mx_quantize(x, xq, xs, M, H, ptm.PT_MXFP4_E2M1, 1, stream=stream)
        ptm.pt_grouped_gemm_fwd(xq, xs, w1q, w1s, hq, hs, lens_d, None, G, M, 2 * I, H,
                                ptm.PT_MXFP4_E2M1, 1, ptm.PT_EPI_SWIGLU_MXFP4, workspace=WS[0], stream=stream)
        ptm.pt_grouped_gemm_fwd(hq, hs, w2q, w2s, out, None, lens_d, None, G, M, H, I,
                                ptm.PT_MXFP4_E2M1, 1, ptm.PT_EPI_NONE, workspace=WS[0], stream=stream)

    _, per = time_launches(mlp, iters, 3, stream)
    flops = 2.0 * M * H * 2 * I + 2.0 * M * I * H
    ne = int((lens > 0).sum())
    nbytes = (ne * (2 * I * H // 2 + 2 * I * H // 32 + H * I // 2 + H * I // 32)
              + M * H * 2 + 2 * (M * I // 2 + M * I // 32) + M * H * 2)
    return summary("MXFP4 expert MLP quantise -> FC1 + SwiGLU + MXFP4 -> FC2, 256 experts, M=49152, "
                   "H=4096, I=2048", "mxfp4", flops, nbytes, per)


def bench_fc2_bwd(dev, stream, iters, lens):
    """FC2's data gradient with the SwiGLU backward fused into its epilogue, at
    the expert-MLP shape in BF16 (256 experts, H = 4096, I = 2048), next to
    the plain data gradient of the same shape."""
    G, M, I, H = 256, int(lens.sum()), 2048, 4096
    lens_d = torch.as_tensor(lens, device=dev)
    dy = synth.randn_bf16((M, H), seed=111, std=1e-2, device=dev)
    w2 = synth.randn_bf16((G, I, H), seed=112, std=H ** -0.5, device=dev)     # [G, K, N] with K = I, N = H
    c = synth.randn_bf16((M, 2 * I), seed=113, std=2.0, device=dev)
    dc = torch.empty((M, 2 * I), dtype=torch.bfloat16, device=dev)
    dx = torch.empty((M, I), dtype=torch.bfloat16, device=dev)
    _, per_f = time_launches(lambda: ptm.pt_grouped_gemm_dgrad_swiglu(
        dy, w2, c, dc, lens_d, None, G, M, H, I, 0, workspace=WS[0], stream=stream), iters, 2, stream)
    _, per_p = time_launches(lambda: ptm.pt_grouped_gemm_dgrad(
        dy, None, w2, None, dx, lens_d, None, G, M, H, I, ptm.PT_BF16, 0, workspace=WS[0], stream=stream),
        iters, 2, stream)
    flops = 2.0 * M * I * H
    w_bytes = bytes_weights(lens, I * H * 2)
    d = summary("BF16 FC2 dgrad + fused SwiGLU backward, 256 experts, M=49152, I=2048, H=4096", "bf16", flops,
                w_bytes + M * H * 2 + 2 * (M * 2 * I * 2), per_f,
                {"plain_dgrad_ms_median": round(float(np.median(per_p)), 4)})
    del dy, w2, c, dc, dx
    torch.cuda.empty_cache()
    return d


def bench_fc2_bwd_mx(dev, stream, iters, lens, dtype):
    """The same FC2 backward with MX operands at the MXFP4 expert-MLP shape:
    dY quantised along H inside the step (pt_mx_quantize), the transposed
    weight cache [G, I, H] quantised along H outside it, dH on the scaled
    matrix cores and the SwiGLU backward in the epilogue."""
    G, M, I, H = 256, int(lens.sum()), 2048, 4096
    fmt = "MXFP4" if dtype == ptm.PT_MXFP4_E2M1 else "MXFP8"
    cb = H // 2 if dtype == ptm.PT_MXFP4_E2M1 else H
    lens_d = torch.as_tensor(lens, device=dev)
    dy = synth.randn_bf16((M, H), seed=111, std=1e-2, device=dev)
    w2t = synth.randn_bf16((G * I, H), seed=112, std=H ** -0.5, device=dev)
    wq = torch.empty((G * I, cb), dtype=torch.uint8, device=dev)
    ws_ = torch.empty((G * I, H // 32), dtype=torch.uint8, device=dev)
    ptm.pt_mx_quantize(w2t, wq, ws_, G * I, H, dtype, 1, stream=stream)
    del w2t
    dq = torch.empty((M, cb), dtype=torch.uint8, device=dev)
    ds = torch.empty((M, H // 32), dtype=torch.uint8, device=dev)
    c = synth.randn_bf16((M, 2 * I), seed=113, std=2.0, device=dev)
    dc = torch.empty((M, 2 * I), dtype=torch.bfloat16, device=dev)

    def step():
        ptm.pt_mx_quantize(dy, dq, ds, M, H, dtype, 1, stream=stream)
        ptm.pt_grouped_gemm_dgrad_swiglu(dq, wq, c, dc, lens_d, None, G, M, H, I, 0, workspace=WS[0],
                                         stream=stream, swiglu_limit=10.0, dtype=dtype, dy_scale=ds, b_scale=ws_)

    _, per = time_launches(step, iters, 2, stream)
    flops = 2.0 * M * I * H
    el = 0.5 if dtype == ptm.PT_MXFP4_E2M1 else 1.0
    w_bytes = bytes_weights(lens, int(I * H * (el + 1 / 32)))
    nbytes = w_bytes + M * H * 2 + int(M * H * (el + 1 / 32)) * 2 + 2 * (M * 2 * I * 2)
    d = summary(f"{fmt} FC2 dgrad + fused clamped SwiGLU backward (dY quantise included), 256 experts, "
                f"M=49152, I=2048, H=4096", "mxfp4" if dtype == ptm.PT_MXFP4_E2M1 else "mxfp8", flops, nbytes, per)
    del dy, wq, ws_, dq, ds, c, dc
    torch.cuda.empty_cache()
    return d


def bench_cfg3_wgrad(dev, stream, iters):
    """The MXFP8 workload's weight gradient: A [65536, 2880] and dY
    [65536, 5760] quantised along tokens in blocks of 32 inside each expert,
    then the weight gradient accumulated into fp32 main_grad [32, 2880, 5760]
    (both transposed to channel rows in the workspace, then the MX kernel)."""
    lens = synth.lens_zipf_distinct(16384, 32, 4, 1.1, seed=3)
    G, M, K, N = 32, int(lens.sum()), 2880, 5760
    lens_d = torch.as_tensor(lens, device=dev)
    a = synth.randn_bf16((M, K), seed=104, device=dev, outlier_frac=0.01, outlier_mult=50.0)
    dy = synth.randn_bf16((M, N), seed=106, std=1e-2, device=dev)
    aq = torch.empty((M, K), dtype=torch.uint8, device=dev)
    as_ = torch.empty((M // 32 + G, K), dtype=torch.uint8, device=dev)
    dq = torch.empty((M, N), dtype=torch.uint8, device=dev)
    ds = torch.empty((M // 32 + G, N), dtype=torch.uint8, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(103)
    mg = torch.randn((G, K, N), generator=g, device=dev, dtype=torch.float32).mul_(1e-3)
    ws = torch.zeros((ptm.pt_grouped_gemm_workspace_size(ptm.PT_OP_WGRAD, G, M, N, K, ptm.PT_MXFP8_E4M3),),
                     dtype=torch.uint8, device=dev)

    def quant():
        ptm.pt_mx_quantize_tokens(a, lens_d, None, aq, as_, G, M, K, ptm.PT_MXFP8_E4M3, workspace=ws, stream=stream)
        ptm.pt_mx_quantize_tokens(dy, lens_d, None, dq, ds, G, M, N, ptm.PT_MXFP8_E4M3, workspace=ws, stream=stream)

    def gemm():
        ptm.pt_grouped_gemm_wgrad(aq, as_, dq, ds, mg, lens_d, None, G, M, N, K, ptm.PT_MXFP8_E4M3, 0, 1,
                                  workspace=ws, stream=stream)

    def step():
        quant()
        gemm()
    _, per = time_launches(step, iters, 3, stream)
    _, per_q = time_launches(quant, iters, 3, stream)
    _, per_g = time_launches(gemm, iters, 3, stream)
    # the same from the bf16 gradients in one call: quantisation along tokens
    # fused into the transpose to the weight gradient's operand layout
    _, per_f = time_launches(lambda: ptm.pt_grouped_gemm_wgrad_quantize(
        a, dy, mg, lens_d, None, G, M, N, K, ptm.PT_MXFP8_E4M3, 0, 1, workspace=ws, stream=stream),
        iters, 3, stream)
    flops = 2.0 * M * K * N
    codes = M * K + M * N + (M // 32 + G) * (K + N)
    nbytes = M * K * 2 + M * N * 2 + 2 * codes + bytes_weights(lens, K * N * 4 * 2)
    w = summary("MXFP8 wgrad (A and dY quantised along tokens + weight gradient into fp32 main_grad), "
                "32 experts, M=65536, K=2880, N=5760", "mxfp8", flops, nbytes, per,
                {"quantize_tokens_ms_median": round(float(np.median(per_q)), 4),
                 "wgrad_only_ms_median": round(float(np.median(per_g)), 4),
                 "fused_quantize_wgrad_ms_median": round(float(np.median(per_f)), 4)})
    del as_, ds, ws
    torch.cuda.empty_cache()
    # FP8 with one factor per tensor: two-pass quantise of A and dY, then the
    # weight gradient (decode, BF16 sums into the workspace, fused main_grad update)
    fa, ma = torch.empty((1,), dtype=torch.float32, device=dev), torch.empty((1,), dtype=torch.float32, device=dev)
    fd, md = torch.empty((1,), dtype=torch.float32, device=dev), torch.empty((1,), dtype=torch.float32, device=dev)
    ws8 = torch.zeros((ptm.pt_grouped_gemm_workspace_size(ptm.PT_OP_WGRAD, G, M, N, K, ptm.PT_FP8_E4M3),),
                      dtype=torch.uint8, device=dev)

    def step8():
        ptm.pt_fp8_quantize(a, aq, ma, fa, 1, M, K, stream=stream)
        ptm.pt_fp8_quantize(dy, dq, md, fd, 1, M, N, stream=stream)
        ptm.pt_grouped_gemm_wgrad(aq, fa, dq, fd, mg, lens_d, None, G, M, N, K, ptm.PT_FP8_E4M3, 0, 1,
                                  workspace=ws8, stream=stream)
    _, per8 = time_launches(step8, iters, 3, stream)
    _, per8f = time_launches(lambda: ptm.pt_grouped_gemm_wgrad_quantize(
        a, dy, mg, lens_d, None, G, M, N, K, ptm.PT_FP8_E4M3, 0, 1, workspace=ws8, stream=stream),
        iters, 3, stream)
    nbytes8 = M * K * 2 * 2 + M * N * 2 * 2 + 2 * (M * K + M * N) + bytes_weights(lens, K * N * 4 * 2)
    w8 = summary("FP8 wgrad with tensor factors (two-pass quantise of A and dY + weight gradient into fp32 "
                 "main_grad), 32 experts, M=65536, K=2880, N=5760", "fp8", flops, nbytes8, per8,
                 {"fused_quantize_wgrad_ms_median": round(float(np.median(per8f)), 4)})
    del a, dy, aq, dq, mg, ws8
    torch.cuda.empty_cache()
    return w, w8


def bench_wgrad_split(dev, stream, iters):
    """BF16 weight gradient with few output tiles per expert (K = N = 512,
    four 256 x 256 tiles each) over the GPT-OSS-20B-like skewed routing (32
    experts, 65536 rows, one of 12541 tokens): with the split reduction's
    workspace, experts are cut into 512-token chunks; without it each
    expert's four tiles reduce all its tokens serially."""
    lens = synth.lens_zipf_distinct(16384, 32, 4, 1.1, seed=3)
    G, M, K, N = 32, int(lens.sum()), 512, 512
    a = synth.randn_bf16((M, K), seed=220, std=K ** -0.5, device=dev)
    dy = synth.randn_bf16((M, N), seed=221, std=1e-2, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(222)
    mg = torch.randn((G, K, N), generator=g, device=dev, dtype=torch.float32).mul_(1e-3)
    lens_d = torch.as_tensor(lens, device=dev)
    ws = torch.zeros(ptm.pt_grouped_gemm_workspace_size(ptm.PT_OP_WGRAD, G, M, N, K, ptm.PT_BF16),
                     dtype=torch.uint8, device=dev)
    _, per_s = time_launches(lambda: ptm.pt_grouped_gemm_wgrad(
        a, None, dy, None, mg, lens_d, None, G, M, N, K, ptm.PT_BF16, 0, 1, workspace=ws, stream=stream),
        iters, 2, stream)
    _, per_n = time_launches(lambda: ptm.pt_grouped_gemm_wgrad(
        a, None, dy, None, mg, lens_d, None, G, M, N, K, ptm.PT_BF16, 0, 1, workspace=WS[0][:1280],
        stream=stream), iters, 2, stream)
    flops = 2.0 * M * K * N
    return summary("BF16 wgrad into fp32 main_grad [32, 512, 512], skewed routing (max 12541 tokens), split "
                   "reduction into 512-token chunks", "bf16", flops,
                   bytes_weights(lens, K * N * 4 * 2) + M * K * 2 + M * N * 2, per_s,
                   {"unsplit_ms_median": round(float(np.median(per_n)), 4), "workspace_bytes": ws.numel()})


def bench_stack(dev, stream, iters):
    """The expert weight stack at the expert-MLP shape: 256 separately
    allocated FC1 weights [2I, H] = [4096, 4096] -> the [G, H, 2I] operand in
    one pass, and both MXFP8 weight caches from one read; the eager
    stack-then-transpose copy is timed beside it for context."""
    G, R, C = 256, 4096, 4096
    ws = [synth.randn_bf16((R, C), seed=300 + g, std=R ** -0.5, device=dev) for g in range(G)]
    addr = ptm.expert_addresses(ws)
    out = torch.empty((G, C, R), dtype=torch.bfloat16, device=dev)
    _, per = time_launches(lambda: ptm.pt_stack_experts(addr, out, G, R, C, 1, stream=stream), iters, 2, stream)
    _, per_eager = time_launches(lambda: torch.stack(ws).transpose(1, 2).contiguous(), max(3, iters // 4), 1, stream)
    nbytes = 2 * G * R * C * 2
    st = summary("expert weight stack + transpose, 256 x [4096, 4096] bf16 -> [256, 4096, 4096]", "bf16", 0,
                 nbytes, per, {"eager_stack_transpose_contiguous_ms_median": round(float(np.median(per_eager)), 4)})
    del out
    torch.cuda.empty_cache()
    q = torch.empty((G, R, C), dtype=torch.uint8, device=dev)
    s = torch.empty((G, R, C // 32), dtype=torch.uint8, device=dev)
    qt = torch.empty((G, C, R), dtype=torch.uint8, device=dev)
    sct = torch.empty((G, C, R // 32), dtype=torch.uint8, device=dev)
    _, per_q = time_launches(lambda: ptm.pt_mx_quantize_experts(addr, q, s, qt, sct, G, R, C, ptm.PT_MXFP8_E4M3,
                                                                stream=stream), iters, 2, stream)
    nbytes_q = G * R * C * 2 + 2 * (G * R * C + G * R * C // 32)
    mq = summary("both MXFP8 weight caches (along K, and transposed along N) from 256 separate [4096, 4096] "
                 "bf16 weights, one read", "mxfp8", 0, nbytes_q, per_q)
    del ws, addr, q, s, qt, sct
    torch.cuda.empty_cache()
    return st, mq


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # 15 untimed steps (~33 ms) cover the engine clock's ramp after idle
    ap.add_argument("--warmup", type=int, default=15)
    ap.add_argument("--headline-only", action="store_true", help="skip per_config workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default=None, help="comma list of per_config keys to run")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB --steps times "
                         "(reference kernel for calibrating HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              f"(this library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    ptm.load()
    make_workspace(dev)
    stream = torch.cuda.current_stream()
    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        _, per = time_launches(lambda: dst.copy_(src), args.steps, args.warmup, stream, flush=False)
        print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n,
                          "ms_mean": float(np.mean(per)), "gbs": 2 * n / (np.mean(per) * 1e-3) / 1e9}))
        return

    log("headline: BF16 FC1 + SwiGLU, 256 experts, M=49152, K=N=4096")
    fc1 = bench_fc1(dev, stream, args.steps, args.warmup)
    kern_ms = float(np.mean(fc1["per"]))
    sec = kern_ms * 1e-3
    value = fc1["flops"] / (fc1["ms_step"] * 1e-3) / 1e12
    roof = roofline(fc1["flops"], fc1["nbytes"], sec, "bf16")
    roof["traffic"] = measured_traffic("fc1_bf16_swiglu")
    lens = fc1["lens"]
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(fc1["ms_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded routing and N(0,1/K) bf16 tensors; no trained weights)",
        "config": {"workload": "BF16 MoE FC1 forward + fused SwiGLU, DeepSeek-V4-Flash-like layer",
                   "experts": 256, "tokens": 8192, "top_k": 6, "rows": int(fc1["M"]),
                   "K": 4096, "N": 4096, "out": [int(fc1["M"]), 2048], "weight_layout": "[G,K,N]",
                   "group_lens_min_p10_median_max": [int(lens.min()), int(np.percentile(lens, 10)),
                                                     int(np.median(lens)), int(lens.max())],
                   "empty_experts": int((lens == 0).sum())},
        "pct_mfma_peak": round(100 * value / PEAK_TFLOPS["bf16"], 2),
        "kernel_ms_mean": round(kern_ms, 4),
        "kernel_ms_median_cache_flushed": round(float(np.median(fc1["per_flush"])), 4),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on a sample of the headline workload")
        rec, err = cpu_baseline(lens, fc1["a"], fc1["b"], fc1["out"], fc1["K"], fc1["N"])
        line["cpu_baseline"] = rec
        line["parity_sample_max_floored_rel_err"] = round(err, 6)
    if not args.headline_only:
        per = {}
        want = set(args.only.split(",")) if args.only else None
        iters = max(5, min(args.steps, 20))
        if want is None or "cfg0" in want:
            log("per_config: tiny")
            per["cfg0_tiny_bf16_fwd"] = bench_cfg0(dev, stream, 50)
        if want is None or "clamp" in want:
            log("per_config: headline with the clamped SwiGLU")
            _, per_c = time_launches(lambda: ptm.pt_grouped_gemm_fwd(
                fc1["a"], None, fc1["b"], None, fc1["out"], None, fc1["lens_d"], None, fc1["G"], fc1["M"], fc1["N"],
                fc1["K"], ptm.PT_BF16, 0, ptm.PT_EPI_SWIGLU, workspace=WS[0], stream=stream, swiglu_limit=10.0),
                iters, 3, stream)
            c_keep = torch.empty((fc1["M"], fc1["N"]), dtype=torch.bfloat16, device=dev)
            _, per_s = time_launches(lambda: ptm.pt_grouped_gemm_fwd_swiglu_save(
                fc1["a"], None, fc1["b"], None, fc1["out"], c_keep, fc1["lens_d"], None, fc1["G"], fc1["M"], fc1["N"],
                fc1["K"], ptm.PT_BF16, 0, workspace=WS[0], stream=stream, swiglu_limit=10.0), iters, 3, stream)
            per["fc1_bf16_swiglu_save"] = summary(
                "BF16 FC1 + clamped SwiGLU that also stores FC1's output [49152, 4096] for the backward", "bf16",
                fc1["flops"], fc1["nbytes"] + fc1["M"] * fc1["N"] * 2, per_s)
            del c_keep
            per["fc1_bf16_swiglu_clamped"] = summary(
                "BF16 FC1 + SwiGLU clamped at swiglu_limit 10, 256 experts, M=49152, K=N=4096", "bf16",
                fc1["flops"], fc1["nbytes"], per_c)
        if want is None or "cfg2" in want:
            log("per_config: dgrad / wgrad")
            per["cfg2_bf16_dgrad"], per["cfg2_bf16_wgrad"] = bench_cfg2(dev, stream, iters, fc1)
        b_keep_lens = fc1["lens"]
        for k in ("a", "b", "out"):
            fc1.pop(k)
        torch.cuda.empty_cache()
        if want is None or "ep" in want:
            log("per_config: one GPU's share of expert parallelism")
            per["ep8_share_bf16_fc1_swiglu"] = bench_ep_share(dev, stream, iters)
            torch.cuda.empty_cache()
        if want is None or "cfg3" in want:
            log("per_config: MXFP8")
            per["cfg3_mxfp8_fwd"], per["cfg3_mxfp8_quantize_A"] = bench_cfg3(dev, stream, iters)
            torch.cuda.empty_cache()
        if want is None or "cfg3la" in want:
            log("per_config: MXFP8 on line-aligned codes")
            per["cfg3_mxfp8_fwd_line_aligned"] = bench_cfg3_aligned(dev, stream, iters)
            torch.cuda.empty_cache()
        if want is None or "cfg3fp8" in want:
            log("per_config: FP8 with tensor scales")
            per["cfg3_fp8_tensor_fwd"], per["cfg3_fp8_rowwise_fwd"] = bench_cfg3_fp8(dev, stream, iters)
            torch.cuda.empty_cache()
        if want is None or "cfg3fp8dgrad" in want:
            log("per_config: FP8 dgrad")
            per["cfg3_fp8_tensor_dgrad"], per["cfg3_fp8_rowwise_dgrad"] = bench_cfg3_fp8_dgrad(dev, stream, iters)
        if want is None or "cfg3dgrad" in want:
            log("per_config: MXFP8 dgrad")
            per["cfg3_mxfp8_dgrad"] = bench_cfg3_dgrad(dev, stream, iters)
            torch.cuda.empty_cache()
        if want is None or "cfg3wgrad" in want:
            log("per_config: MXFP8 wgrad")
            per["cfg3_mxfp8_wgrad"], per["cfg3_fp8_tensor_wgrad"] = bench_cfg3_wgrad(dev, stream, iters)
            torch.cuda.empty_cache()
        if want is None or "wgradsplit" in want:
            log("per_config: split weight gradient")
            per["wgrad_split_skewed_k512"] = bench_wgrad_split(dev, stream, iters)
            torch.cuda.empty_cache()
        if want is None or "stack" in want:
            log("per_config: expert weight stack")
            per["stack_experts_transpose"], per["stack_experts_mxfp8_caches"] = bench_stack(dev, stream, iters)
        if want is None or "cfg4" in want:
            log("per_config: MXFP4 MLP")
            per["cfg4_mxfp4_mlp"] = bench_cfg4(dev, stream, iters, b_keep_lens)
            torch.cuda.empty_cache()
        if want is None or "fc2bwd" in want:
            log("per_config: FC2 dgrad + SwiGLU backward")
            per["fc2_bf16_dgrad_swiglu_bwd"] = bench_fc2_bwd(dev, stream, iters, b_keep_lens)
            per["fc2_mxfp8_dgrad_swiglu_bwd"] = bench_fc2_bwd_mx(dev, stream, iters, b_keep_lens, ptm.PT_MXFP8_E4M3)
            per["fc2_mxfp4_dgrad_swiglu_bwd"] = bench_fc2_bwd_mx(dev, stream, iters, b_keep_lens, ptm.PT_MXFP4_E2M1)
        attach_traffic(per)
        line["per_config"] = per
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
