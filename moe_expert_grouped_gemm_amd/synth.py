"""Seeded synthetic inputs for the grouped GEMM: routing and tensor values.

This module holds no arithmetic of the method itself (no GEMM, no SwiGLU, no
quantisation): it draws expert group sizes from a synthetic router and draws
bf16 tensors / raw MX bytes from seeded generators.  Both the HIP path and the
oracle consume exactly the bits produced here.

Workloads follow the shapes the pages describe: DeepSeek-V4-Flash routes every
token to 6 of 256 experts with hidden size 4096 (blog "Enabling
DeepSeek-V4-Flash Training on AMD Instinct MI355X GPUs with Primus", opening
section and section "Expert parallelism: DeepEP and the grouped GEMM"), and a
GPT-OSS-20B-style MoE (Primus-Turbo README, "What's New": pad-aware paths for
GPT-OSS-20B-style MoE).  No trained router or dataset is involved; group sizes
come from seeded synthetic logits as described per function.
"""
from __future__ import annotations

import numpy as np
import torch


# ----------------------------------------------------------------- routing
def lens_multinomial(M: int, G: int, seed: int, n_empty: int = 1) -> np.ndarray:
    """Tiny case: `n_empty` seeded experts get no rows, the rest share M rows
    by a uniform multinomial draw."""
    rng = np.random.Generator(np.random.PCG64(seed))
    empty = rng.choice(G, size=n_empty, replace=False)
    p = np.ones(G)
    p[empty] = 0.0
    p /= p.sum()
    return rng.multinomial(M, p).astype(np.int64)


def lens_topk_gaussian(tokens: int, G: int, topk: int, seed: int,
                       bias_std: float = 0.5, n_masked: int = 4) -> np.ndarray:
    """Imbalanced routing: logits z[t,e] + b[e] with z ~ N(0,1) per token and
    a per-expert bias b ~ N(0, bias_std^2); `n_masked` seeded experts never
    win; each token takes its top-k experts (ties to the lower index)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    bias = rng.normal(0.0, bias_std, size=G)
    masked = rng.choice(G, size=n_masked, replace=False)
    bias[masked] = -np.inf
    lens = np.zeros(G, np.int64)
    for t0 in range(0, tokens, 1024):
        z = rng.normal(0.0, 1.0, size=(min(1024, tokens - t0), G)) + bias
        top = np.argsort(-z, axis=1, kind="stable")[:, :topk]
        lens += np.bincount(top.ravel(), minlength=G)
    return lens


def lens_zipf_distinct(tokens: int, G: int, topk: int, s: float, seed: int) -> np.ndarray:
    """Skewed routing: expert popularity p_r ~ r^-s over a seeded permutation
    of the experts; each token picks `topk` distinct experts by Gumbel-top-k
    on log p (so no expert can take more rows than there are tokens)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    perm = rng.permutation(G)
    logp = np.empty(G)
    logp[perm] = -s * np.log(np.arange(1, G + 1, dtype=np.float64))
    lens = np.zeros(G, np.int64)
    for t0 in range(0, tokens, 4096):
        n = min(4096, tokens - t0)
        gum = rng.gumbel(size=(n, G)) + logp
        top = np.argsort(-gum, axis=1, kind="stable")[:, :topk]
        lens += np.bincount(top.ravel(), minlength=G)
    return lens


def offsets(lens: np.ndarray) -> np.ndarray:
    """Exclusive prefix sum, G+1 entries (start row of each expert, then M)."""
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


# ----------------------------------------------------------------- tensors
def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def randn_bf16(shape, seed: int, std: float = 1.0, device="cpu",
               outlier_frac: float = 0.0, outlier_mult: float = 50.0,
               chunk_rows: int = 1 << 14) -> torch.Tensor:
    """bf16 tensor of N(0, std^2) values drawn in fp32 and rounded by torch.

    With outlier_frac > 0 a seeded fraction of the elements is multiplied by
    outlier_mult before the rounding.  Drawn in row chunks to bound the
    temporary fp32 memory; the chunking is part of the recipe (same seed,
    same bits).
    """
    shape = tuple(int(s) for s in shape)
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1, shape[-1]) if len(shape) > 1 else out.view(1, -1)
    g = _gen(seed, device)
    for r0 in range(0, flat.shape[0], chunk_rows):
        r1 = min(flat.shape[0], r0 + chunk_rows)
        v = torch.randn((r1 - r0, flat.shape[1]), generator=g, device=device,
                        dtype=torch.float32)
        if std != 1.0:
            v.mul_(std)
        if outlier_frac > 0.0:
            sel = torch.rand(v.shape, generator=g, device=device) < outlier_frac
            v = torch.where(sel, v * outlier_mult, v)
        flat[r0:r1].copy_(v)
    return out


def random_mx_codes(rows: int, cols: int, fmt: str, seed: int, device="cpu",
                    scale_lo: int = 120, scale_hi: int = 134):
    """Random MX operand: uniform finite element codes and E8M0 scale bytes in
    [scale_lo, scale_hi].  fmt is "e4m3" ([rows, cols] bytes) or "e2m1"
    ([rows, cols/2] bytes, two codes each).  Returns (codes, scales) uint8."""
    g = _gen(seed, device)
    if fmt == "e4m3":
        q = torch.randint(0, 256, (rows, cols), generator=g, device=device, dtype=torch.int32)
        # 0x7F and 0xFF encode NaN: move them to the neighbouring finite code
        q = torch.where((q & 0x7F) == 0x7F, q - 1, q).to(torch.uint8)
    elif fmt == "e2m1":
        q = torch.randint(0, 256, (rows, cols // 2), generator=g, device=device,
                          dtype=torch.int32).to(torch.uint8)
    else:
        raise ValueError(fmt)
    s = torch.randint(scale_lo, scale_hi + 1, (rows, cols // 32), generator=g,
                      device=device, dtype=torch.int32).to(torch.uint8)
    return q, s


def integer_bf16(shape, seed: int, lo: int = -4, hi: int = 4, device="cpu") -> torch.Tensor:
    """bf16 tensor of small integers in [lo, hi] (exactly representable)."""
    g = _gen(seed, device)
    v = torch.randint(lo, hi + 1, tuple(shape), generator=g, device=device, dtype=torch.int32)
    return v.to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw uint16 bits of a bf16 tensor, on the host."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().numpy().view(np.uint8)
