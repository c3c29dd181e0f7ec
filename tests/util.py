"""Test helpers: device/host conversions and the tolerance metrics.

Tolerances (written here once, used by every parity test):
  * BF16 outputs: max_i |x_i - r_i| / max(|r_i|, rms(r)) <= 1e-2, per expert
    and over all rows, where r is the oracle's exact binary64 result.  The
    rms floor keeps outputs near zero (where any fp32 summation order gives
    a large relative error) from deciding the test.
  * MX outputs: ||x - r||_2 / ||r||_2 <= 2e-2, per expert and over all rows,
    with r the oracle on the same MX operand bytes (exactly dequantised).
  * Quantise outputs and scale bytes: bit-exact.
"""
import numpy as np
import torch

BF16_TOL = 1e-2
MX_TOL = 2e-2


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().numpy().view(np.uint8)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def floored_rel_err(x: np.ndarray, r: np.ndarray) -> float:
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    if r.size == 0:
        return 0.0
    floor = max(float(np.sqrt(np.mean(r * r))), 1e-30)
    return float(np.max(np.abs(x - r) / np.maximum(np.abs(r), floor)))


def norm_err(x: np.ndarray, r: np.ndarray) -> float:
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    d = float(np.linalg.norm(r))
    return float(np.linalg.norm(x - r)) / max(d, 1e-300)


def per_group_max(metric, x, r, group_of_row):
    """Worst metric over the experts present in the sample, and overall."""
    worst = metric(x, r)
    for g in np.unique(group_of_row):
        sel = group_of_row == g
        worst = max(worst, metric(x[sel], r[sel]))
    return worst


def group_of_rows(lens: np.ndarray, rows: np.ndarray) -> np.ndarray:
    offs = np.concatenate([[0], np.cumsum(lens)])
    return np.searchsorted(offs, rows, side="right") - 1


def sample_rows(lens: np.ndarray, per_group: int, seed: int, max_groups=None) -> np.ndarray:
    """First, last and `per_group` random rows of each (or of a seeded subset
    of) non-empty expert, sorted."""
    rng = np.random.default_rng(seed)
    offs = np.concatenate([[0], np.cumsum(lens)])
    groups = [g for g in range(len(lens)) if lens[g] > 0]
    if max_groups is not None and len(groups) > max_groups:
        groups = sorted(rng.choice(groups, size=max_groups, replace=False))
    rows = []
    for g in groups:
        a, b = offs[g], offs[g + 1]
        rows += [a, b - 1]
        rows += list(rng.integers(a, b, size=min(per_group, b - a)))
    return np.unique(np.array(rows, np.int64))


def dev_i64(x, device) -> torch.Tensor:
    return torch.as_tensor(np.asarray(x, np.int64), device=device)


# Workspaces for the persistent kernels: "static" (none: fixed tile order),
# "queue" (the per-XCD tile queues), "swz" (the full size for an MX forward of
# the given shape: queues plus stage-major copies of the scales).  They are
# filled with 0xFF so that a launch relying on leftover contents, rather than
# on what it writes first, goes wrong.
SCHEDS = ["static", "queue"]
MX_SCHEDS = ["static", "queue", "swz"]


def make_ws(device, sched, G=1, M=1, N=1, K=32, dtype=None):
    if sched == "static":
        return None
    import moe_expert_grouped_gemm_amd as ptm
    if sched == "queue":
        n = ptm.pt_grouped_gemm_workspace_size(ptm.PT_OP_FWD, 1, 1, 1, 1, ptm.PT_BF16)
    else:
        n = ptm.pt_grouped_gemm_workspace_size(ptm.PT_OP_FWD, G, M, N, K, dtype)
    return torch.full((n,), 0xFF, dtype=torch.uint8, device=device)
