"""CPU check of the library's integer MX rules in common.hpp, compiled for
the host: the E8M0 scale rule that every SwiGLU -> MXFP4 epilogue uses
(mx_scale_byte) and the integer encoder of the 128 x 256 kernels' epilogue
(mx_encode; the 256 x 256 kernels encode with the hardware conversion the
row quantiser uses, pinned on the GPU).  Compared byte for byte with the
oracle's quantiser over every finite bf16 pattern combined with every scale
byte a 32-value block holding it can reach.

Construction: for each exponent field `ea` of a block maximum (from emax,
where the scale byte first leaves 0, up to 254), blocks hold one element
2^(ea - 127) and then 31 patterns from all those whose exponent field is at
most `ea` (both signs, zeros and subnormals included), so the block maximum
keeps exponent field `ea` and the scale byte is clamp(ea - emax, 0, 254).
Every (pattern, reachable scale byte) pair appears at least once: about
8.4 million for each element format.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

from conftest import ROOT

SRC = os.path.join(ROOT, "tests", "csrc", "mx_encode_host.cpp")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def host_encoder(tmp_path_factory):
    so = str(tmp_path_factory.mktemp("enc") / "mx_encode_host.so")
    subprocess.run([HIPCC, "-x", "hip", "--offload-host-only", "-O2", "-std=c++17", "-shared", "-fPIC", SRC,
                    "-o", so], check=True)
    lib = ctypes.CDLL(so)
    fn = lib.ptgg_host_mx_encode_blocks
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]

    def run(x: np.ndarray, fmt: int):
        x = np.ascontiguousarray(x, np.uint16)
        nb = x.size // 32
        q = np.zeros(nb * (32 if fmt == 0 else 16), np.uint8)
        s = np.zeros(nb, np.uint8)
        assert fn(x.ctypes.data, nb, fmt, q.ctypes.data, s.ctypes.data) == 0
        return q.reshape(nb, -1), s
    return run


def exhaustive_blocks(emax: int) -> np.ndarray:
    """[nblocks, 32] bf16 bit patterns, as described in the module docstring."""
    mant = np.arange(128, dtype=np.uint16)
    blocks = []
    for ea in range(emax, 255):
        efs = np.arange(ea + 1, dtype=np.uint16)
        mags = ((efs[:, None] << 7) | mant[None, :]).ravel()
        pats = np.concatenate([mags, mags | np.uint16(0x8000)])
        pad = (-pats.size) % 31
        pats = np.concatenate([pats, np.zeros(pad, np.uint16)]).reshape(-1, 31)
        head = np.full((pats.shape[0], 1), ea << 7, np.uint16)
        blocks.append(np.concatenate([head, pats], axis=1))
    return np.concatenate(blocks)


@pytest.mark.parametrize("fmt,emax", [(0, 8), (1, 2)], ids=["e4m3", "e2m1"])
def test_epilogue_encoder_matches_oracle_exhaustively(orc, host_encoder, fmt, emax):
    x = exhaustive_blocks(emax)
    # every finite pattern with every reachable scale byte is present
    ef = (x[:, 1:] >> 7) & 0xFF
    assert ef.max() <= 254
    assert len(np.unique(x[:, 1:])) == 2 * 255 * 128
    q, s = host_encoder(x, fmt)
    rq, rs = orc.mx_quantize(x, orc.E4M3 if fmt == 0 else orc.E2M1)
    assert (s == rs.ravel()).all()
    assert (s == np.clip((x[:, 0] >> 7).astype(np.int64) - emax, 0, 254)).all()
    bad = np.nonzero((q != rq).any(axis=1))[0]
    assert bad.size == 0, f"{bad.size} blocks differ, first {x[bad[0]].tolist()}"


def test_harness_is_sensitive(orc, host_encoder):
    # a planted error in the oracle's output (one code off by one) is caught
    x = exhaustive_blocks(8)[:2000]
    q, s = host_encoder(x, 0)
    rq, rs = orc.mx_quantize(x, orc.E4M3)
    rq = rq.copy()
    rq[1234, 7] ^= 1
    assert (q != rq).any()
