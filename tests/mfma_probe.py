"""Build and call the MFMA probe (tests/mfma_probe.hip): test infrastructure
that runs the 16x16x32 MFMA instructions directly, so the oracle's block rule
can be checked against the instruction with any accumulator input."""
import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mfma_probe.hip")
LIB = os.path.join(HERE, "libmfma_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build() -> str:
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
           SRC, "-o", tmp]
    subprocess.run(cmd, check=True, capture_output=True)
    os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is not built (python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB)
        L.mfma_probe.restype = ctypes.c_int
        L.mfma_probe.argtypes = [ctypes.c_int] + [ctypes.c_void_p] * 4 + [ctypes.c_int] * 2
        _lib = L
    return _lib


def to_lanes(A, B, C):
    """A [n, 16, 32 s], B [n, 32 s, 16] (16-bit patterns), C [n, 16, 16] float32 ->
    per-lane operand slots [n, s, 64, 8] and accumulator slots [n, 64, 4]."""
    n, _, K = A.shape
    s = K // 32
    lane = np.arange(64)
    r, g = lane % 16, lane // 16
    Al = np.empty((n, s, 64, 8), np.uint16)
    Bl = np.empty((n, s, 64, 8), np.uint16)
    for t in range(s):
        k = 32 * t + 8 * g[:, None] + np.arange(8)[None, :]
        Al[:, t] = A[:, r[:, None], k]
        Bl[:, t] = B[:, k, r[:, None]]
    rows = 4 * g[:, None] + np.arange(4)[None, :]
    Cl = np.ascontiguousarray(C[:, rows, r[:, None]])
    return Al, Bl, Cl


def from_lanes(Dl):
    n = Dl.shape[0]
    D = np.zeros((n, 16, 16), np.float32)
    lane = np.arange(64)
    r, g = lane % 16, lane // 16
    rows = 4 * g[:, None] + np.arange(4)[None, :]
    D[:, rows, r[:, None]] = Dl
    return D


def run(dtype: int, A, B, C):
    """D = the chained MFMAs over K = A.shape[2] (a multiple of 32) from C, on the GPU."""
    import torch
    Al, Bl, Cl = to_lanes(A, B, C)
    n, s = Al.shape[0], Al.shape[1]
    ta = torch.from_numpy(np.ascontiguousarray(Al).view(np.int16)).cuda()
    tb = torch.from_numpy(np.ascontiguousarray(Bl).view(np.int16)).cuda()
    tc = torch.from_numpy(Cl).cuda()
    td = torch.empty_like(tc)
    assert ta.numel() == n * s * 64 * 8 and tc.numel() == n * 64 * 4
    rc = lib().mfma_probe(dtype, ta.data_ptr(), tb.data_ptr(), tc.data_ptr(), td.data_ptr(), n, s)
    if rc != 0:
        raise RuntimeError(f"mfma_probe failed: hipError {rc}")
    return from_lanes(td.cpu().numpy())
