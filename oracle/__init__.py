"""CPU oracle for the deterministic gated FFN -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or falls back to it, and the two share
no code.  BF16 and FP16 tensors cross this interface as ``numpy.uint16`` bit
patterns; functions with a ``dtype`` argument take "bf16" (default) or "fp16".

``dgf_oracle.c`` is the tree oracle (canonical leaf/tree of RL-Kernel PR #325,
section "Design"); ``fp64.py`` is the float64 brute-force FFN used as an
independent accuracy reference.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dgf_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (plain C11, OpenMP, no FP contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=gnu11", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        L.oracle_block_step.restype = ctypes.c_float
        L.oracle_block_step.argtypes = [ctypes.c_float, P, I64, P, I64, ctypes.c_int]
        L.oracle_leaf_f32.restype = ctypes.c_float
        L.oracle_leaf_f32.argtypes = [P, I64, P, I64, I64]
        L.oracle_dot_tree.restype = ctypes.c_uint16
        L.oracle_dot_tree.argtypes = [P, I64, P, I64, I64]
        L.oracle_dot_subtree.restype = ctypes.c_uint16
        L.oracle_dot_subtree.argtypes = [P, I64, P, I64, I64, I64, I64]
        L.oracle_gemm_tree.restype = None
        L.oracle_gemm_tree.argtypes = [P, I64, I64, P, I64, I64, P, I64, I64, I64, I64]
        L.oracle_tree_combine.restype = ctypes.c_int
        L.oracle_tree_combine.argtypes = [ctypes.POINTER(P), ctypes.c_int, P, I64]
        L.oracle_tree_combine_typed.restype = ctypes.c_int
        L.oracle_tree_combine_typed.argtypes = [ctypes.POINTER(P), ctypes.c_int, P, I64, ctypes.c_int]
        L.oracle_f16_to_f32.restype = ctypes.c_float
        L.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_f32_to_f16.restype = ctypes.c_uint16
        L.oracle_f32_to_f16.argtypes = [ctypes.c_float]
        for f in ("oracle_sigma", "oracle_silu", "oracle_dsilu"):
            getattr(L, f).restype = ctypes.c_float
            getattr(L, f).argtypes = [ctypes.c_float]
        L.oracle_act_fwd.restype = None
        L.oracle_act_fwd.argtypes = [P, P, P, I64]
        L.oracle_act_bwd.restype = None
        L.oracle_act_bwd.argtypes = [P, P, P, P, P, P, I64]
        L.oracle_ffn_fwd.restype = None
        L.oracle_ffn_fwd.argtypes = [P] * 8 + [I64] * 3
        L.oracle_ffn_bwd.restype = None
        L.oracle_ffn_bwd.argtypes = [P] * 17 + [I64] * 3
        # the same functions for a stored type (0 BF16, 1 FP16) given first
        Ci = ctypes.c_int
        L.oracle_block_step_t.restype = ctypes.c_float
        L.oracle_block_step_t.argtypes = [Ci, ctypes.c_float, P, I64, P, I64, Ci]
        L.oracle_block_chains_t.restype = None
        L.oracle_block_chains_t.argtypes = [Ci, P, P, P, P, I64, Ci]
        L.oracle_leaf_f32_t.restype = ctypes.c_float
        L.oracle_leaf_f32_t.argtypes = [Ci, P, I64, P, I64, I64]
        L.oracle_dot_tree_t.restype = ctypes.c_uint16
        L.oracle_dot_tree_t.argtypes = [Ci, P, I64, P, I64, I64]
        L.oracle_dot_subtree_t.restype = ctypes.c_uint16
        L.oracle_dot_subtree_t.argtypes = [Ci, P, I64, P, I64, I64, I64, I64]
        L.oracle_gemm_tree_t.restype = None
        L.oracle_gemm_tree_t.argtypes = [Ci, P, I64, I64, P, I64, I64, P, I64, I64, I64, I64]
        L.oracle_act_fwd_t.restype = None
        L.oracle_act_fwd_t.argtypes = [Ci, P, P, P, I64]
        L.oracle_act_bwd_t.restype = None
        L.oracle_act_bwd_t.argtypes = [Ci, P, P, P, P, P, P, I64]
        L.oracle_ffn_fwd_t.restype = None
        L.oracle_ffn_fwd_t.argtypes = [Ci] + [P] * 8 + [I64] * 3
        L.oracle_ffn_bwd_t.restype = None
        L.oracle_ffn_bwd_t.argtypes = [Ci] + [P] * 17 + [I64] * 3
        _lib = L
    return _lib


_ELEM = {"bf16": 0, "fp16": 1}


def _dt(dtype: str) -> int:
    if dtype not in _ELEM:
        raise ValueError(f"stored type must be bf16 or fp16, got {dtype!r}")
    return _ELEM[dtype]


def _u16(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"expected uint16 BF16 bit patterns, got {a.dtype}")
    return np.ascontiguousarray(a)


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


# ------------------------------------------------------------------ BF16 helpers
def f32_to_bf16_bits(x) -> np.ndarray:
    """Round-to-nearest-even FP32 -> BF16 bits (NaN kept quiet)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = ((u & 0x7F800000) == 0x7F800000) & ((u & 0x7FFFFF) != 0)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return np.where(nan, ((u >> 16) | 0x40).astype(np.uint16), r)


def bf16_bits_to_f32(h) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bits_to_f32(h, dtype: str = "bf16") -> np.ndarray:
    """Stored bits -> float32 (exact for both types)."""
    if _dt(dtype) == 1:
        return np.asarray(h, dtype=np.uint16).view(np.float16).astype(np.float32)
    return bf16_bits_to_f32(h)


# ------------------------------------------------------------------ leaf and tree
def block_step(acc: float, a, b, dtype: str = "bf16") -> np.float32:
    a, b = _u16(a), _u16(b)
    assert a.shape == b.shape and a.ndim == 1 and a.size <= 8
    return np.float32(lib().oracle_block_step_t(_dt(dtype), ctypes.c_float(acc), _p(a), 1, _p(b), 1, a.size))


def block_chains(acc0, a, b, dtype: str = "bf16") -> np.ndarray:
    """Rows r of a, b [n, k] as block steps of 8 in ascending k from acc0[r]
    (float32): what a chain of matrix-core instructions computes per output."""
    a, b = _u16(a), _u16(b)
    acc0 = np.ascontiguousarray(np.asarray(acc0, np.float32)).ravel()
    n, k = a.shape
    assert b.shape == (n, k) and acc0.size == n
    out = np.zeros(n, np.float32)
    lib().oracle_block_chains_t(_dt(dtype), _p(acc0), _p(a), _p(b), _p(out), n, k)
    return out


def leaf_f32(a, b, dtype: str = "bf16") -> np.float32:
    a, b = _u16(a), _u16(b)
    assert a.shape == b.shape and a.ndim == 1 and a.size <= 64
    return np.float32(lib().oracle_leaf_f32_t(_dt(dtype), _p(a), 1, _p(b), 1, a.size))


def dot_tree(a, b, dtype: str = "bf16") -> int:
    """Canonical tree of sum_k a[k]*b[k] -> stored bits."""
    a, b = _u16(a), _u16(b)
    assert a.shape == b.shape and a.ndim == 1
    return int(lib().oracle_dot_tree_t(_dt(dtype), _p(a), 1, _p(b), 1, a.size))


def dot_subtree(a, b, leaf_lo: int, leaf_hi: int, dtype: str = "bf16") -> int:
    """Tree over leaves [leaf_lo, leaf_hi) of the full-length reduction a.b."""
    a, b = _u16(a), _u16(b)
    return int(lib().oracle_dot_subtree_t(_dt(dtype), _p(a), 1, _p(b), 1, a.size, leaf_lo, leaf_hi))


def gemm_tree(A, B, layout: str = "NT", dtype: str = "bf16") -> np.ndarray:
    """Tree GEMM over K.  NT: A [M,K], B [N,K] -> C [M,N] = A B^T.
    NN: A [M,K], B [K,N] -> A B.  TN: A [K,M], B [K,N] -> A^T B."""
    A, B = _u16(A), _u16(B)
    if layout == "NT":
        M, K = A.shape; N, K2 = B.shape
        sam, sak, sbk, sbn = K, 1, 1, K
    elif layout == "NN":
        M, K = A.shape; K2, N = B.shape
        sam, sak, sbk, sbn = K, 1, N, 1
    elif layout == "TN":
        K, M = A.shape; K2, N = B.shape
        sam, sak, sbk, sbn = 1, M, N, 1
    else:
        raise ValueError(layout)
    assert K == K2
    C = np.zeros((M, N), np.uint16)
    lib().oracle_gemm_tree_t(_dt(dtype), _p(A), sam, sak, _p(B), sbk, sbn, _p(C), N, M, N, K)
    return C


def tree_combine(parts) -> np.ndarray:
    parts = [_u16(p).ravel() for p in parts]
    n = parts[0].size
    assert all(p.size == n for p in parts)
    arr = (ctypes.c_void_p * len(parts))(*[p.ctypes.data for p in parts])
    out = np.zeros(n, np.uint16)
    rc = lib().oracle_tree_combine(arr, len(parts), _p(out), n)
    if rc != 0:
        raise ValueError(f"unsupported part count {len(parts)}")
    return out


_DTYPES = {"bf16": (0, np.uint16), "fp16": (1, np.uint16), "fp32": (2, np.float32)}


def tree_combine_typed(parts, dtype: str) -> np.ndarray:
    """The balanced rank tree over S parts in BF16, FP16 (bit patterns as
    uint16) or FP32 (float32 arrays)."""
    code, np_t = _DTYPES[dtype]
    parts = [np.ascontiguousarray(np.asarray(p).astype(np_t, copy=False)).ravel() for p in parts]
    n = parts[0].size
    assert all(p.size == n for p in parts)
    arr = (ctypes.c_void_p * len(parts))(*[p.ctypes.data for p in parts])
    out = np.zeros(n, np_t)
    rc = lib().oracle_tree_combine_typed(arr, len(parts), out.ctypes.data, n, code)
    if rc != 0:
        raise ValueError(f"unsupported part count {len(parts)} or dtype {dtype}")
    return out


def f16_to_f32(h: int) -> np.float32:
    return np.float32(lib().oracle_f16_to_f32(int(h)))


def f32_to_f16(x) -> int:
    return int(lib().oracle_f32_to_f16(ctypes.c_float(float(x))))


# ------------------------------------------------------------------ activation
def sigma(g: float) -> np.float32:
    return np.float32(lib().oracle_sigma(ctypes.c_float(g)))


def silu(g: float) -> np.float32:
    return np.float32(lib().oracle_silu(ctypes.c_float(g)))


def dsilu(g: float) -> np.float32:
    return np.float32(lib().oracle_dsilu(ctypes.c_float(g)))


def act_fwd(g, u, dtype: str = "bf16") -> np.ndarray:
    g, u = _u16(g), _u16(u)
    a = np.zeros_like(g)
    lib().oracle_act_fwd_t(_dt(dtype), _p(g), _p(u), _p(a), g.size)
    return a


def act_bwd(da, g, u, dtype: str = "bf16"):
    da, g, u = _u16(da), _u16(g), _u16(u)
    dg, du, a = np.zeros_like(g), np.zeros_like(g), np.zeros_like(g)
    lib().oracle_act_bwd_t(_dt(dtype), _p(da), _p(g), _p(u), _p(dg), _p(du), _p(a), g.size)
    return dg, du, a


# ------------------------------------------------------------------ FFN
def ffn_fwd(x, w_gate, w_up, w_down, dtype: str = "bf16"):
    """Returns dict with g, u, a, y (stored bits)."""
    x, wg, wu, wd = _u16(x), _u16(w_gate), _u16(w_up), _u16(w_down)
    M, H = x.shape
    I = wg.shape[0]
    assert wg.shape == (I, H) and wu.shape == (I, H) and wd.shape == (H, I)
    g = np.zeros((M, I), np.uint16); u = np.zeros_like(g); a = np.zeros_like(g)
    y = np.zeros((M, H), np.uint16)
    lib().oracle_ffn_fwd_t(_dt(dtype), _p(x), _p(wg), _p(wu), _p(wd), _p(g), _p(u), _p(a), _p(y), M, H, I)
    return {"g": g, "u": u, "a": a, "y": y}


def ffn_bwd(dy, x, g, u, w_gate, w_up, w_down, dtype: str = "bf16"):
    """Returns dict with dA, dG, dU, a, G, U, dX, dW_gate, dW_up, dW_down."""
    dy, x, g, u = _u16(dy), _u16(x), _u16(g), _u16(u)
    wg, wu, wd = _u16(w_gate), _u16(w_up), _u16(w_down)
    M, H = x.shape
    I = wg.shape[0]
    assert dy.shape == (M, H) and g.shape == (M, I) and u.shape == (M, I)
    z = lambda *s: np.zeros(s, np.uint16)
    da, dg, du, a = z(M, I), z(M, I), z(M, I), z(M, I)
    gl, ul, dx = z(M, H), z(M, H), z(M, H)
    dwg, dwu, dwd = z(I, H), z(I, H), z(H, I)
    lib().oracle_ffn_bwd_t(_dt(dtype), _p(dy), _p(x), _p(g), _p(u), _p(wg), _p(wu), _p(wd),
                           _p(da), _p(dg), _p(du), _p(a), _p(gl), _p(ul), _p(dx),
                           _p(dwg), _p(dwu), _p(dwd), M, H, I)
    return {"dA": da, "dG": dg, "dU": du, "a": a, "G": gl, "U": ul, "dX": dx,
            "dW_gate": dwg, "dW_up": dwu, "dW_down": dwd}
