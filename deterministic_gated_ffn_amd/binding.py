"""Python binding of libdgf (include/dgf.h): argument marshalling only.

Every step of the path runs in the HIP library; this module turns torch
tensors into device pointers, leading dimensions and the current HIP stream,
allocates outputs and the workspace the library asks for, and raises on any
non-OK status.  There is no fallback: without the built library (or without a
GPU) every call raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdgf.so")
_lib = None

DGF_NT, DGF_NN, DGF_TN = 0, 1, 2
_LAYOUTS = {"NT": DGF_NT, "NN": DGF_NN, "TN": DGF_TN}

STATUS = {0: "DGF_OK", 1: "DGF_EINVAL", 2: "DGF_EUNSUPPORTED", 3: "DGF_EWORKSPACE", 4: "DGF_EHIP"}

# (name, restype, argtypes) of every exported entry point
_P, _I64, _SZ, _I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
SIGNATURES = {
    "dgf_abi_version": (_I, []),
    "dgf_leaf_size": (_I, []),
    "dgf_last_error": (ctypes.c_char_p, []),
    "dgf_ffn_fwd_workspace": (_SZ, [_I64, _I64, _I64]),
    "dgf_ffn_fwd": (_I, [_P, _I64, _P, _I64, _P, _I64, _P, _I64, _P, _I64, _P, _P, _I64,
                         _I64, _I64, _I64, _P, _SZ, _P]),
    "dgf_ffn_fwd_static": (_I, [_P, _I64, _P, _I64, _P, _I64, _P, _I64, _P, _I64, _P, _P, _I64,
                                _I64, _I64, _I64, _P]),
    "dgf_ffn_bwd_workspace": (_SZ, [_I64, _I64, _I64]),
    "dgf_ffn_bwd": (_I, [_P, _I64, _P, _I64, _P, _P, _I64, _P, _I64, _P, _I64, _P, _I64,
                         _P, _P, _P, _I64, _P, _I64, _P, _I64, _P, _I64,
                         _I64, _I64, _I64, _P, _SZ, _P]),
    "dgf_tree_combine": (_I, [ctypes.POINTER(_P), _I, _P, _I64, _P]),
    "dgf_tree_combine_typed": (_I, [ctypes.POINTER(_P), _I, _P, _I64, _I, _P]),
    "dgf_gemm_tree_workspace": (_SZ, [_I, _I64, _I64, _I64]),
    "dgf_gemm_tree": (_I, [_I, _P, _I64, _P, _I64, _P, _I64, _I64, _I64, _I64, _P, _SZ, _P]),
    "dgf_act_fwd": (_I, [_P, _P, _P, _I64, _P]),
    "dgf_act_bwd": (_I, [_P, _P, _P, _P, _P, _P, _I64, _P]),
    "dgf_ffn_fwd_typed": (_I, [_P, _I64, _P, _I64, _P, _I64, _P, _I64, _P, _I64, _P, _P, _I64,
                               _I64, _I64, _I64, _P, _SZ, _I, _P]),
    "dgf_ffn_bwd_typed": (_I, [_P, _I64, _P, _I64, _P, _P, _I64, _P, _I64, _P, _I64, _P, _I64,
                               _P, _P, _P, _I64, _P, _I64, _P, _I64, _P, _I64,
                               _I64, _I64, _I64, _P, _SZ, _I, _P]),
    "dgf_gemm_tree_typed": (_I, [_I, _P, _I64, _P, _I64, _P, _I64, _I64, _I64, _I64, _P, _SZ, _I, _P]),
    "dgf_act_fwd_typed": (_I, [_P, _P, _P, _I64, _I, _P]),
    "dgf_act_bwd_typed": (_I, [_P, _P, _P, _P, _P, _P, _I64, _I, _P]),
    "dgf_profile_begin": (_I, [ctypes.POINTER(_P), _I]),
    "dgf_profile_end": (_I, []),
    "dgf_profile_name": (ctypes.c_char_p, [_I]),
}


class DgfError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: {STATUS.get(status, status)}: {msg}")
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Load libdgf.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"libdgf.so not built at {_LIB_PATH}: run `python -m deterministic_gated_ffn_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int, where: str):
    if status != 0:
        raise DgfError(status, where, load().dgf_last_error().decode())


def _stream(stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _on(stream):
    """Allocate on the launch stream: outputs and the workspace come from that
    stream's pool, so the caching allocator cannot hand a block to another
    stream while the launched kernels still use it."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


DGF_BF16, DGF_FP16, DGF_FP32 = 0, 1, 2
# stored types of the FFN and the tree GEMM: BF16 (the untyped entry points) or FP16
_STORED = {torch.bfloat16: DGF_BF16, torch.float16: DGF_FP16}


def _stored(*ts) -> int:
    """The dtype code shared by every given tensor (BF16 or FP16)."""
    dt = ts[0].dtype
    if dt not in _STORED:
        raise TypeError(f"expected bfloat16 or float16 tensors, got {dt}")
    for t in ts:
        if t.dtype != dt:
            raise TypeError(f"all tensors must share one dtype ({dt} and {t.dtype} given)")
    return _STORED[dt]


def _mat(t: torch.Tensor, name: str):
    """(pointer, leading dimension) of a row-major BF16 or FP16 matrix view on the GPU."""
    if t.dtype not in _STORED:
        raise TypeError(f"{name}: expected bfloat16 or float16, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: expected a GPU tensor")
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name}: expected a 2-D row-major view (stride(1) == 1)")
    return t.data_ptr(), t.stride(0)


def _empty(rows: int, cols: int, like: torch.Tensor, ld: int | None = None) -> torch.Tensor:
    """Row-major [rows, cols] of like's dtype whose leading dimension is a multiple of 8."""
    ld = ld or ((cols + 7) // 8) * 8
    buf = torch.empty((rows, ld), dtype=like.dtype, device=like.device)
    return buf[:, :cols]


def _workspace(nbytes: int, like: torch.Tensor) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=like.device)


# ---------------------------------------------------------------- entry points
def abi_version() -> int:
    return load().dgf_abi_version()


def leaf_size() -> int:
    return load().dgf_leaf_size()


def ffn_fwd(x, w_gate, w_up, w_down, training: bool = False, out=None, stream=None):
    """y = W_down (silu(W_gate x) * (W_up x)) through the canonical tree, in the
    tensors' stored type (BF16: dgf_ffn_fwd, FP16: dgf_ffn_fwd_typed).
    Returns y, or (y, g, u) when training."""
    with _on(stream):
        return _ffn_fwd(x, w_gate, w_up, w_down, training, out, stream)


def _ffn_fwd(x, w_gate, w_up, w_down, training, out, stream):
    L = load()
    dt = _stored(x, w_gate, w_up, w_down, *([out] if out is not None else []))
    M, H = x.shape
    I = w_gate.shape[0]
    y = out if out is not None else _empty(M, H, x)
    g = u = None
    gp = up = None
    ld_gu = 0
    if training:
        g, u = _empty(M, I, x), _empty(M, I, x)
        gp, up, ld_gu = g.data_ptr(), u.data_ptr(), g.stride(0)
    ws = _workspace(L.dgf_ffn_fwd_workspace(M, H, I), x)
    xp, ldx = _mat(x, "x"); wg, ldwg = _mat(w_gate, "w_gate"); wu, ldwu = _mat(w_up, "w_up")
    wd, ldwd = _mat(w_down, "w_down"); yp, ldy = _mat(y, "y")
    if dt == DGF_BF16:
        _check(L.dgf_ffn_fwd(xp, ldx, wg, ldwg, wu, ldwu, wd, ldwd, yp, ldy, gp, up, ld_gu,
                             M, H, I, ws.data_ptr(), ws.numel(), _stream(stream)), "dgf_ffn_fwd")
    else:
        _check(L.dgf_ffn_fwd_typed(xp, ldx, wg, ldwg, wu, ldwu, wd, ldwd, yp, ldy, gp, up, ld_gu,
                                   M, H, I, ws.data_ptr(), ws.numel(), dt, _stream(stream)), "dgf_ffn_fwd_typed")
    return (y, g, u) if training else y


STATIC_SCRATCH_BYTES = 16 << 20  # DGF_STATIC_SCRATCH_BYTES


def ffn_fwd_static(x, w_gate, w_up, w_down, y, g=None, u=None, stream=None):
    """dgf_ffn_fwd_static: the forward into caller-given y (and g, u when
    training) with the library's own scratch; allocates nothing."""
    L = load()
    if (g is None) != (u is None):
        raise ValueError("give both g and u (training) or neither (inference)")
    if _stored(x, w_gate, w_up, w_down, y, *([g, u] if g is not None else [])) != DGF_BF16:
        raise TypeError("dgf_ffn_fwd_static takes bfloat16 tensors only")
    M, H = x.shape
    I = w_gate.shape[0]
    xp, ldx = _mat(x, "x"); wg, ldwg = _mat(w_gate, "w_gate"); wu, ldwu = _mat(w_up, "w_up")
    wd, ldwd = _mat(w_down, "w_down"); yp, ldy = _mat(y, "y")
    gp = up = None
    ld_gu = 0
    if g is not None:
        (gp, ld_gu), (up, ldu) = _mat(g, "g"), _mat(u, "u")
        if ldu != ld_gu:
            raise ValueError("g and u must share a leading dimension")
    _check(L.dgf_ffn_fwd_static(xp, ldx, wg, ldwg, wu, ldwu, wd, ldwd, yp, ldy, gp, up, ld_gu, M, H, I,
                                _stream(stream)), "dgf_ffn_fwd_static")
    return y


def ffn_bwd(dy, x, g, u, w_gate, w_up, w_down, lanes: bool = False, stream=None):
    """Returns dict dX, dW_gate, dW_up, dW_down (and G, U lanes if lanes=True),
    in the tensors' stored type (BF16: dgf_ffn_bwd, FP16: dgf_ffn_bwd_typed)."""
    with _on(stream):
        return _ffn_bwd(dy, x, g, u, w_gate, w_up, w_down, lanes, stream)


def _ffn_bwd(dy, x, g, u, w_gate, w_up, w_down, lanes, stream):
    L = load()
    dt = _stored(dy, x, g, u, w_gate, w_up, w_down)
    M, H = x.shape
    I = w_gate.shape[0]
    dx = _empty(M, H, x)
    gl = _empty(M, H, x, ld=dx.stride(0)) if lanes else None
    ul = _empty(M, H, x, ld=dx.stride(0)) if lanes else None
    dwg, dwu, dwd = _empty(I, H, x), _empty(I, H, x), _empty(H, I, x)
    ws = _workspace(L.dgf_ffn_bwd_workspace(M, H, I), x)
    dyp, lddy = _mat(dy, "dy"); xp, ldx = _mat(x, "x"); gp, ldg = _mat(g, "g"); upp, ldu = _mat(u, "u")
    if ldg != ldu:
        raise ValueError("g and u must share a leading dimension")
    wg, ldwg = _mat(w_gate, "w_gate"); wu, ldwu = _mat(w_up, "w_up"); wd, ldwd = _mat(w_down, "w_down")
    args = (dyp, lddy, xp, ldx, gp, upp, ldg, wg, ldwg, wu, ldwu, wd, ldwd,
            dx.data_ptr(), gl.data_ptr() if lanes else None, ul.data_ptr() if lanes else None,
            dx.stride(0), dwg.data_ptr(), dwg.stride(0), dwu.data_ptr(), dwu.stride(0),
            dwd.data_ptr(), dwd.stride(0), M, H, I, ws.data_ptr(), ws.numel())
    if dt == DGF_BF16:
        _check(L.dgf_ffn_bwd(*args, _stream(stream)), "dgf_ffn_bwd")
    else:
        _check(L.dgf_ffn_bwd_typed(*args, dt, _stream(stream)), "dgf_ffn_bwd_typed")
    r = {"dX": dx, "dW_gate": dwg, "dW_up": dwu, "dW_down": dwd}
    if lanes:
        r["G"], r["U"] = gl, ul
    return r


_COMBINE_DTYPES = {torch.bfloat16: DGF_BF16, torch.float16: DGF_FP16, torch.float32: DGF_FP32}


def tree_combine(parts, out=None, stream=None):
    """Balanced combine of S in {1,2,4,8} equally sized tensors (rank order);
    BF16, FP16 or FP32, all parts of one dtype."""
    with _on(stream):
        return _tree_combine(parts, out, stream)


def _tree_combine(parts, out, stream):
    L = load()
    parts = list(parts)
    n = parts[0].numel()
    dt = parts[0].dtype
    if dt not in _COMBINE_DTYPES:
        raise ValueError(f"tree_combine takes bfloat16, float16 or float32, not {dt}")
    for t in parts:
        if t.dtype != dt or not t.is_cuda or t.numel() != n or not t.is_contiguous():
            raise ValueError("parts must be contiguous GPU tensors of one dtype and size")
    out = out if out is not None else torch.empty_like(parts[0])
    arr = (ctypes.c_void_p * len(parts))(*[t.data_ptr() for t in parts])
    if dt == torch.bfloat16:
        _check(L.dgf_tree_combine(arr, len(parts), out.data_ptr(), n, _stream(stream)), "dgf_tree_combine")
    else:
        _check(L.dgf_tree_combine_typed(arr, len(parts), out.data_ptr(), n, _COMBINE_DTYPES[dt], _stream(stream)),
               "dgf_tree_combine_typed")
    return out


def tree_combine_ptrs(ptrs, S: int, out_ptr: int, n: int, stream=None, dtype: int = DGF_BF16):
    """Raw-pointer form (offset or unaligned views)."""
    L = load()
    arr = (ctypes.c_void_p * len(ptrs))(*ptrs)
    _check(L.dgf_tree_combine_typed(arr, S, out_ptr, n, dtype, _stream(stream)), "dgf_tree_combine_typed")


def gemm_tree(layout: str, A, B, out=None, stream=None):
    """NT: A [M,K], B [N,K]; NN: A [M,K], B [K,N]; TN: A [K,M], B [K,N] -> C [M,N],
    in the operands' stored type (BF16: dgf_gemm_tree, FP16: dgf_gemm_tree_typed)."""
    with _on(stream):
        return _gemm_tree(layout, A, B, out, stream)


def _gemm_tree(layout, A, B, out, stream):
    L = load()
    dt = _stored(A, B, *([out] if out is not None else []))
    lay = _LAYOUTS[layout]
    if layout == "NT":
        (M, K), N = A.shape, B.shape[0]
    elif layout == "NN":
        (M, K), N = A.shape, B.shape[1]
    else:
        (K, M), N = A.shape, B.shape[1]
    C = out if out is not None else _empty(M, N, A)
    ws = _workspace(L.dgf_gemm_tree_workspace(lay, M, N, K), A)
    ap, lda = _mat(A, "A"); bp, ldb = _mat(B, "B"); cp, ldc = _mat(C, "C")
    if dt == DGF_BF16:
        _check(L.dgf_gemm_tree(lay, ap, lda, bp, ldb, cp, ldc, M, N, K, ws.data_ptr(), ws.numel(), _stream(stream)),
               "dgf_gemm_tree")
    else:
        _check(L.dgf_gemm_tree_typed(lay, ap, lda, bp, ldb, cp, ldc, M, N, K, ws.data_ptr(), ws.numel(), dt,
                                     _stream(stream)), "dgf_gemm_tree_typed")
    return C


def _flat(t: torch.Tensor, name: str) -> int:
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous GPU tensor")
    return t.data_ptr()


def act_fwd(g, u, stream=None):
    """a = rnd(silu(g) u) elementwise in the stored type of g and u."""
    L = load()
    dt = _stored(g, u)
    if u.numel() != g.numel():
        raise ValueError("g and u must have the same size")
    with _on(stream):
        a = torch.empty_like(g)
    gp, up = _flat(g, "g"), _flat(u, "u")
    if dt == DGF_BF16:
        _check(L.dgf_act_fwd(gp, up, a.data_ptr(), g.numel(), _stream(stream)), "dgf_act_fwd")
    else:
        _check(L.dgf_act_fwd_typed(gp, up, a.data_ptr(), g.numel(), dt, _stream(stream)), "dgf_act_fwd_typed")
    return a


def act_bwd(da, g, u, stream=None):
    """dG, dU and the recomputed a elementwise in the stored type of da, g, u."""
    L = load()
    dt = _stored(da, g, u)
    if u.numel() != g.numel() or da.numel() != g.numel():
        raise ValueError("da, g and u must have the same size")
    with _on(stream):
        dg, du, a = torch.empty_like(g), torch.empty_like(g), torch.empty_like(g)
    ptrs = (_flat(da, "da"), _flat(g, "g"), _flat(u, "u"), dg.data_ptr(), du.data_ptr(), a.data_ptr(), g.numel())
    if dt == DGF_BF16:
        _check(L.dgf_act_bwd(*ptrs, _stream(stream)), "dgf_act_bwd")
    else:
        _check(L.dgf_act_bwd_typed(*ptrs, dt, _stream(stream)), "dgf_act_bwd_typed")
    return dg, du, a


class KernelTimer:
    """Times every kernel the library launches between start() and stop() with
    HIP events recorded on the launch stream (the library's timing hook)."""

    def __init__(self, max_kernels: int = 4096):
        self.n = max_kernels
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(2 * max_kernels)]
        s = torch.cuda.current_stream()
        for e in self.events:  # materialise the underlying HIP events
            e.record(s)
        torch.cuda.synchronize()
        self._arr = (ctypes.c_void_p * (2 * max_kernels))(*[e.cuda_event for e in self.events])
        self.count = 0
        self.names = []

    def start(self):
        _check(load().dgf_profile_begin(self._arr, self.n), "dgf_profile_begin")

    def stop(self):
        L = load()
        self.count = L.dgf_profile_end()
        self.names = [L.dgf_profile_name(k).decode() for k in range(min(self.count, self.n))]
        return self

    def durations_ms(self):
        """[(name, ms)] for each timed launch (call after synchronising)."""
        return [(self.names[k], self.events[2 * k].elapsed_time(self.events[2 * k + 1]))
                for k in range(min(self.count, self.n))]
