"""Float64 brute-force FFN -- TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The exact-arithmetic reference of the bias-free gated FFN of RL-Kernel PR #325
(section "Design"): y = W_down (silu(W_gate x) * (W_up x)), weights [out, in],
and its analytic backward, all in float64 from the same BF16 inputs, with no
intermediate rounding.  It measures how far the BF16-staged tree result is from
the mathematical function (relative L2).
"""
import numpy as np


def _f64(bits, dtype="bf16"):
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "fp16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ffn_fwd(x, w_gate, w_up, w_down, dtype="bf16"):
    x, wg, wu, wd = (_f64(t, dtype) for t in (x, w_gate, w_up, w_down))
    g = x @ wg.T
    u = x @ wu.T
    s = g / (1.0 + np.exp(-g))
    a = s * u
    return {"g": g, "u": u, "a": a, "y": a @ wd.T}


def ffn_bwd(dy, x, w_gate, w_up, w_down, dtype="bf16"):
    dy, x, wg, wu, wd = (_f64(t, dtype) for t in (dy, x, w_gate, w_up, w_down))
    g = x @ wg.T
    u = x @ wu.T
    sig = 1.0 / (1.0 + np.exp(-g))
    s = g * sig
    ds = sig * (1.0 + g * (1.0 - sig))
    a = s * u
    da = dy @ wd
    du = da * s
    dg = da * u * ds
    gl = dg @ wg
    ul = du @ wu
    return {"dA": da, "dG": dg, "dU": du, "G": gl, "U": ul, "dX": gl + ul,
            "dW_gate": dg.T @ x, "dW_up": du.T @ x, "dW_down": dy.T @ a}


def rel_l2(approx_bits, ref64, dtype="bf16"):
    a = _f64(approx_bits, dtype)
    d = np.linalg.norm((a - ref64).ravel())
    n = np.linalg.norm(np.asarray(ref64).ravel())
    return float(d / n) if n > 0 else float(d)
