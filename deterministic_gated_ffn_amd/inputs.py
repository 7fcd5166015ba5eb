"""Seeded synthetic inputs for the deterministic gated FFN.

This module holds input generation only -- no step of the FFN's arithmetic --
so that the HIP path's tests and the CPU oracle can be fed the same tensors.

Recipe (the pages load no model or dataset: RL-Kernel PR #325, section "Note"):
  * tiny case (M=4, H=256, I=768): one CPU generator seeded 0, drawn in the order
    x, W_gate, W_up, W_down, dY; standard normal in FP32, weights scaled by 0.02,
    then rounded to BF16 (nearest even);
  * Qwen3-8B-shaped cases (H=4096, I=12288): weights from a generator seeded 0
    (W_gate, W_up, W_down, each N(0,1)*0.02); activations from a generator
    seeded 1 as x_full [4096, H] then dY_full [4096, H] (N(0,1)); a case with M
    tokens uses rows [0, M), so M = 1/8/32/4096 share their first rows.  The
    M=4096 case is read as 8 sequences x 512 tokens, sequence-major.
Weights use the [out, in] layout (PR #325, section "Operator test matrix").
"""
from __future__ import annotations

import functools
import hashlib

import numpy as np
import torch

QWEN3_8B_H = 4096
QWEN3_8B_I = 12288
FULL_ROWS = 4096


def _randn(gen: torch.Generator, shape, scale: float | None = None) -> torch.Tensor:
    t = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if scale is not None:
        t = t * scale
    return t.to(torch.bfloat16)


def tiny_case(M: int = 4, H: int = 256, I: int = 768, seed: int = 0) -> dict:
    """The tiny fwd+bwd case; CPU BF16 tensors."""
    gen = torch.Generator("cpu").manual_seed(seed)
    x = _randn(gen, (M, H))
    w_gate = _randn(gen, (I, H), 0.02)
    w_up = _randn(gen, (I, H), 0.02)
    w_down = _randn(gen, (H, I), 0.02)
    dy = _randn(gen, (M, H))
    return {"x": x, "w_gate": w_gate, "w_up": w_up, "w_down": w_down, "dy": dy}


@functools.lru_cache(maxsize=4)
def ffn_weights(H: int = QWEN3_8B_H, I: int = QWEN3_8B_I, seed: int = 0):
    gen = torch.Generator("cpu").manual_seed(seed)
    w_gate = _randn(gen, (I, H), 0.02)
    w_up = _randn(gen, (I, H), 0.02)
    w_down = _randn(gen, (H, I), 0.02)
    return w_gate, w_up, w_down


@functools.lru_cache(maxsize=2)
def _activations_full(H: int, rows: int, seed: int):
    gen = torch.Generator("cpu").manual_seed(seed)
    x_full = _randn(gen, (rows, H))
    dy_full = _randn(gen, (rows, H))
    return x_full, dy_full


def activations(M: int, H: int = QWEN3_8B_H, seed: int = 1, rows: int = FULL_ROWS):
    """x[:M], dY[:M] of the shared 4096-row draws (CPU BF16)."""
    if M > rows:
        raise ValueError(f"M={M} exceeds the {rows} generated rows")
    x_full, dy_full = _activations_full(H, rows, seed)
    return x_full[:M], dy_full[:M]


def qwen3_case(M: int, H: int = QWEN3_8B_H, I: int = QWEN3_8B_I, wseed: int = 0, aseed: int = 1) -> dict:
    w_gate, w_up, w_down = ffn_weights(H, I, wseed)
    x, dy = activations(M, H, aseed)
    return {"x": x, "w_gate": w_gate, "w_up": w_up, "w_down": w_down, "dy": dy}


def bits(t: torch.Tensor) -> np.ndarray:
    """BF16 tensor -> numpy uint16 bit patterns (host copy)."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def from_bits(a: np.ndarray) -> torch.Tensor:
    """numpy uint16 bit patterns -> CPU BF16 tensor."""
    a = np.ascontiguousarray(np.asarray(a, dtype=np.uint16))
    return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)


def sha256(t: torch.Tensor) -> str:
    return hashlib.sha256(bits(t).tobytes()).hexdigest()
