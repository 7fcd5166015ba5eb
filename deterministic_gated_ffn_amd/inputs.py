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
The FP16 cases draw the same FP32 values and round them to FP16 instead
(nearest even); every value of these distributions is in FP16's normal range
or a subnormal, none overflows.
"""
from __future__ import annotations

import functools
import hashlib

import numpy as np
import torch

QWEN3_8B_H = 4096
QWEN3_8B_I = 12288
FULL_ROWS = 4096


STORED = (torch.bfloat16, torch.float16)


def _randn(gen: torch.Generator, shape, scale: float | None = None, dtype=torch.bfloat16) -> torch.Tensor:
    t = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if scale is not None:
        t = t * scale
    return t.to(dtype)


def tiny_case(M: int = 4, H: int = 256, I: int = 768, seed: int = 0, dtype=torch.bfloat16) -> dict:
    """The tiny fwd+bwd case; CPU tensors of the stored type."""
    gen = torch.Generator("cpu").manual_seed(seed)
    x = _randn(gen, (M, H), dtype=dtype)
    w_gate = _randn(gen, (I, H), 0.02, dtype)
    w_up = _randn(gen, (I, H), 0.02, dtype)
    w_down = _randn(gen, (H, I), 0.02, dtype)
    dy = _randn(gen, (M, H), dtype=dtype)
    return {"x": x, "w_gate": w_gate, "w_up": w_up, "w_down": w_down, "dy": dy}


@functools.lru_cache(maxsize=4)
def ffn_weights(H: int = QWEN3_8B_H, I: int = QWEN3_8B_I, seed: int = 0, dtype=torch.bfloat16):
    gen = torch.Generator("cpu").manual_seed(seed)
    w_gate = _randn(gen, (I, H), 0.02, dtype)
    w_up = _randn(gen, (I, H), 0.02, dtype)
    w_down = _randn(gen, (H, I), 0.02, dtype)
    return w_gate, w_up, w_down


@functools.lru_cache(maxsize=2)
def _activations_full(H: int, rows: int, seed: int, dtype=torch.bfloat16):
    gen = torch.Generator("cpu").manual_seed(seed)
    x_full = _randn(gen, (rows, H), dtype=dtype)
    dy_full = _randn(gen, (rows, H), dtype=dtype)
    return x_full, dy_full


def activations(M: int, H: int = QWEN3_8B_H, seed: int = 1, rows: int = FULL_ROWS, dtype=torch.bfloat16):
    """x[:M], dY[:M] of the shared 4096-row draws (CPU, stored type)."""
    if M > rows:
        raise ValueError(f"M={M} exceeds the {rows} generated rows")
    x_full, dy_full = _activations_full(H, rows, seed, dtype)
    return x_full[:M], dy_full[:M]


def qwen3_case(M: int, H: int = QWEN3_8B_H, I: int = QWEN3_8B_I, wseed: int = 0, aseed: int = 1,
               dtype=torch.bfloat16) -> dict:
    w_gate, w_up, w_down = ffn_weights(H, I, wseed, dtype)
    x, dy = activations(M, H, aseed, dtype=dtype)
    return {"x": x, "w_gate": w_gate, "w_up": w_up, "w_down": w_down, "dy": dy}


def bits(t: torch.Tensor) -> np.ndarray:
    """BF16 or FP16 tensor -> numpy uint16 bit patterns (host copy)."""
    assert t.dtype in STORED, t.dtype
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def from_bits(a: np.ndarray, dtype=torch.bfloat16) -> torch.Tensor:
    """numpy uint16 bit patterns -> CPU tensor of the stored type."""
    a = np.ascontiguousarray(np.asarray(a, dtype=np.uint16))
    return torch.from_numpy(a.view(np.int16).copy()).view(dtype)


def sha256(t: torch.Tensor) -> str:
    return hashlib.sha256(bits(t).tobytes()).hexdigest()
