"""The FP32 leaf's declared block rule against the matrix-core instructions
themselves: v_mfma_f32_16x16x32_bf16 and v_mfma_f32_16x16x32_f16, run directly
by the test probe (tests/mfma_probe.hip) on crafted operands and accumulators,
against the oracle's block steps from the same accumulator.  This reproduces,
from the repository, the measurement behind the leaf reading (the pages fix
an FP32 leaf but not its order: "feat(ffn): add deterministic distributed
Triton FFN for ROCm", section "Design"; FP16 and BF16 follow one tree:
"[PERF][distributed]: optimize deterministic ROCm collectives with HIP IPC",
section "Determinism and correctness")."""
import numpy as np
import pytest
import torch

import oracle
from tests import mfma_probe

pytestmark = pytest.mark.gpu

# (fraction bits, exponent bias, largest normal exponent) of the stored types
FMT = {"bf16": (7, 127, 127), "fp16": (10, 15, 15)}
CODE = {"bf16": 0, "fp16": 1}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the GPU tests need an MI355X")
    mfma_probe.lib()


def elems(rng, fmt, shape, lo, hi, sub=0.0, zero=0.0, sign=True):
    """Values with exponents in [lo, hi] (clamped to the format's normal range),
    a fraction `sub` of them subnormal and `zero` of them zero."""
    fb, bias, emax = FMT[fmt]
    lo, hi = max(lo, 1 - bias), min(hi, emax)
    e = rng.integers(lo, hi + 1, size=shape) + bias
    m = rng.integers(0, 1 << fb, size=shape)
    s = (rng.integers(0, 2, size=shape) << 15) if sign else np.zeros(shape, np.int64)
    b = s | (e << fb) | m
    if sub:
        b = np.where(rng.random(shape) < sub, s | rng.integers(1, 1 << fb, size=shape), b)
    if zero:
        b = np.where(rng.random(shape) < zero, 0, b)
    return b.astype(np.uint16)


def f32s(rng, shape, lo, hi, subnormal=0.0):
    e = rng.integers(lo, hi + 1, size=shape) + 127
    m = rng.integers(0, 1 << 23, size=shape)
    s = rng.integers(0, 2, size=shape)
    u = (s << 31) | (e << 23) | m
    if subnormal:
        u = np.where(rng.random(shape) < subnormal, (s << 31) | rng.integers(1, 1 << 23, size=shape), u)
    return u.astype(np.uint32).view(np.float32)


def from_float(x, fmt):
    x = np.asarray(x, np.float32)
    if fmt == "fp16":
        return x.astype(np.float16).view(np.uint16)
    return oracle.f32_to_bf16_bits(x)


def case(fmt, dist, n, rng, K=32):
    """A [n, 16, K], B [n, K, 16] stored bits and C [n, 16, 16] FP32."""
    A_shape, B_shape, C_shape = (n, 16, K), (n, K, 16), (n, 16, 16)
    zc = np.zeros(C_shape, np.float32)
    hi = min(FMT[fmt][2], 80)  # BF16: products stay far below FP32's range
    if dist == "int":
        A = from_float(rng.integers(-8, 9, A_shape), fmt)
        B = from_float(rng.integers(-8, 9, B_shape), fmt)
        return A, B, rng.integers(-100, 100, C_shape).astype(np.float32)
    if dist == "wide":
        return elems(rng, fmt, A_shape, -14, hi // 2), elems(rng, fmt, B_shape, -14, hi // 2), zc
    if dist == "wide_acc":
        return (elems(rng, fmt, A_shape, -14, hi // 2), elems(rng, fmt, B_shape, -14, hi // 2),
                f32s(rng, C_shape, -40, 40))
    if dist == "cancel":
        A = elems(rng, fmt, A_shape, -4, 4)
        h = K // 2
        A[:, :, h:] = A[:, :, :h] ^ np.uint16(0x8000)
        A[:, :, ::5] = elems(rng, fmt, (n, 16, len(range(0, K, 5))), -14, -8)
        one = from_float(np.ones(1), fmt)[0]
        B = np.where(rng.random(B_shape) < 0.3, elems(rng, fmt, B_shape, -2, 2), one).astype(np.uint16)
        C = np.where(rng.random(C_shape) < 0.5, f32s(rng, C_shape, -20, 5), 0).astype(np.float32)
        return A, B, C
    if dist == "subnormal":
        return elems(rng, fmt, A_shape, -14, -10, sub=0.5), elems(rng, fmt, B_shape, -14, hi, sub=0.3), zc
    if dist == "subnormal_acc":
        return (elems(rng, fmt, A_shape, -14, -10, sub=0.5), elems(rng, fmt, B_shape, -14, 0, sub=0.5),
                f32s(rng, C_shape, -60, -20))
    if dist == "ties":
        a = np.where(rng.random(A_shape) < 0.3, 2.0 ** -rng.integers(8, 14, A_shape), 0)
        a = a * np.where(rng.random(A_shape) < 0.7, 1, -1)
        a[:, :, 0] = 1.0
        one = from_float(np.ones(1), fmt)[0]
        B = np.where(rng.random(B_shape) < 0.5, one, elems(rng, fmt, B_shape, -12, -6)).astype(np.uint16)
        C = np.where(rng.random(C_shape) < 0.5, f32s(rng, C_shape, 0, 8), 0).astype(np.float32)
        return from_float(a, fmt), B, C
    if dist == "tiny_acc":
        # tiny products against FP32 subnormal and near-subnormal accumulators
        lo = -14 if fmt == "fp16" else -70
        A = elems(rng, fmt, A_shape, lo, lo + 6, sub=0.4)
        B = elems(rng, fmt, B_shape, lo, lo + 6, sub=0.4)
        return A, B, f32s(rng, C_shape, -126, -100, subnormal=0.5)
    if dist == "big_acc":
        lo = 10 if fmt == "fp16" else 30
        return (elems(rng, fmt, A_shape, lo, lo + 5), elems(rng, fmt, B_shape, lo, lo + 5),
                f32s(rng, C_shape, 20, 120))
    if dist == "signed_zero":
        # zero results: -0 and +0 accumulators over blocks of zero products, and
        # (BF16) block sums of a few products near 2^-152, which FP32 rounds to
        # zero or to its smallest subnormals
        lo = -14 if fmt == "fp16" else -77
        A = elems(rng, fmt, A_shape, lo, lo + 1, zero=0.7)
        B = elems(rng, fmt, B_shape, lo, lo + 1, zero=0.3)
        A[:, ::2, 8:16] = np.where(rng.random((n, 8, 8)) < 0.5, 0x8000, 0)  # a zero block in half the rows
        A[:, ::4, :] = np.where(rng.random((n, 4, K)) < 0.5, 0x8000, 0)  # only zero blocks in a quarter
        C = np.where(rng.random(C_shape) < 0.5, np.float32(-0.0), np.float32(0.0))
        C = np.where(rng.random(C_shape) < 0.2, f32s(rng, C_shape, -149, -149, subnormal=1.0), C)
        return A, B, C.astype(np.float32)
    if dist == "overflow":
        # past FP32's range: BF16 products up to 2^130 (those of 2^128 and more are
        # infinities of their sign) against infinite, NaN, large and zero
        # accumulators; FP16 products stay finite, so there only the accumulators
        lo, hi = (56, 64) if fmt == "bf16" else (8, 15)
        A = elems(rng, fmt, A_shape, lo, hi, zero=0.85)
        B = elems(rng, fmt, B_shape, lo, hi)
        pick = rng.random(C_shape)
        C = np.where(pick < 0.2, np.float32(np.inf), np.where(pick < 0.4, np.float32(-np.inf),
                     np.where(pick < 0.5, np.float32(np.nan), np.where(pick < 0.75, f32s(rng, C_shape, 120, 127), 0))))
        return A, B, C.astype(np.float32)
    if dist == "special":
        # infinite and NaN operands beside zeros and ordinary values: an infinity
        # times a nonzero value is an infinity of the product's sign, times zero a
        # NaN; a NaN operand, or infinities of both signs, give NaN
        A = elems(rng, fmt, A_shape, -4, 4, zero=0.3)
        B = elems(rng, fmt, B_shape, -4, 4, zero=0.3)
        inf, nan = (0x7F80, 0x7FC0) if fmt == "bf16" else (0x7C00, 0x7E00)
        pa = rng.random(A_shape)
        A = np.where(pa < 0.015, np.uint16(inf), np.where(pa < 0.03, np.uint16(inf | 0x8000),
                     np.where(pa < 0.035, np.uint16(nan), A))).astype(np.uint16)
        pb = rng.random(B_shape)
        B = np.where(pb < 0.01, np.uint16(inf), B).astype(np.uint16)
        C = np.where(rng.random(C_shape) < 0.1, np.float32(-np.inf), f32s(rng, C_shape, -4, 4)).astype(np.float32)
        return A, B, C
    assert dist == "mixed"
    A = elems(rng, fmt, A_shape, -14, hi // 2, sub=0.1, zero=0.25)
    B = elems(rng, fmt, B_shape, -14, hi // 2, sub=0.1)
    C = np.where(rng.random(C_shape) < 0.5, f32s(rng, C_shape, -30, 30), 0).astype(np.float32)
    return A, B, C


def expected(fmt, A, B, C):
    n, _, K = A.shape
    a = np.ascontiguousarray(np.repeat(A[:, :, None, :], 16, axis=2)).reshape(n * 256, K)
    b = np.ascontiguousarray(np.repeat(np.transpose(B, (0, 2, 1))[:, None, :, :], 16, axis=1)).reshape(n * 256, K)
    return oracle.block_chains(C.reshape(-1), a, b, fmt).reshape(n, 16, 16)


DISTS = ["int", "wide", "wide_acc", "cancel", "subnormal", "subnormal_acc", "ties", "tiny_acc", "big_acc", "mixed",
         "signed_zero", "overflow", "special"]


@pytest.mark.parametrize("fmt", ["bf16", "fp16"])
@pytest.mark.parametrize("dist", DISTS)
def test_one_mfma_from_an_accumulator(fmt, dist):
    # one 16x16x32 MFMA: four blocks of 8 in ascending k from the accumulator C
    rng = np.random.default_rng(DISTS.index(dist) * 2 + (fmt == "fp16"))
    A, B, C = case(fmt, dist, 96, rng)
    got = mfma_probe.run(CODE[fmt], A, B, C)
    want = expected(fmt, A, B, C)
    bad = got.view(np.uint32) != want.view(np.uint32)
    assert not bad.any(), (f"{fmt} {dist}: {int(bad.sum())}/{bad.size} outputs differ from the block rule; "
                           f"first at {np.argwhere(bad)[:3].tolist()}")
    if dist == "int":  # exact sums: every order agrees, which checks the lane layout
        exact = np.einsum("nik,nkj->nij", oracle.bits_to_f32(A, fmt).astype(np.float64),
                          oracle.bits_to_f32(B, fmt).astype(np.float64)) + C
        assert np.array_equal(got, exact.astype(np.float32))


@pytest.mark.parametrize("fmt", ["bf16", "fp16"])
@pytest.mark.parametrize("dist", ["wide", "cancel", "subnormal", "ties", "mixed"])
def test_two_chained_mfmas_make_a_leaf(fmt, dist):
    # the library's leaf: K 0..31 then 32..63 from a zero accumulator
    rng = np.random.default_rng(100 + DISTS.index(dist) * 2 + (fmt == "fp16"))
    A, B, _ = case(fmt, dist, 64, rng, K=64)
    C = np.zeros((64, 16, 16), np.float32)
    got = mfma_probe.run(CODE[fmt], A, B, C)
    want = expected(fmt, A, B, C)
    bad = got.view(np.uint32) != want.view(np.uint32)
    assert not bad.any(), f"{fmt} {dist}: {int(bad.sum())}/{bad.size} leaves differ from the block rule"
    # and they are the oracle's leaves
    i, j = 3, 5
    for c in range(0, 64, 16):
        assert np.float32(oracle.leaf_f32(A[c, i], np.ascontiguousarray(B[c, :, j]), fmt)) == got[c, i, j]
