"""Parsers for the hand-worked fixtures under tests/golden/."""
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def parse_value(tok: str) -> Fraction:
    """'1', '-5', '2^-8', '1.5*2^-24', '3*2^-8', '-2^-12' -> exact Fraction."""
    tok = tok.strip()
    sign = 1
    if tok.startswith("-"):
        sign, tok = -1, tok[1:]
    coef, pw = Fraction(1), Fraction(1)
    if "*" in tok:
        c, p = tok.split("*")
        coef = Fraction(c)
        tok = p
    if tok.startswith("2^"):
        pw = Fraction(2) ** int(tok[2:])
    else:
        coef *= Fraction(tok)
    return sign * coef * pw


def bf16_bits_exact(v: Fraction) -> int:
    """Exact BF16 encoding of a value that must be representable: normal
    (1.m * 2^e, e >= -126) or subnormal (m * 2^-133, exponent field 0)."""
    if v == 0:
        return 0
    s = 0x8000 if v < 0 else 0
    v = abs(v)
    sub = v / Fraction(2) ** -133
    if v < Fraction(2) ** -126:
        assert sub.denominator == 1 and 0 < sub < 128, f"not representable in BF16: {v}"
        return s | int(sub)
    e = 0
    while v >= 2:
        v /= 2; e += 1
    while v < 1:
        v *= 2; e -= 1
    m = (v - 1) * 128
    assert m.denominator == 1, f"not representable in BF16: {v}"
    assert e + 127 < 255, f"past the BF16 range: {v}"
    return s | ((e + 127) << 7) | int(m)


def f16_bits_exact(v: Fraction) -> int:
    """Exact FP16 encoding of a value that must be representable: normal
    (1.m * 2^e, -14 <= e <= 15, 10 fraction bits) or subnormal (m * 2^-24)."""
    if v == 0:
        return 0
    s = 0x8000 if v < 0 else 0
    v = abs(v)
    if v < Fraction(2) ** -14:
        sub = v / Fraction(2) ** -24
        assert sub.denominator == 1 and 0 < sub < 1024, f"not representable in FP16: {v}"
        return s | int(sub)
    e = 0
    while v >= 2:
        v /= 2; e += 1
    while v < 1:
        v *= 2; e -= 1
    m = (v - 1) * 1024
    assert m.denominator == 1, f"not representable in FP16: {v}"
    assert e + 15 < 31, f"past the FP16 range: {v}"
    return s | ((e + 15) << 10) | int(m)


_ENC = {"bf16": (bf16_bits_exact, 0x3F80), "fp16": (f16_bits_exact, 0x3C00)}


def load_table(name: str):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append([c.strip() for c in line.split("|")])
    return rows


def _vector(n: int, spec: str, fmt: str = "bf16") -> np.ndarray:
    enc, one = _ENC[fmt]
    v = np.zeros(n, np.uint16)
    if spec == "ones":
        v[:] = one
    else:
        for it in spec.split():
            i, val = it.split(":"); v[int(i)] = enc(parse_value(val))
    return v


def tree_cases(fmt: str = "bf16"):
    name_ = {"bf16": "tree_cases.txt", "fp16": "tree_f16_cases.txt"}[fmt]
    out = []
    for name, K, xs, ws, exp, why in load_table(name_):
        K = int(K)
        out.append((name, _vector(K, xs, fmt), _vector(K, ws, fmt), int(exp, 16), why))
    return out


def _stored(tok: str, enc) -> int:
    """An operand token: 'inf', '-inf', 'nan' (the stored type's infinities and
    a quiet NaN), or an exact value as parse_value reads it."""
    special = {"inf": 0x7F80, "-inf": 0xFF80, "nan": 0x7FC0} if enc is bf16_bits_exact else \
              {"inf": 0x7C00, "-inf": 0xFC00, "nan": 0x7E00}
    return special[tok] if tok in special else enc(parse_value(tok))


def block_cases(fmt: str = "bf16"):
    enc = _ENC[fmt][0]
    name_ = {"bf16": "block_rule_cases.txt", "fp16": "block_rule_f16_cases.txt"}[fmt]
    out = []
    for name, acc, av, bv, exp, why in load_table(name_):
        a = np.array([_stored(t, enc) for t in av.split()], np.uint16)
        b = np.array([_stored(t, enc) for t in bv.split()], np.uint16)
        accf = np.array([int(acc, 16)], np.uint32).view(np.float32)[0]
        out.append((name, accf, a, b, int(exp, 16), why))
    return out


def leaf_cases(fmt: str = "bf16"):
    name_ = {"bf16": "leaf_cases.txt", "fp16": "leaf_f16_cases.txt"}[fmt]
    out = []
    for name, n, av, bv, exp, why in load_table(name_):
        n = int(n)
        out.append((name, _vector(n, av, fmt), _vector(n, bv, fmt), int(exp, 16), why))
    return out


def act_cases():
    out = []
    for name, g, u, da, output, exp, other, why in load_table("act_cases.txt"):
        vals = [bf16_bits_exact(parse_value(t)) for t in (g, u, da)]
        out.append((name, *vals, output, int(exp, 16), int(other, 16), why))
    return out
