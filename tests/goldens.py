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


def load_table(name: str):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append([c.strip() for c in line.split("|")])
    return rows


def tree_cases():
    out = []
    for name, K, xs, ws, exp, why in load_table("tree_cases.txt"):
        K = int(K)
        x = np.zeros(K, np.uint16)
        if xs == "ones":
            x[:] = 0x3F80
        else:
            for it in xs.split():
                i, v = it.split(":"); x[int(i)] = bf16_bits_exact(parse_value(v))
        w = np.zeros(K, np.uint16)
        for it in ws.split():
            i, v = it.split(":"); w[int(i)] = bf16_bits_exact(parse_value(v))
        out.append((name, x, w, int(exp, 16), why))
    return out


def block_cases():
    out = []
    for name, acc, av, bv, exp, why in load_table("block_rule_cases.txt"):
        a = np.array([bf16_bits_exact(parse_value(t)) for t in av.split()], np.uint16)
        b = np.array([bf16_bits_exact(parse_value(t)) for t in bv.split()], np.uint16)
        accf = np.array([int(acc, 16)], np.uint32).view(np.float32)[0]
        out.append((name, accf, a, b, int(exp, 16), why))
    return out


def _vector(n: int, spec: str) -> np.ndarray:
    v = np.zeros(n, np.uint16)
    if spec == "ones":
        v[:] = 0x3F80
    else:
        for it in spec.split():
            i, val = it.split(":"); v[int(i)] = bf16_bits_exact(parse_value(val))
    return v


def leaf_cases():
    out = []
    for name, n, av, bv, exp, why in load_table("leaf_cases.txt"):
        n = int(n)
        out.append((name, _vector(n, av), _vector(n, bv), int(exp, 16), why))
    return out


def act_cases():
    out = []
    for name, g, u, da, output, exp, other, why in load_table("act_cases.txt"):
        vals = [bf16_bits_exact(parse_value(t)) for t in (g, u, da)]
        out.append((name, *vals, output, int(exp, 16), int(other, 16), why))
    return out
