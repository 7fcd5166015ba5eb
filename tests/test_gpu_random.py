"""Seeded random sweep against the oracle: tree GEMMs in the three layouts and
the FFN forward and backward, in BF16 and FP16 storage, over random shapes
(ragged K, any H and I, token counts across every kernel's range; the dX
lanes and the forward without allocation on some cases) and value mixes (scaled
normals, exponents spread over 24 binades, sparse values, small integers),
with padded leading dimensions.  Large scales push FP16 stage boundaries past
65504, so infinities and NaN flow into later GEMMs: results must still equal
the oracle bit for bit, except that a NaN matches any NaN (the sign and
payload of a NaN made by an FP32 operation are not part of the definition;
"feat(ffn): add deterministic distributed Triton FFN for ROCm", section
"Design", fixes the tree, and the leaf's block rule covers infinities)."""
import numpy as np
import pytest
import torch

import oracle
from deterministic_gated_ffn_amd import binding as dgf

pytestmark = pytest.mark.gpu

CASES = 480


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the GPU tests need an MI355X")
    dgf.load()


def gen(rng, fmt, shape, kind):
    if kind == "normal":
        x = rng.standard_normal(shape).astype(np.float32) * rng.choice([1.0, 0.02, 30.0])
    elif kind == "wide":
        x = (rng.standard_normal(shape) * 2.0 ** rng.integers(-12, 12, shape)).astype(np.float32)
    elif kind == "sparse":
        x = np.where(rng.random(shape) < 0.3, rng.standard_normal(shape), 0).astype(np.float32)
    else:
        x = rng.integers(-4, 5, shape).astype(np.float32)
    if fmt == "fp16":
        return np.clip(x, -60000, 60000).astype(np.float16).view(np.uint16)
    return oracle.f32_to_bf16_bits(x)


def dev(rng, bits, fmt):
    R, C = bits.shape
    ld = ((C + 7) // 8) * 8 + int(rng.choice([0, 8]))
    full = np.zeros((R, ld), np.uint16)
    full[:, :C] = bits
    t = torch.from_numpy(full.view(np.int16)).cuda()
    return t.view(torch.float16 if fmt == "fp16" else torch.bfloat16)[:, :C]


def host(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def mismatches(got, want, fmt):
    emask, fmask = (0x7C00, 0x3FF) if fmt == "fp16" else (0x7F80, 0x7F)
    nan = lambda b: ((b & emask) == emask) & ((b & fmask) != 0)
    want = np.asarray(want, np.uint16).reshape(got.shape)
    return int(((got != want) & ~(nan(got) & nan(want))).sum())


def test_random_gemms_and_ffns_match_the_oracle():
    rng = np.random.default_rng(2024)
    failures = []
    for case in range(CASES):
        fmt = str(rng.choice(["bf16", "fp16"]))
        kind = str(rng.choice(["normal", "wide", "sparse", "ints"]))
        dt = [] if fmt == "bf16" else ["fp16"]
        if rng.random() < 0.65:
            layout = str(rng.choice(["NT", "NN", "TN"]))
            M = int(rng.integers(1, 40) if rng.random() < 0.5 else rng.integers(40, 300))
            N = int(rng.integers(1, 400))
            K = int(rng.integers(1, 130) if rng.random() < 0.5 else rng.integers(130, 3000))
            if layout == "TN" and rng.random() < 0.7:
                K = int(rng.integers(1, 65))
            A, Bnk = gen(rng, fmt, (M, K), kind), gen(rng, fmt, (N, K), kind)
            a, b = {"NT": (A, Bnk), "NN": (A, np.ascontiguousarray(Bnk.T)),
                    "TN": (np.ascontiguousarray(A.T), np.ascontiguousarray(Bnk.T))}[layout]
            want = oracle.gemm_tree(a, b, layout, *dt)
            got = host(dgf.gemm_tree(layout, dev(rng, a, fmt), dev(rng, b, fmt)))
            bad = mismatches(got, want, fmt)
            tag = f"gemm {fmt} {layout} {kind} M={M} N={N} K={K}"
        else:
            M = int(rng.integers(1, 40) if rng.random() < 0.5 else rng.integers(40, 260))
            H, I = int(rng.integers(1, 320)), int(rng.integers(1, 480))
            x, dy = gen(rng, fmt, (M, H), "normal"), gen(rng, fmt, (M, H), "normal")
            wg, wu, wd = gen(rng, fmt, (I, H), kind), gen(rng, fmt, (I, H), kind), gen(rng, fmt, (H, I), kind)
            o = oracle.ffn_fwd(x, wg, wu, wd, *dt)
            ob = oracle.ffn_bwd(dy, x, o["g"], o["u"], wg, wu, wd, *dt)
            W = [dev(rng, w, fmt) for w in (wg, wu, wd)]
            xd = dev(rng, x, fmt)
            y, g, u = dgf.ffn_fwd(xd, *W, training=True)
            lanes = bool(rng.random() < 0.3)
            r = dgf.ffn_bwd(dev(rng, dy, fmt), xd, g, u, *W, lanes=lanes)
            outs = [(y, o["y"]), (g, o["g"]), (u, o["u"]), (r["dX"], ob["dX"]), (r["dW_gate"], ob["dW_gate"]),
                    (r["dW_up"], ob["dW_up"]), (r["dW_down"], ob["dW_down"])]
            if lanes:
                outs += [(r["G"], ob["G"]), (r["U"], ob["U"])]
            if fmt == "bf16" and rng.random() < 0.3:
                # the entry point without allocation, into a padded y of its own
                ys = torch.empty(M, (H + 7) // 8 * 8, dtype=torch.bfloat16, device="cuda")[:, :H]
                outs.append((dgf.ffn_fwd_static(xd, *W, ys), o["y"]))
            bad = sum(mismatches(host(t), ref, fmt) for t, ref in outs)
            tag = f"ffn {fmt} {kind} M={M} H={H} I={I} lanes={lanes}"
        if bad:
            failures.append(f"case {case}: {tag}: {bad} mismatches")
    torch.cuda.synchronize()
    assert not failures, "\n".join(failures[:10])


def test_random_bit_patterns_through_combine_and_activation():
    # every 16-bit pattern is fair game here (NaN, infinities, subnormals, -0):
    # the rank-tree combine in BF16, FP16 and FP32, and the activation forward
    # and backward, against the oracle; a NaN matches any NaN
    rng = np.random.default_rng(77)
    failures = []
    for case in range(48):
        S = int(rng.choice([1, 2, 4, 8]))
        n = int(rng.integers(1, 100) if rng.random() < 0.3 else rng.integers(100, 60000))
        cd = str(rng.choice(["bf16", "fp16", "fp32"]))
        if cd == "fp32":
            with np.errstate(over="ignore"):  # values past FP32's range become infinities on purpose
                parts = [(rng.standard_normal(n) * 2.0 ** rng.integers(-140, 128, n)).astype(np.float32)
                         for _ in range(S)]
            for p in parts:
                p[rng.random(n) < 0.01] = np.float32(np.inf)
                p[rng.random(n) < 0.01] = np.float32(-0.0)
            want = oracle.tree_combine_typed(parts, "fp32")
            got = dgf.tree_combine([torch.from_numpy(p).cuda() for p in parts]).cpu().numpy()
            bad = int(((got.view(np.uint32) != want.view(np.uint32)) & ~(np.isnan(got) & np.isnan(want))).sum())
        else:
            parts = [rng.integers(0, 65536, n, dtype=np.uint64).astype(np.uint16) for _ in range(S)]
            want = oracle.tree_combine_typed(parts, cd)
            tdt = torch.float16 if cd == "fp16" else torch.bfloat16
            got = host(dgf.tree_combine([torch.from_numpy(p.view(np.int16)).cuda().view(tdt) for p in parts]))
            bad = mismatches(got, want, cd)
        if bad:
            failures.append(f"combine {cd} S={S} n={n}: {bad} mismatches")
        ad = str(rng.choice(["bf16", "fp16"]))
        m = int(rng.integers(1, 40000))
        G, U, DA = (rng.integers(0, 65536, m, dtype=np.uint64).astype(np.uint16) for _ in range(3))
        tdt = torch.float16 if ad == "fp16" else torch.bfloat16
        dv = lambda b: torch.from_numpy(b.view(np.int16)).cuda().view(tdt)
        bad = mismatches(host(dgf.act_fwd(dv(G), dv(U))), oracle.act_fwd(G, U, ad), ad)
        for got, want in zip(dgf.act_bwd(dv(DA), dv(G), dv(U)), oracle.act_bwd(DA, G, U, ad)):
            bad += mismatches(host(got), want, ad)
        if bad:
            failures.append(f"act {ad} n={m}: {bad} mismatches")
    torch.cuda.synchronize()
    assert not failures, "\n".join(failures[:10])
