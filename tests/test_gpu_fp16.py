"""GPU parity of the FFN in FP16 storage: the HIP path (the *_typed entry
points through the C ABI) against the CPU oracle in FP16, bitwise.  FP32,
FP16 and BF16 follow one tree ("[PERF][distributed]: optimize deterministic
ROCm collectives with HIP IPC", section "Determinism and correctness"); the
FP16 leaf's block rule is the oracle's, with FP16 exponents."""
import zlib

import numpy as np
import pytest
import torch

import oracle
from oracle import fp64
from deterministic_gated_ffn_amd import binding as dgf
from deterministic_gated_ffn_amd import inputs

pytestmark = pytest.mark.gpu
F16 = torch.float16


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the GPU tests need an MI355X")
    dgf.load()
    return torch.device("cuda:0")


def h(x):
    """float values -> FP16 bits (nearest even)."""
    return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


def dev(bits):
    return inputs.from_bits(bits, F16).cuda()


def bits(t):
    return inputs.bits(t)


def padded(b, ld_extra=8):
    R, C = b.shape
    ld = ((C + 7) // 8) * 8 + ld_extra
    full = np.zeros((R, ld), np.uint16)
    full[:, :C] = b
    return dev(full)[:, :C]


def ordinal(b):
    b = np.asarray(b, np.uint16).astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)


def assert_bitwise(got, expected_bits, name):
    g = bits(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.uint16)
    e = np.asarray(expected_bits, np.uint16).reshape(g.shape)
    bad = g != e
    n = int(bad.sum())
    if n:
        d = np.abs(ordinal(g) - ordinal(e))[bad]
        idx = np.argwhere(bad)[:5].tolist()
        pytest.fail(f"{name}: {n}/{g.size} mismatches; max ulp {d.max()}, >1 ulp: {(d > 1).sum()}; first at {idx}")


def rnd(rng, shape, scale=1.0):
    return h(rng.standard_normal(shape) * scale)


def wide(rng, shape, lo=-14, hi=15, sub=0.0):
    """FP16 values with random exponents in [lo, hi], a fraction `sub` of them subnormal."""
    e = rng.integers(lo, hi + 1, size=shape) + 15
    m = rng.integers(0, 1024, size=shape)
    s = rng.integers(0, 2, size=shape)
    b = (s << 15) | (e << 10) | m
    if sub:
        b = np.where(rng.random(shape) < sub, (s << 15) | rng.integers(1, 1024, size=shape), b)
    return b.astype(np.uint16)


# ---------------------------------------------------------------- the FP16 leaf
@pytest.mark.parametrize("dist", ["wide", "cancel", "subnormal", "ties", "tiny", "large"])
@pytest.mark.parametrize("K", [8, 32, 64, 128, 200])
def test_f16_leaf_block_rule_adversarial(dist, K):
    # v_mfma_f32_16x16x32_f16 inside the tree GEMM on inputs that separate the
    # declared block rule from other summation orders and alignments
    rng = np.random.default_rng(zlib.crc32(f"f16/{dist}/{K}".encode()))
    M, N = 32, 48
    # (exponent ranges keep every sum finite, or, for "large", of one sign: an
    # infinity never meets one of the other sign, so no NaN arises)
    if dist == "wide":
        A, B = wide(rng, (M, K), -14, 3), wide(rng, (N, K), -14, 3)
    elif dist == "cancel":
        A = wide(rng, (M, K), -4, 4)
        A[:, K // 2:] = A[:, :K - K // 2][:, :K // 2] ^ np.uint16(0x8000)
        A[:, ::7] = wide(rng, (M, len(range(0, K, 7))), -14, -8)
        B = np.where(rng.random((N, K)) < 0.3, wide(rng, (N, K), -2, 2), np.uint16(0x3C00)).astype(np.uint16)
    elif dist == "subnormal":
        # FP16-subnormal operands (exponent -14 for the grid) against large and small ones
        A = wide(rng, (M, K), -14, -10, sub=0.5)
        B = np.where(rng.random((N, K)) < 0.5, wide(rng, (N, K), 8, 15), wide(rng, (N, K), -14, 0, sub=0.3))
        B = B.astype(np.uint16)
    elif dist == "ties":
        A = h(np.where(rng.random((M, K)) < 0.3, 2.0 ** -rng.integers(8, 14, (M, K)), 0)
              * np.where(rng.random((M, K)) < 0.7, 1, -1))
        A[:, 0] = 0x3C00
        B = np.where(rng.random((N, K)) < 0.5, np.uint16(0x3C00), wide(rng, (N, K), -12, -6)).astype(np.uint16)
    elif dist == "tiny":
        A, B = wide(rng, (M, K), -14, -9, sub=0.3), wide(rng, (N, K), -14, -9, sub=0.3)
    else:  # positive products up to 2^14: some leaves (K <= 64) or nodes overflow FP16 to +infinity
        lo, hi = (1, 6) if K <= 64 else (0, 5)
        A, B = wide(rng, (M, K), lo, hi) & np.uint16(0x7FFF), wide(rng, (N, K), lo, hi) & np.uint16(0x7FFF)
    expect = oracle.gemm_tree(A, B, "NT", "fp16")
    got = dgf.gemm_tree("NT", dev(A), dev(B))
    torch.cuda.synchronize()
    assert_bitwise(got, expect, f"fp16 leaf {dist} K={K}")


@pytest.mark.parametrize("dist", ["wide", "cancel", "subnormal", "ties", "tiny", "negzero", "large"])
@pytest.mark.parametrize("K", [200, 640, 1536, 2048])
def test_f16_tiled_tree_adversarial(dist, K):
    # The tiled kernel (128 tokens and more) keeps FP16 tree values as packed
    # pairs and adds two nodes with one packed FP16 add; these inputs make the
    # nodes round at ties, sum in the FP16 subnormal range, cancel to zero,
    # meet negative zeros (leaves of tiny negative products round to -0) and
    # overflow to infinity.  K = 200 ends in a partial leaf, K = 640 splits
    # into lower subtrees of 2 and 3 leaves, K = 1536 into eight of 3 and K =
    # 2048 into eight of 4 (both in the deferred form).
    rng = np.random.default_rng(zlib.crc32(f"f16/tiled/{dist}/{K}".encode()))
    M, N = 160, 144
    if dist == "wide":
        A, B = wide(rng, (M, K), -14, 3), wide(rng, (N, K), -14, 3)
    elif dist == "cancel":
        A = wide(rng, (M, K), -4, 4)
        A[:, K // 2:] = A[:, :K - K // 2][:, :K // 2] ^ np.uint16(0x8000)
        B = np.where(rng.random((N, K)) < 0.1, wide(rng, (N, K), -2, 2), np.uint16(0x3C00)).astype(np.uint16)
    elif dist == "subnormal":
        A = wide(rng, (M, K), -14, -10, sub=0.5)
        B = np.where(rng.random((N, K)) < 0.5, wide(rng, (N, K), 0, 4), wide(rng, (N, K), -14, 0, sub=0.3))
        B = B.astype(np.uint16)
    elif dist == "ties":
        A = h(np.where(rng.random((M, K)) < 0.3, 2.0 ** -rng.integers(9, 13, (M, K)), 0)
              * np.where(rng.random((M, K)) < 0.7, 1, -1))
        A[:, ::64] = 0x3C00
        B = np.full((N, K), 0x3C00, np.uint16)
    elif dist == "tiny":
        A, B = wide(rng, (M, K), -14, -9, sub=0.3), wide(rng, (N, K), -14, -9, sub=0.3)
    elif dist == "negzero":
        # subnormal operands of at most 2^-20: every leaf is below 2^-25 and
        # rounds to a zero of its sign; whole leaves of B share a sign, mostly
        # negative, so that some rows have only negative leaves
        A = rng.integers(1, 17, size=(M, K)).astype(np.uint16)
        sgn = (rng.random((N, (K + 63) // 64)) < 0.92).repeat(64, axis=1)[:, :K].astype(np.uint16)
        B = (rng.integers(1, 17, size=(N, K)).astype(np.uint16) | (sgn << 15)).astype(np.uint16)
        B[rng.random((N, K)) < 0.02] = 0
    else:  # positive products up to 2^10: leaves and nodes overflow FP16 to +infinity
        A, B = wide(rng, (M, K), 0, 5) & np.uint16(0x7FFF), wide(rng, (N, K), 0, 5) & np.uint16(0x7FFF)
    expect = oracle.gemm_tree(A, B, "NT", "fp16")
    got = dgf.gemm_tree("NT", padded(A), padded(B))
    torch.cuda.synchronize()
    assert_bitwise(got, expect, f"fp16 tiled {dist} K={K}")
    if dist == "negzero":
        assert (expect == 0x8000).any() and (expect == 0).any(), "the case should make zeros of both signs"
    if dist == "large":
        assert (expect == 0x7C00).any(), "the case should overflow"


SHAPES = [(1, 16, 64), (4, 48, 256), (5, 33, 100), (16, 20, 24), (17, 100, 1000), (32, 64, 4096),
          (33, 40, 768), (3, 7, 8), (40, 130, 520), (2, 1, 12288), (3, 24, 65600)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_f16_gemm_tree_matches_oracle(layout, M, N, K):
    rng = np.random.default_rng(M * 1000 + N * 10 + K + 16)
    A = rnd(rng, (M, K)); Bnk = rnd(rng, (N, K), 0.02)
    if layout == "NT":
        a, b = A, Bnk
    elif layout == "NN":
        a, b = A, np.ascontiguousarray(Bnk.T)
    else:
        a, b = np.ascontiguousarray(A.T), np.ascontiguousarray(Bnk.T)
    expect = oracle.gemm_tree(a, b, layout, "fp16")
    got = dgf.gemm_tree(layout, padded(a), padded(b))
    torch.cuda.synchronize()
    assert_bitwise(got, expect, f"fp16 {layout} {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(128, 128, 64), (130, 200, 100), (256, 64, 4096), (300, 257, 1000),
                                   (256, 256, 12288), (129, 17, 520), (200, 1000, 8)])
def test_f16_tiled_gemm_matches_oracle(M, N, K):
    rng = np.random.default_rng(M * 7 + N * 3 + K + 16)
    A, B = rnd(rng, (M, K)), rnd(rng, (N, K), 0.05)
    expect = oracle.gemm_tree(A, B, "NT", "fp16")
    got = dgf.gemm_tree("NT", padded(A), padded(B))
    torch.cuda.synchronize()
    assert_bitwise(got, expect, f"fp16 NT {M}x{N}x{K}")


# ---------------------------------------------------------------- activation
def test_f16_activation_exhaustive_over_gate_values():
    rng = np.random.default_rng(2)
    g = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    g = g[np.isfinite(g.view(np.float16))]
    u = rnd(rng, g.size); da = rnd(rng, g.size)
    a_ref = oracle.act_fwd(g, u, "fp16")
    dg_ref, du_ref, a2_ref = oracle.act_bwd(da, g, u, "fp16")
    gd, ud, dad = dev(g), dev(u), dev(da)
    a = dgf.act_fwd(gd, ud)
    dg, du, a2 = dgf.act_bwd(dad, gd, ud)
    torch.cuda.synchronize()
    assert_bitwise(a, a_ref, "a")
    assert_bitwise(dg, dg_ref, "dG")
    assert_bitwise(du, du_ref, "dU")
    assert_bitwise(a2, a2_ref, "a (backward)")


# ---------------------------------------------------------------- the FFN
def test_f16_tiny_ffn_forward_backward_bitwise():
    c = inputs.tiny_case(dtype=F16)
    b = {k: bits(v) for k, v in c.items()}
    o = oracle.ffn_fwd(b["x"], b["w_gate"], b["w_up"], b["w_down"], "fp16")
    ob = oracle.ffn_bwd(b["dy"], b["x"], o["g"], o["u"], b["w_gate"], b["w_up"], b["w_down"], "fp16")
    d = {k: v.cuda() for k, v in c.items()}
    y, g, u = dgf.ffn_fwd(d["x"], d["w_gate"], d["w_up"], d["w_down"], training=True)
    y_inf = dgf.ffn_fwd(d["x"], d["w_gate"], d["w_up"], d["w_down"])
    r = dgf.ffn_bwd(d["dy"], d["x"], g, u, d["w_gate"], d["w_up"], d["w_down"], lanes=True)
    torch.cuda.synchronize()
    assert y.dtype == F16 and r["dX"].dtype == F16
    assert_bitwise(g, o["g"], "g"); assert_bitwise(u, o["u"], "u"); assert_bitwise(y, o["y"], "y")
    assert_bitwise(y_inf, o["y"], "y (inference)")
    for k in ("dX", "G", "U", "dW_gate", "dW_up", "dW_down"):
        assert_bitwise(r[k], ob[k], k)
    f = fp64.ffn_fwd(b["x"], b["w_gate"], b["w_up"], b["w_down"], "fp16")
    fb = fp64.ffn_bwd(b["dy"], b["x"], b["w_gate"], b["w_up"], b["w_down"], "fp16")
    assert fp64.rel_l2(bits(y), f["y"], "fp16") <= 2e-3
    for k in ("dX", "dW_gate", "dW_up", "dW_down"):
        assert fp64.rel_l2(bits(r[k]), fb[k], "fp16") <= 2e-3, k


# every kernel family: fused gate/up (M <= 32), all-K down (M <= 18), streaming
# (33..127 tokens), tiled (128+), the generic NT/NN kernels, one-leaf and
# transposed weight gradients; ragged sizes throughout
@pytest.mark.parametrize("M,H,I", [(1, 64, 64), (3, 128, 320), (20, 256, 768), (37, 200, 136), (64, 128, 256),
                                   (17, 960, 1000), (32, 2112, 136), (9, 4096, 40), (65, 128, 72),
                                   (130, 256, 200), (256, 192, 520), (3, 198, 512), (16, 136, 1536),
                                   (12, 16, 12288), (23, 16, 12288), (8, 512, 4810)])
def test_f16_ffn_other_shapes_bitwise(M, H, I):
    rng = np.random.default_rng(M + H + I + 16)
    x, dy = rnd(rng, (M, H)), rnd(rng, (M, H))
    wg, wu, wd = rnd(rng, (I, H), 0.02), rnd(rng, (I, H), 0.02), rnd(rng, (H, I), 0.02)
    o = oracle.ffn_fwd(x, wg, wu, wd, "fp16")
    ob = oracle.ffn_bwd(dy, x, o["g"], o["u"], wg, wu, wd, "fp16")
    y, g, u = dgf.ffn_fwd(padded(x), padded(wg), padded(wu), padded(wd), training=True)
    r = dgf.ffn_bwd(padded(dy), padded(x), g, u, padded(wg), padded(wu), padded(wd), lanes=True)
    torch.cuda.synchronize()
    assert_bitwise(y, o["y"], "y"); assert_bitwise(g, o["g"], "g")
    for k in ("dX", "G", "U", "dW_gate", "dW_up", "dW_down"):
        assert_bitwise(r[k], ob[k], k)


@pytest.fixture(scope="module")
def qwen16():
    wg, wu, wd = inputs.ffn_weights(dtype=F16)
    return (wg, wu, wd), (wg.cuda(), wu.cuda(), wd.cuda())


def test_f16_full_size_forward_backward_vs_oracle(qwen16):
    # M = 32 tokens, H = 4096, I = 12288 in FP16
    (wg_c, wu_c, wd_c), (wg, wu, wd) = qwen16
    x_c, dy_c = inputs.activations(32, dtype=F16)
    x, dy = x_c.cuda(), dy_c.cuda()
    y, g, u = dgf.ffn_fwd(x, wg, wu, wd, training=True)
    y_inf = dgf.ffn_fwd(x, wg, wu, wd)
    r = dgf.ffn_bwd(dy, x, g, u, wg, wu, wd, lanes=True)
    torch.cuda.synchronize()
    B = {k: bits(v) for k, v in (("x", x_c), ("dy", dy_c), ("wg", wg_c), ("wu", wu_c), ("wd", wd_c))}
    o = oracle.ffn_fwd(B["x"], B["wg"], B["wu"], B["wd"], "fp16")
    for k, t in (("g", g), ("u", u), ("y", y)):
        assert_bitwise(t, o[k], k)
    assert_bitwise(y_inf, o["y"], "y (inference)")
    da = oracle.gemm_tree(B["dy"], B["wd"], "NN", "fp16")
    dg, du, a = oracle.act_bwd(da, o["g"], o["u"], "fp16")
    G = oracle.gemm_tree(dg, B["wg"], "NN", "fp16"); U = oracle.gemm_tree(du, B["wu"], "NN", "fp16")
    assert_bitwise(r["G"], G, "G lane"); assert_bitwise(r["U"], U, "U lane")
    assert_bitwise(dgf.gemm_tree("NN", dy, wd), da, "dA")
    assert_bitwise(r["dX"], oracle.tree_combine_typed([G, U], "fp16").reshape(G.shape), "dX")
    rows = np.random.default_rng(0).choice(12288, 48, replace=False)
    rows_h = np.random.default_rng(1).choice(4096, 48, replace=False)
    assert_bitwise(bits(r["dW_gate"])[rows], oracle.gemm_tree(np.ascontiguousarray(dg[:, rows]), B["x"], "TN", "fp16"),
                   "dW_gate rows")
    assert_bitwise(bits(r["dW_up"])[rows], oracle.gemm_tree(np.ascontiguousarray(du[:, rows]), B["x"], "TN", "fp16"),
                   "dW_up rows")
    assert_bitwise(bits(r["dW_down"])[rows_h],
                   oracle.gemm_tree(np.ascontiguousarray(B["dy"][:, rows_h]), a, "TN", "fp16"), "dW_down rows")
    f = fp64.ffn_fwd(B["x"], B["wg"], B["wu"], B["wd"], "fp16")
    assert fp64.rel_l2(bits(y), f["y"], "fp16") <= 2e-3
    fb = fp64.ffn_bwd(B["dy"], B["x"], B["wg"], B["wu"], B["wd"], "fp16")
    assert fp64.rel_l2(bits(r["dX"]), fb["dX"], "fp16") <= 2e-3
    # repeatable, and the same rows at fewer tokens (every forward path)
    assert (bits(dgf.ffn_fwd(x, wg, wu, wd)) == bits(y)).all()
    for M in (1, 8, 17, 18, 19, 24):
        assert (bits(dgf.ffn_fwd(x[:M], wg, wu, wd)) == bits(y)[:M]).all(), M


def test_f16_long_sequence_sampled_vs_oracle(qwen16):
    # M = 4096 tokens in FP16: the tiled kernel in both passes; sampled rows and
    # I-slices against the oracle, as for BF16
    (wg_c, wu_c, wd_c), (wg, wu, wd) = qwen16
    M, I = 4096, 12288
    x_c, dy_c = inputs.activations(M, dtype=F16)
    x, dy = x_c.cuda(), dy_c.cuda()
    y, g, u = dgf.ffn_fwd(x, wg, wu, wd, training=True)
    r = dgf.ffn_bwd(dy, x, g, u, wg, wu, wd)
    torch.cuda.synchronize()
    B = {k: bits(v) for k, v in (("x", x_c), ("dy", dy_c), ("wg", wg_c), ("wu", wu_c), ("wd", wd_c))}
    rng = np.random.default_rng(4097)
    ms = np.unique(np.concatenate([[0, 511, 512, 4095], rng.choice(M, 3, replace=False)]))
    cols = np.unique(np.concatenate([[0, I - 1], rng.choice(I, 4, replace=False)]))
    o = oracle.ffn_fwd(B["x"][ms], B["wg"], B["wu"], B["wd"], "fp16")
    for k, t in (("g", g), ("u", u), ("y", y)):
        assert_bitwise(bits(t)[ms], o[k], f"{k} rows")
    ob = oracle.ffn_bwd(B["dy"][ms], B["x"][ms], o["g"], o["u"], B["wg"], B["wu"], B["wd"], "fp16")
    assert_bitwise(bits(r["dX"])[ms], ob["dX"], "dX rows")
    wg_s = np.ascontiguousarray(B["wg"][cols]); wu_s = np.ascontiguousarray(B["wu"][cols])
    wd_s = np.ascontiguousarray(B["wd"][:, cols])
    os_ = oracle.ffn_fwd(B["x"], wg_s, wu_s, wd_s, "fp16")
    obs = oracle.ffn_bwd(B["dy"], B["x"], os_["g"], os_["u"], wg_s, wu_s, wd_s, "fp16")
    assert_bitwise(bits(r["dW_gate"])[cols], obs["dW_gate"], "dW_gate rows")
    assert_bitwise(bits(r["dW_up"])[cols], obs["dW_up"], "dW_up rows")
    assert_bitwise(bits(r["dW_down"])[:, cols], obs["dW_down"], "dW_down columns")
    fs = fp64.ffn_bwd(B["dy"], B["x"], wg_s, wu_s, wd_s, "fp16")
    assert fp64.rel_l2(bits(r["dW_gate"])[cols], fs["dW_gate"], "fp16") <= 2e-3


def test_f16_and_bf16_calls_interleave():
    # the stored type is per call: alternating calls give each type's own bits
    c16 = inputs.tiny_case(dtype=F16); c16 = {k: v.cuda() for k, v in c16.items()}
    c32 = inputs.tiny_case(); c32 = {k: v.cuda() for k, v in c32.items()}
    y16 = dgf.ffn_fwd(c16["x"], c16["w_gate"], c16["w_up"], c16["w_down"])
    yb = dgf.ffn_fwd(c32["x"], c32["w_gate"], c32["w_up"], c32["w_down"])
    y16b = dgf.ffn_fwd(c16["x"], c16["w_gate"], c16["w_up"], c16["w_down"])
    torch.cuda.synchronize()
    assert y16.dtype == F16 and yb.dtype == torch.bfloat16
    assert (bits(y16) == bits(y16b)).all()
    b = {k: bits(v) for k, v in inputs.tiny_case().items()}
    assert (bits(yb) == oracle.ffn_fwd(b["x"], b["w_gate"], b["w_up"], b["w_down"])["y"]).all()
    with pytest.raises(TypeError):
        dgf.ffn_fwd(c16["x"], c32["w_gate"], c16["w_up"], c16["w_down"])
