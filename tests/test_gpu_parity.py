"""GPU parity: the HIP path through the C ABI against the CPU oracle, element by
element, bitwise (0 mismatches), plus run-to-run and shard invariance and the
float64 relative-L2 bound.  The oracle's readings are in oracle/dgf_oracle.c."""
import zlib

import numpy as np
import pytest
import torch

import oracle
from oracle import fp64
from deterministic_gated_ffn_amd import binding as dgf
from deterministic_gated_ffn_amd import inputs

pytestmark = pytest.mark.gpu

F2B = oracle.f32_to_bf16_bits
B2F = oracle.bf16_bits_to_f32


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the GPU tests need an MI355X")
    dgf.load()
    return torch.device("cuda:0")


def dev(bits_or_t):
    if isinstance(bits_or_t, np.ndarray):
        return inputs.from_bits(bits_or_t).cuda()
    return bits_or_t.cuda()


def ordinal(b):
    b = np.asarray(b, np.uint16).astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)


def assert_bitwise(got, expected_bits, name):
    """0 mismatching BF16 bit patterns; on failure report the ulp distances."""
    g = inputs.bits(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.uint16)
    e = np.asarray(expected_bits, np.uint16).reshape(g.shape)
    bad = g != e
    n = int(bad.sum())
    if n:
        d = np.abs(ordinal(g) - ordinal(e))[bad]
        idx = np.argwhere(bad)[:5].tolist()
        pytest.fail(f"{name}: {n}/{g.size} mismatches (exact fraction {1 - n / g.size:.6f}); "
                    f"max ulp {d.max()}, >1 ulp: {(d > 1).sum()}; first at {idx}")


def assert_bitwise_nan(got, expected_bits, name):
    """Bitwise, except that a NaN matches any NaN: the sign and payload of a NaN
    made by an FP32 operation (infinities of both signs) are not part of the
    definition."""
    g = inputs.bits(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.uint16)
    e = np.asarray(expected_bits, np.uint16).reshape(g.shape)
    isnan = lambda b: ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)
    bad = (g != e) & ~(isnan(g) & isnan(e))
    n = int(bad.sum())
    if n:
        pytest.fail(f"{name}: {n}/{g.size} mismatches (NaN against NaN allowed); first at {np.argwhere(bad)[:5].tolist()}")


def rnd(rng, shape, scale=1.0):
    return F2B((rng.standard_normal(shape) * scale).astype(np.float32))


def wide(rng, shape, lo=-20, hi=20):
    """BF16 values with random exponents in [lo, hi] (stresses the block rule)."""
    e = rng.integers(lo, hi + 1, size=shape) + 127
    m = rng.integers(0, 128, size=shape)
    s = rng.integers(0, 2, size=shape)
    return ((s << 15) | (e << 7) | m).astype(np.uint16)


def padded(bits, ld_extra=8):
    """GPU view of a [R, C] matrix whose leading dimension exceeds its width."""
    R, C = bits.shape
    ld = ((C + 7) // 8) * 8 + ld_extra
    full = np.zeros((R, ld), np.uint16)
    full[:, :C] = bits
    return dev(full)[:, :C]


# ---------------------------------------------------------------- tree GEMMs
SHAPES = [(1, 16, 64), (4, 48, 256), (5, 33, 100), (16, 20, 24), (17, 100, 1000), (32, 64, 4096),
          (33, 40, 768), (64, 16, 192), (3, 7, 8), (40, 130, 520), (2, 1, 12288),
          # past the streaming kernel's 1024 leaves: the generic tree GEMM with its LDS stack and K split
          (3, 24, 65600)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_gemm_tree_matches_oracle(layout, M, N, K):
    rng = np.random.default_rng(M * 1000 + N * 10 + K)
    A = rnd(rng, (M, K)); Bnk = rnd(rng, (N, K), 0.02)
    if layout == "NT":
        a, b = A, Bnk
    elif layout == "NN":
        a, b = A, np.ascontiguousarray(Bnk.T)
    else:
        a, b = np.ascontiguousarray(A.T), np.ascontiguousarray(Bnk.T)
    expect = oracle.gemm_tree(a, b, layout)
    got = dgf.gemm_tree(layout, padded(a), padded(b))
    torch.cuda.synchronize()
    assert_bitwise(got, expect, f"{layout} {M}x{N}x{K}")


# many tokens: the tiled kernel (128 x 128 output tiles, K pieces of lower
# subtrees of at most 4 leaves under an LDS-parked top of up to 3 levels)
# The streaming kernel is compiled per launch for the largest leaf count of
# its waves (1..4, the waves holding that many or one fewer), with or without
# a partial last leaf, at one or two token tiles: K over 8 waves gives 1..4
# leaves per wave (512 .. 2048), the same with a partial last leaf (500 ..
# 2000), 10 and 33 leaves (waves of unequal counts); N = 96 leaves a ragged
# column tile in every layout.
@pytest.mark.parametrize("M", [16, 32])
@pytest.mark.parametrize("K", [512, 1024, 1536, 2048, 500, 1000, 1500, 2000, 640, 2112])
@pytest.mark.parametrize("layout", ["NT", "NN"])
def test_streaming_kernel_leaf_counts(layout, K, M):
    N = 96
    rng = np.random.default_rng(7 * K + M)
    A = rnd(rng, (M, K)); Bnk = rnd(rng, (N, K), 0.02)
    b = Bnk if layout == "NT" else np.ascontiguousarray(Bnk.T)
    expect = oracle.gemm_tree(A, b, layout)
    got = dgf.gemm_tree(layout, padded(A), padded(b))
    torch.cuda.synchronize()
    assert_bitwise(got, expect, f"{layout} {M}x{N}x{K}")


MM_SHAPES = [(128, 128, 64), (130, 200, 100), (256, 64, 4096), (300, 257, 1000), (256, 256, 12288), (129, 17, 520),
             (512, 384, 3000), (200, 1000, 8)]


@pytest.mark.parametrize("M,N,K", MM_SHAPES)
def test_tiled_gemm_matches_oracle(M, N, K):
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    A, B = rnd(rng, (M, K)), rnd(rng, (N, K), 0.05)
    expect = oracle.gemm_tree(A, B, "NT")
    got = dgf.gemm_tree("NT", padded(A), padded(B))
    torch.cuda.synchronize()
    assert_bitwise(got, expect, f"NT {M}x{N}x{K}")


def subnormal_mix(rng, shape):
    """Half BF16 subnormals (exponent field 0, any nonzero fraction), half
    normals just above them (exponents -126..-110), random signs."""
    sub = rng.integers(1, 128, size=shape)
    nrm = wide(rng, shape, -126, -110)
    s = rng.integers(0, 2, size=shape) << 15
    return np.where(rng.random(shape) < 0.5, s | sub, nrm).astype(np.uint16)


def sparse_tiny(rng, shape, p=0.8):
    """+-2^-76 at a fraction p of the positions, zeros elsewhere: against 2^-76
    its products are +-2^-152, so a block's sum of a few of them is too small
    for FP32 and rounds to zero (the block rule makes that zero +0)."""
    v = np.where(rng.random(shape) < 0.5, np.uint16(0x1980 | 0x8000), np.uint16(0x1980))  # -+2^-76
    return np.where(rng.random(shape) < p, v, np.uint16(0)).astype(np.uint16)


@pytest.mark.parametrize("dist", ["wide", "wide60", "cancel", "tiny", "ties", "subnormal", "subnormal_tiny",
                                  "zero_sums", "overflow"])
@pytest.mark.parametrize("K", [8, 32, 64, 128, 200])
def test_leaf_block_rule_adversarial(dist, K):
    # The FP32 leaf's accumulation rule on inputs that separate it from other
    # summation orders (wide exponents, cancellation, near-ties, tiny products).
    rng = np.random.default_rng(zlib.crc32(f"{dist}/{K}".encode()))
    M, N = 32, 48
    if dist == "wide":
        A, B = wide(rng, (M, K)), wide(rng, (N, K))
    elif dist == "wide60":
        A, B = wide(rng, (M, K), -60, 60), wide(rng, (N, K), -60, 60)
    elif dist == "cancel":
        A = wide(rng, (M, K), -6, 6); B = F2B(np.ones((N, K), np.float32))
        A[:, K // 2:] = A[:, :K - K // 2][:, :K // 2] ^ np.uint16(0x8000)
        A[:, ::7] = wide(rng, (M, len(range(0, K, 7))), -40, -20)
        B = np.where(rng.random((N, K)) < 0.2, wide(rng, (N, K), -2, 2), B).astype(np.uint16)
    elif dist == "tiny":
        A, B = wide(rng, (M, K), -70, -55), wide(rng, (N, K), -70, -55)
    elif dist == "subnormal":
        # BF16-subnormal operands against large ones: products in the normal FP32 range,
        # where the subnormal's exponent (-126 for the block grid) decides what is cut
        A, B = subnormal_mix(rng, (M, K)), wide(rng, (N, K), 90, 126)
    elif dist == "subnormal_tiny":
        # ... and against small ones: products and sums in the FP32 subnormal range
        A, B = subnormal_mix(rng, (M, K)), wide(rng, (N, K), -30, 10)
    elif dist == "zero_sums":
        A, B = sparse_tiny(rng, (M, K)), np.full((N, K), np.uint16(0x1980), np.uint16)
    elif dist == "overflow":
        # products up to 2^130: those of 2^128 and more are infinities of their sign
        A, B = wide(rng, (M, K), 56, 64), wide(rng, (N, K), 56, 64)
        A[rng.random((M, K)) < 0.85] = 0
    else:
        A = F2B((np.where(rng.random((M, K)) < 0.3, 2.0 ** -rng.integers(22, 27, (M, K)), 0)
                 * np.where(rng.random((M, K)) < 0.7, 1, -1)).astype(np.float32))
        A[:, 0] = F2B(np.ones(M, np.float32))
        B = F2B(np.ones((N, K), np.float32))
    expect = oracle.gemm_tree(A, B, "NT")
    got = dgf.gemm_tree("NT", dev(A), dev(B))
    torch.cuda.synchronize()
    (assert_bitwise_nan if dist == "overflow" else assert_bitwise)(got, expect, f"leaf {dist} K={K}")


def signed_per_leaf(rng, bits, K, p_neg=0.92):
    """bits with one sign for each 64-element leaf of a row, negative with
    probability p_neg, so that whole leaves of products share a sign (and some
    rows have only negative leaves)."""
    rows = bits.shape[0]
    s = (rng.random((rows, (K + 63) // 64)) < p_neg).repeat(64, axis=1)[:, :K].astype(np.uint16)
    return ((bits & np.uint16(0x7FFF)) | (s << 15)).astype(np.uint16)


@pytest.mark.parametrize("dist", ["wide", "cancel", "ties", "tiny", "subnormal_tiny", "negzero", "zero_sums",
                                  "overflow"])
@pytest.mark.parametrize("K", [200, 640, 1536, 2048])
def test_tiled_tree_adversarial(dist, K):
    # The tiled kernel (128 tokens and more) on inputs whose leaves and tree
    # nodes round at ties, sum in the FP32 subnormal range, cancel to zero or
    # are negative zeros (leaves of tiny negative products round to -0; the
    # node of two -0 children is -0, of -0 and +0 is +0).  K = 200 ends in a
    # partial leaf, K = 640 splits into lower subtrees of 2 and 3 leaves, K =
    # 1536 into eight of 3 and K = 2048 into eight of 4 (both whole: the
    # deferred form where the stored type uses it).
    rng = np.random.default_rng(zlib.crc32(f"tiled/{dist}/{K}".encode()))
    M, N = 160, 144
    if dist == "wide":
        A, B = wide(rng, (M, K), -30, 30), wide(rng, (N, K), -30, 30)
    elif dist == "cancel":
        A = wide(rng, (M, K), -6, 6)
        A[:, K // 2:] = A[:, :K - K // 2][:, :K // 2] ^ np.uint16(0x8000)
        B = np.where(rng.random((N, K)) < 0.1, wide(rng, (N, K), -2, 2), F2B(np.ones((N, K), np.float32)))
        B = B.astype(np.uint16)
    elif dist == "ties":
        A = F2B((np.where(rng.random((M, K)) < 0.3, 2.0 ** -rng.integers(6, 10, (M, K)), 0)
                 * np.where(rng.random((M, K)) < 0.7, 1, -1)).astype(np.float32))
        A[:, ::64] = F2B(np.ones((M, len(range(0, K, 64))), np.float32))
        B = F2B(np.ones((N, K), np.float32))
    elif dist == "tiny":
        A, B = wide(rng, (M, K), -70, -55), wide(rng, (N, K), -70, -55)
    elif dist == "subnormal_tiny":
        A, B = subnormal_mix(rng, (M, K)), wide(rng, (N, K), -30, 10)
    elif dist == "zero_sums":
        A, B = sparse_tiny(rng, (M, K)), np.full((N, K), np.uint16(0x1980), np.uint16)
    elif dist == "overflow":
        A, B = wide(rng, (M, K), 56, 64), wide(rng, (N, K), 56, 64)
        A[rng.random((M, K)) < 0.85] = 0
    else:  # products of about 2^-146: every leaf rounds to a zero of its sign
        A = wide(rng, (M, K), -74, -72) & np.uint16(0x7FFF)
        B = signed_per_leaf(rng, wide(rng, (N, K), -74, -72), K)
        B[rng.random((N, K)) < 0.02] = 0
    expect = oracle.gemm_tree(A, B, "NT")
    got = dgf.gemm_tree("NT", padded(A), padded(B))
    torch.cuda.synchronize()
    (assert_bitwise_nan if dist == "overflow" else assert_bitwise)(got, expect, f"tiled {dist} K={K}")
    if dist == "negzero":
        assert (expect == 0x8000).any() and (expect == 0).any(), "the case should make zeros of both signs"


def test_gemm_k_zero_and_m_zero():
    A = torch.zeros((4, 0), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((8, 0), dtype=torch.bfloat16, device="cuda")
    C = dgf.gemm_tree("NT", A, B)
    torch.cuda.synchronize()
    assert (C.float() == 0).all()
    assert (inputs.bits(C) == 0).all()  # the empty tree is +0
    A0 = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    assert dgf.gemm_tree("NT", A0, torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda")).shape == (0, 8)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
def test_ffn_with_no_tokens(dt):
    # M = 0: the forward and dX are empty; each weight gradient is the tree over
    # K = M = 0 leaves, +0 as in the oracle, written over whatever dW held
    H, I = 40, 72
    rng = np.random.default_rng(3)
    w = [torch.from_numpy(rng.standard_normal(s).astype(np.float32) * 0.02).to(dt).cuda()
         for s in ((I, H), (I, H), (H, I))]
    x = torch.zeros((0, H), dtype=dt, device="cuda")
    y, g, u = dgf.ffn_fwd(x, *w, training=True)
    assert y.shape == (0, H) and g.shape == (0, I) and u.shape == (0, I)
    dw = [torch.full(s, float("nan"), dtype=dt, device="cuda") for s in ((I, H), (I, H), (H, I))]
    dx = torch.empty((0, H), dtype=dt, device="cuda")
    L = dgf.load()
    st = L.dgf_ffn_bwd_typed(None, H, None, H, None, None, I, w[0].data_ptr(), H, w[1].data_ptr(), H,
                             w[2].data_ptr(), I, dx.data_ptr(), None, None, H, dw[0].data_ptr(), H,
                             dw[1].data_ptr(), H, dw[2].data_ptr(), I, 0, H, I, None, 0,
                             dgf.DGF_FP16 if dt == torch.float16 else dgf.DGF_BF16,
                             torch.cuda.current_stream().cuda_stream)
    assert st == 0, L.dgf_last_error()
    r = dgf.ffn_bwd(torch.zeros((0, H), dtype=dt, device="cuda"), x, g, u, *w)
    torch.cuda.synchronize()
    hb = lambda shape: np.zeros(shape, np.uint16)
    zx, zu = hb((0, H)), hb((0, I))
    o = oracle.ffn_bwd(zx, zx, zu, zu, hb((I, H)), hb((I, H)), hb((H, I)),
                       *([] if dt == torch.bfloat16 else ["fp16"]))
    for got, name in zip(dw + [r["dW_gate"], r["dW_up"], r["dW_down"]], ["dW_gate", "dW_up", "dW_down"] * 2):
        assert (inputs.bits(got) == np.asarray(o[name], np.uint16)).all(), name
    assert r["dX"].shape == (0, H)


# ---------------------------------------------------------------- activation
def test_activation_exhaustive_over_gate_values():
    rng = np.random.default_rng(1)
    g = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    gf = B2F(g)
    g = g[np.isfinite(gf)]
    u = rnd(rng, g.size); da = rnd(rng, g.size)
    a_ref = oracle.act_fwd(g, u)
    dg_ref, du_ref, a2_ref = oracle.act_bwd(da, g, u)
    gd, ud, dad = dev(g), dev(u), dev(da)
    a = dgf.act_fwd(gd, ud)
    dg, du, a2 = dgf.act_bwd(dad, gd, ud)
    torch.cuda.synchronize()
    assert_bitwise(a, a_ref, "a")
    assert_bitwise(dg, dg_ref, "dG")
    assert_bitwise(du, du_ref, "dU")
    assert_bitwise(a2, a2_ref, "a (backward)")


# ---------------------------------------------------------------- combine
@pytest.mark.parametrize("S", [1, 2, 4, 8])
@pytest.mark.parametrize("n", [1, 7, 8, 1000, 4097])
def test_tree_combine(S, n):
    rng = np.random.default_rng(S * 7 + n)
    parts = [rnd(rng, n) for _ in range(S)]
    expect = oracle.tree_combine(parts)
    got = dgf.tree_combine([dev(p) for p in parts])
    torch.cuda.synchronize()
    assert_bitwise(got, expect, f"combine S={S} n={n}")
    # offset (unaligned) views take the element path with the same arithmetic
    bufs = [torch.zeros(n + 1, dtype=torch.bfloat16, device="cuda") for _ in range(S)]
    for b, p in zip(bufs, parts):
        b[1:] = dev(p)
    out = torch.zeros(n + 1, dtype=torch.bfloat16, device="cuda")
    dgf.tree_combine_ptrs([b.data_ptr() + 2 for b in bufs], S, out.data_ptr() + 2, n)
    torch.cuda.synchronize()
    assert_bitwise(out[1:], expect, f"combine offset S={S} n={n}")
    # in place into parts[0]
    p0 = [dev(p) for p in parts]
    dgf.tree_combine(p0, out=p0[0])
    torch.cuda.synchronize()
    assert_bitwise(p0[0], expect, f"combine in place S={S} n={n}")


@pytest.mark.parametrize("dtype", ["fp16", "fp32"])
@pytest.mark.parametrize("S", [1, 2, 4, 8])
@pytest.mark.parametrize("n", [1, 5, 8, 1000, 4099])
def test_tree_combine_fp16_fp32(dtype, S, n):
    # the same rank tree in FP16 and FP32, against the oracle, bitwise; values
    # over a wide exponent range (FP16 subnormals and overflow included)
    rng = np.random.default_rng(S * 31 + n + (7 if dtype == "fp16" else 0))
    tdt = torch.float16 if dtype == "fp16" else torch.float32
    if dtype == "fp16":
        parts = [(rng.standard_normal(n) * 2.0 ** rng.integers(-26, 11, n)).astype(np.float16) for _ in range(S)]
        raw = [p.view(np.uint16) for p in parts]
        expect = oracle.tree_combine_typed(raw, "fp16")
        to_dev = lambda p: torch.from_numpy(p.view(np.int16).copy()).view(torch.float16).cuda()
        bits_of = lambda t: t.detach().cpu().view(torch.int16).numpy().view(np.uint16)
    else:
        parts = [(rng.standard_normal(n) * 10.0 ** rng.integers(-30, 30, n)).astype(np.float32) for _ in range(S)]
        raw = parts
        expect = oracle.tree_combine_typed(raw, "fp32").view(np.uint32)
        to_dev = lambda p: torch.from_numpy(p.copy()).cuda()
        bits_of = lambda t: t.detach().cpu().numpy().view(np.uint32)
    got = dgf.tree_combine([to_dev(p) for p in parts])
    torch.cuda.synchronize()
    assert (bits_of(got) == expect).all(), f"{dtype} S={S} n={n}: {(bits_of(got) != expect).sum()} mismatches"
    # offset views (one element in): the element path, same arithmetic
    bufs = [torch.zeros(n + 1, dtype=tdt, device="cuda") for _ in range(S)]
    for b, p in zip(bufs, parts):
        b[1:] = to_dev(p)
    out = torch.zeros(n + 1, dtype=tdt, device="cuda")
    es = bufs[0].element_size()
    dgf.tree_combine_ptrs([b.data_ptr() + es for b in bufs], S, out.data_ptr() + es, n,
                          dtype=dgf.DGF_FP16 if dtype == "fp16" else dgf.DGF_FP32)
    torch.cuda.synchronize()
    assert (bits_of(out[1:]) == expect).all(), f"{dtype} offset S={S} n={n}"


def test_tree_combine_hand_worked_and_errors():
    one, a = 0x3F80, 0x3B80
    vals = np.array([one, a, a, a, a, a, a, a], np.uint16)
    parts = [dev(np.array([v], np.uint16)) for v in vals]
    assert int(inputs.bits(dgf.tree_combine(parts))[0]) == 0x3F83
    with pytest.raises(dgf.DgfError):
        dgf.tree_combine(parts[:3])


# ---------------------------------------------------------------- the FFN
def _tiny():
    c = inputs.tiny_case()
    return c, {k: inputs.bits(v) for k, v in c.items()}


def test_tiny_ffn_forward_backward_bitwise():
    c, b = _tiny()
    o = oracle.ffn_fwd(b["x"], b["w_gate"], b["w_up"], b["w_down"])
    ob = oracle.ffn_bwd(b["dy"], b["x"], o["g"], o["u"], b["w_gate"], b["w_up"], b["w_down"])
    d = {k: v.cuda() for k, v in c.items()}
    y, g, u = dgf.ffn_fwd(d["x"], d["w_gate"], d["w_up"], d["w_down"], training=True)
    y_inf = dgf.ffn_fwd(d["x"], d["w_gate"], d["w_up"], d["w_down"])
    r = dgf.ffn_bwd(d["dy"], d["x"], g, u, d["w_gate"], d["w_up"], d["w_down"], lanes=True)
    torch.cuda.synchronize()
    assert_bitwise(g, o["g"], "g"); assert_bitwise(u, o["u"], "u"); assert_bitwise(y, o["y"], "y")
    assert_bitwise(y_inf, o["y"], "y (inference)")
    for k in ("dX", "G", "U", "dW_gate", "dW_up", "dW_down"):
        assert_bitwise(r[k], ob[k], k)
    f = fp64.ffn_fwd(b["x"], b["w_gate"], b["w_up"], b["w_down"])
    fb = fp64.ffn_bwd(b["dy"], b["x"], b["w_gate"], b["w_up"], b["w_down"])
    assert fp64.rel_l2(inputs.bits(y), f["y"]) <= 1e-2
    for k in ("dX", "dW_gate", "dW_up", "dW_down"):
        assert fp64.rel_l2(inputs.bits(r[k]), fb[k]) <= 1e-2, k


@pytest.mark.parametrize("M,H,I", [(1, 64, 64), (3, 128, 320), (20, 256, 768), (37, 200, 136), (64, 128, 256),
                                   (5, 512, 200), (17, 960, 1000), (32, 2112, 136), (9, 4096, 40), (32, 576, 24),
                                   (65, 128, 72), (100, 256, 200), (130, 256, 200), (256, 192, 520),
                                   # down projection over all K per workgroup (M <= 18): 1..32 leaves per wave,
                                   # ragged H
                                   (3, 198, 512), (11, 64, 1024), (16, 136, 1536), (16, 96, 2048), (5, 40, 3072),
                                   (8, 72, 4096), (15, 48, 6144), (12, 16, 12288), (2, 32, 8192), (16, 24, 16384),
                                   (4, 8, 512), (2, 1, 1024),
                                   # ... and with two token tiles (17, 18 tokens); from 19 the streaming kernel
                                   (17, 64, 1024), (18, 200, 1536), (18, 16, 12288),
                                   (19, 64, 1024), (20, 200, 1536), (24, 136, 3072), (23, 16, 12288),
                                   # fused gate/up with more 16-column tiles than workgroups, unevenly
                                   # spread (301 and 514 tiles, the last one ragged)
                                   (8, 512, 4810), (32, 576, 8220)])
def test_ffn_other_shapes_bitwise(M, H, I):
    rng = np.random.default_rng(M + H + I)
    x, dy = rnd(rng, (M, H)), rnd(rng, (M, H))
    wg, wu, wd = rnd(rng, (I, H), 0.02), rnd(rng, (I, H), 0.02), rnd(rng, (H, I), 0.02)
    o = oracle.ffn_fwd(x, wg, wu, wd)
    ob = oracle.ffn_bwd(dy, x, o["g"], o["u"], wg, wu, wd)
    y, g, u = dgf.ffn_fwd(padded(x), padded(wg), padded(wu), padded(wd), training=True)
    r = dgf.ffn_bwd(padded(dy), padded(x), g, u, padded(wg), padded(wu), padded(wd), lanes=True)
    torch.cuda.synchronize()
    assert_bitwise(y, o["y"], "y")
    for k in ("dX", "G", "U", "dW_gate", "dW_up", "dW_down"):
        assert_bitwise(r[k], ob[k], k)


@pytest.mark.parametrize("M,H,I", [(48, 1024, 3072), (200, 512, 1536), (130, 256, 4096)])
def test_inference_forward_many_tokens(M, H, I):
    # The inference forward (no g/u saved) past 32 tokens: the streaming
    # gate/up GEMM (33..127 tokens) or the tiled one (128 and more) with the
    # activation in the join, then the down projection.  Against the oracle,
    # and the same y bits as the training forward (PR #325, "Correctness
    # results": training and inference forward agree).
    rng = np.random.default_rng(M * 3 + H + I)
    x = rnd(rng, (M, H))
    wg, wu, wd = rnd(rng, (I, H), 0.02), rnd(rng, (I, H), 0.02), rnd(rng, (H, I), 0.02)
    o = oracle.ffn_fwd(x, wg, wu, wd)
    xd, wgd, wud, wdd = padded(x), padded(wg), padded(wu), padded(wd)
    y_inf = dgf.ffn_fwd(xd, wgd, wud, wdd)
    y_tr, g, u = dgf.ffn_fwd(xd, wgd, wud, wdd, training=True)
    torch.cuda.synchronize()
    assert_bitwise(y_inf, o["y"], f"y (inference) M={M}")
    assert_bitwise(y_tr, o["y"], f"y (training) M={M}")
    assert_bitwise(g, o["g"], "g"); assert_bitwise(u, o["u"], "u")


# ---------------------------------------------------------------- Qwen3-8B shapes
@pytest.fixture(scope="module")
def qwen_weights():
    wg, wu, wd = inputs.ffn_weights()
    return (wg, wu, wd), (wg.cuda(), wu.cuda(), wd.cuda())


def test_repeat_and_batch_invariance(qwen_weights):
    _, (wg, wu, wd) = qwen_weights
    x32, dy32 = (t.cuda() for t in inputs.activations(32))
    ys = [inputs.bits(dgf.ffn_fwd(x32, wg, wu, wd)) for _ in range(3)]
    assert all((y == ys[0]).all() for y in ys), "forward not bitwise repeatable"
    y, g, u = dgf.ffn_fwd(x32, wg, wu, wd, training=True)
    b1 = dgf.ffn_bwd(dy32, x32, g, u, wg, wu, wd)
    b2 = dgf.ffn_bwd(dy32, x32, g, u, wg, wu, wd)
    torch.cuda.synchronize()
    assert (inputs.bits(y) == ys[0]).all(), "training forward differs from inference"
    for k in b1:
        assert (inputs.bits(b1[k]) == inputs.bits(b2[k])).all(), f"{k} not bitwise repeatable"
    # every forward path (one or two token tiles, all-K or split-K down projection) gives the same rows
    for M in (1, 8, 16, 17, 24, 25):
        yM = inputs.bits(dgf.ffn_fwd(x32[:M], wg, wu, wd))
        assert (yM == ys[0][:M]).all(), f"M={M} rows differ from the M=32 rows"
    # other buffers for the same weights, another stream: the same bits
    wg2, wu2, wd2 = wg.clone(), wu.clone(), wd.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        y3, g3, u3 = dgf.ffn_fwd(x32, wg2, wu2, wd2, training=True)
        b3 = dgf.ffn_bwd(dy32, x32, g3, u3, wg2, wu2, wd2)
    side.synchronize()
    assert (inputs.bits(y3) == ys[0]).all(), "forward differs on other buffers / another stream"
    for k in b1:
        assert (inputs.bits(b3[k]) == inputs.bits(b1[k])).all(), f"{k} differs on other buffers / another stream"


def test_full_size_forward_backward_vs_oracle(qwen_weights):
    (wg_c, wu_c, wd_c), (wg, wu, wd) = qwen_weights
    x_c, dy_c = inputs.activations(32)
    x, dy = x_c.cuda(), dy_c.cuda()
    y, g, u = dgf.ffn_fwd(x, wg, wu, wd, training=True)
    r = dgf.ffn_bwd(dy, x, g, u, wg, wu, wd, lanes=True)
    torch.cuda.synchronize()
    B = {k: inputs.bits(v) for k, v in (("x", x_c), ("dy", dy_c), ("wg", wg_c), ("wu", wu_c), ("wd", wd_c))}
    o = oracle.ffn_fwd(B["x"], B["wg"], B["wu"], B["wd"])
    for k, t in (("g", g), ("u", u), ("y", y)):
        assert_bitwise(t, o[k], k)
    # backward: all of dA-driven dX; dW on sampled rows (the oracle is slow at 50M outputs)
    da = oracle.gemm_tree(B["dy"], B["wd"], "NN")
    dg, du, a = oracle.act_bwd(da, o["g"], o["u"])
    G = oracle.gemm_tree(dg, B["wg"], "NN"); U = oracle.gemm_tree(du, B["wu"], "NN")
    assert_bitwise(r["G"], G, "G lane"); assert_bitwise(r["U"], U, "U lane")
    # the standalone dA tree GEMM (K = H along the rows of W_down) at the full shape
    assert_bitwise(dgf.gemm_tree("NN", dy, wd), da, "dA")
    assert_bitwise(r["dX"], oracle.tree_combine([G, U]).reshape(G.shape), "dX")
    rows = np.random.default_rng(0).choice(12288, 48, replace=False)
    rows_h = np.random.default_rng(1).choice(4096, 48, replace=False)
    dwg_ref = oracle.gemm_tree(np.ascontiguousarray(dg[:, rows]), B["x"], "TN")
    dwu_ref = oracle.gemm_tree(np.ascontiguousarray(du[:, rows]), B["x"], "TN")
    dwd_ref = oracle.gemm_tree(np.ascontiguousarray(B["dy"][:, rows_h]), a, "TN")
    assert_bitwise(r["dW_gate"][rows.tolist()], dwg_ref, "dW_gate rows")
    assert_bitwise(r["dW_up"][rows.tolist()], dwu_ref, "dW_up rows")
    assert_bitwise(r["dW_down"][rows_h.tolist()], dwd_ref, "dW_down rows")
    # float64 brute force: relative L2 <= 1e-2
    f = fp64.ffn_fwd(B["x"], B["wg"], B["wu"], B["wd"])
    assert fp64.rel_l2(inputs.bits(y), f["y"]) <= 1e-2
    fb = fp64.ffn_bwd(B["dy"], B["x"], B["wg"], B["wu"], B["wd"])
    assert fp64.rel_l2(inputs.bits(r["dX"]), fb["dX"]) <= 1e-2
    assert fp64.rel_l2(inputs.bits(r["dW_gate"])[rows], fb["dW_gate"][rows]) <= 1e-2


@pytest.fixture(scope="module")
def qwen_oracle_m32(qwen_weights):
    """The oracle's M=32 forward and the dX part of the backward at the full shape."""
    (wg_c, wu_c, wd_c), _ = qwen_weights
    x_c, dy_c = inputs.activations(32)
    B = {k: inputs.bits(v) for k, v in (("x", x_c), ("dy", dy_c), ("wg", wg_c), ("wu", wu_c), ("wd", wd_c))}
    o = oracle.ffn_fwd(B["x"], B["wg"], B["wu"], B["wd"])
    da = oracle.gemm_tree(B["dy"], B["wd"], "NN")
    dg, du, _ = oracle.act_bwd(da, o["g"], o["u"])
    G = oracle.gemm_tree(dg, B["wg"], "NN"); U = oracle.gemm_tree(du, B["wu"], "NN")
    return {"y": o["y"], "g": o["g"], "dA": da, "G": G, "U": U, "dX": oracle.tree_combine([G, U]).reshape(G.shape)}


@pytest.mark.parametrize("S", [2, 4, 8])
def test_shard_invariance(qwen_weights, qwen_oracle_m32, S):
    # Contiguous K shards computed as separate partial GEMMs and combined with the
    # balanced tree equal the unsharded result bit for bit (PR #325 "Design").
    _, (wg, wu, wd) = qwen_weights
    H, I = 4096, 12288
    x, dy = (t.cuda() for t in inputs.activations(32))
    y, g, u = dgf.ffn_fwd(x, wg, wu, wd, training=True)
    full = dgf.ffn_bwd(dy, x, g, u, wg, wu, wd, lanes=True)
    Is, Hs = I // S, H // S
    # I-shards: the forward's down projection (K = I) and the backward's dX lanes (K = I)
    ys, Gs, Us = [], [], []
    for r in range(S):
        sl = slice(r * Is, (r + 1) * Is)
        yr, gr, ur = dgf.ffn_fwd(x, wg[sl], wu[sl], wd[:, sl], training=True)
        br = dgf.ffn_bwd(dy, x, gr, ur, wg[sl], wu[sl], wd[:, sl], lanes=True)
        ys.append(yr.contiguous()); Gs.append(br["G"].contiguous()); Us.append(br["U"].contiguous())
        # dW under I-shards are slices of the unsharded dW (K = M is not sharded)
        assert (inputs.bits(br["dW_gate"]) == inputs.bits(full["dW_gate"][sl])).all()
        assert (inputs.bits(br["dW_down"]) == inputs.bits(full["dW_down"][:, sl])).all()
    y_c = dgf.tree_combine(ys)
    G_c, U_c = dgf.tree_combine(Gs), dgf.tree_combine(Us)
    dx_c = dgf.tree_combine([G_c, U_c])  # gate lane first, then up
    # H-shards: gate/up (K = H) and dA (K = H)
    g_parts = [dgf.gemm_tree("NT", x[:, r * Hs:(r + 1) * Hs], wg[:, r * Hs:(r + 1) * Hs]).contiguous() for r in range(S)]
    da_parts = [dgf.gemm_tree("NN", dy[:, r * Hs:(r + 1) * Hs], wd[r * Hs:(r + 1) * Hs]).contiguous() for r in range(S)]
    g_c = dgf.tree_combine(g_parts)
    da_c = dgf.tree_combine(da_parts)
    da_full = dgf.gemm_tree("NN", dy, wd)
    torch.cuda.synchronize()
    for got, ref, name in ((y_c, y, "y"), (G_c, full["G"], "G"), (U_c, full["U"], "U"), (dx_c, full["dX"], "dX"),
                           (g_c, g, "g"), (da_c, da_full, "dA")):
        gb, rb = inputs.bits(got), inputs.bits(ref.contiguous())
        assert int((gb != rb).sum()) == 0, f"S={S} {name}: {(gb != rb).sum()} mismatches vs unsharded"
        # and the combined shards against the oracle's unsharded result directly
        assert_bitwise(got, qwen_oracle_m32[name], f"S={S} combined {name} vs oracle")


def test_bad_arguments_raise():
    x = torch.zeros((4, 256), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((768, 256), dtype=torch.bfloat16, device="cuda")
    wd = torch.zeros((256, 768), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dgf.DgfError) as e:
        dgf.ffn_fwd(x[:, 1:], w[:, 1:], w[:, 1:], wd[1:])  # misaligned views
    assert e.value.status == 1


def test_long_sequence_sampled_vs_oracle(qwen_weights):
    # M = 4096 tokens (8 sequences x 512), the compute-bound shape: the whole
    # forward and backward run on the GPU; the oracle checks sampled token rows
    # of g, u, y and dX (every output depends on its own token row only) and
    # sampled I-slices of the weight gradients (dW_gate/dW_up rows and dW_down
    # columns depend only on their slice of I, with K = all 4096 tokens).
    (wg_c, wu_c, wd_c), (wg, wu, wd) = qwen_weights
    M, H, I = 4096, 4096, 12288
    x_c, dy_c = inputs.activations(M)
    x, dy = x_c.cuda(), dy_c.cuda()
    y, g, u = dgf.ffn_fwd(x, wg, wu, wd, training=True)
    r = dgf.ffn_bwd(dy, x, g, u, wg, wu, wd)
    torch.cuda.synchronize()
    B = {k: inputs.bits(v) for k, v in (("x", x_c), ("dy", dy_c), ("wg", wg_c), ("wu", wu_c), ("wd", wd_c))}
    rng = np.random.default_rng(4096)
    ms = np.unique(np.concatenate([[0, 511, 512, 4095], rng.choice(M, 4, replace=False)]))
    cols = np.unique(np.concatenate([[0, I - 1], rng.choice(I, 6, replace=False)]))
    # token rows
    o = oracle.ffn_fwd(B["x"][ms], B["wg"], B["wu"], B["wd"])
    for k, t in (("g", g), ("u", u), ("y", y)):
        assert_bitwise(inputs.bits(t)[ms], o[k], f"{k} rows")
    ob = oracle.ffn_bwd(B["dy"][ms], B["x"][ms], o["g"], o["u"], B["wg"], B["wu"], B["wd"])
    assert_bitwise(inputs.bits(r["dX"])[ms], ob["dX"], "dX rows")
    # I-slices of the weight gradients
    wg_s = np.ascontiguousarray(B["wg"][cols]); wu_s = np.ascontiguousarray(B["wu"][cols])
    wd_s = np.ascontiguousarray(B["wd"][:, cols])
    os_ = oracle.ffn_fwd(B["x"], wg_s, wu_s, wd_s)
    obs = oracle.ffn_bwd(B["dy"], B["x"], os_["g"], os_["u"], wg_s, wu_s, wd_s)
    assert_bitwise(inputs.bits(g)[:, cols], os_["g"], "g columns")
    assert_bitwise(inputs.bits(r["dW_gate"])[cols], obs["dW_gate"], "dW_gate rows")
    assert_bitwise(inputs.bits(r["dW_up"])[cols], obs["dW_up"], "dW_up rows")
    assert_bitwise(inputs.bits(r["dW_down"])[:, cols], obs["dW_down"], "dW_down columns")
    # float64 brute force on the same samples: relative L2 <= 1e-2
    f = fp64.ffn_fwd(B["x"][ms], B["wg"], B["wu"], B["wd"])
    assert fp64.rel_l2(inputs.bits(y)[ms], f["y"]) <= 1e-2
    fb = fp64.ffn_bwd(B["dy"][ms], B["x"][ms], B["wg"], B["wu"], B["wd"])
    assert fp64.rel_l2(inputs.bits(r["dX"])[ms], fb["dX"]) <= 1e-2
    fs = fp64.ffn_bwd(B["dy"], B["x"], wg_s, wu_s, wd_s)
    for k in ("dW_gate", "dW_up"):
        assert fp64.rel_l2(inputs.bits(r[k])[cols], fs[k]) <= 1e-2, k
    assert fp64.rel_l2(inputs.bits(r["dW_down"])[:, cols], fs["dW_down"]) <= 1e-2


def test_token_shard_weight_gradients(qwen_weights):
    # Token (context-parallel) shards of the weight gradients.  The pages
    # gather whole token sequences before the weight-gradient GEMMs so that
    # their K tree is the unsharded one (PR #325, section "Design").  K = M is
    # the token axis, so 512-token shards of the M=4096 case are 8-leaf
    # subtrees of that tree: per-shard backward passes combined with the
    # balanced tree reproduce the unsharded weight gradients bit for bit.
    (wg_c, wu_c, wd_c), (wg, wu, wd) = qwen_weights
    M, S = 4096, 8
    x_c, dy_c = inputs.activations(M)
    x, dy = x_c.cuda(), dy_c.cuda()
    y, g, u = dgf.ffn_fwd(x, wg, wu, wd, training=True)
    full = dgf.ffn_bwd(dy, x, g, u, wg, wu, wd)
    Ms = M // S
    parts = {k: [] for k in ("dW_gate", "dW_up", "dW_down")}
    for r in range(S):
        sl = slice(r * Ms, (r + 1) * Ms)
        br = dgf.ffn_bwd(dy[sl], x[sl], g[sl], u[sl], wg, wu, wd)
        # dX rows are local to their tokens
        assert (inputs.bits(br["dX"]) == inputs.bits(full["dX"][sl])).all()
        for k in parts:
            parts[k].append(br[k].contiguous())
    combined = {}
    for k, ps in parts.items():
        got = dgf.tree_combine(ps)
        torch.cuda.synchronize()
        gb, rb = inputs.bits(got), inputs.bits(full[k].contiguous())
        assert int((gb != rb).sum()) == 0, f"{k}: {(gb != rb).sum()} mismatches vs unsharded"
        combined[k] = gb.reshape(full[k].shape)
    # the combined shards against the oracle directly, on sampled I-slices (every
    # dW_gate/dW_up row and dW_down column depends on its own slice of I only)
    B = {k: inputs.bits(v) for k, v in (("x", x_c), ("dy", dy_c), ("wg", wg_c), ("wu", wu_c), ("wd", wd_c))}
    cols = np.unique(np.concatenate([[0, 12287], np.random.default_rng(512).choice(12288, 2, replace=False)]))
    wg_s, wu_s = np.ascontiguousarray(B["wg"][cols]), np.ascontiguousarray(B["wu"][cols])
    wd_s = np.ascontiguousarray(B["wd"][:, cols])
    os_ = oracle.ffn_fwd(B["x"], wg_s, wu_s, wd_s)
    obs = oracle.ffn_bwd(B["dy"], B["x"], os_["g"], os_["u"], wg_s, wu_s, wd_s)
    assert_bitwise(combined["dW_gate"][cols], obs["dW_gate"], "combined dW_gate rows vs oracle")
    assert_bitwise(combined["dW_up"][cols], obs["dW_up"], "combined dW_up rows vs oracle")
    assert_bitwise(combined["dW_down"][:, cols], obs["dW_down"], "combined dW_down columns vs oracle")


def test_sub_leaf_token_shards_need_the_gather():
    # Shards smaller than one 64-token leaf are not subtrees: combining their
    # partial weight gradients rounds each part to BF16 on its own and differs
    # from the unsharded leaf, which is why the tokens are gathered first
    # (PR #325, section "Design"); the gathered tokens give the unsharded
    # result.  Checked against the oracle.
    rng = np.random.default_rng(7)
    M, H, I = 32, 64, 48
    dg, x = rnd(rng, (M, I)), rnd(rng, (M, H))
    full = oracle.gemm_tree(dg, x, "TN")
    parts = [oracle.gemm_tree(np.ascontiguousarray(dg[r * 8:(r + 1) * 8]), np.ascontiguousarray(x[r * 8:(r + 1) * 8]), "TN")
             for r in range(4)]
    combined = oracle.tree_combine(parts).reshape(full.shape)
    assert (combined != full).sum() > 0  # per-shard rounding changes the result
    got = dgf.gemm_tree("TN", dev(dg), dev(x))  # the gathered tokens: one leaf over all 32
    torch.cuda.synchronize()
    assert_bitwise(got, full, "gathered dW")


def test_kernel_timing_hook_keeps_results_and_times_each_launch():
    """The timing hook hands its events to the launches themselves: the timed
    call gives the same bits, every launch gets a positive duration, and the
    durations fit inside the call's own wall time."""
    rng = np.random.default_rng(11)
    M, H, I = 32, 512, 1024
    x = dev(rnd(rng, (M, H)))
    wg, wu, wd = (dev(rnd(rng, s, 0.02)) for s in ((I, H), (I, H), (H, I)))
    y0 = inputs.bits(dgf.ffn_fwd(x, wg, wu, wd))
    timer = dgf.KernelTimer(max_kernels=16)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    timer.start()
    y1 = dgf.ffn_fwd(x, wg, wu, wd)
    timer.stop()
    e1.record()
    torch.cuda.synchronize()
    assert (inputs.bits(y1) == y0).all(), "a timed call changed the result"
    d = timer.durations_ms()
    assert timer.count == len(d) >= 2
    assert d[0][0] == "gate/up + act"
    assert all(ms > 0 for _, ms in d), d
    assert sum(ms for _, ms in d) <= e0.elapsed_time(e1) * 1.05, (d, e0.elapsed_time(e1))


def test_kernel_timing_hook_spans_a_two_kernel_step():
    """tree_combine over a length that is not a multiple of 8 runs a vector body
    and a scalar tail: one timed step whose interval covers both kernels."""
    rng = np.random.default_rng(12)
    n = 1 << 20
    parts = [dev(rnd(rng, (n + 3,))) for _ in range(4)]
    ref = dgf.tree_combine(parts)
    timer = dgf.KernelTimer(max_kernels=4)
    timer.start()
    got = dgf.tree_combine(parts)
    timer.stop()
    torch.cuda.synchronize()
    assert (inputs.bits(got) == inputs.bits(ref)).all()
    d = timer.durations_ms()
    assert timer.count == 1 and len(d) == 1 and d[0][0] == "tree_combine" and d[0][1] > 0, d


def test_concurrent_calls_on_two_streams():
    """The library keeps no device state: two training steps enqueued on two
    streams at once, each with its own buffers, give the bits of one step alone."""
    rng = np.random.default_rng(13)
    M, H, I = 32, 512, 1536
    x, dy = dev(rnd(rng, (M, H))), dev(rnd(rng, (M, H)))
    wg, wu, wd = (dev(rnd(rng, s, 0.02)) for s in ((I, H), (I, H), (H, I)))
    y0, g0, u0 = dgf.ffn_fwd(x, wg, wu, wd, training=True)
    r0 = dgf.ffn_bwd(dy, x, g0, u0, wg, wu, wd)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        for st in streams:
            with torch.cuda.stream(st):
                y, g, u = dgf.ffn_fwd(x, wg, wu, wd, training=True)
                outs.append((y, dgf.ffn_bwd(dy, x, g, u, wg, wu, wd)))
    torch.cuda.synchronize()
    for y, r in outs:
        assert (inputs.bits(y) == inputs.bits(y0)).all()
        for k in r0:
            assert (inputs.bits(r[k]) == inputs.bits(r0[k])).all(), k


@pytest.mark.parametrize("M", [5, 32, 48, 200])
@pytest.mark.parametrize("outs", ["lanes", "gate_lane_and_dx", "up_lane_only", "dx_only"])
def test_bwd_dx_outputs_in_any_combination(M, outs):
    # dx and the two lanes are each optional (at least one given): every
    # combination writes exactly the outputs given, each equal to the oracle's
    # (the lanes G and U, and dX = bf16(G + U) with the gate lane first)
    H, I, ld_h, ld_i = 196, 516, 200, 520
    rng = np.random.default_rng(M)
    f = lambda r, c, s=1.0: F2B((rng.standard_normal((r, c)) * s).astype(np.float32))
    x, dy = f(M, H), f(M, H)
    wg, wu, wd = f(I, H, 0.02), f(I, H, 0.02), f(H, I, 0.02)
    o = oracle.ffn_fwd(x, wg, wu, wd)
    ob = oracle.ffn_bwd(dy, x, o["g"], o["u"], wg, wu, wd)

    def padded(b, ld):
        full = np.zeros((b.shape[0], ld), np.uint16)
        full[:, :b.shape[1]] = b
        return torch.from_numpy(full.view(np.int16)).cuda()

    X, DY = padded(x, ld_h), padded(dy, ld_h)
    G_, U_ = padded(o["g"], ld_i), padded(o["u"], ld_i)
    WG, WU, WD = padded(wg, ld_h), padded(wu, ld_h), padded(wd, ld_i)
    nan = lambda r, c: torch.full((r, c), 0x7FC0, dtype=torch.int16, device="cuda")
    dx, gl, ul = nan(M, ld_h), nan(M, ld_h), nan(M, ld_h)
    dwg, dwu, dwd = nan(I, ld_h), nan(I, ld_h), nan(H, ld_i)
    want = {"lanes": ("G", "U"), "gate_lane_and_dx": ("G", "dX"), "up_lane_only": ("U",), "dx_only": ("dX",)}[outs]
    bufs = {"dX": dx, "G": gl, "U": ul}
    ptr = lambda k: bufs[k].data_ptr() if k in want else None
    L = dgf.load()
    ws = torch.empty(max(L.dgf_ffn_bwd_workspace(M, H, I), 16), dtype=torch.uint8, device="cuda")
    st = L.dgf_ffn_bwd(DY.data_ptr(), ld_h, X.data_ptr(), ld_h, G_.data_ptr(), U_.data_ptr(), ld_i,
                       WG.data_ptr(), ld_h, WU.data_ptr(), ld_h, WD.data_ptr(), ld_i,
                       ptr("dX"), ptr("G"), ptr("U"), ld_h, dwg.data_ptr(), ld_h, dwu.data_ptr(), ld_h,
                       dwd.data_ptr(), ld_i, M, H, I, ws.data_ptr(), ws.numel(),
                       torch.cuda.current_stream().cuda_stream)
    assert st == 0, L.dgf_last_error()
    torch.cuda.synchronize()
    host = lambda t, c: t.cpu().numpy().view(np.uint16)[:, :c]
    for k, buf in bufs.items():
        got = host(buf, H)
        if k in want:
            assert (got == ob[k]).all(), f"M={M} {outs} {k}: {(got != ob[k]).sum()} differ from the oracle"
        else:
            assert (got == 0x7FC0).all(), f"M={M} {outs}: {k} was not asked for but was written"
    for k, buf, c in (("dW_gate", dwg, H), ("dW_up", dwu, H), ("dW_down", dwd, I)):
        assert (host(buf, c) == ob[k]).all(), f"M={M} {outs} {k}"
