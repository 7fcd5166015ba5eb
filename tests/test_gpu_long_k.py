"""GPU parity at very long K: trees of thousands of leaves, far past the FFN's
H and I, in the generic tree GEMM (per-wave subtrees of hundreds of leaves,
their pending nodes on an LDS stack of matching depth), the streaming kernel
at its deepest K split (32 pieces, a 32-part join), and the FFN with one of H
and I in the tens of thousands.  Every result is compared bit for bit with
the oracle ("feat(ffn): add deterministic distributed Triton FFN for ROCm",
section "Design": the same canonical tree at any K)."""
import numpy as np
import pytest
import torch

import oracle
from deterministic_gated_ffn_amd import binding as dgf

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the GPU tests need an MI355X")
    dgf.load()


def bits(rng, fmt, shape, scale=1.0):
    x = rng.standard_normal(shape).astype(np.float32) * scale
    if fmt == "fp16":
        return x.astype(np.float16).view(np.uint16)
    return oracle.f32_to_bf16_bits(x)


def dev(bits_, fmt, pad=8):
    R, C = bits_.shape
    full = np.zeros((R, (C + 7) // 8 * 8 + pad), np.uint16)
    full[:, :C] = bits_
    t = torch.from_numpy(full.view(np.int16)).cuda()
    return t.view(torch.float16 if fmt == "fp16" else torch.bfloat16)[:, :C]


def host(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("layout,fmt,M,N,K", [
    ("NT", "bf16", 4, 24, (1 << 20) + 37),   # 16,385 leaves, the last partial
    ("NN", "bf16", 4, 24, (1 << 20) + 37),
    ("NN", "fp16", 4, 24, (1 << 20) + 37),
    ("NT", "bf16", 40, 40, 300_037),         # two token tiles, 4,689 leaves
    ("NT", "bf16", 130, 16, 100_003),        # five token tiles, 1,563 leaves
    ("NT", "bf16", 8, 64, 65_536 - 5),       # 1,024 leaves: 32 K pieces of 4-leaf wave subtrees
    ("NN", "fp16", 20, 72, 65_536 + 64),     # 1,025 leaves
])
def test_long_k_tree_gemm(layout, fmt, M, N, K):
    rng = np.random.default_rng(K + M)
    A, Bnk = bits(rng, fmt, (M, K)), bits(rng, fmt, (N, K))
    b = Bnk if layout == "NT" else np.ascontiguousarray(Bnk.T)
    want = np.asarray(oracle.gemm_tree(A, b, layout, *([] if fmt == "bf16" else ["fp16"])), np.uint16)
    got = host(dgf.gemm_tree(layout, dev(A, fmt), dev(b, fmt)))
    torch.cuda.synchronize()
    bad = int((got != want.reshape(got.shape)).sum())
    assert bad == 0, f"{layout} {fmt} M={M} N={N} K={K}: {bad} of {got.size} differ from the oracle"


@pytest.mark.parametrize("fmt,M,H,I", [
    ("bf16", 4, 64, 40_000),   # down GEMM and dX lanes over 625 leaves
    ("fp16", 4, 64, 40_000),
    ("bf16", 8, 40_000, 64),   # gate/up and dA over 625 leaves
])
def test_long_k_ffn(fmt, M, H, I):
    rng = np.random.default_rng(H + I)
    dt = [] if fmt == "bf16" else ["fp16"]
    x, dy = bits(rng, fmt, (M, H)), bits(rng, fmt, (M, H))
    wg, wu, wd = bits(rng, fmt, (I, H), 0.02), bits(rng, fmt, (I, H), 0.02), bits(rng, fmt, (H, I), 0.02)
    o = oracle.ffn_fwd(x, wg, wu, wd, *dt)
    ob = oracle.ffn_bwd(dy, x, o["g"], o["u"], wg, wu, wd, *dt)
    W = [dev(w, fmt) for w in (wg, wu, wd)]
    xd = dev(x, fmt)
    y, g, u = dgf.ffn_fwd(xd, *W, training=True)
    r = dgf.ffn_bwd(dev(dy, fmt), xd, g, u, *W, lanes=True)
    torch.cuda.synchronize()
    for name, t, ref in (("y", y, o["y"]), ("g", g, o["g"]), ("u", u, o["u"]), ("dX", r["dX"], ob["dX"]),
                         ("G", r["G"], ob["G"]), ("U", r["U"], ob["U"]), ("dW_gate", r["dW_gate"], ob["dW_gate"]),
                         ("dW_up", r["dW_up"], ob["dW_up"]), ("dW_down", r["dW_down"], ob["dW_down"])):
        got = host(t)
        bad = int((got != np.asarray(ref, np.uint16).reshape(got.shape)).sum())
        assert bad == 0, f"{fmt} M={M} H={H} I={I} {name}: {bad} of {got.size} differ from the oracle"
