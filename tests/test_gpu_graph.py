"""GPU: the library's calls captured in a HIP graph and replayed.

Every entry point only enqueues kernels on the caller's stream: no
allocation, no memset, no synchronisation, no stream query.  So a training
step (the forward with g and u saved, then the backward) and the forward
without allocation can be captured once and replayed.  Each replay runs on
new inputs copied into the captured tensors, with eager library calls and
synchronisations between replays, and must equal the eager step on the same
inputs bit for bit; the first replay is also checked against the oracle."""
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


def rand_bits(rng, shape, scale=1.0):
    return oracle.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * scale)


def to_dev(b):
    return torch.from_numpy(b.view(np.int16)).cuda().view(torch.bfloat16)


def host(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def step(x, dy, w):
    y, g, u = dgf.ffn_fwd(x, *w, training=True)
    r = dgf.ffn_bwd(dy, x, g, u, *w)
    return {"y": y, "g": g, "u": u, "dX": r["dX"], "dW_gate": r["dW_gate"], "dW_up": r["dW_up"],
            "dW_down": r["dW_down"]}


# 48 tokens: the streaming kernels at two token tiles with their K-piece joins;
# 160 tokens: the tiled kernel, with the transposed weight copies of the backward
@pytest.mark.parametrize("M,H,I", [(48, 512, 1536), (160, 256, 640)])
def test_training_step_replays_from_a_hip_graph(M, H, I):
    rng = np.random.default_rng(M + H + I)
    hw = [rand_bits(rng, (I, H), 0.02), rand_bits(rng, (I, H), 0.02), rand_bits(rng, (H, I), 0.02)]
    w = [to_dev(b) for b in hw]
    batches = [(rand_bits(rng, (M, H)), rand_bits(rng, (M, H))) for _ in range(4)]
    x, dy = to_dev(batches[0][0]), to_dev(batches[0][1])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(x, dy, w)  # warm the allocator on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = step(x, dy, w)

    for i, (xb, dyb) in enumerate(batches):
        x.copy_(to_dev(xb))
        dy.copy_(to_dev(dyb))
        graph.replay()
        eager = step(x.clone(), dy.clone(), w)
        torch.cuda.synchronize()
        for k, t in out.items():
            got, want = host(t), host(eager[k])
            assert (got == want).all(), f"replay {i} M={M} {k}: {(got != want).sum()} differ from the eager call"
        if i == 0:
            o = oracle.ffn_fwd(xb, *hw)
            ob = oracle.ffn_bwd(dyb, xb, o["g"], o["u"], *hw)
            ref = {"y": o["y"], "g": o["g"], "u": o["u"], **{k: ob[k] for k in ("dX", "dW_gate", "dW_up", "dW_down")}}
            for k, t in out.items():
                got = host(t)
                bad = int((got != np.asarray(ref[k], np.uint16).reshape(got.shape)).sum())
                assert bad == 0, f"replay 0 M={M} {k}: {bad} differ from the oracle"


def test_static_forward_replays_from_a_hip_graph():
    M, H, I = 40, 512, 1536
    rng = np.random.default_rng(5)
    w = [to_dev(rand_bits(rng, (I, H), 0.02)), to_dev(rand_bits(rng, (I, H), 0.02)),
         to_dev(rand_bits(rng, (H, I), 0.02))]
    x = to_dev(rand_bits(rng, (M, H)))
    y = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    dgf.ffn_fwd_static(x, *w, y)  # resolves the scratch array's address before the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dgf.ffn_fwd_static(x, *w, y)
    for i in range(4):
        x.copy_(to_dev(rand_bits(rng, (M, H))))
        graph.replay()
        want = dgf.ffn_fwd(x.clone(), *w)
        torch.cuda.synchronize()
        assert (host(y) == host(want)).all(), f"replay {i}: {(host(y) != host(want)).sum()} differ"
