"""GPU: calls on caller-chosen streams, and the two-stream schedule of the dX
lanes (RL-Kernel PR #325, section "Communication overlap assessment"), against
the library's own backward and the oracle, bitwise."""
import numpy as np
import pytest
import torch

import oracle
from deterministic_gated_ffn_amd import binding as dgf
from deterministic_gated_ffn_amd import inputs
from deterministic_gated_ffn_amd import schedules

pytestmark = pytest.mark.gpu

F2B = oracle.f32_to_bf16_bits


def rnd(rng, shape, scale=1.0):
    return F2B((rng.standard_normal(shape) * scale).astype(np.float32))


def dev(bits):
    return inputs.from_bits(bits).cuda()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the GPU tests need an MI355X")
    dgf.load()


def test_explicit_stream_argument_while_the_current_stream_allocates():
    # Every wrapper allocates its outputs and workspace on the stream it
    # launches on.  While the calls run on a side stream, the current stream
    # allocates and overwrites fresh tensors: the caching allocator must not
    # hand them the side stream's blocks, so the results keep their bits.
    rng = np.random.default_rng(21)
    M, H, I = 32, 1024, 3072
    x, dy = dev(rnd(rng, (M, H))), dev(rnd(rng, (M, H)))
    wg, wu, wd = (dev(rnd(rng, s, 0.02)) for s in ((I, H), (I, H), (H, I)))
    y0, g0, u0 = dgf.ffn_fwd(x, wg, wu, wd, training=True)
    r0 = dgf.ffn_bwd(dy, x, g0, u0, wg, wu, wd)
    c0 = dgf.gemm_tree("NN", dy, wd)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(4):
        y, g, u = dgf.ffn_fwd(x, wg, wu, wd, training=True, stream=side)
        r = dgf.ffn_bwd(dy, x, g, u, wg, wu, wd, stream=side)
        c = dgf.gemm_tree("NN", dy, wd, stream=side)
        outs.append((y, r, c))
        # the current stream churns through allocations of the same sizes and writes them
        junk = [torch.full((sz,), 7, dtype=torch.uint8, device="cuda")
                for sz in (dgf.load().dgf_ffn_bwd_workspace(M, H, I), M * H * 2, I * H * 2, M * I * 2)]
        del junk
    side.synchronize()
    torch.cuda.synchronize()
    for y, r, c in outs:
        assert (inputs.bits(y) == inputs.bits(y0)).all()
        assert (inputs.bits(c) == inputs.bits(c0)).all()
        for k in r0:
            assert (inputs.bits(r[k]) == inputs.bits(r0[k])).all(), k


@pytest.mark.parametrize("M,H,I", [(32, 4096, 12288), (8, 1024, 3072), (5, 512, 1000)])
def test_two_stream_lanes_equal_the_fused_backward_and_the_oracle(M, H, I):
    # G and U as two NN tree GEMMs on two streams, joined by events, then the
    # ordered add as the two-part rank tree: the same bits as the one-launch
    # lanes of dgf_ffn_bwd and as the oracle's gate-first dX.
    if (M, H, I) == (32, 4096, 12288):
        wg_c, wu_c, wd_c = inputs.ffn_weights()
        x_c, dy_c = inputs.activations(32)
        B = {k: inputs.bits(v) for k, v in (("x", x_c), ("dy", dy_c), ("wg", wg_c), ("wu", wu_c), ("wd", wd_c))}
    else:
        rng = np.random.default_rng(M + H + I)
        B = {"x": rnd(rng, (M, H)), "dy": rnd(rng, (M, H)), "wg": rnd(rng, (I, H), 0.02),
             "wu": rnd(rng, (I, H), 0.02), "wd": rnd(rng, (H, I), 0.02)}
    d = {k: dev(v) for k, v in B.items()}
    y, g, u = dgf.ffn_fwd(d["x"], d["wg"], d["wu"], d["wd"], training=True)
    fused = dgf.ffn_bwd(d["dy"], d["x"], g, u, d["wg"], d["wu"], d["wd"], lanes=True)
    dA = dgf.gemm_tree("NN", d["dy"], d["wd"])
    dG, dU, _ = dgf.act_bwd(dA, g, u)
    two = schedules.TwoStreamLanes()
    runs = [two(dG, dU, d["wg"], d["wu"]) for _ in range(3)]
    serial = schedules.serial_lanes(dG, dU, d["wg"], d["wu"])
    torch.cuda.synchronize()
    ref = {k: inputs.bits(fused[k]) for k in ("dX", "G", "U")}
    for dX, G, U in runs + [serial]:
        assert (inputs.bits(G) == ref["G"]).all()
        assert (inputs.bits(U) == ref["U"]).all()
        assert (inputs.bits(dX) == ref["dX"]).all()
    # the oracle's gate-first dX
    o = oracle.ffn_fwd(B["x"], B["wg"], B["wu"], B["wd"])
    da = oracle.gemm_tree(B["dy"], B["wd"], "NN")
    odg, odu, _ = oracle.act_bwd(da, o["g"], o["u"])
    OG, OU = oracle.gemm_tree(odg, B["wg"], "NN"), oracle.gemm_tree(odu, B["wu"], "NN")
    odx = oracle.tree_combine([OG, OU]).reshape(OG.shape)
    assert (inputs.bits(runs[0][0]) == odx).all(), int((inputs.bits(runs[0][0]) != odx).sum())
    assert (inputs.bits(runs[0][1]) == OG).all()


def test_concurrent_calls_from_two_host_threads():
    # The library keeps no shared state between calls (the error message and
    # the timing hook are per thread), so two host threads may drive it at once,
    # each on a stream of its own (ctypes releases the GIL during each call).
    # Every result must equal the same call made alone; the second thread's
    # errors must not leak into the first thread's message.
    import threading

    M, H, I = 40, 512, 1536
    rng = np.random.default_rng(11)
    f = lambda shape, s=1.0: torch.from_numpy(rng.standard_normal(shape).astype(np.float32) * s).to(torch.bfloat16).cuda()
    w = [f((I, H), 0.02), f((I, H), 0.02), f((H, I), 0.02)]
    work = [(f((M, H)), f((M, H))) for _ in range(2)]

    def run(x, dy):
        y, g, u = dgf.ffn_fwd(x, *w, training=True)
        r = dgf.ffn_bwd(dy, x, g, u, *w)
        return [y, r["dX"], r["dW_gate"], r["dW_up"], r["dW_down"]]

    alone = [[inputs.bits(t) for t in run(x, dy)] for x, dy in work]
    torch.cuda.synchronize()
    got = [None, None]
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(5):
                    outs = run(*work[i])
                    if i == 1:  # a rejected call on this thread only: x's leading dimension is not a multiple of 8
                        bad_x = torch.zeros((M, H + 1), dtype=torch.bfloat16, device="cuda")[:, :H]
                        with pytest.raises(dgf.DgfError, match="leading dimension"):
                            dgf.ffn_fwd(bad_x, *w)
                s.synchronize()
            got[i] = [inputs.bits(t) for t in outs]
        except Exception as e:  # reported by the main thread
            errors.append(f"thread {i}: {e!r}")

    before = dgf.load().dgf_last_error()
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for i in range(2):
        for k, (a, b) in enumerate(zip(got[i], alone[i])):
            assert (a == b).all(), f"thread {i} output {k}: {(a != b).sum()} differ from the call made alone"
    assert dgf.load().dgf_last_error() == before  # the other thread's error stayed on that thread
