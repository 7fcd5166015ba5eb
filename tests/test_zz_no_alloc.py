"""GPU: the forward without a workspace (dgf_ffn_fwd_static, for callers that
cannot allocate) through the C ABI, against dgf_ffn_fwd with a caller
workspace, bitwise: two calls in a row, the second smaller, in training and
inference mode; and the size limit."""
import ctypes

import numpy as np
import pytest
import torch

from deterministic_gated_ffn_amd import binding as dgf
from deterministic_gated_ffn_amd import inputs

pytestmark = pytest.mark.gpu


def _bf16(rng, shape, scale=1.0):
    return (torch.from_numpy(rng.standard_normal(shape).astype(np.float32)) * scale).to(torch.bfloat16).cuda()


def _call_static(L, x, wg, wu, wd, y, g=None, u=None):
    ptr = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
    return L.dgf_ffn_fwd_static(ptr(x), x.stride(0), ptr(wg), wg.stride(0), ptr(wu), wu.stride(0), ptr(wd), wd.stride(0),
                                ptr(y), y.stride(0), ptr(g), ptr(u), g.stride(0) if g is not None else 0,
                                x.shape[0], x.shape[1], wg.shape[0], ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def test_static_forward_matches_the_workspace_forward():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the GPU tests need an MI355X")
    L = dgf.load()
    rng = np.random.default_rng(77)
    H, I = 4096, 12288
    wg, wu, wd = _bf16(rng, (I, H), 0.02), _bf16(rng, (I, H), 0.02), _bf16(rng, (H, I), 0.02)
    # two calls in a row, the second with a smaller input: the scratch keeps the
    # first call's contents, which the second must not depend on
    for M in (48, 32, 8):
        x = _bf16(rng, (M, H))
        y_ref, g_ref, u_ref = dgf.ffn_fwd(x, wg, wu, wd, training=True)
        y_inf_ref = dgf.ffn_fwd(x, wg, wu, wd)
        y = torch.full((M, H), 3.0, dtype=torch.bfloat16, device="cuda")
        g = torch.full((M, I), 3.0, dtype=torch.bfloat16, device="cuda")
        u = torch.full((M, I), 3.0, dtype=torch.bfloat16, device="cuda")
        assert _call_static(L, x, wg, wu, wd, y, g, u) == 0, L.dgf_last_error()
        y2 = torch.full((M, H), 3.0, dtype=torch.bfloat16, device="cuda")
        assert _call_static(L, x, wg, wu, wd, y2) == 0, L.dgf_last_error()
        torch.cuda.synchronize()
        for got, ref, name in ((y, y_ref, "y"), (g, g_ref, "g"), (u, u_ref, "u"), (y2, y_inf_ref, "y (inference)")):
            gb, rb = inputs.bits(got), inputs.bits(ref.contiguous())
            assert (gb == rb).all(), f"M={M} {name}: {(gb != rb).sum()} mismatches"
    # the binding wrapper takes the same path
    x = _bf16(rng, (5, H))
    y = torch.empty((5, H), dtype=torch.bfloat16, device="cuda")
    dgf.ffn_fwd_static(x, wg, wu, wd, y)
    ref = dgf.ffn_fwd(x, wg, wu, wd)
    torch.cuda.synchronize()
    assert (inputs.bits(y) == inputs.bits(ref)).all()


def test_static_forward_rejects_problems_past_its_scratch():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the GPU tests need an MI355X")
    L = dgf.load()
    H, I, M = 4096, 12288, 256
    assert L.dgf_ffn_fwd_workspace(M, H, I) > dgf.STATIC_SCRATCH_BYTES
    x = torch.zeros((M, H), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((I, H), dtype=torch.bfloat16, device="cuda")
    wd = torch.zeros((H, I), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros((M, H), dtype=torch.bfloat16, device="cuda")
    st = _call_static(L, x, w, w, wd, y)
    assert st == 2, st  # DGF_EUNSUPPORTED, nothing enqueued
    assert b"scratch" in L.dgf_last_error()
    with pytest.raises(dgf.DgfError):
        dgf.ffn_fwd_static(x, w, w, wd, y)
