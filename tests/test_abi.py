"""The C-ABI library loads and exports every entry point include/dgf.h declares;
argument validation answers before any HIP call (no GPU needed here)."""
import ctypes
import os
import re

import pytest

from deterministic_gated_ffn_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dgf.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dgf_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.lib_path()):
        pytest.fail("libdgf.so is not built (python -m deterministic_gated_ffn_amd.build)")
    return binding.load()


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("dgf_ffn_fwd", "dgf_ffn_bwd", "dgf_tree_combine", "dgf_tree_combine_typed", "dgf_gemm_tree",
                     "dgf_act_fwd", "dgf_act_bwd", "dgf_last_error", "dgf_ffn_fwd_typed", "dgf_ffn_bwd_typed",
                     "dgf_gemm_tree_typed", "dgf_act_fwd_typed", "dgf_act_bwd_typed"):
        assert required in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in binding.SIGNATURES, f"binding lacks {name}"


def test_constants(lib):
    assert lib.dgf_abi_version() == 2
    assert lib.dgf_leaf_size() == 64


def test_workspace_queries(lib):
    assert lib.dgf_ffn_fwd_workspace(0, 4096, 12288) == 0
    assert lib.dgf_ffn_fwd_workspace(32, 4096, 12288) >= 32 * 12288 * 2
    assert lib.dgf_ffn_bwd_workspace(32, 4096, 12288) >= 32 * 12288 * 2 * 5
    assert lib.dgf_gemm_tree_workspace(binding.DGF_NT, 4, 4, 4) == 0
    assert lib.dgf_gemm_tree_workspace(binding.DGF_TN, 4, 4, 4) == 0  # one leaf: operands read in place
    assert lib.dgf_gemm_tree_workspace(binding.DGF_TN, 4, 4, 100) > 0  # transposed copies


FAKE = 1 << 20  # a 16-byte aligned stand-in address; never dereferenced by these calls


def test_fwd_validation(lib):
    st = lib.dgf_ffn_fwd(None, 256, FAKE, 256, FAKE, 256, FAKE, 768, FAKE, 256, None, None, 0,
                         4, 256, 768, FAKE, 1 << 20, None)
    assert st == 1 and b"x is NULL" in lib.dgf_last_error()
    st = lib.dgf_ffn_fwd(FAKE + 2, 256, FAKE, 256, FAKE, 256, FAKE, 768, FAKE, 256, None, None, 0,
                         4, 256, 768, FAKE, 1 << 20, None)
    assert st == 1 and b"aligned" in lib.dgf_last_error()
    st = lib.dgf_ffn_fwd(FAKE, 100, FAKE, 256, FAKE, 256, FAKE, 768, FAKE, 256, None, None, 0,
                         4, 256, 768, FAKE, 1 << 20, None)
    assert st == 1 and b"leading dimension" in lib.dgf_last_error()
    st = lib.dgf_ffn_fwd(FAKE, 260, FAKE, 256, FAKE, 256, FAKE, 768, FAKE, 256, None, None, 0,
                         4, 256, 768, FAKE, 1 << 20, None)
    assert st == 1 and b"multiple of 8" in lib.dgf_last_error()
    st = lib.dgf_ffn_fwd(FAKE, 256, FAKE, 256, FAKE, 256, FAKE, 768, FAKE, 256, FAKE, None, 768,
                         4, 256, 768, FAKE, 1 << 20, None)
    assert st == 1 and b"g_save" in lib.dgf_last_error()
    st = lib.dgf_ffn_fwd(FAKE, 256, FAKE, 256, FAKE, 256, FAKE, 768, FAKE, 256, None, None, 0,
                         4, 256, 768, FAKE, 16, None)
    assert st == 3 and b"workspace" in lib.dgf_last_error()
    st = lib.dgf_ffn_fwd(FAKE, 256, FAKE, 256, FAKE, 256, FAKE, 768, FAKE, 256, None, None, 0,
                         -1, 256, 768, FAKE, 1 << 20, None)
    assert st == 1
    # M = 0: nothing to do, no launch
    assert lib.dgf_ffn_fwd(None, 0, None, 0, None, 0, None, 0, None, 0, None, None, 0,
                           0, 256, 768, None, 0, None) == 0


def test_bwd_validation(lib):
    args = [FAKE, 256, FAKE, 256, FAKE, FAKE, 768, FAKE, 256, FAKE, 256, FAKE, 768,
            None, None, None, 256, FAKE, 256, FAKE, 256, FAKE, 768, 4, 256, 768, FAKE, 1 << 24, None]
    assert lib.dgf_ffn_bwd(*args) == 1 and b"no dX output" in lib.dgf_last_error()
    args[13] = FAKE
    args[17] = None
    assert lib.dgf_ffn_bwd(*args) == 1 and b"dw_gate" in lib.dgf_last_error()
    args[17] = FAKE
    args[-2] = 100
    assert lib.dgf_ffn_bwd(*args) == 3
    # no tokens: the weight gradients are still written (+0), so their buffers are checked
    empty = [None, 256, None, 256, None, None, 768, FAKE, 256, FAKE, 256, FAKE, 768,
             None, None, None, 256, None, 256, FAKE, 256, FAKE, 768, 0, 256, 768, None, 0, None]
    assert lib.dgf_ffn_bwd(*empty) == 1 and b"dw_gate" in lib.dgf_last_error()


def test_combine_validation(lib):
    arr = (ctypes.c_void_p * 3)(FAKE, FAKE, FAKE)
    assert lib.dgf_tree_combine(arr, 3, FAKE, 10, None) == 2
    assert b"S=3" in lib.dgf_last_error()
    arr8 = (ctypes.c_void_p * 8)(*([FAKE] * 8))
    assert lib.dgf_tree_combine(arr8, 8, FAKE, 0, None) == 0      # n = 0: no launch
    assert lib.dgf_tree_combine(arr8, 8, None, 10, None) == 1
    assert lib.dgf_tree_combine(arr8, 8, FAKE + 1, 10, None) == 1
    assert lib.dgf_tree_combine(arr8, 8, FAKE, -1, None) == 1
    arr2 = (ctypes.c_void_p * 2)(FAKE, None)
    assert lib.dgf_tree_combine(arr2, 2, FAKE, 10, None) == 1


def test_typed_combine_validation(lib):
    arr4 = (ctypes.c_void_p * 4)(*([FAKE] * 4))
    assert lib.dgf_tree_combine_typed(arr4, 4, FAKE, 0, binding.DGF_FP32, None) == 0  # n = 0: no launch
    assert lib.dgf_tree_combine_typed(arr4, 4, FAKE, 10, 7, None) == 1
    assert b"dtype" in lib.dgf_last_error()
    assert lib.dgf_tree_combine_typed(arr4, 3, FAKE, 10, binding.DGF_FP16, None) == 2
    assert lib.dgf_tree_combine_typed(arr4, 4, FAKE + 2, 10, binding.DGF_FP32, None) == 1  # FP32 needs 4-byte alignment
    assert b"aligned" in lib.dgf_last_error()
    assert lib.dgf_tree_combine_typed(arr4, 4, FAKE + 1, 10, binding.DGF_FP16, None) == 1
    assert lib.dgf_tree_combine_typed(arr4, 4, None, 10, binding.DGF_BF16, None) == 1


def test_gemm_validation(lib):
    assert lib.dgf_gemm_tree(7, FAKE, 8, FAKE, 8, FAKE, 8, 4, 4, 4, None, 0, None) == 1
    assert lib.dgf_gemm_tree(binding.DGF_NT, FAKE, 8, FAKE, 8, FAKE, 8, 0, 4, 4, None, 0, None) == 0
    # TN past one leaf needs transposed copies in the workspace
    assert lib.dgf_gemm_tree(binding.DGF_TN, FAKE, 8, FAKE, 8, FAKE, 8, 4, 4, 100, None, 0, None) == 3
    assert lib.dgf_gemm_tree(binding.DGF_NN, FAKE, 4, FAKE, 8, FAKE, 8, 4, 4, 8, None, 0, None) == 1
    # a 128-row tile's byte offsets must stay below 2^31: leading dimensions below 2^23, K at most 2^23
    assert lib.dgf_gemm_tree(binding.DGF_NT, FAKE, 1 << 23, FAKE, 8, FAKE, 8, 4, 4, 4, None, 0, None) == 2
    assert b"leading dimension" in lib.dgf_last_error()
    assert lib.dgf_gemm_tree(binding.DGF_NT, FAKE, (1 << 23) + 8, FAKE, (1 << 23) + 8, FAKE, 8,
                             4, 4, (1 << 23) + 8, None, 0, None) == 2
    assert lib.dgf_act_fwd(None, FAKE, FAKE, 10, None) == 1
    assert lib.dgf_act_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == 0


def test_typed_entry_points_validate_the_dtype(lib):
    # FP32 has no declared leaf: unsupported; an unknown code: invalid; both before any HIP call
    fwd = lambda dt, M=4: lib.dgf_ffn_fwd_typed(FAKE, 256, FAKE, 256, FAKE, 256, FAKE, 768, FAKE, 256, None, None, 0,
                                                M, 256, 768, FAKE, 1 << 30, dt, None)
    assert fwd(binding.DGF_FP32) == 2
    assert b"FP32" in lib.dgf_last_error()
    assert fwd(9) == 1
    assert b"dtype" in lib.dgf_last_error()
    assert fwd(binding.DGF_FP16, M=0) == 0  # empty input: no launch
    assert lib.dgf_ffn_fwd_typed(None, 256, FAKE, 256, FAKE, 256, FAKE, 768, FAKE, 256, None, None, 0,
                                 4, 256, 768, FAKE, 1 << 30, binding.DGF_FP16, None) == 1
    assert b"x" in lib.dgf_last_error()
    bwd = lambda dt: lib.dgf_ffn_bwd_typed(FAKE, 256, FAKE, 256, FAKE, FAKE, 768, FAKE, 256, FAKE, 256, FAKE, 768,
                                           FAKE, None, None, 256, FAKE, 256, FAKE, 256, FAKE, 768, 4, 256, 768,
                                           FAKE, 0, dt, None)
    assert bwd(binding.DGF_FP32) == 2
    assert bwd(binding.DGF_FP16) == 3  # reaches the workspace check: no workspace given
    gemm = lambda dt: lib.dgf_gemm_tree_typed(binding.DGF_TN, FAKE, 8, FAKE, 8, FAKE, 8, 4, 4, 100, None, 0, dt, None)
    assert gemm(binding.DGF_FP32) == 2 and gemm(-1) == 1 and gemm(binding.DGF_FP16) == 3
    assert lib.dgf_act_fwd_typed(FAKE, FAKE, FAKE, 10, binding.DGF_FP32, None) == 2
    assert lib.dgf_act_fwd_typed(None, FAKE, FAKE, 10, binding.DGF_FP16, None) == 1
    assert lib.dgf_act_bwd_typed(FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, binding.DGF_FP16, None) == 0
    assert lib.dgf_act_bwd_typed(FAKE, FAKE, FAKE, FAKE, FAKE, None, 10, 5, None) == 1


def test_profile_hook_validation(lib):
    assert lib.dgf_profile_begin(None, 1) == 1
    assert lib.dgf_profile_begin(None, -1) == 1
    arr = (ctypes.c_void_p * 2)(FAKE, None)
    assert lib.dgf_profile_begin(arr, 1) == 1
    assert b"NULL" in lib.dgf_last_error()
    # no events: nothing is recorded, and a call that launches nothing counts nothing
    assert lib.dgf_profile_begin(None, 0) == 0
    arr4 = (ctypes.c_void_p * 4)(*([FAKE] * 4))
    assert lib.dgf_tree_combine_typed(arr4, 4, FAKE, 0, binding.DGF_BF16, None) == 0
    assert lib.dgf_profile_end() == 0
    assert lib.dgf_profile_name(0) == b""
    assert lib.dgf_profile_name(-1) == b""


def test_static_forward_binding_checks_its_arguments(lib):
    # the entry point without allocation takes BF16 only and both saves or neither;
    # the binding refuses other calls before anything reaches the library
    import torch
    t16 = torch.zeros(4, 8, dtype=torch.float16)
    tb = torch.zeros(4, 8, dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="bfloat16"):
        binding.ffn_fwd_static(t16, t16, t16, t16, t16)
    with pytest.raises(ValueError, match="both g and u"):
        binding.ffn_fwd_static(tb, tb, tb, tb, tb, g=tb)


C_CALLER = r"""
#include <stdio.h>
#include <string.h>
#include "dgf.h"

int main(void) {
    if (dgf_abi_version() != 2 || dgf_leaf_size() != 64) return 1;
    size_t ws = dgf_ffn_fwd_workspace(32, 4096, 12288);
    /* a NULL input is refused before any HIP call */
    dgf_status st = dgf_ffn_fwd(NULL, 4096, NULL, 4096, NULL, 4096, NULL, 12288, NULL, 4096,
                                NULL, NULL, 0, 32, 4096, 12288, NULL, ws, NULL);
    if (st != DGF_EINVAL || strlen(dgf_last_error()) == 0) return 2;
    printf("%zu %d %s\n", ws, (int)st, dgf_last_error());
    return 0;
}
"""


def test_header_compiles_and_links_as_plain_c(lib, tmp_path):
    # the boundary is a C ABI: the header compiles as C11 with warnings as
    # errors, and a C program links the library and gets its validation
    import subprocess
    src = tmp_path / "caller.c"
    src.write_text(C_CALLER)
    exe = tmp_path / "caller"
    libdir = os.path.dirname(binding.lib_path())
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-L", libdir, "-ldgf", f"-Wl,-rpath,{libdir}", "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, (out.returncode, out.stdout, out.stderr)
    ws, st, msg = out.stdout.split(" ", 2)
    assert int(ws) == lib.dgf_ffn_fwd_workspace(32, 4096, 12288) and int(st) == 1 and msg.strip()
