"""Host logic of bench.py that needs no GPU: the algorithmic byte counts and
the ulp distance used to report the step's agreement with the oracle."""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def test_ordinal_is_the_ulp_distance():
    b = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x3F80, 0x3F81, 0x7F7F, 0xFF7F], np.uint16)
    o = bench.ordinal(b)
    assert o[0] == o[1] == 0                        # +0 and -0
    assert o[2] - o[3] == 2                         # the two smallest subnormals straddle zero
    assert o[5] - o[4] == 1                         # 1.0 and the next BF16 up
    assert o[6] == -o[7] and o[6] == 0x7F7F         # largest finite values, both signs
    assert (np.diff(bench.ordinal(np.arange(0, 0x7F80, dtype=np.uint16))) == 1).all()


def test_step_bytes_count_each_operand_once():
    H, I, BF = bench.H, bench.I, 2
    W = H * I * BF
    for M in (1, 8, 32):
        act_mh, act_mi = M * H * BF, M * I * BF
        # three weights read in the forward; the backward reads them again and writes three gradients
        assert bench.step_bytes(M) >= 9 * W
        assert bench.kernel_bytes("gate/up + act", M) == 2 * W + act_mh + 3 * act_mi
        assert bench.kernel_bytes("down join", M) is None
    assert bench.step_bytes(32) == 910426112
