"""Host-side schedules composed of the C-ABI calls (no arithmetic here).

Two-stream dX lanes (RL-Kernel PR #325, section "Communication overlap
assessment": the pages' next step runs the up-lane dX GEMM on a second stream
beside the gate lane, then adds the two in order).  The gate lane
G = T_I(dG W_gate) and the up lane U = T_I(dU W_up) are independent tree GEMMs;
each runs as one `dgf_gemm_tree` NN call on its own stream, both streams wait
for the caller's stream first, the caller's stream waits for both through
events, and the ordered add dX = bf16(G + U) (gate lane first) is the rank
tree over the two lanes, `dgf_tree_combine({G, U}, 2)`.  The order of the
add is fixed by the combine, so the bits do not depend on which lane ends
first.  The library's own backward runs both lanes in one launch instead
(`dgf_ffn_bwd`); this schedule is the alternative the pages name.
"""
from __future__ import annotations

import torch

from . import binding as dgf


class TwoStreamLanes:
    """Holds the two side streams (default priority) and their events."""

    def __init__(self, device=None):
        self.gate_stream = torch.cuda.Stream(device=device)
        self.up_stream = torch.cuda.Stream(device=device)
        self.gate_done = torch.cuda.Event()
        self.up_done = torch.cuda.Event()

    def __call__(self, dG, dU, w_gate, w_up):
        """Returns (dX, G, U), all ready on the caller's current stream."""
        cur = torch.cuda.current_stream()
        self.gate_stream.wait_stream(cur)
        self.up_stream.wait_stream(cur)
        G = dgf.gemm_tree("NN", dG, w_gate, stream=self.gate_stream)
        self.gate_done.record(self.gate_stream)
        U = dgf.gemm_tree("NN", dU, w_up, stream=self.up_stream)
        self.up_done.record(self.up_stream)
        cur.wait_event(self.gate_done)
        cur.wait_event(self.up_done)
        # the lanes were allocated on the side streams; the caller's stream uses them from here on
        G.record_stream(cur)
        U.record_stream(cur)
        for t in (dG, w_gate):
            t.record_stream(self.gate_stream)
        for t in (dU, w_up):
            t.record_stream(self.up_stream)
        dX = dgf.tree_combine([G.contiguous(), U.contiguous()]).view(G.shape[0], -1)
        return dX, G, U


def serial_lanes(dG, dU, w_gate, w_up):
    """The same two lane GEMMs and ordered add on the caller's stream, one after the other."""
    G = dgf.gemm_tree("NN", dG, w_gate)
    U = dgf.gemm_tree("NN", dU, w_up)
    dX = dgf.tree_combine([G.contiguous(), U.contiguous()]).view(G.shape[0], -1)
    return dX, G, U
