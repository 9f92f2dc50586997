"""The fused attention call captured once in a HIP graph and replayed.

Every call on the per-call path only launches kernels on the caller's stream
(the plan's workspace is allocated and cleared at plan creation; counters and
cursors are reset by kernels, never by memset nodes), so the five calls of
one attention step can be captured and replayed.  Each replay, with eager
calls and synchronisations between replays, must give exactly the eager
result, also after new inputs are copied into the captured buffers.
"""
import numpy as np
import pytest
import torch

from block_sparse_spatiotemporal_amd import fva, synth
from tests._helpers import to_dev

pytestmark = pytest.mark.gpu

CASES = [
    synth.scaled(synth.WORKLOADS["wan1.3b_480p"], H=3, grid=(9, 10, 13)),
    synth.scaled(synth.WORKLOADS["wan_720p_hilbert_sub"], H=2, grid=(7, 9, 14)),
    synth.scaled(synth.WORKLOADS["hetero_slack"], H=4, grid=(6, 9, 13)),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_fused_call_replays_in_a_hip_graph(w):
    plan = fva.Plan(w.B, w.H, w.D, w.grid, tile=w.tile, order=w.order, sub=w.sub, dtype=w.dtype)
    q, k, v, meta = synth.make(w)
    p = meta["p_head"].tolist() * w.B if isinstance(w.p, tuple) else float(meta["p_head"][0])
    qd, kd, vd = (to_dev(x, w.dtype) for x in (q, k, v))
    # inputs the graph reads, and a second input set copied in later
    qg, kg, vg = qd.clone(), kd.clone(), vd.clone()
    q2, k2, v2 = qd.flip(1).contiguous(), kd.flip(1).contiguous(), vd.roll(7, 1).contiguous()

    def eager(qx, kx, vx):
        b = fva.Buffers(plan)
        o = torch.empty_like(qx)
        fva.attention_call(plan, qx, kx, vx, o, p, w.k_min, b, slack=w.slack, fused=True)
        torch.cuda.synchronize()
        return o, b

    ref1, b1 = eager(qd, kd, vd)
    ref2, b2 = eager(q2, k2, v2)

    bufs = fva.Buffers(plan)
    out = torch.empty_like(qd)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # one uncaptured call on the capture stream's kind of stream
        fva.attention_call(plan, qg, kg, vg, out, p, w.k_min, bufs, slack=w.slack, fused=True)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fva.attention_call(plan, qg, kg, vg, out, p, w.k_min, bufs, slack=w.slack, fused=True)
    torch.cuda.synchronize()

    for i in range(4):
        # eager work on the same plan between replays
        e, _ = eager(qd, kd, vd)
        assert torch.equal(e, ref1)
        out.fill_(float("nan"))
        bufs.row_ptr.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref1), f"replay {i}"
        assert torch.equal(bufs.row_ptr, b1.row_ptr), f"replay {i} lists"
    # new contents in the captured inputs
    qg.copy_(q2), kg.copy_(k2), vg.copy_(v2)
    for i in range(2):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref2), f"replay {i} on new inputs"
        n = int(b2.row_ptr[-1].item())
        assert torch.equal(bufs.row_ptr, b2.row_ptr) and torch.equal(bufs.col_idx[:n], b2.col_idx[:n])
    del g
    torch.cuda.synchronize()
