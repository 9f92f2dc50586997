"""Selection parity in the direction the scores flow: the oracle's own fp64
pooled scores of sampled heads at full workload shapes, rounded once to fp32,
are fed to fva_select (scores_in, so pooling and scoring are skipped) and the
CSR lists must equal the oracle's Top-p / Top-k floor selection ("FVAttn"
review, sections 00 and 02) on that same fp32 array bit for bit; with median
slack fill ("FVAttn" section 02) the lifted lists must match too.

The sampled heads are gathered into a plan of B = 1 and H = number of heads
on the workload's full grid (tile or Hilbert order, sub-block scoring as the
workload has it), so every row of every sampled head is compared.
"""
import numpy as np
import pytest
import torch

from block_sparse_spatiotemporal_amd import fva, synth
from oracle import fva_oracle as O

pytestmark = pytest.mark.gpu

# (workload, sampled (b, h) heads): densest and sparsest kinds of head where
# the workload varies its smoothing or p per head
CASES = [
    ("wan14b_480p_cfg", [(0, 0), (1, 17), (0, 39), (1, 5)]),
    ("wan_720p_hilbert_sub", [(0, 3), (0, 29)]),
    ("hetero_slack", [(0, 0), (0, 7), (0, 21), (0, 33)]),
]


def _oracle_scores(w, q, k, heads):
    opl = O.plan(w.grid, tile=w.tile, order=w.order, sub=w.sub)
    out = []
    for b, h in heads:
        q64 = synth.to_f64(q[b:b + 1, :, h:h + 1, :], w.dtype)
        k64 = synth.to_f64(k[b:b + 1, :, h:h + 1, :], w.dtype)
        qb = O.pool(O.permute(q64, opl), opl)
        kp = O.permute(k64, opl)
        if opl.n_sub:
            kbs, empty = O.pool_sub(kp, opl)
            out.append(O.score_sub(qb, kbs, empty)[0, 0])
        else:
            out.append(O.score(qb, O.pool(kp, opl))[0, 0])
    return np.stack(out)[None]          # [1, len(heads), n_blk, n_blk] fp64


@pytest.mark.parametrize("name,heads", CASES, ids=[c[0] for c in CASES])
def test_select_bit_exact_on_oracle_pooled_scores(name, heads):
    w = synth.WORKLOADS[name]
    q, k, _, meta = synth.make(w, heads=heads)
    S32 = _oracle_scores(w, q, k, heads).astype(np.float32)
    H = len(heads)
    p_head = np.array([meta["p_head"][h] for _, h in heads], dtype=np.float32)
    per_head = isinstance(w.p, tuple)
    plan = fva.Plan(1, H, w.D, w.grid, tile=w.tile, order=w.order, sub=w.sub, dtype=w.dtype)
    assert plan.n_blk == S32.shape[-1]
    bufs = fva.Buffers(plan)
    p_arg = p_head.tolist() if per_head else float(p_head[0])
    fva.fva_select(plan, None, None, p_arg, w.k_min, bufs.row_ptr, bufs.col_idx, slack=w.slack,
                   scores_in=torch.from_numpy(S32).cuda(), head_nnz=bufs.head_nnz)
    torch.cuda.synchronize()
    rp_ref, ci_ref = O.select(S32, p_head, w.k_min)
    if w.slack == "median":
        rp_ref, ci_ref = O.slack_fill(S32, rp_ref, ci_ref)
    rp = bufs.row_ptr.cpu().numpy()
    assert np.array_equal(rp, rp_ref)
    assert np.array_equal(bufs.col_idx[: rp[-1]].cpu().numpy(), ci_ref)
    assert np.array_equal(bufs.head_nnz.cpu().numpy(), O.head_nnz(rp_ref, 1, H, plan.n_blk))
    plan.destroy()
