"""Full-size workloads, in the launch configuration bench.py times (the fused
calls fva_permute_pool, fva_select_pooled and fva_attention_raster, persistent
schedule, default group and ring depth), checked against the oracle on what
the oracle can compute in a test's time:

* selection bit-exact: the oracle's Top-p / floor (and slack fill) fed the
  GPU's own fp32 scores must reproduce the GPU's CSR lists;
* scores of sampled heads within 1e-7 relative of the oracle's fp64 pooling
  and scoring, and those heads' lists epsilon-valid against fp64 scores;
* attention outputs of sampled query blocks within 2e-2 of the oracle run on
  the GPU's lists.
"""
import numpy as np
import pytest
import torch

from block_sparse_spatiotemporal_amd import fva, synth
from oracle import fva_oracle as O
from tests._helpers import eps_valid, to_dev

pytestmark = pytest.mark.gpu

# (workload, sampled (b, h) heads, query blocks sampled per head)
CASES = [
    ("wan14b_480p_cfg", [(0, 0), (1, 17), (0, 39)], 6),
    ("wan_720p_hilbert_sub", [(0, 3), (0, 29)], 4),
    ("hetero_slack", [(0, 0), (0, 21)], 6),
]


def _run(name):
    w = synth.WORKLOADS[name]
    q, k, v, meta = synth.make(w)
    plan = fva.Plan(w.B, w.H, w.D, w.grid, tile=w.tile, order=w.order, sub=w.sub, dtype=w.dtype)
    bufs = fva.Buffers(plan)
    qd, kd, vd = to_dev(q, w.dtype), to_dev(k, w.dtype), to_dev(v, w.dtype)
    out = torch.empty_like(qd)
    S = torch.empty(w.B, w.H, plan.n_blk, plan.n_blk, dtype=torch.float32, device="cuda")
    p_head = meta["p_head"]
    p = p_head.tolist() if isinstance(w.p, tuple) else float(p_head[0])
    fva.attention_call(plan, qd, kd, vd, out, p, w.k_min, bufs, slack=w.slack, scores_out=S, fused=True)
    torch.cuda.synchronize()
    rp = bufs.row_ptr.cpu().numpy().astype(np.int64)
    ci = bufs.col_idx[: rp[-1]].cpu().numpy().astype(np.int64)
    res = dict(w=w, q=q, k=k, v=v, p_head=p_head, rp=rp, ci=ci, S=S.cpu().numpy(),
               out=out, head_nnz=bufs.head_nnz.cpu().numpy(), n_blk=plan.n_blk)
    del qd, kd, vd, S, bufs
    plan.destroy()
    return res


@pytest.fixture(scope="module", params=CASES, ids=[c[0] for c in CASES])
def run(request):
    name, heads, nq = request.param
    r = _run(name)
    r["heads"], r["nq"] = heads, nq
    yield r
    torch.cuda.empty_cache()


def test_csr_well_formed(run):
    w, rp, ci, n = run["w"], run["rp"], run["ci"], run["n_blk"]
    n_rows = w.B * w.H * n
    assert len(rp) == n_rows + 1 and rp[0] == 0 and np.all(np.diff(rp) >= min(w.k_min, n))
    assert ci.min() >= 0 and ci.max() < n
    for r in range(0, n_rows, 997):   # ascending, no repeats
        assert np.all(np.diff(ci[rp[r]:rp[r + 1]]) > 0)
    per_head = np.add.reduceat(np.diff(rp), np.arange(0, n_rows, n))
    assert np.array_equal(per_head, run["head_nnz"])


def test_selection_bit_exact_on_gpu_scores(run):
    """Oracle selection (+ slack) over every row, fed the GPU's fp32 scores."""
    w, n = run["w"], run["n_blk"]
    S = run["S"]
    p_head = run["p_head"]
    rp_o, ci_o = O.select(S.astype(np.float32), p_head, w.k_min)
    if w.slack == "median":
        rp_o, ci_o = O.slack_fill(S.astype(np.float32), rp_o, ci_o)
    assert np.array_equal(rp_o, run["rp"])
    assert np.array_equal(ci_o, run["ci"])


def _head64(a, b, h, dtype):
    return synth.to_f64(a[b:b + 1, :, h:h + 1, :], dtype)


def test_sampled_heads_scores_lists_and_outputs(run):
    w, n, rp, ci = run["w"], run["n_blk"], run["rp"], run["ci"]
    opl = O.plan(w.grid, tile=w.tile, order=w.order, sub=w.sub)
    rng = np.random.default_rng(7)
    for b, h in run["heads"]:
        q64, k64, v64 = (_head64(run[t], b, h, w.dtype) for t in ("q", "k", "v"))
        qp, kp, vp = O.permute(q64, opl), O.permute(k64, opl), O.permute(v64, opl)
        qb = O.pool(qp, opl)
        if opl.n_sub:
            kbs, empty = O.pool_sub(kp, opl)
            ref = O.score_sub(qb, kbs, empty)[0, 0]
        else:
            ref = O.score(qb, O.pool(kp, opl))[0, 0]
        got = run["S"][b, h].astype(np.float64)
        assert np.all(np.abs(got - ref) <= 1e-7 * ref + 1e-12), f"scores of head {(b, h)}"
        base = (b * w.H + h) * n
        p = float(np.float32(run["p_head"][h]))   # p is per head index, shared by the batch
        if w.slack == "none":
            for I in range(n):
                ok, why = eps_valid(ci[rp[base + I]:rp[base + I + 1]], ref[I], p, w.k_min)
                assert ok, f"head {(b, h)} row {I}: {why}"
        # attention of sampled query blocks, on the GPU's lists
        rows = rng.choice(n, size=run["nq"], replace=False)
        rp_h = np.zeros(n + 1, dtype=np.int64)
        cols = []
        for I in range(n):
            sel = ci[rp[base + I]:rp[base + I + 1]] if I in rows else np.zeros(0, dtype=np.int64)
            cols.append(sel)
            rp_h[I + 1] = rp_h[I] + len(sel)
        o_ref = O.attention(qp, kp, vp, rp_h, np.concatenate(cols), opl)[0, 0]
        o_gpu = O.permute(synth.to_f64(run["out"][b:b + 1, :, h:h + 1, :].float().cpu().numpy(), "f32"), opl)[0, 0]
        for I in rows:
            valid = opl.perm[I * 64:(I + 1) * 64] >= 0
            d = np.abs(o_gpu[I * 64:(I + 1) * 64][valid] - o_ref[I * 64:(I + 1) * 64][valid]).max()
            assert d < 2e-2, f"head {(b, h)} query block {I}: max abs {d}"
