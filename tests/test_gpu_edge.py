"""Edge cases of the GPU path against the CPU oracle, through the C ABI:

* attention on any valid CSR (the header's contract): empty rows, repeated
  ids, ids outside [0, n_blk) and unsorted rows give the result of the
  cleaned lists, bit for bit, and within tolerance of the oracle;
* grids smaller than one tile and barely larger (one token up to two blocks
  per axis), end to end, fused and separate calls;
* the largest plan the selection supports, 4096 blocks per head: the CSR is
  bit-exact against the oracle's selection on the GPU's scores, the scores
  match the oracle's fp64 pooling and scoring, and sampled query blocks
  match the oracle's attention on the GPU's lists.
"""
import numpy as np
import pytest
import torch

from block_sparse_spatiotemporal_amd import fva, synth
from oracle import fva_oracle as O
from tests._helpers import eps_valid, inputs, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _plan(w):
    return fva.Plan(w.B, w.H, w.D, w.grid, tile=w.tile, order=w.order, sub=w.sub, dtype=w.dtype)


def _csr(rows):
    rp = np.zeros(len(rows) + 1, dtype=np.int64)
    for i, r in enumerate(rows):
        rp[i + 1] = rp[i] + len(r)
    ci = np.concatenate([np.asarray(r, dtype=np.int64) for r in rows]) if rp[-1] else np.zeros(0, np.int64)
    return rp, ci


@pytest.mark.parametrize("dtype,D,tol", [("bf16", 128, 2e-2), ("f32", 64, 1e-4)])
def test_attention_accepts_any_valid_csr(dtype, D, tol):
    w = synth.scaled(synth.WORKLOADS["wan1.3b_480p"], H=2, D=D, grid=(6, 9, 13), dtype=dtype)
    plan = _plan(w)
    opl = O.plan(w.grid)
    (q, k, v), (q64, k64, v64), _ = inputs(w)
    b = fva.Buffers(plan)
    for x, dst, lay in ((q, b.q, fva.LAYOUT_ROWS), (k, b.k, fva.LAYOUT_ROWS), (v, b.vt, fva.LAYOUT_VT)):
        fva.fva_permute(plan, to_dev(x, dtype), dst, lay)
    n = plan.n_blk
    rng = np.random.default_rng(11)
    clean, messy = [], []
    for r in range(plan.n_rows):
        if r % 7 == 3:                    # empty row
            ids = np.zeros(0, np.int64)
        else:
            ids = np.sort(rng.choice(n, size=int(rng.integers(1, n + 1)), replace=False))
        clean.append(ids)
        m = list(ids) + list(rng.choice(ids, size=min(3, len(ids)))) if len(ids) else []
        m += [-1, n, n + 5] if r % 3 == 0 else []
        m = np.array(m, dtype=np.int64)
        rng.shuffle(m)
        messy.append(m)
    outs = []
    for rows in (clean, messy):
        rp, ci = _csr(rows)
        rpd = torch.from_numpy(rp.astype(np.int32)).cuda()
        cid = torch.from_numpy(ci.astype(np.int32)).cuda() if len(ci) else torch.zeros(1, dtype=torch.int32,
                                                                                     device="cuda")
        o = torch.full_like(b.o, float("nan"))
        fva.fva_attention(plan, b.q, b.k, b.vt, rpd, cid, o)
        r_out = torch.full_like(to_dev(q, dtype), float("nan"))
        fva.fva_attention_raster(plan, b.q, b.k, b.vt, rpd, cid, r_out)
        outs.append((o, r_out))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    rp, ci = _csr(clean)
    ref = O.attention(O.permute(q64, opl), O.permute(k64, opl), O.permute(v64, opl), rp, ci, opl)
    got = to_f64(outs[0][0])
    assert np.max(np.abs(got - ref)) < tol
    # empty rows and pad positions are exact zeros
    for r in range(plan.n_rows):
        if len(clean[r]) == 0:
            bh, I = divmod(r, n)
            assert np.all(got.reshape(-1, plan.info.n_pad, D)[bh, I * 64:(I + 1) * 64] == 0)
    assert np.max(np.abs(to_f64(outs[0][1]) - O.unpermute(ref, opl))) < tol


@pytest.mark.parametrize("grid", [(1, 1, 1), (2, 3, 5), (4, 4, 4), (5, 4, 7), (8, 8, 8)])
@pytest.mark.parametrize("fused", [False, True])
def test_tiny_grids_end_to_end(grid, fused):
    w = synth.scaled(synth.WORKLOADS["wan1.3b_480p"], H=2, grid=grid, k_min=2)
    plan = _plan(w)
    opl = O.plan(w.grid)
    if w.n_tokens > 1:
        (q, k, v), (q64, k64, v64), meta = inputs(w)
    else:   # the generator standardises over the tokens, which one token cannot: seeded normals
        rng = np.random.default_rng(5)
        q, k, v = (synth.f32_to_bf16_bits(rng.standard_normal((w.B, 1, w.H, w.D), dtype=np.float32))
                   for _ in range(3))
        q64, k64, v64 = (synth.to_f64(x, w.dtype) for x in (q, k, v))
    b = fva.Buffers(plan)
    out = torch.full_like(to_dev(q, w.dtype), float("nan"))
    fva.attention_call(plan, to_dev(q, w.dtype), to_dev(k, w.dtype), to_dev(v, w.dtype), out, w.p, w.k_min, b,
                       fused=fused)
    torch.cuda.synchronize()
    n = plan.n_blk
    rp = b.row_ptr.cpu().numpy().astype(np.int64)
    ci = b.col_idx[: rp[-1]].cpu().numpy().astype(np.int64)
    S64 = O.score(O.pool(O.permute(q64, opl), opl), O.pool(O.permute(k64, opl), opl))
    for r in range(plan.n_rows):
        bh, I = divmod(r, n)
        ok, why = eps_valid(ci[rp[r]:rp[r + 1]], S64.reshape(-1, n, n)[bh, I], float(np.float32(w.p)), w.k_min)
        assert ok, (r, why)
    ref = O.unpermute(O.attention(O.permute(q64, opl), O.permute(k64, opl), O.permute(v64, opl), rp, ci, opl), opl)
    assert np.max(np.abs(to_f64(out) - ref)) < 2e-2


def test_largest_supported_plan_4096_blocks():
    w = synth.scaled(synth.WORKLOADS["wan1.3b_480p"], B=1, H=1, D=64, grid=(64, 64, 64))
    plan = _plan(w)
    assert plan.n_blk == 4096
    opl = O.plan(w.grid)
    q, k, v, meta = synth.make(w)
    b = fva.Buffers(plan)
    out = torch.empty_like(to_dev(q, w.dtype))
    S = torch.empty(1, 1, 4096, 4096, dtype=torch.float32, device="cuda")
    fva.attention_call(plan, to_dev(q, w.dtype), to_dev(k, w.dtype), to_dev(v, w.dtype), out, w.p, w.k_min, b,
                       scores_out=S, fused=True)
    torch.cuda.synchronize()
    rp = b.row_ptr.cpu().numpy().astype(np.int64)
    ci = b.col_idx[: rp[-1]].cpu().numpy().astype(np.int64)
    Sg = S.cpu().numpy()
    # selection bit-exact on the GPU's own fp32 scores
    rp_o, ci_o = O.select(Sg.astype(np.float32), meta["p_head"], w.k_min)
    assert np.array_equal(rp_o, rp) and np.array_equal(ci_o, ci)
    # scores against fp64 pooling and scoring
    qp = O.permute(synth.to_f64(q, w.dtype), opl)
    kp = O.permute(synth.to_f64(k, w.dtype), opl)
    vp = O.permute(synth.to_f64(v, w.dtype), opl)
    ref_s = O.score(O.pool(qp, opl), O.pool(kp, opl))[0, 0]
    assert np.all(np.abs(Sg[0, 0].astype(np.float64) - ref_s) <= 1e-7 * ref_s + 1e-12)
    # attention of sampled query blocks (first, last and one in between)
    rows = [0, 2047, 4095]
    sub = [ci[rp[I]:rp[I + 1]] if I in rows else np.zeros(0, np.int64) for I in range(4096)]
    rp_s, ci_s = _csr(sub)
    o_ref = O.attention(qp, kp, vp, rp_s, ci_s, opl)[0, 0]
    o_gpu = O.permute(synth.to_f64(out.float().cpu().numpy(), "f32"), opl)[0, 0]
    for I in rows:
        valid = opl.perm[I * 64:(I + 1) * 64] >= 0
        d = np.abs(o_gpu[I * 64:(I + 1) * 64][valid] - o_ref[I * 64:(I + 1) * 64][valid]).max()
        assert d < 2e-2, (I, d)
