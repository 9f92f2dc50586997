"""GPU path against the CPU oracle, element by element, through the C ABI.

Tolerances: block lists bit-exact when selection reads the oracle's scores;
end-to-end lists epsilon-valid (1e-6) against the oracle's fp64 scores;
attention max-abs 2e-2 (bf16) / 1e-4 (fp32) against the oracle run on the
same block lists; permutation bitwise.
"""
import math

import numpy as np
import pytest
import torch

from block_sparse_spatiotemporal_amd import fva, synth
from oracle import fva_oracle as O
from tests._helpers import eps_valid, inputs, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _plan_and_inputs(w, **kw):
    (q, k, v), (q64, k64, v64), meta = inputs(w)
    plan = fva.Plan(w.B, w.H, w.D, w.grid, tile=w.tile, order=w.order, sub=w.sub, dtype=w.dtype, **kw)
    opl = O.plan(w.grid, tile=w.tile, order=w.order, sub=w.sub)
    return plan, opl, (to_dev(q, w.dtype), to_dev(k, w.dtype), to_dev(v, w.dtype)), (q64, k64, v64), meta


def _vt_expected(v_perm64, D):
    """VT layout from block-order rows, written from the header's formula."""
    B, H, n_pad, _ = v_perm64.shape
    out = np.empty((B, H, n_pad // 64, 2, D, 32))
    slot_of = []
    for k in range(32):
        c, r = k // 16, k % 16
        slot_of.append(16 * c + 8 * ((r // 4) % 2) + (r % 4) + 4 * (r // 8))
    blocks = v_perm64.reshape(B, H, n_pad // 64, 2, 32, D)
    for k in range(32):
        out[:, :, :, :, :, slot_of[k]] = blocks[:, :, :, :, k, :]
    return out.reshape(B, H, n_pad, D)


SMALL = [
    synth.scaled(synth.WORKLOADS["tiny_f32"]),
    synth.scaled(synth.WORKLOADS["wan1.3b_480p"], H=2, grid=(9, 10, 13)),
    synth.scaled(synth.WORKLOADS["wan_720p_hilbert_sub"], H=2, grid=(7, 9, 14)),
    synth.scaled(synth.WORKLOADS["wan1.3b_480p"], H=2, D=64, grid=(5, 12, 11)),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: f"{w.name}-{w.grid}-D{w.D}")
def test_permute_unpermute_bitwise(w):
    plan, opl, (q, k, v), (q64, k64, v64), _ = _plan_and_inputs(w)
    b = fva.Buffers(plan)
    fva.fva_permute(plan, q, b.q, fva.LAYOUT_ROWS)
    fva.fva_permute(plan, v, b.vt, fva.LAYOUT_VT)
    out = torch.empty_like(q)
    fva.fva_unpermute(plan, b.q, out)
    torch.cuda.synchronize()
    assert np.array_equal(to_f64(b.q), O.permute(q64, opl))
    assert np.array_equal(to_f64(b.vt), _vt_expected(O.permute(v64, opl), w.D))
    assert torch.equal(out, q)


@pytest.mark.parametrize("w", SMALL, ids=lambda w: f"{w.name}-{w.grid}-D{w.D}")
def test_scores_match_oracle(w):
    plan, opl, (q, k, v), (q64, k64, v64), _ = _plan_and_inputs(w)
    b = fva.Buffers(plan)
    fva.fva_permute(plan, q, b.q)
    fva.fva_permute(plan, k, b.k)
    S = torch.empty(w.B, w.H, plan.n_blk, plan.n_blk, dtype=torch.float32, device="cuda")
    fva.fva_select(plan, b.q, b.k, 0.9, 4, b.row_ptr, b.col_idx, scores_out=S)
    torch.cuda.synchronize()
    qp, kp = O.permute(q64, opl), O.permute(k64, opl)
    qb = O.pool(qp, opl)
    if opl.n_sub:
        kbs, empty = O.pool_sub(kp, opl)
        ref = O.score_sub(qb, kbs, empty)
    else:
        ref = O.score(qb, O.pool(kp, opl))
    got = S.cpu().numpy().astype(np.float64)
    # fp64 logits, one fp32 rounding at the end: |dS| <= 2^-24 S
    assert np.all(np.abs(got - ref) <= 1e-7 * ref + 1e-38), np.max(np.abs(got - ref) / (ref + 1e-38))
    assert np.allclose(got.sum(-1), 1.0, atol=1e-5)


def _random_scores(B, H, n, rng, ties=True):
    S = rng.dirichlet(np.full(n, 0.3), size=(B, H, n))
    if ties:
        S[..., 1::7] = S[..., 0:1]        # many exact ties per row
    return S.astype(np.float32)


@pytest.mark.parametrize("n_grid,B,H,k_min,p", [
    ((4, 8, 16), 1, 3, 0, 0.9),           # 32 blocks
    ((4, 8, 16), 2, 2, 5, [0.5, 0.99, 0.7, 1.0]),
    ((21, 30, 52), 1, 2, 16, 0.9),        # 624 blocks
    ((21, 45, 80), 1, 1, 32, 0.95),       # 1440 blocks
    ((9, 10, 13), 1, 4, 200, 0.3),        # floor above n
])
def test_select_bit_exact_on_oracle_scores(n_grid, B, H, k_min, p):
    rng = np.random.default_rng(hash((n_grid, B, H)) % 2 ** 32)
    plan = fva.Plan(B, H, 128, n_grid)
    n = plan.n_blk
    S = _random_scores(B, H, n, rng)
    S[0, 0, 0, :] = 0.0
    S[0, 0, 0, 3] = np.nan
    S[0, 0, 0, 5] = 0.7
    S[0, -1, -1, :] = np.float32(1.0 / n)  # all equal
    b = fva.Buffers(plan)
    sin = torch.from_numpy(S).cuda()
    fva.fva_select(plan, None, None, p, k_min, b.row_ptr, b.col_idx, scores_in=sin, head_nnz=b.head_nnz)
    torch.cuda.synchronize()
    ps = p if isinstance(p, list) else [p] * (B * H)
    rows = [O.select_row(S[bb, h, i], ps[bb * H + h], k_min)
            for bb in range(B) for h in range(H) for i in range(n)]
    rp_ref, ci_ref = O.to_csr(rows)
    rp = b.row_ptr.cpu().numpy()
    assert np.array_equal(rp, rp_ref)
    assert np.array_equal(b.col_idx[: rp[-1]].cpu().numpy(), ci_ref)
    assert np.array_equal(b.head_nnz.cpu().numpy(), O.head_nnz(rp_ref, B, H, n))


@pytest.mark.parametrize("flat_heads", [0, 2])
def test_slack_fill_bit_exact_on_oracle_scores(flat_heads):
    # flat heads: every score equal and a low p, so the head falls short of
    # the median and its fill is decided by the pair index alone
    rng = np.random.default_rng(5)
    B, H = 1, 9
    plan = fva.Plan(B, H, 128, (9, 10, 13))
    n = plan.n_blk
    S = _random_scores(B, H, n, rng)
    p = rng.uniform(0.3, 0.99, size=H).astype(np.float32)
    S[0, :flat_heads] = np.float32(1.0 / n)
    p[:flat_heads] = 0.1
    b = fva.Buffers(plan)
    fva.fva_select(plan, None, None, p.tolist(), 2, b.row_ptr, b.col_idx, slack="median",
                   scores_in=torch.from_numpy(S).cuda(), head_nnz=b.head_nnz)
    torch.cuda.synchronize()
    rows = [O.select_row(S[0, h, i], p[h], 2) for h in range(H) for i in range(n)]
    rp0, ci0 = O.to_csr(rows)
    rp_ref, ci_ref = O.slack_fill(S, rp0, ci0)
    rp = b.row_ptr.cpu().numpy()
    assert np.array_equal(rp, rp_ref)
    assert np.array_equal(b.col_idx[: rp[-1]].cpu().numpy(), ci_ref)


def _oracle_scores(w, opl, q64, k64):
    qp, kp = O.permute(q64, opl), O.permute(k64, opl)
    qb = O.pool(qp, opl)
    if opl.n_sub:
        kbs, empty = O.pool_sub(kp, opl)
        return O.score_sub(qb, kbs, empty)
    return O.score(qb, O.pool(kp, opl))


@pytest.mark.parametrize("w", SMALL + [synth.scaled(synth.WORKLOADS["tiny_f32_indep"])],
                         ids=lambda w: f"{w.name}-{w.grid}-D{w.D}")
@pytest.mark.parametrize("sched", ["persistent", "plain"])
def test_end_to_end_vs_oracle(w, sched):
    plan, opl, (q, k, v), (q64, k64, v64), meta = _plan_and_inputs(w)
    b = fva.Buffers(plan)
    out = torch.empty_like(q)
    p = meta["p_head"][0] if not isinstance(w.p, tuple) else meta["p_head"].tolist()
    fva.attention_call(plan, q, k, v, out, p, w.k_min, b, sched=sched)
    torch.cuda.synchronize()
    # selection: epsilon-valid against the oracle's fp64 scores
    S64 = _oracle_scores(w, opl, q64, k64)
    rp = b.row_ptr.cpu().numpy().astype(np.int64)
    ci = b.col_idx[: rp[-1]].cpu().numpy().astype(np.int64)
    rows = O.from_csr(rp, ci)
    n = plan.n_blk
    for r, G in enumerate(rows):
        bh, i = divmod(r, n)
        ok, why = eps_valid(G, S64.reshape(-1, n, n)[bh, i], float(np.float32(meta["p_head"][bh % w.H])), w.k_min)
        assert ok, (r, why)
        assert np.all(np.diff(G) > 0)
    # attention on the GPU's own lists
    ref = O.unpermute(O.attention(O.permute(q64, opl), O.permute(k64, opl), O.permute(v64, opl), rp, ci, opl), opl)
    tol = 2e-2 if w.dtype == "bf16" else 1e-4
    err = np.max(np.abs(to_f64(out) - ref))
    assert err < tol, err


@pytest.mark.parametrize("qscale", [1.0, 8.0])
def test_exact_scale_form_vs_oracle(monkeypatch, qscale):
    """FVA_ATTN_EXACT_SCALE=1 keeps S exact in fp32 and applies the scale
    per score.  With Q times 8 (exact in bf16) the logits of a row span
    tens of log2 units; the exact-scale form stays within the bf16 output
    tolerance of the oracle there, and the default form (scale folded into a
    bf16 rounding of Q) stays within it at the inputs' own scale."""
    w = synth.scaled(synth.WORKLOADS["wan1.3b_480p"], H=2, grid=(9, 10, 13))
    plan, opl, (q, k, v), (q64, k64, v64), _ = _plan_and_inputs(w)
    q = q * qscale
    q64 = q64 * qscale
    errs = {}
    for mode in ("exact", "fold"):
        if mode == "exact":
            monkeypatch.setenv("FVA_ATTN_EXACT_SCALE", "1")
        else:
            monkeypatch.delenv("FVA_ATTN_EXACT_SCALE", raising=False)
        b = fva.Buffers(plan)
        out = torch.empty_like(q)
        fva.attention_call(plan, q, k, v, out, 0.9, 16, b)
        torch.cuda.synchronize()
        rp = b.row_ptr.cpu().numpy().astype(np.int64)
        ci = b.col_idx[: rp[-1]].cpu().numpy().astype(np.int64)
        ref = O.unpermute(O.attention(O.permute(q64, opl), O.permute(k64, opl), O.permute(v64, opl), rp, ci, opl), opl)
        errs[mode] = float(np.max(np.abs(to_f64(out) - ref)))
    print(f"q x {qscale}: max abs error exact-scale {errs['exact']:.3g}, folded {errs['fold']:.3g}")
    assert errs["exact"] < 2e-2
    if qscale == 1.0:
        assert errs["fold"] < 2e-2


def test_persistent_and_plain_bitwise_equal():
    w = synth.scaled(synth.WORKLOADS["wan1.3b_480p"], H=3, grid=(9, 10, 13))
    plan, opl, (q, k, v), _, meta = _plan_and_inputs(w)
    outs = []
    for sched in ("persistent", "plain", "persistent"):
        b = fva.Buffers(plan)
        out = torch.empty_like(q)
        fva.attention_call(plan, q, k, v, out, 0.9, 16, b, sched=sched)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


@pytest.mark.parametrize("dtype,tol", [("bf16", 2e-2), ("f32", 1e-4)])
def test_p1_equals_dense_attention(dtype, tol):
    w = synth.scaled(synth.WORKLOADS["wan1.3b_480p"], H=2, D=64, grid=(5, 6, 13), dtype=dtype)
    plan, opl, (q, k, v), (q64, k64, v64), _ = _plan_and_inputs(w)
    b = fva.Buffers(plan)
    out = torch.empty_like(q)
    fva.attention_call(plan, q, k, v, out, 1.0, 0, b)
    torch.cuda.synchronize()
    assert b.row_ptr[-1].item() == plan.n_rows * plan.n_blk
    t = lambda a: torch.from_numpy(a).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(t(q64), t(k64), t(v64)).permute(0, 2, 1, 3).numpy()
    assert np.max(np.abs(to_f64(out) - ref)) < tol


def test_attention_rows_sum_to_one_and_pad_rows_zero():
    w = synth.scaled(synth.WORKLOADS["wan1.3b_480p"], H=2, grid=(9, 10, 13))
    plan, opl, (q, k, v), _, _ = _plan_and_inputs(w)
    b = fva.Buffers(plan)
    fva.fva_permute(plan, q, b.q)
    fva.fva_permute(plan, k, b.k)
    ones = torch.ones_like(v)
    fva.fva_permute(plan, ones, b.vt, fva.LAYOUT_VT)
    fva.fva_select(plan, b.q, b.k, 0.8, 3, b.row_ptr, b.col_idx)
    fva.fva_attention(plan, b.q, b.k, b.vt, b.row_ptr, b.col_idx, b.o)
    torch.cuda.synchronize()
    o = to_f64(b.o)
    valid = opl.perm >= 0
    assert np.all(o[:, :, ~valid] == 0)
    assert np.max(np.abs(o[:, :, valid] - 1.0)) < 1e-2


def test_wg_times_recorded():
    w = synth.scaled(synth.WORKLOADS["wan1.3b_480p"], H=2, grid=(9, 10, 13))
    plan, _, (q, k, v), _, _ = _plan_and_inputs(w)
    b = fva.Buffers(plan)
    out = torch.empty_like(q)
    wt = torch.zeros(2 * plan.info.max_wg, dtype=torch.int64, device="cuda")
    fva.attention_call(plan, q, k, v, out, 0.9, 16, b, wg_times=wt)
    torch.cuda.synchronize()
    t = wt.cpu().numpy().reshape(-1, 2)
    used = t[t[:, 0] > 0]
    assert len(used) > 0 and np.all(used[:, 1] >= used[:, 0])


def test_launch_shapes_bitwise_equal(monkeypatch):
    """Group size, query-block pairing, LDS ring depth, XCD chunk, work-list
    order and schedule change only which rows share a workgroup and the
    order they are taken in, never a row's arithmetic: outputs are bitwise
    equal."""
    w = synth.scaled(synth.WORKLOADS["wan1.3b_480p"], H=3, grid=(9, 10, 13))
    plan, opl, (q, k, v), _, meta = _plan_and_inputs(w)
    ref = None
    for group, stages, chunk, sched, order, pair in [
            ("1", "3", "32", "persistent", "0", "0"), ("2", "2", "16", "plain", "1", "1"),
            ("4", "4", "1", "persistent", "1", "1"), ("2", "3", "32", "persistent", "0", "1"),
            ("4", "2", "64", "plain", "0", "0"), ("2", "4", "8", "plain", "1", "0"),
            ("2", "4", "32", "persistent", "1", "1"), ("1", "4", "8", "persistent", "1", "0"),
            ("2", "4", "1000", "persistent", "1", "0")]:
        monkeypatch.setenv("FVA_ATTN_GROUP", group)
        monkeypatch.setenv("FVA_ATTN_STAGES", stages)
        monkeypatch.setenv("FVA_ATTN_CHUNK", chunk)
        monkeypatch.setenv("FVA_ATTN_ORDER", order)
        monkeypatch.setenv("FVA_ATTN_PAIR", pair)
        b = fva.Buffers(plan)
        out = torch.empty_like(q)
        fva.attention_call(plan, q, k, v, out, 0.9, 16, b, sched=sched)
        torch.cuda.synchronize()
        if ref is None:
            ref = out
        else:
            assert torch.equal(out, ref), (group, stages, chunk, sched, order, pair)


@pytest.mark.parametrize("w", SMALL, ids=lambda w: f"{w.name}-{w.grid}-D{w.D}")
@pytest.mark.parametrize("sched", ["persistent", "plain"])
def test_attention_raster_equals_attention_unpermute(w, sched):
    """fva_attention_raster writes each row straight to its raster position:
    bit for bit fva_attention + fva_unpermute, and within tolerance of the
    oracle on the same lists."""
    plan, opl, (q, k, v), (q64, k64, v64), meta = _plan_and_inputs(w)
    p = meta["p_head"][0] if not isinstance(w.p, tuple) else meta["p_head"].tolist()
    b = fva.Buffers(plan)
    ref = torch.empty_like(q)
    fva.attention_call(plan, q, k, v, ref, p, w.k_min, b, sched=sched)
    got = torch.full_like(q, float("nan"))
    fva.fva_attention_raster(plan, b.q, b.k, b.vt, b.row_ptr, b.col_idx, got, sched=sched)
    got2 = torch.full_like(q, float("nan"))
    fva.attention_call(plan, q, k, v, got2, p, w.k_min, fva.Buffers(plan), sched=sched, fused=True)
    torch.cuda.synchronize()
    assert torch.equal(got, ref) and torch.equal(got2, ref)
    rp = b.row_ptr.cpu().numpy().astype(np.int64)
    ci = b.col_idx[: rp[-1]].cpu().numpy().astype(np.int64)
    o64 = O.unpermute(O.attention(O.permute(q64, opl), O.permute(k64, opl), O.permute(v64, opl), rp, ci, opl), opl)
    assert np.max(np.abs(to_f64(got) - o64)) < (2e-2 if w.dtype == "bf16" else 1e-4)


@pytest.mark.parametrize("w", SMALL, ids=lambda w: f"{w.name}-{w.grid}-D{w.D}")
def test_permute_pool_and_select_pooled_equal_separate_path(w):
    """fva_permute_pool writes what fva_permute writes, and fva_select_pooled
    gives the lists (and fp32 scores) fva_select gives on the same tensors:
    the fused means are the same bits."""
    plan, opl, (q, k, v), _, meta = _plan_and_inputs(w)
    p = meta["p_head"][0] if not isinstance(w.p, tuple) else meta["p_head"].tolist()
    d = plan.desc
    sq = (d.batch, d.heads, plan.n_blk, plan.n_blk)
    a, b = fva.Buffers(plan), fva.Buffers(plan)
    s_a = torch.empty(sq, dtype=torch.float32, device="cuda")
    s_b = torch.empty(sq, dtype=torch.float32, device="cuda")
    fva.fva_permute(plan, q, a.q)
    fva.fva_permute(plan, k, a.k)
    fva.fva_select(plan, a.q, a.k, p, w.k_min, a.row_ptr, a.col_idx, slack=w.slack, scores_out=s_a)
    b.q.fill_(float("nan"))
    fva.fva_permute_pool(plan, q, b.q, "q")
    fva.fva_permute_pool(plan, k, b.k, "k")
    fva.fva_select_pooled(plan, p, w.k_min, b.row_ptr, b.col_idx, slack=w.slack, scores_out=s_b)
    torch.cuda.synchronize()
    assert torch.equal(a.q, b.q) and torch.equal(a.k, b.k)
    assert torch.equal(s_a, s_b)
    assert torch.equal(a.row_ptr, b.row_ptr)
    n = int(a.row_ptr[-1].item())
    assert torch.equal(a.col_idx[:n], b.col_idx[:n])


def test_select_pooled_needs_both_pools():
    w = synth.scaled(synth.WORKLOADS["wan1.3b_480p"], H=2, grid=(9, 10, 13))
    plan, _, (q, k, v), _, _ = _plan_and_inputs(w)
    b = fva.Buffers(plan)
    with pytest.raises(fva.FvaError) as e:
        fva.fva_select_pooled(plan, 0.9, 16, b.row_ptr, b.col_idx)
    assert e.value.code == fva.FVA_EINVAL
    with pytest.raises(fva.FvaError) as e:   # neither Q nor K
        fva.fva_permute_pool(plan, q, b.q, 7)
    assert e.value.code == fva.FVA_EINVAL
    fva.fva_permute_pool(plan, q, b.q, "q")
    with pytest.raises(fva.FvaError):
        fva.fva_select_pooled(plan, 0.9, 16, b.row_ptr, b.col_idx)
    fva.fva_permute_pool(plan, k, b.k, "k")
    fva.fva_select_pooled(plan, 0.9, 16, b.row_ptr, b.col_idx)
    # a select that pools its own inputs replaces the means: pooled again needed
    fva.fva_select(plan, b.q, b.k, 0.9, 16, b.row_ptr, b.col_idx)
    with pytest.raises(fva.FvaError):
        fva.fva_select_pooled(plan, 0.9, 16, b.row_ptr, b.col_idx)
    torch.cuda.synchronize()
