"""Selection reuse across denoising steps ("DFSAttn" explainer, trick 3):
fva_mask_overlap against the oracle's set counts, and attention on a cached
selection against the oracle run on the same cached lists."""
import numpy as np
import pytest
import torch

from block_sparse_spatiotemporal_amd import fva, synth
from oracle import fva_oracle as O
from tests._helpers import to_dev

pytestmark = pytest.mark.gpu


def _rand_csr(rng, rows, n, junk=False):
    lists = []
    for _ in range(rows):
        m = int(rng.integers(0, n + 1))
        ids = rng.choice(n, size=m, replace=False)
        if junk and m:   # repeats and ids outside the plan: rows are read as sets of plan blocks
            ids = np.concatenate([ids, ids[:2], [n + 3, -1]])
        lists.append(ids.astype(np.int32))
    rp = np.zeros(rows + 1, dtype=np.int64)
    rp[1:] = np.cumsum([len(x) for x in lists])
    return rp, np.concatenate(lists) if lists else np.zeros(0, np.int32)


@pytest.mark.parametrize("junk", [False, True])
def test_mask_overlap_matches_oracle_on_random_lists(junk):
    rng = np.random.default_rng(9 + junk)
    B, H, D, grid = 1, 3, 64, (8, 16, 16)
    plan = fva.Plan(B, H, D, grid, dtype="f32")
    n = plan.n_blk
    (ra, ca), (rb, cb) = _rand_csr(rng, plan.n_rows, n, junk), _rand_csr(rng, plan.n_rows, n, junk)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    got = fva.fva_mask_overlap(plan, dev(ra), dev(ca), dev(rb), dev(cb)).cpu().numpy()
    assert np.array_equal(got, O.mask_overlap(ra, ca, rb, cb, B, H, n))


def test_cached_selection_across_drifting_steps():
    """Step 1's inputs drift from step 0's; the step-0 lists are reused for
    step 1.  Overlap counts are exact, and attention on the cached lists is
    the oracle's attention on those lists."""
    w = synth.scaled(synth.WORKLOADS["wan1.3b_480p"], H=2, grid=(9, 10, 13))
    q0, k0, v0, _ = synth.make(w)
    rng = np.random.default_rng(21)
    drift = lambda a: synth.f32_to_bf16_bits(
        (synth.bf16_bits_to_f32(a) + 0.25 * rng.standard_normal(a.shape)).astype(np.float32))
    q1, k1 = drift(q0), drift(k0)
    plan = fva.Plan(w.B, w.H, w.D, w.grid)
    b0, b1 = fva.Buffers(plan), fva.Buffers(plan)
    out0, out1, out_c = (torch.empty_like(to_dev(q0, "bf16")) for _ in range(3))
    fva.attention_call(plan, to_dev(q0, "bf16"), to_dev(k0, "bf16"), to_dev(v0, "bf16"), out0, w.p, w.k_min, b0)
    fva.attention_call(plan, to_dev(q1, "bf16"), to_dev(k1, "bf16"), to_dev(v0, "bf16"), out1, w.p, w.k_min, b1)
    counts = fva.fva_mask_overlap(plan, b0.row_ptr, b0.col_idx, b1.row_ptr, b1.col_idx).cpu().numpy()
    # step 1 with the cached step-0 lists (b1 holds step 1's permuted Q, K, V)
    fva.fva_attention(plan, b1.q, b1.k, b1.vt, b0.row_ptr, b0.col_idx, b1.o)
    fva.fva_unpermute(plan, b1.o, out_c)
    torch.cuda.synchronize()
    rp0 = b0.row_ptr.cpu().numpy().astype(np.int64)
    ci0 = b0.col_idx[: rp0[-1]].cpu().numpy().astype(np.int64)
    rp1 = b1.row_ptr.cpu().numpy().astype(np.int64)
    ci1 = b1.col_idx[: rp1[-1]].cpu().numpy().astype(np.int64)
    want = O.mask_overlap(rp0, ci0, rp1, ci1, w.B, w.H, plan.n_blk)
    assert np.array_equal(counts, want)
    assert np.all(counts[:, 0] <= counts[:, 1]) and np.all(counts[:, 0] > 0)
    opl = O.plan(w.grid)
    f = lambda a: synth.to_f64(a, "bf16")
    ref = O.unpermute(O.attention(O.permute(f(q1), opl), O.permute(f(k1), opl), O.permute(f(v0), opl), rp0, ci0, opl), opl)
    assert float(np.abs(out_c.float().cpu().numpy() - ref).max()) < 2e-2


def test_reuse_drift_over_steps():
    """Steps 1..4 of a seeded random walk on Q, K, V (drift std 0.1 per step):
    at each step the step-0 selection is reused and compared with a fresh
    one.  The per-head overlap counts equal the oracle's; the Jaccard ratio
    and the output change caused by reuse are recorded (printed) per step,
    and the output on the cached lists stays the oracle's attention on them."""
    w = synth.scaled(synth.WORKLOADS["wan1.3b_480p"], H=2, grid=(9, 10, 13))
    q0, k0, v0, _ = synth.make(w)
    plan = fva.Plan(w.B, w.H, w.D, w.grid)
    opl = O.plan(w.grid)
    f = lambda a: synth.to_f64(a, "bf16")
    b0, bs = fva.Buffers(plan), fva.Buffers(plan)
    out0 = torch.empty_like(to_dev(q0, "bf16"))
    fva.attention_call(plan, to_dev(q0, "bf16"), to_dev(k0, "bf16"), to_dev(v0, "bf16"), out0, w.p, w.k_min, b0)
    torch.cuda.synchronize()
    rp0 = b0.row_ptr.cpu().numpy().astype(np.int64)
    ci0 = b0.col_idx[: rp0[-1]].cpu().numpy().astype(np.int64)
    for step in range(1, 5):
        q, k, v = (synth.drift(w, x, t, step) for t, x in enumerate((q0, k0, v0)))
        qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
        fresh, cached = torch.empty_like(qd), torch.empty_like(qd)
        fva.attention_call(plan, qd, kd, vd, fresh, w.p, w.k_min, bs)
        fva.fva_attention_raster(plan, bs.q, bs.k, bs.vt, b0.row_ptr, b0.col_idx, cached)
        counts = fva.fva_mask_overlap(plan, b0.row_ptr, b0.col_idx, bs.row_ptr, bs.col_idx).cpu().numpy()
        torch.cuda.synchronize()
        rps = bs.row_ptr.cpu().numpy().astype(np.int64)
        cis = bs.col_idx[: rps[-1]].cpu().numpy().astype(np.int64)
        assert np.array_equal(counts, O.mask_overlap(rp0, ci0, rps, cis, w.B, w.H, plan.n_blk))
        jac = counts[:, 0].sum() / counts[:, 1].sum()
        diff = (cached.float() - fresh.float()).abs()
        ref = O.unpermute(O.attention(O.permute(f(q), opl), O.permute(f(k), opl), O.permute(f(v), opl),
                                      rp0, ci0, opl), opl)
        assert float(np.abs(cached.float().cpu().numpy() - ref).max()) < 2e-2
        print(f"drift step {step}: jaccard {jac:.4f}, reuse output change max {diff.max().item():.4e} "
              f"mean {diff.mean().item():.4e}")
