"""Pins for the oracle's block-sparse attention gradients: finite
differences of the oracle's own forward, and at p = 1 the dense gradients of
an fp64 softmax attention differentiated by torch autograd."""
import numpy as np
import torch

from oracle import fva_oracle as O


def _toy(seed, grid=(4, 4, 8), D=8, sel=None):
    rng = np.random.default_rng(seed)
    pl = O.plan(grid)
    N = int(np.prod(grid))
    x = lambda: rng.standard_normal((1, N, 1, D))
    q, k, v, do = (O.permute(x(), pl) for _ in range(4))
    n = pl.n_blk
    rows = sel if sel is not None else [np.sort(rng.choice(n, size=rng.integers(1, n + 1), replace=False)) for _ in range(n)]
    rp, ci = O.to_csr(rows)
    return pl, q, k, v, do, rp, ci


def test_gradients_match_finite_differences():
    pl, q, k, v, do, rp, ci = _toy(0)
    dq, dk, dv = O.attention_backward(q, k, v, do, rp, ci, pl)
    f = lambda q_, k_, v_: float((O.attention(q_, k_, v_, rp, ci, pl) * do).sum())
    rng = np.random.default_rng(1)
    h = 1e-6
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(12):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            plus, minus = arr.copy(), arr.copy()
            plus[idx] += h
            minus[idx] -= h
            args = {"q": (q, k, v), "k": (q, k, v), "v": (q, k, v)}[name]
            a = [x.copy() for x in args]
            pos = "qkv".index(name)
            a[pos] = plus
            fp = f(*a)
            a[pos] = minus
            fm = f(*a)
            num = (fp - fm) / (2 * h)
            assert abs(num - grad[idx]) <= 1e-6 * max(1.0, abs(num)), (name, idx, num, grad[idx])


def test_dense_lists_match_autograd():
    grid, D = (4, 4, 4), 8
    pl = O.plan(grid)
    n = pl.n_blk
    pl_, q, k, v, do, rp, ci = _toy(2, grid=grid, D=D, sel=[np.arange(n)] * n)
    tq, tk, tv = (torch.tensor(a[0, 0], dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    p = torch.softmax(tq @ tk.T / np.sqrt(D), dim=-1)
    (p @ tv * torch.tensor(do[0, 0])).sum().backward()
    dq, dk, dv = O.attention_backward(q, k, v, do, rp, ci, pl)
    for g, t in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.allclose(g[0, 0], t.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_pad_rows_get_zero_gradients():
    pl, q, k, v, do, rp, ci = _toy(3, grid=(3, 4, 6))    # padded to 4 x 4 x 8
    dq, dk, dv = O.attention_backward(q, k, v, do, rp, ci, pl)
    pad = pl.perm < 0
    assert pad.any()
    for g in (dq, dk, dv):
        assert np.all(g[:, :, pad, :] == 0)


def test_lse_single_valid_key_is_its_score():
    """Grid 5x5x5 pads to 8x8x8: the far corner block holds one valid token,
    so a row listing only that block has lse = s * log2(e) exactly."""
    grid, D = (5, 5, 5), 8
    pl = O.plan(grid)
    rng = np.random.default_rng(4)
    N = int(np.prod(grid))
    q, k = (O.permute(rng.standard_normal((1, N, 1, D)), pl) for _ in range(2))
    corner = [j for j in range(pl.n_blk) if (pl.perm[j * 64:(j + 1) * 64] >= 0).sum() == 1]
    assert len(corner) == 1
    J = corner[0]
    kt = pl.perm[J * 64:(J + 1) * 64] >= 0
    rp, ci = O.to_csr([np.array([J])] * pl.n_blk)
    lse = O.attention_lse(q, k, rp, ci, pl)
    kj = k[0, 0, J * 64 + np.nonzero(kt)[0][0]]
    valid = pl.perm >= 0
    expect = (q[0, 0] @ kj) / np.sqrt(D) / np.log(2.0)
    assert np.allclose(lse[0, 0][valid], expect[valid], rtol=0, atol=1e-12)
    assert np.all(lse[0, 0][~valid] == 0)


def test_lse_equal_keys_adds_log2_count():
    """All keys equal: every score of a row is the same s, so lse = s log2 e +
    log2(number of valid listed keys)."""
    grid, D = (4, 4, 12), 8
    pl = O.plan(grid)
    rng = np.random.default_rng(5)
    N = int(np.prod(grid))
    q = O.permute(rng.standard_normal((1, N, 1, D)), pl)
    k = O.permute(np.broadcast_to(rng.standard_normal((1, 1, 1, D)), (1, N, 1, D)).copy(), pl)
    rows = [np.array([0]), np.array([1, 2]), np.array([0, 1, 2])]
    rp, ci = O.to_csr(rows)
    lse = O.attention_lse(q, k, rp, ci, pl)
    kk = k[0, 0, 0]
    for i, sel in enumerate(rows):
        s = q[0, 0, i * 64:(i + 1) * 64] @ kk / np.sqrt(D)
        assert np.allclose(lse[0, 0, i * 64:(i + 1) * 64], s / np.log(2.0) + np.log2(64 * len(sel)), atol=1e-12)


def test_lse_rebuilds_attention_output():
    """o_i = sum_j 2^(s_ij log2 e - lse_i) v_j reproduces the oracle's
    attention output (which normalises on its own)."""
    pl, q, k, v, do, rp, ci = _toy(6, grid=(3, 4, 6))
    lse = O.attention_lse(q, k, rp, ci, pl)
    o = O.attention(q, k, v, rp, ci, pl)
    valid = pl.perm >= 0
    D = q.shape[-1]
    for I in range(pl.n_blk):
        rows = np.nonzero(valid[I * 64:(I + 1) * 64])[0] + I * 64
        blocks = ci[rp[I]:rp[I + 1]]
        keys = np.concatenate([np.nonzero(valid[j * 64:(j + 1) * 64])[0] + j * 64 for j in blocks])
        s = q[0, 0, rows] @ k[0, 0, keys].T / np.sqrt(D)
        P = np.exp2(s / np.log(2.0) - lse[0, 0, rows][:, None])
        assert np.allclose(P @ v[0, 0, keys], o[0, 0, rows], atol=1e-12)


def test_mask_transpose_small_example_and_involution():
    # B*H = 2 heads of 3 blocks; rows as sets with a repeat and an out-of-range id
    rows = [[2, 0, 2], [], [1, 7], [0], [0, 1, 2], [-1]]
    rp, ci = O.to_csr([np.array(r, dtype=np.int64) for r in rows])
    trp, tci = O.mask_transpose(rp, ci, 1, 2, 3)
    got = O.from_csr(trp, tci)
    want = [[0], [2], [0], [0, 1], [1], [1]]
    assert [list(g) for g in got] == want
    brp, bci = O.mask_transpose(trp, tci, 1, 2, 3)
    clean = [sorted({x for x in r if 0 <= x < 3}) for r in rows]
    assert [list(g) for g in O.from_csr(brp, bci)] == clean
