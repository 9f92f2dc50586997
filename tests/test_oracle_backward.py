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
