"""Shared test utilities: moving seeded inputs to the GPU and the end-to-end
selection acceptance rule."""
import numpy as np
import torch

from block_sparse_spatiotemporal_amd import synth


def to_dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    """Storage array (uint16 bf16 bits or float32) -> contiguous GPU tensor."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.cuda()


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def inputs(w, heads=None):
    """Seeded raster Q, K, V (storage arrays) plus fp64 views for the oracle."""
    q, k, v, meta = synth.make(w, heads=heads)
    f = lambda a: synth.to_f64(a, w.dtype)
    return (q, k, v), (f(q), f(k), f(v)), meta


def eps_valid(G, s64, p, k_min, eps=1e-6):
    """Acceptance of a GPU block set G for one row against the oracle's fp64
    scores s64: at least the floor; every kept block scores at least every
    dropped block minus eps; above the floor, the kept mass reaches p - eps and
    without its lowest block stays below p + eps."""
    n = len(s64)
    G = np.asarray(sorted(set(int(j) for j in G)))
    floor = min(int(k_min), n)
    if len(G) < floor:
        return False, "below floor"
    if p >= 1:
        return (len(G) == n), "p>=1 must keep all"
    keep = np.zeros(n, dtype=bool)
    keep[G] = True
    if keep.all():
        lo_in, hi_out = s64.min(), -np.inf
    else:
        lo_in, hi_out = s64[keep].min(), s64[~keep].max()
    if lo_in < hi_out - eps:
        return False, f"order violated {lo_in} < {hi_out}"
    if len(G) > floor:
        mass = s64[keep].sum()
        if mass < p - eps and not keep.all():
            return False, f"mass {mass} < p"
        if mass - lo_in >= p + eps:
            return False, f"not minimal: {mass - lo_in} >= p"
    return True, ""
