"""Seeded synthetic attention inputs shaped like video-DiT latents.

This module only draws random numbers, smooths them over the (t, h, w) token
grid and rounds them to the storage dtype.  It holds no step of the sparse
attention method (no pooling, scoring, selection or attention), so the CPU
oracle and the GPU path can both consume its output without sharing any of
the method's arithmetic.

Workloads (the shapes the pages measure on are Wan-style 480P / 720P video
latents; the model weights and prompts are not available, so these fields
stand in for the attention inputs in shape and structure only):

* ``tiny_f32``         B1 H2 D64 fp32, grid 8x16x16, tile 4x4x4 (32 blocks).
                       Q and K share one N(0,1) vector per tile plus 0.5*N(0,1)
                       per-token noise; V ~ N(0,1).  p 0.9, k_min 4.
* ``tiny_f32_indep``   as above but Q and K draw independent tile vectors.
* ``wan1.3b_480p``     B1 H12 D128 bf16, grid 21x30x52 (32,760 tokens), one
                       smooth field per (b, h) (Gaussian sigma 3 tokens,
                       standardised per channel); Q = F + 0.3 e_Q,
                       K = F + 0.3 e_K; V ~ N(0,1).  p 0.9, k_min 16.
* ``wan14b_480p_cfg``  B2 H40, as above with sigma_h ~ U(1, 8) per head,
                       shared by the CFG pair; each (b, h) has its own field.
* ``wan_720p_hilbert_sub``  B1 H40, grid 21x45x80 (75,600 tokens), sigma 3,
                       Hilbert order, (2,2,2) sub-block scoring, p 0.95,
                       k_min 32.
* ``hetero_slack``     B1 H40, grid 21x30x52; 36 heads as 480P sigma 3, 4 heads
                       (chosen by seed) near-dense: Q and K independent
                       standardised sigma 0.5 fields; p_h ~ U(0.5, 0.99) per
                       head, k_min 16, slack fill to the median.

Every random stream is keyed by ``SeedSequence(seed, spawn_key=(b, h, tensor))``
so the bytes do not depend on generation order or thread count.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
from scipy.ndimage import gaussian_filter1d

# tensor ids inside a spawn key
_T_FIELD, _T_Q, _T_K, _T_V, _T_FIELD_K, _T_DO = 0, 1, 2, 3, 4, 5
_HEAD_PARAMS = 1000  # spawn-key slot for per-head parameters


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    D: int
    grid: tuple
    dtype: str            # "bf16" or "f32"
    kind: str             # "tile_shared", "tile_indep", "smooth"
    p: object             # float, or ("uniform", lo, hi) per head
    k_min: int
    seed: int
    sigma: object = 3.0   # float, or ("uniform", lo, hi) per head
    tile: tuple = (4, 4, 4)
    order: str = "tile"   # "tile" or "hilbert"
    sub: tuple = (0, 0, 0)
    slack: str = "none"   # "none" or "median"
    near_dense_frac: float = 0.0
    noise: float = 0.3

    @property
    def n_tokens(self) -> int:
        t, h, w = self.grid
        return t * h * w


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_f32", 1, 2, 64, (8, 16, 16), "f32", "tile_shared", 0.9, 4, 1),
        Workload("tiny_f32_indep", 1, 2, 64, (8, 16, 16), "f32", "tile_indep", 0.9, 4, 11),
        Workload("wan1.3b_480p", 1, 12, 128, (21, 30, 52), "bf16", "smooth", 0.9, 16, 2),
        Workload("wan14b_480p_cfg", 2, 40, 128, (21, 30, 52), "bf16", "smooth", 0.9, 16, 3,
                 sigma=("uniform", 1.0, 8.0)),
        Workload("wan_720p_hilbert_sub", 1, 40, 128, (21, 45, 80), "bf16", "smooth", 0.95, 32, 4,
                 order="hilbert", sub=(2, 2, 2)),
        Workload("hetero_slack", 1, 40, 128, (21, 30, 52), "bf16", "smooth",
                 ("uniform", 0.5, 0.99), 16, 5, slack="median", near_dense_frac=0.1),
    ]
}


def scaled(w: Workload, **changes) -> Workload:
    """A copy of ``w`` with some fields replaced (smaller grids for tests)."""
    return dataclasses.replace(w, **changes)


# ---------------------------------------------------------------- rounding
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16.  Inputs here are finite.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array (uint16 bf16 bits or float32) to float64, exactly."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


# ---------------------------------------------------------------- fields
def _smoothing_matrix(n: int, sigma: float) -> np.ndarray:
    """Dense n x n operator of a 1-D Gaussian filter (reflect boundary,
    truncated at 4 sigma): column j is the filtered unit impulse at j."""
    eye = np.eye(n, dtype=np.float64)
    return gaussian_filter1d(eye, sigma, axis=0, mode="reflect", truncate=4.0)


def smooth_field(rng: np.random.Generator, grid, d: int, sigma: float) -> np.ndarray:
    """White N(0,1) noise on (t, h, w, d), Gaussian-filtered over t, h, w,
    then standardised per channel to mean 0 and std 1 over the tokens.
    Returns float32 of shape (t*h*w, d)."""
    t, h, w = grid
    x = rng.standard_normal((t, h, w, d), dtype=np.float32)
    at = _smoothing_matrix(t, sigma).astype(np.float32)
    ah = _smoothing_matrix(h, sigma).astype(np.float32)
    aw = _smoothing_matrix(w, sigma).astype(np.float32)
    x = (at @ x.reshape(t, -1)).reshape(t, h, w, d)
    x = np.matmul(ah, x.transpose(1, 0, 2, 3).reshape(h, -1)).reshape(h, t, w, d).transpose(1, 0, 2, 3)
    x = np.matmul(aw, x.transpose(2, 0, 1, 3).reshape(w, -1)).reshape(w, t, h, d).transpose(1, 2, 0, 3)
    x = np.ascontiguousarray(x).reshape(t * h * w, d)
    mean = x.mean(axis=0, dtype=np.float64)
    std = x.std(axis=0, dtype=np.float64)
    return ((x - mean) / std).astype(np.float32)


def _tile_index(grid, tile) -> np.ndarray:
    """Raster token index -> raster index of its tile (for the tiny inputs)."""
    t, h, w = grid
    tt, th, tw = tile
    tc, hc, wc = np.meshgrid(np.arange(t), np.arange(h), np.arange(w), indexing="ij")
    nh = -(-h // th)
    nw = -(-w // tw)
    return (((tc // tt) * nh + hc // th) * nw + wc // tw).reshape(-1)


def _rng(seed: int, *key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def head_params(w: Workload):
    """Per-head parameters drawn once per workload: sigma_h, p_h and the set
    of near-dense heads."""
    rng = _rng(w.seed, _HEAD_PARAMS)
    if isinstance(w.sigma, tuple):
        sig = rng.uniform(w.sigma[1], w.sigma[2], size=w.H)
    else:
        sig = np.full(w.H, float(w.sigma))
    if isinstance(w.p, tuple):
        p = rng.uniform(w.p[1], w.p[2], size=w.H).astype(np.float32)
    else:
        p = np.full(w.H, w.p, dtype=np.float32)
    n_dense = int(round(w.near_dense_frac * w.H))
    dense = np.zeros(w.H, dtype=bool)
    if n_dense:
        dense[rng.choice(w.H, n_dense, replace=False)] = True
    return sig, p, dense


def _one_head(w: Workload, b: int, h: int, sig: float, dense: bool):
    n, d = w.n_tokens, w.D
    if w.kind in ("tile_shared", "tile_indep"):
        tix = _tile_index(w.grid, w.tile)
        n_t = int(tix.max()) + 1
        cq = _rng(w.seed, b, h, _T_FIELD).standard_normal((n_t, d))
        ck = cq if w.kind == "tile_shared" else _rng(w.seed, b, h, _T_FIELD_K).standard_normal((n_t, d))
        q = cq[tix] + 0.5 * _rng(w.seed, b, h, _T_Q).standard_normal((n, d))
        k = ck[tix] + 0.5 * _rng(w.seed, b, h, _T_K).standard_normal((n, d))
    elif dense:
        q = smooth_field(_rng(w.seed, b, h, _T_FIELD), w.grid, d, 0.5)
        k = smooth_field(_rng(w.seed, b, h, _T_FIELD_K), w.grid, d, 0.5)
    else:
        f = smooth_field(_rng(w.seed, b, h, _T_FIELD), w.grid, d, sig)
        q = f + w.noise * _rng(w.seed, b, h, _T_Q).standard_normal((n, d), dtype=np.float32)
        k = f + w.noise * _rng(w.seed, b, h, _T_K).standard_normal((n, d), dtype=np.float32)
    v = _rng(w.seed, b, h, _T_V).standard_normal((n, d), dtype=np.float32)
    out = []
    for x in (q, k, v):
        x = np.asarray(x, dtype=np.float32)
        out.append(f32_to_bf16_bits(x) if w.dtype == "bf16" else x)
    return out


def make(w: Workload, threads: int | None = None, heads=None):
    """Generate raster Q, K, V of shape [B, N, H, D].

    Storage is uint16 bfloat16 bit patterns for ``bf16`` workloads and float32
    otherwise.  ``heads`` optionally restricts generation to a list of
    (b, h) pairs (the other heads are left zero).
    Returns (q, k, v, meta) where meta holds per-head p and sigma.
    """
    sig, p, dense = head_params(w)
    st = np.uint16 if w.dtype == "bf16" else np.float32
    shape = (w.B, w.n_tokens, w.H, w.D)
    q, k, v = (np.zeros(shape, dtype=st) for _ in range(3))
    pairs = heads if heads is not None else [(b, h) for b in range(w.B) for h in range(w.H)]

    def work(bh):
        b, h = bh
        qq, kk, vv = _one_head(w, b, h, float(sig[h]), bool(dense[h]))
        q[b, :, h, :] = qq
        k[b, :, h, :] = kk
        v[b, :, h, :] = vv

    nthr = threads or min(16, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(max_workers=nthr) as ex:
        list(ex.map(work, pairs))
    meta = {"p_head": p, "sigma_head": sig, "near_dense": dense}
    return q, k, v, meta


def make_dout(w: Workload, threads: int | None = None, heads=None, scale: float = 1.0):
    """Seeded output gradient dO of shape [B, N, H, D] for the backward
    pass: N(0, scale^2) per element, one independent stream per (b, h), in
    the workload's storage type (``heads`` as for ``make``)."""
    st = np.uint16 if w.dtype == "bf16" else np.float32
    out = np.zeros((w.B, w.n_tokens, w.H, w.D), dtype=st)
    pairs = heads if heads is not None else [(b, h) for b in range(w.B) for h in range(w.H)]

    def work(bh):
        b, h = bh
        x = scale * _rng(w.seed, b, h, _T_DO).standard_normal((w.n_tokens, w.D), dtype=np.float32)
        out[b, :, h, :] = f32_to_bf16_bits(x) if w.dtype == "bf16" else x

    nthr = threads or min(16, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(max_workers=nthr) as ex:
        list(ex.map(work, pairs))
    return out


_DRIFT = 1001   # spawn-key slot for the drift streams (apart from any (b, h, tensor) key)


def drift(w: Workload, x: np.ndarray, tensor: int, step: int, step_std: float = 0.1) -> np.ndarray:
    """Inputs of a later denoising step: ``x`` (a storage array from ``make``)
    after ``step`` steps of a seeded random walk, i.e. plus
    N(0, step * step_std^2) per element, one independent stream per
    (tensor, step) pair, re-rounded to the workload's storage type.
    ``tensor`` names the stream (0: Q, 1: K, 2: V)."""
    f = bf16_bits_to_f32(x) if w.dtype == "bf16" else np.asarray(x, dtype=np.float32)
    rng = _rng(w.seed, _DRIFT, tensor, step)
    y = f + np.float32(step_std * np.sqrt(step)) * rng.standard_normal(f.shape, dtype=np.float32)
    return f32_to_bf16_bits(y) if w.dtype == "bf16" else y.astype(np.float32)
