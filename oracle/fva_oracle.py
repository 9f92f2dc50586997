"""Plain, slow, fp64 CPU oracle for training-free block-sparse spatiotemporal
attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code with the HIP library.

Sources (the pages this follows; cited by title and section):

* [FVAttn]  "FVAttn: Adaptive Sparse Attention with Runtime Load Balancing for
  Video Generation" (review page), sections 00 and 02: a routing front end that
  keeps blocks by adaptive Top-p with a Top-k safety floor over video-aware
  blocks, and that spends spare capacity on extra high-value blocks.
* [VSA]  Video Sparse Attention explainer page, dialogue and section 3: tokens
  are pooled in small (4,4,4) cubes, cube-level importance is predicted from the
  pooled tiles, and token-level attention runs only inside the chosen tiles.
* [DFSAttn]  "DFSAttn: Dynamic Fine-grained Sparse Attention for Efficient Video
  Generation" explainer page, tricks 1 and 2: a 3D Hilbert-curve reordering so
  that sequence neighbours are space-time neighbours, and block scores formed by
  summing finer sub-block scores.

Readings where the pages are silent (each one stated where it is used):

* pooling is the arithmetic mean over the valid (non-pad) tokens of a cube;
* the cube score is softmax over key cubes of q_bar . k_bar / sqrt(D);
* Top-p keeps the shortest prefix, in (score desc, block id asc) order, whose
  mass reaches p; p >= 1 keeps everything; the floor is
  k = max(k_p, min(k_min, n_blk));
* the selection mass is an exact fixed-point sum: each fp32 score s, clamped
  to [0, 1] (NaN counts as 0), contributes floor(s * 2**47) and the threshold
  is ceil(p * 2**47);
* sub-block scoring splits the key side only: the softmax runs over every
  non-empty (block, sub-block) pair and a block's score is the sum over its
  sub-blocks;
* slack fill lifts every head whose block count is below the lower median of
  the call's heads up to that median, adding unselected (I, J) pairs in
  (score desc, I asc, J asc) order;
* attention uses scale 1/sqrt(D); pad keys and unselected blocks are left out
  of the softmax; pad query rows of the permuted output are zero.

Parity pins for every function live in ``tests/test_oracle.py``.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

PAD = -1
FIX_BITS = 47
FIX_ONE = 1 << FIX_BITS


# --------------------------------------------------------------------------
# 3D Hilbert index (J. Skilling, "Programming the Hilbert curve", AIP Conf.
# Proc. 707, 2004): coordinates -> "transposed" index by undoing the excess
# rotations level by level, Gray-encoding across axes, then reading the bits
# of the three transposed words interleaved, most significant level first.
# Used by [DFSAttn] trick 1.
# --------------------------------------------------------------------------
def hilbert_key(coords, bits: int) -> int:
    """Hilbert index of integer coordinates (x0, x1, x2) on the 2**bits cube."""
    x = [int(c) for c in coords]
    n = len(x)
    q = 1 << (bits - 1)
    while q > 1:
        low = q - 1
        for i in range(n):
            if x[i] & q:
                x[0] ^= low                      # flip the low bits of axis 0
            else:
                swap = (x[0] ^ x[i]) & low       # exchange low bits of 0 and i
                x[0] ^= swap
                x[i] ^= swap
        q >>= 1
    for i in range(1, n):                        # Gray encode across axes
        x[i] ^= x[i - 1]
    fix = 0
    q = 1 << (bits - 1)
    while q > 1:
        if x[n - 1] & q:
            fix ^= q - 1
        q >>= 1
    for i in range(n):
        x[i] ^= fix
    key = 0
    for level in range(bits - 1, -1, -1):
        for i in range(n):
            key = (key << 1) | ((x[i] >> level) & 1)
    return key


# --------------------------------------------------------------------------
# Plan: padding, block order and per-position tables.  [VSA] section 3 (cube
# tiles), [DFSAttn] trick 1 (Hilbert order).  Tokens are in raster ("book")
# order n = (t*H + h)*W + w; a block is 64 consecutive permuted positions.
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Plan:
    grid: tuple
    tile: tuple
    padded: tuple
    order: str
    sub: tuple
    n_blk: int
    n_pad: int
    perm: np.ndarray        # [n_pad] raster index of each permuted position or PAD
    coords: np.ndarray      # [n_pad, 3] padded-grid coordinate of each position
    cnt: np.ndarray         # [n_blk] valid tokens per block
    sub_id: np.ndarray      # [n_pad] sub-block index within the block (or -1)
    n_sub: int

    @property
    def blk_size(self) -> int:
        return self.tile[0] * self.tile[1] * self.tile[2]

    @property
    def inv(self) -> np.ndarray:
        """[N] permuted position of each raster token."""
        out = np.empty(self.grid[0] * self.grid[1] * self.grid[2], dtype=np.int64)
        valid = self.perm >= 0
        out[self.perm[valid]] = np.nonzero(valid)[0]
        return out


def plan(grid, tile=(4, 4, 4), order="tile", sub=(0, 0, 0)) -> Plan:
    T, H, W = grid
    tt, th, tw = tile
    Tp, Hp, Wp = (-(-T // tt) * tt, -(-H // th) * th, -(-W // tw) * tw)
    pts = [(t, h, w) for t in range(Tp) for h in range(Hp) for w in range(Wp)]
    if order == "tile":
        nh, nw = Hp // th, Wp // tw

        def key(c):
            t, h, w = c
            blk = ((t // tt) * nh + h // th) * nw + w // tw
            loc = ((t % tt) * th + h % th) * tw + w % tw
            return blk * (tt * th * tw) + loc
    elif order == "hilbert":
        bits = max(1, math.ceil(math.log2(max(Tp, Hp, Wp))))

        def key(c):
            return hilbert_key(c, bits)
    else:
        raise ValueError(order)
    pts.sort(key=key)
    coords = np.array(pts, dtype=np.int64)
    n_pad = len(pts)
    bs = tt * th * tw
    valid = (coords[:, 0] < T) & (coords[:, 1] < H) & (coords[:, 2] < W)
    raster = (coords[:, 0] * H + coords[:, 1]) * W + coords[:, 2]
    perm = np.where(valid, raster, PAD)
    n_blk = n_pad // bs
    cnt = valid.reshape(n_blk, bs).sum(axis=1)
    sub = tuple(sub)
    if any(sub):
        st, sh, sw = sub
        sid = (((coords[:, 0] % tt) // st) * (th // sh) + (coords[:, 1] % th) // sh) * (tw // sw) \
            + (coords[:, 2] % tw) // sw
        n_sub = (tt // st) * (th // sh) * (tw // sw)
    else:
        sid = np.full(n_pad, -1, dtype=np.int64)
        n_sub = 0
    return Plan(tuple(grid), tuple(tile), (Tp, Hp, Wp), order, sub, n_blk, n_pad, perm, coords,
                cnt, sid, n_sub)


def permute(x_raster: np.ndarray, pl: Plan) -> np.ndarray:
    """[B, N, H, D] raster -> [B, H, N_pad, D] block order, pad rows zero."""
    B, N, H, D = x_raster.shape
    out = np.zeros((B, H, pl.n_pad, D), dtype=np.float64)
    valid = pl.perm >= 0
    out[:, :, valid, :] = np.transpose(x_raster, (0, 2, 1, 3))[:, :, pl.perm[valid], :]
    return out


def unpermute(x_perm: np.ndarray, pl: Plan) -> np.ndarray:
    """[B, H, N_pad, D] block order -> [B, N, H, D] raster; pads dropped."""
    return np.transpose(x_perm[:, :, pl.inv, :], (0, 2, 1, 3)).copy()


# --------------------------------------------------------------------------
# Coarse stage: [VSA] dialogue and section 3 (pool cubes, score tiles).
# --------------------------------------------------------------------------
def pool(x_perm: np.ndarray, pl: Plan) -> np.ndarray:
    """Mean over the valid tokens of each block: [B, H, n_blk, D]."""
    B, H, _, D = x_perm.shape
    bs = pl.blk_size
    out = np.empty((B, H, pl.n_blk, D))
    valid = pl.perm >= 0
    for j in range(pl.n_blk):
        rows = np.nonzero(valid[j * bs:(j + 1) * bs])[0] + j * bs
        out[:, :, j, :] = x_perm[:, :, rows, :].mean(axis=2)
    return out


def pool_sub(x_perm: np.ndarray, pl: Plan):
    """Mean over the valid tokens of each (block, sub-block) pair
    ([DFSAttn] trick 2).  Returns ([B, H, n_blk, n_sub, D], empty[n_blk, n_sub])."""
    B, H, _, D = x_perm.shape
    bs, ns = pl.blk_size, pl.n_sub
    out = np.zeros((B, H, pl.n_blk, ns, D))
    empty = np.ones((pl.n_blk, ns), dtype=bool)
    valid = pl.perm >= 0
    for j in range(pl.n_blk):
        for s in range(ns):
            sel = np.nonzero(valid[j * bs:(j + 1) * bs] & (pl.sub_id[j * bs:(j + 1) * bs] == s))[0]
            if len(sel):
                empty[j, s] = False
                out[:, :, j, s, :] = x_perm[:, :, sel + j * bs, :].mean(axis=2)
    return out, empty


def score(qbar: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """S[b,h,I,:] = softmax_J(qbar_I . kbar_J / sqrt(D))  ([VSA] section 3)."""
    D = qbar.shape[-1]
    z = np.einsum("bhid,bhjd->bhij", qbar, kbar) / math.sqrt(D)
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def score_sub(qbar: np.ndarray, kbar_sub: np.ndarray, empty: np.ndarray) -> np.ndarray:
    """Block score = sum of sub-block scores, the softmax running over every
    non-empty (block, sub-block) key ([DFSAttn] trick 2)."""
    B, H, n, ns, D = kbar_sub.shape
    flat = kbar_sub.reshape(B, H, n * ns, D)
    z = np.einsum("bhid,bhjd->bhij", qbar, flat) / math.sqrt(D)
    z = np.where(empty.reshape(-1)[None, None, None, :], -np.inf, z)
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    prob = e / e.sum(axis=-1, keepdims=True)
    return prob.reshape(B, H, n, n, ns).sum(axis=-1)


# --------------------------------------------------------------------------
# Routing: [FVAttn] sections 00 and 02 (Top-p with a Top-k floor).
# --------------------------------------------------------------------------
def clamp_scores(s) -> np.ndarray:
    """fp32 view used by selection: NaN and s <= 0 -> +0, s > 1 -> 1."""
    s = np.asarray(s, dtype=np.float32)
    s = np.where(s > 0, s, np.float32(0))      # NaN compares false
    return np.minimum(s, np.float32(1)).astype(np.float32)


def fixed_mass(s32: np.ndarray) -> np.ndarray:
    """floor(s * 2**47) of clamped fp32 scores, exact (int64).

    s is an fp32 value in [0, 1]; s * 2**47 is exact in fp64 (a power-of-two
    scaling of a 24-bit significand) and below 2**53, so the floor is exact.
    """
    v = np.asarray(s32, dtype=np.float32).astype(np.float64) * float(FIX_ONE)
    return np.floor(v).astype(np.int64)


def fixed_threshold(p) -> int:
    return int(math.ceil(float(np.float32(p)) * FIX_ONE))


def rank_order(s32: np.ndarray) -> np.ndarray:
    """Block ids by (score desc, id asc)."""
    s32 = np.asarray(s32, dtype=np.float32)
    ids = np.arange(len(s32))
    return np.lexsort((ids, -s32.astype(np.float64)))


def select_row(s_row, p: float, k_min: int) -> np.ndarray:
    """Blocks one query block keeps, ascending."""
    s32 = clamp_scores(s_row)
    n = len(s32)
    order = rank_order(s32)
    if float(np.float32(p)) >= 1.0:
        k_p = n
    else:
        prefix = np.cumsum(fixed_mass(s32)[order])      # int64, < 2**63 for n < 2**16
        hit = np.nonzero(prefix >= fixed_threshold(p))[0]
        k_p = int(hit[0]) + 1 if len(hit) else n
    k = max(k_p, min(int(k_min), n))
    return np.sort(order[:k])


def select(S: np.ndarray, p_head, k_min: int):
    """CSR over flattened rows r = (b*H + h)*n_blk + I: (row_ptr, col_idx)."""
    B, H, n, _ = S.shape
    p_head = np.broadcast_to(np.asarray(p_head, dtype=np.float32), (H,))
    rows = []
    for b in range(B):
        for h in range(H):
            for i in range(n):
                rows.append(select_row(S[b, h, i], p_head[h], k_min))
    return to_csr(rows)


def to_csr(rows):
    row_ptr = np.zeros(len(rows) + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum([len(r) for r in rows])
    col_idx = np.concatenate([np.asarray(r, dtype=np.int64) for r in rows]) if rows else np.zeros(0, np.int64)
    return row_ptr, col_idx


def from_csr(row_ptr, col_idx):
    return [np.asarray(col_idx[row_ptr[r]:row_ptr[r + 1]]) for r in range(len(row_ptr) - 1)]


def head_nnz(row_ptr, B: int, H: int, n: int) -> np.ndarray:
    rp = np.asarray(row_ptr, dtype=np.int64)
    return np.array([rp[(bh + 1) * n] - rp[bh * n] for bh in range(B * H)], dtype=np.int64)


def slack_fill(S: np.ndarray, row_ptr, col_idx):
    """Lift light heads to the lower median block count ([FVAttn] section 02,
    slack-aware augmentation, one-GPU reading)."""
    B, H, n, _ = S.shape
    rows = from_csr(row_ptr, col_idx)
    nnz = head_nnz(row_ptr, B, H, n)
    target = int(np.sort(nnz)[(len(nnz) - 1) // 2])
    for bh in range(B * H):
        need = target - int(nnz[bh])
        if need <= 0:
            continue
        s32 = clamp_scores(S.reshape(B * H, n, n)[bh]).reshape(-1)
        chosen = np.zeros(n * n, dtype=bool)
        for i in range(n):
            chosen[i * n + rows[bh * n + i]] = True
        lin = np.nonzero(~chosen)[0]                      # linear index i*n + j
        order = np.lexsort((lin, -s32[lin].astype(np.float64)))
        add = lin[order[:need]]
        for i in range(n):
            extra = add[add // n == i] % n
            if len(extra):
                rows[bh * n + i] = np.sort(np.concatenate([rows[bh * n + i], extra]))
    return to_csr(rows)


# --------------------------------------------------------------------------
# Fine stage: [VSA] section 3 (token attention inside the chosen tiles only).
# --------------------------------------------------------------------------
def attention(q_perm, k_perm, v_perm, row_ptr, col_idx, pl: Plan) -> np.ndarray:
    """O_perm[b,h,i] = sum_j softmax_j(q_i . k_j / sqrt(D)) v_j over the valid
    key tokens j of the selected blocks of i's block; pad queries give 0."""
    B, H, n_pad, D = q_perm.shape
    n, bs = pl.n_blk, pl.blk_size
    out = np.zeros(q_perm.shape[:3] + v_perm.shape[3:], dtype=np.float64)
    valid = pl.perm >= 0
    scale = 1.0 / math.sqrt(D)
    for b in range(B):
        for h in range(H):
            for i in range(n):
                r = (b * H + h) * n + i
                blocks = col_idx[row_ptr[r]:row_ptr[r + 1]]
                qrows = np.nonzero(valid[i * bs:(i + 1) * bs])[0] + i * bs
                if len(blocks) == 0 or len(qrows) == 0:
                    continue
                krows = np.concatenate([np.nonzero(valid[j * bs:(j + 1) * bs])[0] + j * bs for j in blocks])
                z = q_perm[b, h, qrows] @ k_perm[b, h, krows].T * scale
                z -= z.max(axis=1, keepdims=True)
                e = np.exp(z)
                out[b, h, qrows] = (e / e.sum(axis=1, keepdims=True)) @ v_perm[b, h, krows]
    return out


def run(q, k, v, pl: Plan, p_head, k_min: int, slack: str = "none"):
    """Whole path on raster fp64 inputs; returns every intermediate."""
    qp, kp, vp = permute(q, pl), permute(k, pl), permute(v, pl)
    qbar = pool(qp, pl)
    if pl.n_sub:
        kbs, empty = pool_sub(kp, pl)
        S = score_sub(qbar, kbs, empty)
    else:
        S = score(qbar, pool(kp, pl))
    row_ptr, col_idx = select(S, p_head, k_min)
    if slack == "median":
        row_ptr, col_idx = slack_fill(S, row_ptr, col_idx)
    o_perm = attention(qp, kp, vp, row_ptr, col_idx, pl)
    return dict(q_perm=qp, k_perm=kp, v_perm=vp, qbar=qbar, scores=S, row_ptr=row_ptr,
                col_idx=col_idx, o_perm=o_perm, o=unpermute(o_perm, pl))


# --------------------------------------------------------------------------
# 3D rotary position encoding with a global time index ([CausalRoPE-SP]
# "Accelerating Video Generation Inference with Sequential-Parallel 3D
# Positional Encoding Using a Global Time Index", section 2.2: each chunk of
# frames uses t_global = t_local + s with its start frame s, so a chunk can be
# encoded without the rest of the sequence).  Readings (the page gives no
# split or convention): the D/2 rotation pairs are split as evenly as
# possible over the (t, h, w) axes, t first; pair p rotates dims (2p, 2p+1);
# within an axis with P pairs, pair i turns by pos * base**(-i / P).
def rope_pairs(head_dim: int):
    """Number of rotation pairs given to the t, h and w axes."""
    n = head_dim // 2
    q, r = divmod(n, 3)
    # the remainder goes one pair at a time to t, then h
    return q + (1 if r > 0 else 0), q + (1 if r > 1 else 0), q


def rope_angles(grid, head_dim: int, t_offset: int = 0, base: float = 10000.0):
    """Angle of every rotation pair at every raster token: [N, D/2] (fp64)."""
    T, Hh, W = grid
    counts = rope_pairs(head_dim)
    t, h, w = np.meshgrid(np.arange(T) + t_offset, np.arange(Hh), np.arange(W), indexing="ij")
    pos = [t.reshape(-1), h.reshape(-1), w.reshape(-1)]
    cols = []
    for axis, P in enumerate(counts):
        inv = base ** (-np.arange(P, dtype=np.float64) / P)
        cols.append(pos[axis][:, None].astype(np.float64) * inv[None, :])
    return np.concatenate(cols, axis=1)


def rope(x_raster: np.ndarray, grid, t_offset: int = 0, base: float = 10000.0) -> np.ndarray:
    """Rotate raster [B, N, H, D] fp64 tokens by their 3D position."""
    D = x_raster.shape[-1]
    ang = rope_angles(grid, D, t_offset, base)[None, :, None, :]     # [1, N, 1, D/2]
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x_raster[..., 0::2], x_raster[..., 1::2]
    out = np.empty_like(x_raster)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


# --------------------------------------------------------------------------
# Mask reuse across denoising steps ([DFSAttn] trick 3: blocks that mattered
# at an earlier step are kept instead of re-evaluated; "FVAttn" section 02
# makes the same selection per step).  The decision to reuse a cached mask
# reads how much two selections agree: per (b, h), the sizes of the
# intersection and of the union of the kept (I, J) pairs.
def mask_overlap(rp_a, ci_a, rp_b, ci_b, B: int, H: int, n_blk: int) -> np.ndarray:
    """[B*H, 2] int64: |A & B| and |A | B| over the (I, J) pairs of each head."""
    a_rows, b_rows = from_csr(rp_a, ci_a), from_csr(rp_b, ci_b)
    out = np.zeros((B * H, 2), dtype=np.int64)
    for r in range(B * H * n_blk):
        sa = set(int(j) for j in a_rows[r] if 0 <= j < n_blk)   # rows are sets of plan blocks
        sb = set(int(j) for j in b_rows[r] if 0 <= j < n_blk)
        out[r // n_blk, 0] += len(sa & sb)
        out[r // n_blk, 1] += len(sa | sb)
    return out


# --------------------------------------------------------------------------
# Static calibrated selections ("Calibrated Sparse Attention" page: an
# offline pass keeps the block patterns that stay stable across calibration
# inputs, per layer, head and diffusion step, and inference then skips the
# rest).  Reading: count, per (b, h, I, J), in how many calibration runs the
# pair was selected; keep the pairs selected in at least min_count runs
# (min_count 1: the union of the runs; min_count = runs: their intersection).
def calib_counts(csrs, B: int, H: int, n_blk: int) -> np.ndarray:
    """[B*H*n_blk, n_blk] int64 selection counts over a list of (row_ptr, col_idx)."""
    counts = np.zeros((B * H * n_blk, n_blk), dtype=np.int64)
    for rp, ci in csrs:
        for r, row in enumerate(from_csr(rp, ci)):
            for j in set(int(x) for x in row if 0 <= x < n_blk):
                counts[r, j] += 1
    return counts


def calib_select(counts: np.ndarray, min_count: int):
    """CSR (ascending ids) of the pairs counted at least min_count times."""
    rows = [np.nonzero(c >= min_count)[0] for c in counts]
    return to_csr(rows)


# --------------------------------------------------------------------------
# Backward pass of the block-sparse attention on the same lists (the pages'
# trained sparse attention, "Video Sparse Attention" explainer section 3,
# needs gradients through the fine stage).  For every valid query token i of
# block I, over the valid key tokens j of I's listed blocks:
#   P_ij = softmax_j(q_i . k_j / sqrt(D)),  o_i = sum_j P_ij v_j
#   dv_j += P_ij do_i;  dP_ij = do_i . v_j;  dS_ij = P_ij (dP_ij - sum_j' P_ij' dP_ij')
#   dq_i = sum_j dS_ij k_j / sqrt(D);  dk_j += dS_ij q_i / sqrt(D)
# (the gradient of o with respect to q, k, v; pad rows get zero gradients).
def attention_backward(q_perm, k_perm, v_perm, do_perm, row_ptr, col_idx, pl: Plan):
    """(dq, dk, dv) in block order, fp64."""
    B, H, n_pad, D = q_perm.shape
    n, bs = pl.n_blk, pl.blk_size
    dq, dk, dv = np.zeros_like(q_perm), np.zeros_like(k_perm), np.zeros_like(v_perm)
    valid = pl.perm >= 0
    scale = 1.0 / math.sqrt(D)
    for b in range(B):
        for h in range(H):
            for i in range(n):
                r = (b * H + h) * n + i
                blocks = col_idx[row_ptr[r]:row_ptr[r + 1]]
                qrows = np.nonzero(valid[i * bs:(i + 1) * bs])[0] + i * bs
                if len(blocks) == 0 or len(qrows) == 0:
                    continue
                krows = np.concatenate([np.nonzero(valid[j * bs:(j + 1) * bs])[0] + j * bs for j in blocks])
                Q, K, V, dO = q_perm[b, h, qrows], k_perm[b, h, krows], v_perm[b, h, krows], do_perm[b, h, qrows]
                z = Q @ K.T * scale
                z -= z.max(axis=1, keepdims=True)
                P = np.exp(z)
                P /= P.sum(axis=1, keepdims=True)
                dP = dO @ V.T
                dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
                dq[b, h, qrows] += dS @ K * scale
                np.add.at(dk[b, h], krows, dS.T @ Q * scale)
                np.add.at(dv[b, h], krows, P.T @ dO)
    return dq, dk, dv


# --------------------------------------------------------------------------
# Softmax normaliser of each query row, the value the backward pass rebuilds
# P from (same lists and scale as ``attention``): in base-2 units,
#   lse_i = log2 sum_j exp(q_i . k_j / sqrt(D))
# over the valid key tokens j of the listed blocks; 0 for pad queries and
# rows with no listed block.  Result [B, H, n_pad].
def attention_lse(q_perm, k_perm, row_ptr, col_idx, pl: Plan) -> np.ndarray:
    B, H, n_pad, D = q_perm.shape
    n, bs = pl.n_blk, pl.blk_size
    out = np.zeros((B, H, n_pad), dtype=np.float64)
    valid = pl.perm >= 0
    scale = 1.0 / math.sqrt(D)
    for b in range(B):
        for h in range(H):
            for i in range(n):
                r = (b * H + h) * n + i
                blocks = col_idx[row_ptr[r]:row_ptr[r + 1]]
                qrows = np.nonzero(valid[i * bs:(i + 1) * bs])[0] + i * bs
                if len(blocks) == 0 or len(qrows) == 0:
                    continue
                krows = np.concatenate([np.nonzero(valid[j * bs:(j + 1) * bs])[0] + j * bs for j in blocks])
                z = q_perm[b, h, qrows] @ k_perm[b, h, krows].T * scale
                m = z.max(axis=1)
                out[b, h, qrows] = (m + np.log(np.exp(z - m[:, None]).sum(axis=1))) / math.log(2.0)
    return out


# Transposed lists: row (b, h, J) holds, ascending, every query block I whose
# row (b, h, I) lists J (rows read as sets, ids outside [0, n_blk) ignored) --
# the key-block-major view the dK / dV gradients are gathered over.
def mask_transpose(row_ptr, col_idx, B: int, H: int, n_blk: int):
    rows = [[] for _ in range(B * H * n_blk)]
    for bh in range(B * H):
        for i in range(n_blk):
            r = bh * n_blk + i
            for j in sorted(set(int(x) for x in col_idx[row_ptr[r]:row_ptr[r + 1]])):
                if 0 <= j < n_blk:
                    rows[bh * n_blk + j].append(i)
    return to_csr([np.array(x, dtype=np.int64) for x in rows])
