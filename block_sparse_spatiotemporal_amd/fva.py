"""ctypes binding of libfva.so (C ABI in include/fva.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Functions keep the C names; tensors are torch tensors on the GPU
(torch provides device memory and streams).  If the library is missing this
module raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfva.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "fva.h")

FVA_OK, FVA_EINVAL, FVA_EUNSUPPORTED, FVA_EHIP, FVA_ENOMEM = range(5)
ORDER = {"tile": 0, "hilbert": 1}
DTYPE = {"bf16": 0, "f32": 1}
LAYOUT_ROWS, LAYOUT_VT = 0, 1
FVA_POOL_Q, FVA_POOL_K = 0, 1
SLACK = {"none": 0, "median": 1}
SCHED = {"persistent": 0, "plain": 1}

c_i32, c_i64, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p


class fva_plan_desc(ctypes.Structure):
    _fields_ = [("batch", c_i32), ("heads", c_i32), ("head_dim", c_i32), ("grid", c_i32 * 3),
                ("tile", c_i32 * 3), ("order", c_i32), ("sub", c_i32 * 3), ("dtype", c_i32)]


class fva_plan_info(ctypes.Structure):
    _fields_ = [("n_tokens", c_i64), ("n_pad", c_i64), ("n_blk", c_i32), ("n_sub", c_i32),
                ("padded", c_i32 * 3), ("n_rows", c_i64), ("max_nnz", c_i64),
                ("workspace_bytes", c_i64), ("max_wg", c_i32)]


class FvaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"fva error {code}: {msg}")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """Open libfva.so (built by block_sparse_spatiotemporal_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        sig = {
            "fva_plan_dims": (c_i32, [P(fva_plan_desc), P(fva_plan_info)]),
            "fva_plan_tables": (c_i32, [P(fva_plan_desc), c_vp, c_vp, c_vp, c_vp]),
            "fva_plan_create": (c_i32, [P(c_vp), P(fva_plan_desc), c_vp]),
            "fva_plan": (c_i32, [P(c_vp), P(fva_plan_desc), c_vp]),
            "fva_attention_static": (c_i32, [P(fva_plan_desc)] + [c_vp] * 7),
            "fva_plan_query": (c_i32, [c_vp, P(fva_plan_info)]),
            "fva_plan_destroy": (None, [c_vp]),
            "fva_permute": (c_i32, [c_vp, c_vp, c_vp, c_i32, c_vp]),
            "fva_permute_rope": (c_i32, [c_vp, c_vp, c_vp, c_i32, ctypes.c_double, c_vp]),
            "fva_permute_pool": (c_i32, [c_vp, c_vp, c_vp, c_i32, c_vp]),
            "fva_select_pooled": (c_i32, [c_vp, P(ctypes.c_float), c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp,
                                          c_vp]),
            "fva_select": (c_i32, [c_vp, c_vp, c_vp, P(ctypes.c_float), c_i32, c_i32, c_i32, c_vp, c_vp,
                                   c_vp, c_vp, c_vp, c_vp]),
            "fva_attention": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp]),
            "fva_attention_raster": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp]),
            "fva_unpermute": (c_i32, [c_vp, c_vp, c_vp, c_vp]),
            "fva_mask_overlap": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
            "fva_p_schedule": (c_i32, [c_i32, c_i32, ctypes.c_float, ctypes.c_float, P(ctypes.c_float)]),
            "fva_mask_accumulate": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp]),
            "fva_mask_from_counts": (c_i32, [c_vp, c_vp, c_i32, c_vp, c_vp, c_vp, c_vp]),
            "fva_attention_lse": (c_i32, [c_vp] * 10),
            "fva_attention_backward": (c_i32, [c_vp] * 14),
            "fva_mask_transpose": (c_i32, [c_vp] * 6),
            "fva_last_error": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def header_symbols() -> list[str]:
    """Entry points declared in include/fva.h."""
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(fva_\w+)\s*\(", txt, re.M)))


def _check(rc: int):
    if rc != FVA_OK:
        raise FvaError(rc, lib().fva_last_error().decode())


def make_desc(batch, heads, head_dim, grid, tile=(4, 4, 4), order="tile", sub=(0, 0, 0), dtype="bf16"):
    d = fva_plan_desc()
    d.batch, d.heads, d.head_dim = batch, heads, head_dim
    d.grid[:] = list(grid)
    d.tile[:] = list(tile)
    d.order = ORDER[order] if isinstance(order, str) else int(order)
    d.sub[:] = list(sub)
    d.dtype = DTYPE[dtype] if isinstance(dtype, str) else int(dtype)
    return d


def fva_plan_dims(desc: fva_plan_desc) -> fva_plan_info:
    info = fva_plan_info()
    _check(lib().fva_plan_dims(ctypes.byref(desc), ctypes.byref(info)))
    return info


def fva_plan_tables(desc: fva_plan_desc):
    """Host tables as numpy arrays: (perm, blk_cnt, blk_mask, sub_id)."""
    import numpy as np
    info = fva_plan_dims(desc)
    perm = np.empty(info.n_pad, np.int32)
    cnt = np.empty(info.n_blk, np.int32)
    mask = np.empty(info.n_blk, np.uint64)
    sid = np.empty(info.n_pad, np.int32)
    _check(lib().fva_plan_tables(ctypes.byref(desc), perm.ctypes.data, cnt.ctypes.data, mask.ctypes.data,
                                 sid.ctypes.data))
    return perm, cnt, mask, sid


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return c_vp(s.cuda_stream)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("tensors must be contiguous CUDA/HIP tensors")
    return c_vp(t.data_ptr())


class Plan:
    """Owns an fva_plan_t; see include/fva.h for the meaning of every field."""

    def __init__(self, batch, heads, head_dim, grid, tile=(4, 4, 4), order="tile", sub=(0, 0, 0),
                 dtype="bf16", stream=None):
        self.desc = make_desc(batch, heads, head_dim, grid, tile, order, sub, dtype)
        self.dtype = dtype
        self.torch_dtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        h = c_vp()
        _check(lib().fva_plan(ctypes.byref(h), ctypes.byref(self.desc), _stream(stream)))
        self.handle = h
        self.info = fva_plan_info()
        _check(lib().fva_plan_query(h, ctypes.byref(self.info)))

    @property
    def n_blk(self):
        return self.info.n_blk

    @property
    def n_pad(self):
        return self.info.n_pad

    @property
    def n_rows(self):
        return self.info.n_rows

    def raster_shape(self):
        d = self.desc
        return (d.batch, self.info.n_tokens, d.heads, d.head_dim)

    def perm_shape(self):
        d = self.desc
        return (d.batch, d.heads, self.info.n_pad, d.head_dim)

    def destroy(self):
        if getattr(self, "handle", None) is not None and _lib is not None:
            lib().fva_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def _expect(t, shape, dtype, name):
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name}: expected {tuple(shape)} {dtype}, got {tuple(t.shape)} {t.dtype}")


def fva_permute(plan: Plan, x_raster, x_perm, layout=LAYOUT_ROWS, stream=None):
    _expect(x_raster, plan.raster_shape(), plan.torch_dtype, "x_raster")
    if x_perm.numel() != plan.desc.batch * plan.desc.heads * plan.n_pad * plan.desc.head_dim \
            or x_perm.dtype != plan.torch_dtype:
        raise ValueError("x_perm has the wrong size or dtype")
    _check(lib().fva_permute(plan.handle, _ptr(x_raster), _ptr(x_perm), int(layout), _stream(stream)))


def fva_permute_rope(plan: Plan, x_raster, x_perm, t_offset=0, base=10000.0, stream=None):
    """Raster -> block-order rows with the 3D rotary encoding applied
    (global time index t + t_offset)."""
    _expect(x_raster, plan.raster_shape(), plan.torch_dtype, "x_raster")
    _expect(x_perm, plan.perm_shape(), plan.torch_dtype, "x_perm")
    _check(lib().fva_permute_rope(plan.handle, _ptr(x_raster), _ptr(x_perm), int(t_offset), float(base),
                                  _stream(stream)))


def fva_p_schedule(step: int, n_steps: int, p_first: float, p_last: float) -> float:
    """Top-p for denoising step ``step`` of ``n_steps`` (the library's schedule)."""
    out = ctypes.c_float()
    _check(lib().fva_p_schedule(int(step), int(n_steps), float(p_first), float(p_last), ctypes.byref(out)))
    return out.value


def fva_mask_overlap(plan: Plan, row_ptr_a, col_idx_a, row_ptr_b, col_idx_b, counts=None, stream=None):
    """Per-head |A & B| and |A | B| of two CSR selections: int64 [B*H, 2]."""
    nbh = plan.desc.batch * plan.desc.heads
    for t, name in ((row_ptr_a, "row_ptr_a"), (row_ptr_b, "row_ptr_b")):
        _expect(t, (plan.n_rows + 1,), torch.int32, name)
    for t, name in ((col_idx_a, "col_idx_a"), (col_idx_b, "col_idx_b")):
        if t.dtype != torch.int32 or not t.is_cuda:
            raise ValueError(f"{name} must be an int32 device tensor")
    if counts is None:
        counts = torch.empty(nbh, 2, dtype=torch.int64, device="cuda")
    _expect(counts, (nbh, 2), torch.int64, "counts")
    _check(lib().fva_mask_overlap(plan.handle, _ptr(row_ptr_a), _ptr(col_idx_a), _ptr(row_ptr_b), _ptr(col_idx_b),
                                  _ptr(counts), _stream(stream)))
    return counts


def fva_mask_accumulate(plan: Plan, row_ptr, col_idx, counts, stream=None):
    """counts[r, J] += 1 for every kept pair of a selection (counts: int32 [n_rows, n_blk])."""
    _expect(row_ptr, (plan.n_rows + 1,), torch.int32, "row_ptr")
    _expect(counts, (plan.n_rows, plan.n_blk), torch.int32, "counts")
    _check(lib().fva_mask_accumulate(plan.handle, _ptr(row_ptr), _ptr(col_idx), _ptr(counts), _stream(stream)))


def fva_mask_from_counts(plan: Plan, counts, min_count, row_ptr, col_idx, head_nnz=None, stream=None):
    """CSR of the pairs counted at least min_count times."""
    _expect(counts, (plan.n_rows, plan.n_blk), torch.int32, "counts")
    _expect(row_ptr, (plan.n_rows + 1,), torch.int32, "row_ptr")
    if col_idx.dtype != torch.int32 or col_idx.numel() < plan.info.max_nnz:
        raise ValueError("col_idx must be int32 with capacity max_nnz")
    _check(lib().fva_mask_from_counts(plan.handle, _ptr(counts), int(min_count), _ptr(row_ptr), _ptr(col_idx),
                                      _ptr(head_nnz), _stream(stream)))


def fva_unpermute(plan: Plan, x_perm, x_raster, stream=None):
    _expect(x_raster, plan.raster_shape(), plan.torch_dtype, "x_raster")
    _expect(x_perm, plan.perm_shape(), plan.torch_dtype, "x_perm")
    _check(lib().fva_unpermute(plan.handle, _ptr(x_perm), _ptr(x_raster), _stream(stream)))


def fva_permute_pool(plan: Plan, x_raster, x_perm, which, stream=None):
    """fva_permute (rows) of Q (which="q") or K (which="k") that also leaves
    the pooled means in the plan's workspace for fva_select_pooled."""
    _expect(x_raster, plan.raster_shape(), plan.torch_dtype, "x_raster")
    _expect(x_perm, plan.perm_shape(), plan.torch_dtype, "x_perm")
    w = {"q": FVA_POOL_Q, "k": FVA_POOL_K}[which] if isinstance(which, str) else int(which)
    _check(lib().fva_permute_pool(plan.handle, _ptr(x_raster), _ptr(x_perm), w, _stream(stream)))


def fva_select_pooled(plan: Plan, p, k_min, row_ptr, col_idx, slack="none", scores_out=None, head_nnz=None,
                      stream=None):
    d = plan.desc
    if scores_out is not None:
        _expect(scores_out, (d.batch, d.heads, plan.n_blk, plan.n_blk), torch.float32, "scores_out")
    _expect(row_ptr, (plan.n_rows + 1,), torch.int32, "row_ptr")
    if col_idx.dtype != torch.int32 or col_idx.numel() < plan.info.max_nnz:
        raise ValueError("col_idx must be int32 with capacity max_nnz")
    if head_nnz is not None:
        _expect(head_nnz, (d.batch * d.heads,), torch.int32, "head_nnz")
    pl = [float(x) for x in (p if hasattr(p, "__len__") else [p])]
    parr = (ctypes.c_float * len(pl))(*pl)
    _check(lib().fva_select_pooled(plan.handle, parr, len(pl), int(k_min),
                                   SLACK[slack] if isinstance(slack, str) else int(slack), _ptr(scores_out),
                                   _ptr(row_ptr), _ptr(col_idx), _ptr(head_nnz), _stream(stream)))


def fva_select(plan: Plan, q_perm, k_perm, p, k_min, row_ptr, col_idx, slack="none", scores_in=None,
               scores_out=None, head_nnz=None, stream=None):
    d = plan.desc
    sq = (d.batch, d.heads, plan.n_blk, plan.n_blk)
    if scores_in is None:
        _expect(q_perm, plan.perm_shape(), plan.torch_dtype, "q_perm")
        _expect(k_perm, plan.perm_shape(), plan.torch_dtype, "k_perm")
    else:
        _expect(scores_in, sq, torch.float32, "scores_in")
    if scores_out is not None:
        _expect(scores_out, sq, torch.float32, "scores_out")
    _expect(row_ptr, (plan.n_rows + 1,), torch.int32, "row_ptr")
    if col_idx.dtype != torch.int32 or col_idx.numel() < plan.info.max_nnz:
        raise ValueError("col_idx must be int32 with capacity max_nnz")
    if head_nnz is not None:
        _expect(head_nnz, (d.batch * d.heads,), torch.int32, "head_nnz")
    pl = [float(x) for x in (p if hasattr(p, "__len__") else [p])]
    parr = (ctypes.c_float * len(pl))(*pl)
    _check(lib().fva_select(plan.handle, _ptr(q_perm) if q_perm is not None else None,
                            _ptr(k_perm) if k_perm is not None else None, parr, len(pl), int(k_min),
                            SLACK[slack] if isinstance(slack, str) else int(slack), _ptr(scores_in),
                            _ptr(scores_out), _ptr(row_ptr), _ptr(col_idx), _ptr(head_nnz), _stream(stream)))


def fva_attention(plan: Plan, q_perm, k_perm, vt_perm, row_ptr, col_idx, o_perm, sched="persistent",
                  wg_times=None, stream=None):
    for t, n in ((q_perm, "q_perm"), (k_perm, "k_perm"), (o_perm, "o_perm")):
        _expect(t, plan.perm_shape(), plan.torch_dtype, n)
    if vt_perm.numel() != o_perm.numel() or vt_perm.dtype != plan.torch_dtype:
        raise ValueError("vt_perm has the wrong size or dtype")
    _expect(row_ptr, (plan.n_rows + 1,), torch.int32, "row_ptr")
    if col_idx.dtype != torch.int32:
        raise ValueError("col_idx must be int32")
    if wg_times is not None and (wg_times.dtype != torch.int64 or wg_times.numel() < 2 * plan.info.max_wg):
        raise ValueError("wg_times must be int64 with 2*max_wg entries")
    _check(lib().fva_attention(plan.handle, _ptr(q_perm), _ptr(k_perm), _ptr(vt_perm), _ptr(row_ptr),
                               _ptr(col_idx), _ptr(o_perm), SCHED[sched] if isinstance(sched, str) else int(sched),
                               _ptr(wg_times), _stream(stream)))


def fva_attention_static(desc: fva_plan_desc, q_perm, k_perm, vt_perm, row_ptr, col_idx, o_perm, stream=None):
    """fva_attention without a plan and without any device allocation (the
    library's static scratch; tile order; persistent schedule)."""
    _check(lib().fva_attention_static(ctypes.byref(desc), _ptr(q_perm), _ptr(k_perm), _ptr(vt_perm),
                                      _ptr(row_ptr), _ptr(col_idx), _ptr(o_perm), _stream(stream)))


def fva_attention_raster(plan: Plan, q_perm, k_perm, vt_perm, row_ptr, col_idx, o_raster, sched="persistent",
                         stream=None):
    for t, n in ((q_perm, "q_perm"), (k_perm, "k_perm")):
        _expect(t, plan.perm_shape(), plan.torch_dtype, n)
    if vt_perm.numel() != q_perm.numel() or vt_perm.dtype != plan.torch_dtype:
        raise ValueError("vt_perm has the wrong size or dtype")
    _expect(o_raster, plan.raster_shape(), plan.torch_dtype, "o_raster")
    _expect(row_ptr, (plan.n_rows + 1,), torch.int32, "row_ptr")
    if col_idx.dtype != torch.int32:
        raise ValueError("col_idx must be int32")
    _check(lib().fva_attention_raster(plan.handle, _ptr(q_perm), _ptr(k_perm), _ptr(vt_perm), _ptr(row_ptr),
                                      _ptr(col_idx), _ptr(o_raster),
                                      SCHED[sched] if isinstance(sched, str) else int(sched), _stream(stream)))


def fva_attention_lse(plan: Plan, q_perm, k_perm, vt_perm, row_ptr, col_idx, o_perm, o32, lse, stream=None):
    for t, n in ((q_perm, "q_perm"), (k_perm, "k_perm"), (o_perm, "o_perm")):
        _expect(t, plan.perm_shape(), plan.torch_dtype, n)
    if vt_perm.numel() != o_perm.numel() or vt_perm.dtype != plan.torch_dtype:
        raise ValueError("vt_perm has the wrong size or dtype")
    _expect(row_ptr, (plan.n_rows + 1,), torch.int32, "row_ptr")
    _expect(lse, plan.perm_shape()[:3], torch.float32, "lse")
    _expect(o32, plan.perm_shape(), torch.float32, "o32")
    _check(lib().fva_attention_lse(plan.handle, _ptr(q_perm), _ptr(k_perm), _ptr(vt_perm), _ptr(row_ptr),
                                   _ptr(col_idx), _ptr(o_perm), _ptr(o32), _ptr(lse), _stream(stream)))


def fva_attention_backward(plan: Plan, q_perm, k_perm, v_perm, o32, lse, do_perm, do_vt,
                           row_ptr, col_idx, dq_perm, dk_perm, dv_perm, stream=None):
    shp = plan.perm_shape()
    for t, n in ((q_perm, "q_perm"), (k_perm, "k_perm"), (v_perm, "v_perm"),
                 (do_perm, "do_perm"), (do_vt, "do_vt"), (dq_perm, "dq_perm"),
                 (dk_perm, "dk_perm"), (dv_perm, "dv_perm")):
        if t.numel() != math.prod(shp) or t.dtype != plan.torch_dtype or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous {plan.torch_dtype} tensor of {math.prod(shp)} elements")
    _expect(o32, shp, torch.float32, "o32")
    _expect(lse, shp[:3], torch.float32, "lse")
    _expect(row_ptr, (plan.n_rows + 1,), torch.int32, "row_ptr")
    if col_idx.dtype != torch.int32:
        raise ValueError("col_idx must be int32")
    _check(lib().fva_attention_backward(plan.handle, _ptr(q_perm), _ptr(k_perm),
                                        _ptr(v_perm), _ptr(o32), _ptr(lse), _ptr(do_perm), _ptr(do_vt),
                                        _ptr(row_ptr), _ptr(col_idx), _ptr(dq_perm), _ptr(dk_perm), _ptr(dv_perm),
                                        _stream(stream)))


def fva_mask_transpose(plan: Plan, row_ptr, col_idx, t_row_ptr, t_col_idx, stream=None):
    _expect(row_ptr, (plan.n_rows + 1,), torch.int32, "row_ptr")
    _expect(t_row_ptr, (plan.n_rows + 1,), torch.int32, "t_row_ptr")
    if col_idx.dtype != torch.int32 or t_col_idx.dtype != torch.int32:
        raise ValueError("col_idx / t_col_idx must be int32")
    _check(lib().fva_mask_transpose(plan.handle, _ptr(row_ptr), _ptr(col_idx), _ptr(t_row_ptr), _ptr(t_col_idx),
                                    _stream(stream)))


class Buffers:
    """Device buffers for one full call on a plan (block-order Q/K/V^T/O,
    CSR lists, per-head counts), allocated once and reused."""

    def __init__(self, plan: Plan):
        dev = torch.device("cuda")
        shp = plan.perm_shape()
        self.q = torch.empty(shp, dtype=plan.torch_dtype, device=dev)
        self.k = torch.empty(shp, dtype=plan.torch_dtype, device=dev)
        self.vt = torch.empty(shp, dtype=plan.torch_dtype, device=dev)
        self.o = torch.empty(shp, dtype=plan.torch_dtype, device=dev)
        self.row_ptr = torch.empty(plan.n_rows + 1, dtype=torch.int32, device=dev)
        self.col_idx = torch.empty(plan.info.max_nnz, dtype=torch.int32, device=dev)
        self.head_nnz = torch.empty(plan.desc.batch * plan.desc.heads, dtype=torch.int32, device=dev)


def attention_call(plan: Plan, q, k, v, out, p, k_min, bufs: Buffers, slack="none", sched="persistent",
                   scores_out=None, wg_times=None, fused=False, stream=None):
    """One full attention call, raster in and raster out:
    permute(Q, K, V) -> select -> attention -> unpermute.  With fused=True
    the permutes of Q and K also pool (fva_permute_pool, fva_select_pooled)
    and the attention writes raster rows itself (fva_attention_raster; bufs.o
    is then not written, and wg_times is not available)."""
    if fused:
        fva_permute_pool(plan, q, bufs.q, "q", stream)
        fva_permute_pool(plan, k, bufs.k, "k", stream)
    else:
        fva_permute(plan, q, bufs.q, LAYOUT_ROWS, stream)
        fva_permute(plan, k, bufs.k, LAYOUT_ROWS, stream)
    fva_permute(plan, v, bufs.vt, LAYOUT_VT, stream)
    if fused:
        fva_select_pooled(plan, p, k_min, bufs.row_ptr, bufs.col_idx, slack=slack, scores_out=scores_out,
                          head_nnz=bufs.head_nnz, stream=stream)
    else:
        fva_select(plan, bufs.q, bufs.k, p, k_min, bufs.row_ptr, bufs.col_idx, slack=slack,
                   scores_out=scores_out, head_nnz=bufs.head_nnz, stream=stream)
    if fused:
        if wg_times is not None:
            raise ValueError("wg_times needs the unfused call")
        fva_attention_raster(plan, bufs.q, bufs.k, bufs.vt, bufs.row_ptr, bufs.col_idx, out, sched=sched,
                             stream=stream)
        return
    fva_attention(plan, bufs.q, bufs.k, bufs.vt, bufs.row_ptr, bufs.col_idx, bufs.o, sched=sched,
                  wg_times=wg_times, stream=stream)
    fva_unpermute(plan, bufs.o, out, stream)


class TrainBuffers:
    """Extra block-order buffers of a training call: V and dO in rows, dO in
    the VT layout, the fp32 output and per-query log-sum-exp of the forward
    pass, the gradients."""

    def __init__(self, plan: Plan):
        dev = torch.device("cuda")
        shp = plan.perm_shape()
        mk = lambda: torch.empty(shp, dtype=plan.torch_dtype, device=dev)
        self.v, self.do, self.do_vt = mk(), mk(), mk()
        self.dq, self.dk, self.dv = mk(), mk(), mk()
        self.lse = torch.empty(shp[:3], dtype=torch.float32, device=dev)
        self.o32 = torch.empty(shp, dtype=torch.float32, device=dev)


def attention_forward_train(plan: Plan, q, k, v, out, p, k_min, bufs: Buffers, tb: TrainBuffers, slack="none",
                            stream=None):
    """Forward pass of a training step: permute, select, attention with the
    per-query log-sum-exp kept for the backward pass, unpermute."""
    fva_permute(plan, q, bufs.q, LAYOUT_ROWS, stream)
    fva_permute(plan, k, bufs.k, LAYOUT_ROWS, stream)
    fva_permute(plan, v, bufs.vt, LAYOUT_VT, stream)
    fva_select(plan, bufs.q, bufs.k, p, k_min, bufs.row_ptr, bufs.col_idx, slack=slack, head_nnz=bufs.head_nnz,
               stream=stream)
    fva_attention_lse(plan, bufs.q, bufs.k, bufs.vt, bufs.row_ptr, bufs.col_idx, bufs.o, tb.o32, tb.lse, stream)
    fva_unpermute(plan, bufs.o, out, stream)


def attention_backward_call(plan: Plan, q, k, v, dout, dq, dk, dv, bufs: Buffers, tb: TrainBuffers, stream=None):
    """Backward pass after attention_forward_train on the same buffers:
    raster dO in, raster dQ, dK, dV out (same lists as the forward pass)."""
    fva_permute(plan, v, tb.v, LAYOUT_ROWS, stream)
    fva_permute(plan, dout, tb.do, LAYOUT_ROWS, stream)
    fva_permute(plan, dout, tb.do_vt, LAYOUT_VT, stream)
    fva_attention_backward(plan, bufs.q, bufs.k, tb.v, tb.o32, tb.lse, tb.do, tb.do_vt,
                           bufs.row_ptr, bufs.col_idx, tb.dq, tb.dk, tb.dv, stream)
    fva_unpermute(plan, tb.dq, dq, stream)
    fva_unpermute(plan, tb.dk, dk, stream)
    fva_unpermute(plan, tb.dv, dv, stream)
