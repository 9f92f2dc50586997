"""fva_attention_static, the entry point for callers that cannot allocate
device memory: through the C ABI, its output equals fva_attention's on a
plan of the same descriptor bit for bit, on two calls in a row (the second
on a smaller shape, so the shared static scratch holds the first call's
contents), and it rejects what it does not support before enqueuing."""
import numpy as np
import pytest
import torch

from block_sparse_spatiotemporal_amd import fva, synth
from tests._helpers import to_dev

pytestmark = pytest.mark.gpu


def _case(name, **changes):
    w = synth.scaled(synth.WORKLOADS[name], **changes) if changes else synth.WORKLOADS[name]
    q, k, v, meta = synth.make(w)
    plan = fva.Plan(w.B, w.H, w.D, w.grid, tile=w.tile, order=w.order, sub=w.sub, dtype=w.dtype)
    bufs = fva.Buffers(plan)
    out = torch.empty_like(to_dev(q, w.dtype))
    p = meta["p_head"].tolist() if isinstance(w.p, tuple) else float(meta["p_head"][0])
    fva.attention_call(plan, to_dev(q, w.dtype), to_dev(k, w.dtype), to_dev(v, w.dtype), out, p, w.k_min, bufs,
                       slack=w.slack)
    return w, plan, bufs


def _check(w, plan, bufs):
    ref = torch.full_like(bufs.o, 7.0)
    got = torch.full_like(bufs.o, -3.0)
    fva.fva_attention(plan, bufs.q, bufs.k, bufs.vt, bufs.row_ptr, bufs.col_idx, ref)
    fva.fva_attention_static(plan.desc, bufs.q, bufs.k, bufs.vt, bufs.row_ptr, bufs.col_idx, got)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got.view(torch.int32),
                       ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref.view(torch.int32))


def test_static_equals_plan_entry_two_calls_second_smaller():
    big = _case("wan14b_480p_cfg", B=1, H=6)       # 624 blocks, 6 heads
    small = _case("wan1.3b_480p", H=2, grid=(9, 10, 13))   # 27 blocks, 2 heads
    _check(*big)
    _check(*small)


def test_static_fp32_and_d64():
    _check(*_case("tiny_f32"))
    _check(*_case("wan1.3b_480p", H=3, D=64, grid=(5, 12, 11)))


def test_static_rejects_before_enqueue():
    w, plan, bufs = _case("wan1.3b_480p", H=1, grid=(4, 8, 8))
    hil = fva.make_desc(1, 1, 128, (4, 8, 8), order="hilbert")
    with pytest.raises(fva.FvaError) as e:
        fva.fva_attention_static(hil, bufs.q, bufs.k, bufs.vt, bufs.row_ptr, bufs.col_idx, bufs.o)
    assert e.value.code == fva.FVA_EUNSUPPORTED
    huge = fva.make_desc(8, 64, 128, (21, 45, 80))     # 737,280 rows: beyond the scratch
    with pytest.raises(fva.FvaError) as e:
        fva.fva_attention_static(huge, bufs.q, bufs.k, bufs.vt, bufs.row_ptr, bufs.col_idx, bufs.o)
    assert e.value.code == fva.FVA_EUNSUPPORTED and "scratch" in str(e.value)
