"""Benchmark one block-sparse attention call (raster Q, K, V -> raster O) on
one MI355X.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--sched persistent|plain] [--no-cpu] [--cpu-heads N] [--unfused]
  python bench.py --copy-probe MIB     # plain device copy of a known size,
                                       # the calibration run for HBM counters

A step is one whole call: permute Q, K, V -> select (pool, score, Top-p with
Top-k floor, CSR) -> block-sparse attention -> unpermute O, on one HIP stream
with the inputs already resident in HBM.  By default the permutes of Q and K
also pool (fva_permute_pool; fva_select_pooled then scores and selects) and
the attention writes O straight to raster order (fva_attention_raster: the
unpermute is its epilogue); with --unfused the same steps run as the six
separate calls fva_permute x3, fva_select, fva_attention, fva_unpermute.  Events recorded
on that stream between the stages of every timed step give the per-stage
times (the attention stage is one kernel launch after the small pairing and
scheduling kernels).
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 vector / matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E peak
ATTN_SOURCE = os.path.join(ROOT, "block_sparse_spatiotemporal_amd", "csrc", "attention.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wan14b_480p_cfg")
    ap.add_argument("--sched", default="persistent", choices=["persistent", "plain"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-backward", action="store_true", help="skip the training-step (backward) timing")
    ap.add_argument("--unfused", action="store_true",
                    help="separate pool (inside fva_select) and unpermute calls")
    ap.add_argument("--cpu-heads", type=int, default=4, help="(b,h) pairs in the CPU oracle sample")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (counter calibration)")
    return ap.parse_args()


def source_digest(path=ATTN_SOURCE):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per attention launch from the committed counter summary,
    if it was taken on the current attention source; else None."""
    path = os.path.join(ROOT, "profiles", f"k_attn_bf16_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_src = re.search(r"source_sha256_16:\s*([0-9a-f]+)", txt)
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not (m_src and m_b) or m_src.group(1) != source_digest():
        return None
    return float(m_b.group(1))


def cpu_baseline(w, q, k, v, n_heads, p_head, gpu_head_nnz, gpu_nnz):
    """The oracle, untuned, on a sample of n_heads (b, h) pairs of the same
    inputs, scaled to one whole call.

    The sample spans the call's range of per-head cost: heads are ranked by
    their kept-block count on the GPU lists and taken at evenly spaced
    quantiles.  Stages whose cost is the same for every head (permute, pool,
    score, select, unpermute) are scaled by the head count; the attention
    stage, whose cost follows the kept blocks, is scaled by the call's kept
    blocks over the sample's (the oracle's own count for the sampled heads)."""
    from block_sparse_spatiotemporal_amd import synth
    from oracle import fva_oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    host_cores = len(os.sched_getaffinity(0))
    all_pairs = [(b, h) for b in range(w.B) for h in range(w.H)]
    n_heads = max(1, min(n_heads, len(all_pairs)))
    ranked = np.argsort(np.asarray(gpu_head_nnz), kind="stable")
    picks = sorted({int(ranked[int((i + 0.5) * len(all_pairs) / n_heads)]) for i in range(n_heads)})
    pairs = [all_pairs[i] for i in picks]
    opl = O.plan(w.grid, tile=w.tile, order=w.order, sub=w.sub)
    t_head, t_attn, nnz_s = 0.0, 0.0, 0
    for b, h in pairs:
        sl = lambda a: synth.to_f64(a[b:b + 1, :, h:h + 1, :], w.dtype)
        qr, kr, vr = sl(q), sl(k), sl(v)
        t0 = time.perf_counter()
        qp, kp, vp = O.permute(qr, opl), O.permute(kr, opl), O.permute(vr, opl)
        qbar = O.pool(qp, opl)
        if opl.n_sub:
            kbs, empty = O.pool_sub(kp, opl)
            S = O.score_sub(qbar, kbs, empty)
        else:
            S = O.score(qbar, O.pool(kp, opl))
        rp, ci = O.select(S, float(p_head[h]), w.k_min)
        t1 = time.perf_counter()
        op = O.attention(qp, kp, vp, rp, ci, opl)
        t2 = time.perf_counter()
        O.unpermute(op, opl)
        t3 = time.perf_counter()
        t_head += (t1 - t0) + (t3 - t2)
        t_attn += t2 - t1
        nnz_s += int(rp[-1])
    s_head = len(all_pairs) / len(pairs)
    s_attn = gpu_nnz / max(nnz_s, 1)
    total = t_head * s_head + t_attn * s_attn
    return {"value": round(total * 1e3, 1), "unit": "ms/call", "cores": int(blas_threads),
            "host_cores": host_cores, "blas_threads": int(blas_threads), "kind": "oracle",
            "sample": f"{len(pairs)} of {len(all_pairs)} (b,h) heads of the same inputs at evenly spaced "
                      f"quantiles of per-head kept blocks ({nnz_s} of {gpu_nnz} kept blocks), full path "
                      f"(plan, permute, pool, score, select, attention, unpermute; no slack fill): "
                      f"per-head stages {t_head:.1f} s scaled x{s_head:g} by heads, attention "
                      f"{t_attn:.1f} s scaled x{s_attn:.2f} by kept blocks"}


def reuse_drift(w, plan, bufs, qd, kd, vd, out, p, sched, steps=4, step_std=0.1):
    """What reusing a selection costs in output: steps 1..steps of a seeded
    random walk on Q, K, V (N(0, step * step_std^2) added per element, torch's
    generator seeded with the workload seed, re-rounded to the input dtype);
    at each step the step-0 lists are reused and compared with a fresh
    selection: Jaccard ratio of the kept (I, J) pairs over all heads, and the
    max / mean absolute change of the output.  Overwrites bufs and out."""
    import torch
    from block_sparse_spatiotemporal_amd import fva
    rp0, ci0 = bufs.row_ptr.clone(), bufs.col_idx.clone()
    fresh, cached = torch.empty_like(out), torch.empty_like(out)
    counts = torch.empty(w.B * w.H, 2, dtype=torch.int64, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed)
    res = []
    for step in range(1, steps + 1):
        sd = step_std * float(np.sqrt(step))
        x = [(t.float() + sd * torch.randn(t.shape, generator=gen, device="cuda")).to(t.dtype) for t in (qd, kd, vd)]
        fva.attention_call(plan, x[0], x[1], x[2], fresh, p, w.k_min, bufs, slack=w.slack, sched=sched, fused=True)
        fva.fva_attention_raster(plan, bufs.q, bufs.k, bufs.vt, rp0, ci0, cached, sched=sched)
        fva.fva_mask_overlap(plan, rp0, ci0, bufs.row_ptr, bufs.col_idx, counts)
        torch.cuda.synchronize()
        c = counts.sum(dim=0).tolist()
        d = (cached.float() - fresh.float()).abs()
        res.append({"step": step, "drift_std": round(sd, 4), "jaccard": round(c[0] / c[1], 4),
                    "max_abs_out_change": round(d.max().item(), 5),
                    "mean_abs_out_change": round(d.mean().item(), 6)})
        del x, d
    return res


def copy_probe(mib, steps):
    import torch
    n = mib * (1 << 20)
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": steps}), flush=True)


def cu_idle(wg):
    """From per-workgroup (start, end) stamps of a persistent launch: idle
    fraction of the launch's workgroup slots over the kernel span, and
    max / mean slot load."""
    wg = wg.reshape(-1, 2).astype(np.int64)
    wg = wg[wg[:, 1] > 0]
    busy = wg[:, 1] - wg[:, 0]
    span = wg[:, 1].max() - wg[:, 0].min()
    return {"slots": int(len(wg)), "idle_frac": round(1.0 - busy.sum() / (len(wg) * span), 4),
            "max_over_mean_load": round(float(busy.max() / busy.mean()), 3)}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; multi-GPU sharding is a design note, "
                                   "not implemented", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    from block_sparse_spatiotemporal_amd import fva, synth

    if args.copy_probe:
        copy_probe(args.copy_probe, args.steps)
        return

    w = synth.WORKLOADS[args.workload]
    q, k, v, meta = synth.make(w)
    dev = (lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()) if w.dtype == "bf16" \
        else (lambda a: torch.from_numpy(a).cuda())
    qd, kd, vd = dev(q), dev(k), dev(v)
    plan = fva.Plan(w.B, w.H, w.D, w.grid, tile=w.tile, order=w.order, sub=w.sub, dtype=w.dtype)
    bufs = fva.Buffers(plan)
    out = torch.empty_like(qd)
    p_head = meta["p_head"]
    p = p_head.tolist() if isinstance(w.p, tuple) else float(p_head[0])

    names = ["permute_q", "permute_k", "permute_v", "select", "attention"] + (["unpermute"] if args.unfused else [])

    def call(ev=None):
        # the C-ABI calls of fva.attention_call, with events between them
        rec = (lambda i: ev[i].record()) if ev else (lambda i: None)
        rec(0)
        if args.unfused:
            fva.fva_permute(plan, qd, bufs.q, fva.LAYOUT_ROWS); rec(1)
            fva.fva_permute(plan, kd, bufs.k, fva.LAYOUT_ROWS); rec(2)
        else:
            fva.fva_permute_pool(plan, qd, bufs.q, "q"); rec(1)
            fva.fva_permute_pool(plan, kd, bufs.k, "k"); rec(2)
        fva.fva_permute(plan, vd, bufs.vt, fva.LAYOUT_VT); rec(3)
        if args.unfused:
            fva.fva_select(plan, bufs.q, bufs.k, p, w.k_min, bufs.row_ptr, bufs.col_idx, slack=w.slack,
                           head_nnz=bufs.head_nnz); rec(4)
        else:
            fva.fva_select_pooled(plan, p, w.k_min, bufs.row_ptr, bufs.col_idx, slack=w.slack,
                                  head_nnz=bufs.head_nnz); rec(4)
        if args.unfused:
            fva.fva_attention(plan, bufs.q, bufs.k, bufs.vt, bufs.row_ptr, bufs.col_idx, bufs.o,
                              sched=args.sched); rec(5)
            fva.fva_unpermute(plan, bufs.o, out); rec(6)
        else:
            fva.fva_attention_raster(plan, bufs.q, bufs.k, bufs.vt, bufs.row_ptr, bufs.col_idx, out,
                                     sched=args.sched); rec(5)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()

    # exactly `steps` timed calls; events on the launch stream between stages
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        call(evs[i])
    torch.cuda.synchronize()
    ms_call = evs[0][0].elapsed_time(evs[-1][len(names)]) / args.steps
    stage = {n: np.array([e[j].elapsed_time(e[j + 1]) for e in evs]) for j, n in enumerate(names)}
    st_mean = {n: float(x.mean()) for n, x in stage.items()}
    st_med = {n: float(np.median(x)) for n, x in stage.items()}
    per_call = np.array([e[0].elapsed_time(e[len(names)]) for e in evs])

    # cold caches: a 512 MB scratch write (twice the 256 MB Infinity Cache,
    # far above the L2s) between calls, each call timed on its own
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    cold = []
    for i in range(min(args.steps, 10)):
        scratch.fill_(i & 0xFF)
        ec = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
        call(ec)
        torch.cuda.synchronize()
        cold.append(ec[0].elapsed_time(ec[len(names)]))
    del scratch

    # the same call captured once in a HIP graph and replayed (fused form only)
    graph_ms = None
    if not args.unfused:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            call()
        torch.cuda.synchronize()
        e_g0, e_g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e_g0.record()
        for _ in range(args.steps):
            graph.replay()
        e_g1.record()
        torch.cuda.synchronize()
        graph_ms = e_g0.elapsed_time(e_g1) / args.steps
        del graph

    # the fused permute + 3D rotary encoding (outside the attention call),
    # timed alone on Q of the same workload
    e_r0, e_r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e_r0.record()
    for _ in range(args.steps):
        fva.fva_permute_rope(plan, qd, bufs.q, t_offset=3)
    e_r1.record()
    torch.cuda.synchronize()
    rope_ms = e_r0.elapsed_time(e_r1) / args.steps

    # a call that reuses the cached selection (no fva_select) and the cost of
    # deciding to: the overlap of two selections
    def call_reuse():
        fva.fva_permute(plan, qd, bufs.q, fva.LAYOUT_ROWS)
        fva.fva_permute(plan, kd, bufs.k, fva.LAYOUT_ROWS)
        fva.fva_permute(plan, vd, bufs.vt, fva.LAYOUT_VT)
        fva.fva_attention_raster(plan, bufs.q, bufs.k, bufs.vt, bufs.row_ptr, bufs.col_idx, out, sched=args.sched)
    counts = torch.empty(w.B * w.H, 2, dtype=torch.int64, device="cuda")
    e_u0, e_u1, e_u2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    e_u0.record()
    for _ in range(args.steps):
        call_reuse()
    e_u1.record()
    for _ in range(args.steps):
        fva.fva_mask_overlap(plan, bufs.row_ptr, bufs.col_idx, bufs.row_ptr, bufs.col_idx, counts)
    e_u2.record()
    torch.cuda.synchronize()
    reuse_ms = e_u0.elapsed_time(e_u1) / args.steps
    overlap_ms = e_u1.elapsed_time(e_u2) / args.steps

    # one extra, untimed call with per-workgroup stamps for the load balance
    wg = torch.zeros(2 * plan.info.max_wg, dtype=torch.int64, device="cuda")
    fva.fva_attention(plan, bufs.q, bufs.k, bufs.vt, bufs.row_ptr, bufs.col_idx, bufs.o, sched=args.sched,
                      wg_times=wg)
    torch.cuda.synchronize()
    balance = cu_idle(wg.cpu().numpy().view(np.uint64)) if args.sched == "persistent" else None

    # training step on the same inputs and lists: the forward pass that keeps
    # lse and the fp32 output, then the backward kernels alone and the whole
    # raster-in / raster-out backward call
    backward = None
    if w.dtype == "bf16" and not args.no_backward:
        dod = dev(synth.make_dout(w))
        tb = fva.TrainBuffers(plan)
        dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
        fva.attention_forward_train(plan, qd, kd, vd, out, p, w.k_min, bufs, tb, slack=w.slack)
        fva.attention_backward_call(plan, qd, kd, vd, dod, dq, dk, dv, bufs, tb)
        torch.cuda.synchronize()
        e_b = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e_b[0].record()
        for _ in range(args.steps):
            fva.fva_attention_lse(plan, bufs.q, bufs.k, bufs.vt, bufs.row_ptr, bufs.col_idx, bufs.o, tb.o32, tb.lse)
        e_b[1].record()
        for _ in range(args.steps):
            fva.fva_attention_backward(plan, bufs.q, bufs.k, tb.v, tb.o32, tb.lse, tb.do, tb.do_vt,
                                       bufs.row_ptr, bufs.col_idx, tb.dq, tb.dk, tb.dv)
        e_b[2].record()
        for _ in range(args.steps):
            fva.attention_backward_call(plan, qd, kd, vd, dod, dq, dk, dv, bufs, tb)
        e_b[3].record()
        torch.cuda.synchronize()
        lse_ms, bwd_ms, bwd_call_ms = (e_b[i].elapsed_time(e_b[i + 1]) / args.steps for i in range(3))
        nnz_b = int(bufs.row_ptr[-1].item())
        # standard count: S recomputed, dP, dQ, dK, dV (five 64x64xD products per block pair)
        bflop = nnz_b * 5 * 2.0 * 64 * 64 * w.D
        backward = {"attention_lse_ms": round(lse_ms, 4), "backward_kernels_ms": round(bwd_ms, 4),
                    "backward_call_ms": round(bwd_call_ms, 4),
                    "backward_tflops": round(bflop / (bwd_ms * 1e-3) / 1e12, 2),
                    "frac_bf16_peak": round(bflop / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                    "flop_count": "5 products of 64x64xD per listed block pair"}
        del dod, tb, dq, dk, dv
        torch.cuda.empty_cache()

    nnz = int(bufs.row_ptr[-1].item())
    head_nnz = bufs.head_nnz.cpu().numpy()
    n_blk = plan.n_blk
    # FLOPs per kept block pair: S = Q K^T and O += P V over 64 queries and
    # 64 keys (4*64*64*D), the work counted with the pad tokens of a kept
    # block included.  The kernel steps over 32-key halves and skips a half
    # whose 32 keys are all padding, so the executed count, which the
    # roofline uses, takes 4*64*32*D per non-empty half of each kept block.
    sparse_flop = nnz * 4.0 * 64 * 64 * w.D
    _, _, bmask, _ = fva.fva_plan_tables(plan.desc)
    halves = ((bmask & np.uint64(0xFFFFFFFF)) != 0).astype(np.int64) + ((bmask >> np.uint64(32)) != 0)
    col = bufs.col_idx[:nnz].cpu().numpy()
    exec_flop = float(halves[col].sum()) * 4.0 * 64 * 32 * w.D
    dense_flop = 4.0 * w.B * w.H * float(w.n_tokens) ** 2 * w.D
    attn_tflops = exec_flop / (st_mean["attention"] * 1e-3) / 1e12
    attn_tflops_padded = sparse_flop / (st_mean["attention"] * 1e-3) / 1e12
    dens = head_nnz / float(n_blk * n_blk)

    # algorithmic bytes of the HBM-bound stages (valid rows at the element size)
    es = 2 if w.dtype == "bf16" else 4
    BH, N, row = w.B * w.H, w.n_tokens, w.D * es
    perm_bytes = BH * (N * row + plan.n_pad * row)        # read valid rows, write every padded row
    unperm_bytes = BH * 2 * N * row
    n_kbar = n_blk * (8 if w.sub[0] else 1)
    sel_bytes = ((2 * BH * N * row if args.unfused else 0)  # pool reads Q and K once (unless fused)
                 + BH * (n_blk + n_kbar) * w.D * 8          # pooled Q, K written (fp64)
                 + BH * n_blk * n_blk * 4                   # fp32 scores, one pass
                 + 4 * nnz + 4 * (plan.n_rows + 1))         # CSR out
    traffic = measured_traffic(w.name)

    res = {
        "metric": "ms/attn call + dense-equiv TFLOPS & MFMA util %, 32760-tok 40-head bf16 at p=0.9",
        "value": round(ms_call, 4),
        "unit": "ms/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_call, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded smooth Gaussian-filtered fields shaped like Wan 480P/720P latents)",
        "config": {"workload": w.name, "batch": w.B, "heads": w.H, "head_dim": w.D, "tokens": w.n_tokens,
                   "grid": list(w.grid), "tile": list(w.tile), "order": w.order, "sub": list(w.sub),
                   "p": w.p if not isinstance(w.p, tuple) else list(w.p), "k_min": w.k_min, "slack": w.slack,
                   "sched": args.sched},
        "dense_equiv_tflops": round(dense_flop / (ms_call * 1e-3) / 1e12, 2),
        "attention_sparse_tflops": round(attn_tflops, 2),
        "mfma_util_pct": round(100.0 * attn_tflops / PEAK_BF16_TFLOPS, 2),
        "executed_tflop_per_call": round(exec_flop / 1e12, 3),
        "sparse_tflop_per_call": round(sparse_flop / 1e12, 3),
        "mfma_util_padded_blocks_pct": round(100.0 * attn_tflops_padded / PEAK_BF16_TFLOPS, 2),
        "flop_count": "mfma_util and roofline: 4*64*32*D per non-empty 32-key half of each kept block "
                      "(executed); *_padded_blocks: 4*64*64*D per kept block",
        "nnz_blocks": nnz,
        "density": {"mean": round(float(dens.mean()), 4), "min": round(float(dens.min()), 4),
                    "max": round(float(dens.max()), 4)},
        "stage_ms_mean": {n: round(x, 4) for n, x in st_mean.items()},
        "stage_ms_median": {n: round(x, 4) for n, x in st_med.items()},
        "call_ms": {"median": round(float(np.median(per_call)), 4), "min": round(float(per_call.min()), 4),
                    "p90": round(float(np.percentile(per_call, 90)), 4)},
        "cold_cache_call_ms": {"median": round(float(np.median(cold)), 4), "min": round(float(np.min(cold)), 4),
                               "calls": len(cold), "scratch_mb_between_calls": 512},
        "core_ms": round(st_mean["select"] + st_mean["attention"], 4),
        "graph_ms_per_call": round(graph_ms, 4) if graph_ms is not None else None,
        "hbm_gbs": {"permute_rows": round(perm_bytes / (st_mean["permute_q"] * 1e-3) / 1e9, 1),
                    "permute_vt": round(perm_bytes / (st_mean["permute_v"] * 1e-3) / 1e9, 1),
                    "select": round(sel_bytes / (st_mean["select"] * 1e-3) / 1e9, 1),
                    **({"unpermute": round(unperm_bytes / (st_mean["unpermute"] * 1e-3) / 1e9, 1)}
                       if args.unfused else {}),
                    "peak": PEAK_HBM_GBS},
        "load_balance": balance,
        "permute_rope_ms": round(rope_ms, 4),
        "reuse": {"ms_per_call_cached_selection": round(reuse_ms, 4), "mask_overlap_ms": round(overlap_ms, 4)},
        "permute_rope_gbs": round(perm_bytes / (rope_ms * 1e-3) / 1e9, 1),
        "training": backward,
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "kernel": "k_attn_bf16 (" + ("fva_attention" if args.unfused else "fva_attention_raster") + ")",
                     "launch_ms": round(st_mean["attention"], 4)},
    }
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_heads, p_head, head_nnz, nnz)
    res["reuse"]["drift"] = reuse_drift(w, plan, bufs, qd, kd, vd, out, p, args.sched)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
