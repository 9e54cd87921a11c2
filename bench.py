#!/usr/bin/env python3
"""Throughput of the neighbour-graph attention hot path on one MI355X.

One step = nl_build (cell-list neighbour rows) + edge_csr (destination CSR) +
block_attn_forward (all attention layers), every input resident in HBM, all
on torch's current stream, no host synchronisation inside the step.  The
workload defaults to the largest one: Fe BCC, 37^3 cubic cells with 5% of
the sites removed (96,241 atoms), rcut 8 A, sel 181, 64 fp32 channels,
4 heads, 2 layers -- the 101,306-site lattice of the deepmd-kit DPA4 issue's
largest run.  Atoms/s = N / step time.

Timing follows the DPA4 issue's protocol (warm-up steps, then timed steps;
20 and 100 by default) with HIP events around every call on the stream the
library launches on; the median and the 10%-trimmed mean (the mlipaudit
page's outlier trimming) are reported per call and per step next to the
wall-clock mean that gives `value`.

Prints one JSON line with the value, a roofline entry for the dominant
kernel (live HIP-event timing of its launches) and the CPU oracle timed on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "atoms/s for NL build + block-dense neighbour attention fwd; % of roofline"
PEAK_TFLOPS = {"f32": 157.3, "f64": 78.6, "f16": 2500.0}   # MI355X dense MFMA peaks
# The f16 split-pair arithmetic (NGA_F32_SPLIT16) runs every contraction on the f16 matrix
# cores as (hi, lo) f16 pairs: four f16 products per fp32 multiply-add.
SPLIT_F16_FACTOR = 4.0
PEAK_HBM_GBS = 8000.0                        # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=5, help="workload key (1..5), default 5")
    ap.add_argument("--split16", action="store_true",
                    help="also time the NGA_F32_SPLIT16 arithmetic (f16 hi/lo pairs) on the same "
                         "inputs and report its time and its difference from the fp32 output")
    ap.add_argument("--no-gather-scatter", action="store_true",
                    help="skip the standalone block_gather / block_scatter leg (the padded "
                         "per-centre block of the workload's features and its scatter back, "
                         "timed after the steps)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--pair-axis", action="store_true",
                    help="also time pair_attn_forward (the ragged pair-axis route) on the same "
                         "inputs, after the timed steps, and report it beside the block-dense "
                         "forward")
    ap.add_argument("--pair-steps", type=int, default=2)
    ap.add_argument("--pair-chunk", type=int, default=1 << 26,
                    help="pairs per chunk of the pair-axis route")
    ap.add_argument("--smooth", action="store_true",
                    help="also time block_attn_forward_smooth (per-segment softmax rescale, "
                         "ln D~ = ln n_i + 1.5) on the same inputs, after the timed steps")
    ap.add_argument("--local-atten", action="store_true",
                    help="also time local_attn_forward (LocalAtten: one query per centre over "
                         "its edges, random centre rows) on the same CSR and edge features")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured as one HIP graph (nga_step_graph_*) on "
                         "the same inputs, replayed --steps times")
    ap.add_argument("--nl-reuse", action="store_true",
                    help="also time neighbour-list reuse: candidate rows at rcut + skin once, "
                         "then nl_refine and nl_max_displacement per step")
    ap.add_argument("--skin", type=float, default=1.0)
    ap.add_argument("--nl-batch", type=int, default=0,
                    help="also time nl_build_batch over this many jittered copies of the "
                         "workload's structure against as many separate nl_build calls")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB "
                         "(reference kernel for HBM counter scaling)")
    return ap.parse_args()


def source_digest(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def attention_sources(variant: str):
    base = "neighbour_graph_attention_amd/csrc/"
    if variant == "fused_f32":
        return [base + "block_attn_f32.hip", base + "block_attn_fused.h"]
    if variant == "fused_f32_split16":
        return [base + "block_attn_fused.hip", base + "block_attn_fused.h"]
    if variant == "fused_f64":
        return [base + "block_attn_f64_fused.hip", base + "block_attn_f64.h"]
    if variant == "mfma_f64":
        return [base + "block_attn_f64.hip", base + "block_attn_f64.h"]
    return [base + "block_attn.hip", base + "gemm_rows.h"]


def load_traffic(variant: str, workload: str):
    """Measured HBM bytes per launch of the attention kernel, if the committed counter summary
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{variant}.{workload}.traffic.json")
    if not os.path.exists(path):
        return None
    doc = json.load(open(path))
    if doc.get("source_sha256") != source_digest(attention_sources(variant)):
        return None
    return float(doc["hbm_bytes_per_launch"])


NL_SOURCES = ["neighbour_graph_attention_amd/csrc/nl_build.hip",
              "neighbour_graph_attention_amd/csrc/scan.hip"]


def load_nl_traffic(workload: str):
    """Measured HBM bytes of one nl_build call (all its kernels), if the committed counter
    summary was taken on the current source; else None."""
    path = os.path.join(ROOT, "profiles", f"nl_build.{workload}.traffic.json")
    if not os.path.exists(path):
        return None
    doc = json.load(open(path))
    if doc.get("source_sha256") != source_digest(NL_SOURCES):
        return None
    return float(doc["hbm_bytes_per_call"])


def cpu_baseline(w, pos, box, rp, x, wt, target_s):
    """The oracle (brute-force rows + naive attention through every layer) on sampled centres."""
    import oracle

    n = pos.shape[0]
    rng = np.random.default_rng(4242)

    def run(m):
        centres = np.sort(rng.choice(n, m, replace=False))
        t0 = time.perf_counter()
        srp, scol, sshift, svec = oracle.nl_rows(pos, box, w.rcut, w.sel, centres)
        xs = np.concatenate([x[rp[i]:rp[i + 1]] for i in centres]).astype(np.float64)
        oracle.attn_naive(srp, xs, wt.astype(np.float64), w.heads)
        return time.perf_counter() - t0

    m0 = min(n, 256)
    t0 = run(m0)
    m = int(min(n, max(m0, m0 * target_s / max(t0, 1e-6))))
    t = run(m)
    return {"value": m / t, "unit": "atoms/s", "cores": oracle.num_threads(), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{m} random centres of {n}: brute-force rows over all atoms and images, "
                      f"then naive attention through {w.layers} layer(s); {t:.1f} s wall"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def robust(ms) -> dict:
    """Mean, median and 10%-trimmed mean (10% cut at each end) of per-call times in ms."""
    a = np.sort(np.asarray(ms, dtype=np.float64))
    k = int(0.1 * a.size)
    trimmed = a[k:a.size - k] if a.size - 2 * k > 0 else a
    return {"mean": float(a.mean()), "median": float(np.median(a)),
            "trimmed_mean_10": float(trimmed.mean()), "min": float(a[0]), "max": float(a[-1])}


def time_pair_axis(nga, torch, dev, stream, row_ptr, x, wt, w, rp, steps, chunk, y_block,
                   attn_ms):
    """The ragged pair-axis route on the same CSR and inputs: one untimed pass, then `steps`
    timed passes (HIP events on the current stream; each pass synchronises once itself to
    plan its chunks, so the events bracket exactly one forward)."""
    counts = np.diff(rp)
    pairs = int(np.sum(counts.astype(np.int64) ** 2))
    # No chunk larger than the whole pair axis (the per-pair buffers are sized by the chunk).
    chunk = int(min(chunk, max(pairs, int(np.max(counts.astype(np.int64) ** 2)), 1)))
    n_chunks, acc = 0, 0
    for c2 in (counts.astype(np.int64) ** 2):
        if acc + c2 > chunk:
            n_chunks, acc = n_chunks + 1, 0
        acc += c2
    n_chunks += 1 if acc > 0 else 0
    ws = nga.Workspace(dev, nga.pair_attn_workspace_bytes(
        nga.NGA_F64 if w.dtype == "f64" else nga.NGA_F32, rp.shape[0] - 1, x.shape[0], w.c,
        w.heads, w.layers, chunk))
    yp = torch.empty_like(x)
    nga.pair_attn_forward(row_ptr, x, wt, w.heads, pair_chunk=chunk, y=yp, ws=ws)
    nga.check_status(ws, "pair_attn_forward")
    times = []
    for _ in range(steps):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        nga.pair_attn_forward(row_ptr, x, wt, w.heads, pair_chunk=chunk, y=yp, ws=ws)
        ev1.record(stream)
        torch.cuda.synchronize(dev)
        times.append(ev0.elapsed_time(ev1))
    nga.check_status(ws, "pair_attn_forward")
    diff = float((yp - y_block).abs().max() / y_block.abs().max())
    ms = float(np.mean(times))
    es = 8 if w.dtype == "f64" else 4
    return {"ms_per_forward": ms, "pairs": pairs, "pair_chunk": chunk, "chunks": n_chunks,
            "pair_tensor_bytes": pairs * w.c * es,
            "workspace_bytes": ws.nbytes, "vs_block_attn_forward": ms / attn_ms,
            "normwise_diff_vs_block": diff, "steps": steps}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only; --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import neighbour_graph_attention_amd as nga
    import workloads as W

    dev = torch.device("cuda:0")
    w = W.WORKLOADS[args.workload]
    pos_np, box = W.workload_positions(w)
    n = pos_np.shape[0]
    pos = torch.from_numpy(pos_np).to(dev)

    # Buffers and workspaces, allocated once.
    nbr = torch.empty((n, w.sel), dtype=torch.int32, device=dev)
    nbr_shift = torch.empty((n, w.sel, 3), dtype=torch.int32, device=dev)
    nnei = torch.empty((n,), dtype=torch.int32, device=dev)
    e_cap = n * w.sel
    csr_out = {
        "row_ptr": torch.empty((n + 1,), dtype=torch.int64, device=dev),
        "col": torch.empty((e_cap,), dtype=torch.int32, device=dev),
        "shift": torch.empty((e_cap, 3), dtype=torch.int32, device=dev),
        "dst": torch.empty((e_cap,), dtype=torch.int32, device=dev),
    }
    ws_nl = nga.Workspace(dev, nga.nl_build_workspace_bytes(n, box, w.rcut))
    ws_csr = nga.Workspace(dev)

    # One untimed pass reads E back (the only host synchronisation of the run).
    nga.nl_build(pos, box, w.rcut, w.sel, nbr=nbr, nbr_shift=nbr_shift, nnei=nnei, ws=ws_nl)
    first = nga.edge_csr(nbr, nbr_shift, nnei, out=csr_out, ws=ws_csr)
    nga.check_status(ws_nl, "nl_build")
    e = first["n_edges"]
    rp = csr_out["row_ptr"].cpu().numpy()

    x_np = W.workload_features(w, e)
    wt_np = W.workload_weights(w)
    x = torch.from_numpy(x_np).to(dev)
    wt = torch.from_numpy(wt_np).to(dev)
    y = torch.empty_like(x)
    dtype_code = nga.NGA_F64 if w.dtype == "f64" else nga.NGA_F32
    variant = nga.attn_variant(dtype_code, w.sel, w.c, w.heads)
    ws_attn = nga.Workspace(dev, nga.block_attn_workspace_bytes(dtype_code, e, w.sel, w.c,
                                                                w.heads, w.layers))
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        nga.nl_build(pos, box, w.rcut, w.sel, nbr=nbr, nbr_shift=nbr_shift, nnei=nnei, ws=ws_nl)
        if ev is not None:
            ev[1].record(stream)
        nga.edge_csr(nbr, nbr_shift, nnei, e_cap=e_cap, read_n_edges=False, out=csr_out,
                     ws=ws_csr)
        if ev is not None:
            ev[2].record(stream)
        nga.block_attn_forward(csr_out["row_ptr"], x, wt, w.heads, w.sel, y=y, ws=ws_attn)
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize(dev)
    t1 = time.perf_counter()
    for ws, name in ((ws_nl, "nl_build"), (ws_csr, "edge_csr"), (ws_attn, "block_attn_forward")):
        nga.check_status(ws, name)
    if not bool(torch.isfinite(y).all()):
        raise RuntimeError("non-finite attention output")

    ms_step = (t1 - t0) * 1e3 / args.steps
    part = np.array([[ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2]),
                      ev[2].elapsed_time(ev[3])] for ev in events])
    nl_ms, csr_ms, attn_ms = (float(v) for v in part.mean(axis=0))
    # Per step on the GPU clock: from the step's first call to the end of its last.
    step_gpu = [ev[0].elapsed_time(ev[3]) for ev in events]
    timing = {"protocol": f"{args.warmup} warm-up steps, then {args.steps} timed steps; HIP "
                          "events around every call on the library's stream",
              "step_ms": robust(step_gpu), "nl_build_ms": robust(part[:, 0]),
              "edge_csr_ms": robust(part[:, 1]), "block_attn_forward_ms": robust(part[:, 2])}

    batch_rec = None
    if args.nl_batch > 0:
        nb = args.nl_batch
        rng_b = np.random.default_rng(800)
        copies = [W.wrap_into_box(pos_np + rng_b.normal(0.0, 0.02, pos_np.shape), box)
                  for _ in range(nb)]
        pos_b = torch.from_numpy(np.concatenate(copies)).to(dev)
        atom_ptr = [k * n for k in range(nb + 1)]
        boxes = [box] * nb
        ws_b = nga.Workspace(dev)
        nbr_b = torch.empty((nb * n, w.sel), dtype=torch.int32, device=dev)
        nsh_b = torch.empty((nb * n, w.sel, 3), dtype=torch.int32, device=dev)
        nn_b = torch.empty((nb * n,), dtype=torch.int32, device=dev)
        singles = [torch.from_numpy(cp).to(dev) for cp in copies]
        ws_s = [nga.Workspace(dev, nga.nl_build_workspace_bytes(n, box, w.rcut)) for _ in range(nb)]
        out_s = [(nbr_b[k * n:(k + 1) * n], nsh_b[k * n:(k + 1) * n], nn_b[k * n:(k + 1) * n])
                 for k in range(nb)]

        def batched():
            nga.nl_build_batch(pos_b, atom_ptr, boxes, w.rcut, w.sel, nbr=nbr_b, nbr_shift=nsh_b,
                               nnei=nn_b, ws=ws_b)

        def separate():
            for k in range(nb):
                nga.nl_build(singles[k], box, w.rcut, w.sel, nbr=out_s[k][0], nbr_shift=out_s[k][1],
                             nnei=out_s[k][2], ws=ws_s[k])

        def wall(fn, k):
            for _ in range(2):
                fn()
            torch.cuda.synchronize(dev)
            t0b = time.perf_counter()
            for _ in range(k):
                fn()
            torch.cuda.synchronize(dev)
            return (time.perf_counter() - t0b) * 1e3 / k

        kb = max(3, args.steps // 5)
        b_ms, s_ms = wall(batched, kb), wall(separate, kb)
        nga.check_status(ws_b, "nl_build_batch")
        batch_rec = {"structures": nb, "atoms_each": n, "batched_ms": b_ms,
                     "separate_ms": s_ms, "speedup": s_ms / b_ms,
                     "note": "wall time per call sequence; the batched call synchronises once "
                             "to upload its structure table"}

    reuse_rec = None
    if args.nl_reuse:
        cand_sel = 512
        ws_cand = nga.Workspace(dev, nga.nl_build_workspace_bytes(n, box, w.rcut + args.skin))
        ws_ref = nga.Workspace(dev)
        cands = nga.nl_build(pos, box, w.rcut + args.skin, cand_sel, ws=ws_cand)
        nga.check_status(ws_cand, "nl_build (candidates)")
        if int(cands[2].max().item()) >= cand_sel:
            raise RuntimeError("candidate rows reach their capacity; lower --skin")
        dmax = torch.empty((1,), dtype=torch.float64, device=dev)
        pos_ref = pos.clone()

        def timed(fn, k):
            for _ in range(args.warmup):
                fn()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(k)]
            for e0, e1 in evs:
                e0.record(stream)
                fn()
                e1.record(stream)
            torch.cuda.synchronize(dev)
            return float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))

        cand_ms = timed(lambda: nga.nl_build(pos, box, w.rcut + args.skin, cand_sel, nbr=cands[0],
                                             nbr_shift=cands[1], nnei=cands[2], ws=ws_cand),
                        max(3, args.steps // 5))
        refine_ms = timed(lambda: nga.nl_refine(pos, box, w.rcut, w.sel, cands[0], cands[1],
                                                cands[2], box, nbr=nbr, nbr_shift=nbr_shift,
                                                nnei=nnei, ws=ws_ref), args.steps)
        disp_ms = timed(lambda: nga.nl_max_displacement(pos, pos_ref, box, out=dmax), args.steps)
        nga.check_status(ws_ref, "nl_refine")
        reuse_rec = {"skin": args.skin, "candidate_rows": cand_sel,
                     "candidate_build_ms": cand_ms, "refine_ms": refine_ms,
                     "max_displacement_ms": disp_ms, "nl_build_ms": nl_ms,
                     "refine_vs_build": refine_ms / nl_ms}

    graph_rec = None
    if args.graph:
        x_cap = torch.zeros((e_cap, w.c), dtype=x.dtype, device=dev)
        x_cap[:e] = x
        g = nga.StepGraph(pos, box, w.rcut, w.sel, x_cap, wt, w.heads)
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize(dev)
        g.check()
        tg0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize(dev)
        tg1 = time.perf_counter()
        g.check()
        if not torch.equal(g.y[:e], y[:e]):
            raise RuntimeError("graph replay differs from the eager step")
        g_ms = (tg1 - tg0) * 1e3 / args.steps
        graph_rec = {"ms_per_step": g_ms, "atoms_per_s": n / (g_ms * 1e-3),
                     "eager_ms_per_step": ms_step, "speedup": ms_step / g_ms}
        del g

    smooth_rec = None
    if args.smooth:
        counts = np.diff(rp)
        ldt_np = np.repeat(np.log(np.maximum(counts, 1)) + 1.5, counts)
        ldt = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(
            ldt_np[None, :, None], (w.layers, e, w.heads)))).to(dev, x.dtype)
        ys = torch.empty_like(x)
        for _ in range(args.warmup):
            nga.block_attn_forward(csr_out["row_ptr"], x, wt, w.heads, w.sel, y=ys, ws=ws_attn,
                                   log_dtilde=ldt)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for e0, e1 in evs:
            e0.record(stream)
            nga.block_attn_forward(csr_out["row_ptr"], x, wt, w.heads, w.sel, y=ys, ws=ws_attn,
                                   log_dtilde=ldt)
            e1.record(stream)
        torch.cuda.synchronize(dev)
        nga.check_status(ws_attn, "block_attn_forward_smooth")
        sm_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
        smooth_rec = {"ms_per_forward": sm_ms, "vs_block_attn_forward": sm_ms / attn_ms,
                      "log_dtilde": "ln(n_i) + 1.5 for every edge and head of centre i"}

    local_rec = None
    if args.local_atten:
        xc = torch.from_numpy(W.make_features(n, w.c, 600, x_np.dtype)).to(dev)
        yc = torch.empty_like(xc)
        ws_loc = nga.Workspace(dev)
        for _ in range(args.warmup):
            nga.local_attn_forward(csr_out["row_ptr"], xc, x, wt, w.heads, yc=yc, ws=ws_loc)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for e0, e1 in evs:
            e0.record(stream)
            nga.local_attn_forward(csr_out["row_ptr"], xc, x, wt, w.heads, yc=yc, ws=ws_loc)
            e1.record(stream)
        torch.cuda.synchronize(dev)
        nga.check_status(ws_loc, "local_attn_forward")
        loc_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
        es = x.element_size()
        # every layer reads the edge rows once; the centre rows are read and written once
        loc_bytes = float(w.layers * e * w.c * es + 2 * n * w.c * es + 8 * (n + 1))
        local_rec = {"ms_per_forward": loc_ms, "algorithmic_bytes": loc_bytes,
                     "achieved_gbs": loc_bytes / (loc_ms * 1e-3) / 1e9,
                     "frac_hbm": loc_bytes / (loc_ms * 1e-3) / 1e9 / PEAK_HBM_GBS}

    gs_rec = None
    if not args.no_gather_scatter:
        # The (nloc, nnei_cap, c) block of the pages' block-dense route, materialised by the
        # standalone copies: gather reads the edge rows and writes every block row (padding
        # included), scatter reads the valid block rows and writes the edge rows.
        ws_gs = nga.Workspace(dev)
        blk = torch.empty((n, w.sel, w.c), dtype=x.dtype, device=dev)
        yg = torch.empty_like(x)
        rp_t = csr_out["row_ptr"]
        nga.block_gather(rp_t, x, w.sel, block=blk, ws=ws_gs)
        nga.block_scatter(rp_t, blk, yg, ws=ws_gs)
        nga.check_status(ws_gs, "block_gather / block_scatter")
        if not torch.equal(yg, x):
            raise RuntimeError("block_scatter(block_gather(x)) differs from x")

        def timed_copy(fn):
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.steps)]
            for _ in range(max(1, args.warmup)):
                fn()
            for e0, e1 in evs:
                e0.record(stream)
                fn()
                e1.record(stream)
            torch.cuda.synchronize(dev)
            return robust([e0.elapsed_time(e1) for e0, e1 in evs])

        g_ms = timed_copy(lambda: nga.block_gather(rp_t, x, w.sel, block=blk, ws=ws_gs))
        s_ms = timed_copy(lambda: nga.block_scatter(rp_t, blk, yg, ws=ws_gs))
        nga.check_status(ws_gs, "block_gather / block_scatter")
        es = x.element_size()
        g_bytes = float(e * w.c * es + n * w.sel * w.c * es + 8 * (n + 1))
        s_bytes = float(2 * e * w.c * es + 8 * (n + 1))

        def rate(nbytes, ms):
            gbs = nbytes / (ms["mean"] * 1e-3) / 1e9
            return {"algorithmic_bytes": nbytes, "ms": ms, "achieved_gbs": gbs,
                    "frac": gbs / PEAK_HBM_GBS}

        gs_rec = {"block_shape": [n, w.sel, w.c],
                  "gather": rate(g_bytes, g_ms), "scatter": rate(s_bytes, s_ms),
                  "bytes_basis": "gather: E*c*s read + N*cap*c*s written (padding rows "
                                 "included) + row_ptr; scatter: 2*E*c*s + row_ptr"}
        del blk, yg

    split_rec = None
    if args.split16 and w.dtype == "f32":
        v16 = nga.attn_variant(nga.NGA_F32_SPLIT16, w.sel, w.c, w.heads)
        ws16 = nga.Workspace(dev, nga.block_attn_workspace_bytes(nga.NGA_F32_SPLIT16, e, w.sel,
                                                                 w.c, w.heads, w.layers))
        y16 = torch.empty_like(x)
        for _ in range(args.warmup):
            nga.block_attn_forward(csr_out["row_ptr"], x, wt, w.heads, w.sel, y=y16, ws=ws16,
                                   split16=True)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for e0, e1 in evs:
            e0.record(stream)
            nga.block_attn_forward(csr_out["row_ptr"], x, wt, w.heads, w.sel, y=y16, ws=ws16,
                                   split16=True)
            e1.record(stream)
        torch.cuda.synchronize(dev)
        nga.check_status(ws16, "block_attn_forward (split16)")
        ms16 = robust([e0.elapsed_time(e1) for e0, e1 in evs])
        diff = float((y16.double() - y.double()).abs().max() / y.double().abs().max())
        fl16 = w.layers * float(np.sum(8.0 * w.c * w.c * np.diff(rp) + 4.0 * w.c * np.diff(rp)
                                      .astype(np.float64) ** 2))
        split_rec = {"kernel": v16, "block_attn_forward_ms": ms16,
                     "vs_fp32_kernel": ms16["mean"] / attn_ms,
                     "frac_of_split_bound": fl16 / (ms16["mean"] * 1e-3) / 1e12
                     / (PEAK_TFLOPS["f16"] / SPLIT_F16_FACTOR),
                     "normwise_diff_vs_fp32_output": diff,
                     "note": "contractions on f16 hi/lo pairs (21-22 significant bits per "
                             "operand); not fp32 arithmetic, asked for only by NGA_F32_SPLIT16"}

    pair_rec = None
    if args.pair_axis:
        pair_rec = time_pair_axis(nga, torch, dev, stream, csr_out["row_ptr"][: n + 1], x, wt, w,
                                  rp, args.pair_steps, args.pair_chunk, y, attn_ms)

    if args.copy_calib_mib > 0:
        nel = args.copy_calib_mib * (1 << 20) // 4
        src = torch.ones(nel, dtype=torch.float32, device=dev)
        dstb = torch.empty_like(src)
        dstb.copy_(src)
        torch.cuda.synchronize(dev)

    counts = np.diff(rp).astype(np.float64)
    proj_flops = w.layers * float(np.sum(8.0 * w.c * w.c * counts))      # Q, K, V, O projections
    attn_flops = w.layers * float(np.sum(4.0 * w.c * counts * counts))   # S = QK^T and O = PV
    flops = proj_flops + attn_flops
    achieved = flops / (attn_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    peak_basis = f"{w.dtype} dense MFMA"
    traffic = load_traffic(variant, w.name)
    nl_bytes = 24.0 * n + 8.0 * (n + 1) + 16.0 * e
    nl_counter = load_nl_traffic(w.name)
    nl_gbs = nl_bytes / ((nl_ms + csr_ms) * 1e-3) / 1e9
    # edge_csr alone: read each kept row entry (j, 3 shifts) and nnei, write col, shift, dst
    # and row_ptr.
    csr_bytes = 16.0 * e + 4.0 * n + 20.0 * e + 8.0 * (n + 1)
    csr_gbs = csr_bytes / (csr_ms * 1e-3) / 1e9

    rec = {
        "metric": METRIC,
        "value": n / (ms_step * 1e-3),
        "unit": "atoms/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "n_atoms": n, "n_edges": e, "rcut": w.rcut, "sel": w.sel,
                   "channels": w.c, "heads": w.heads, "layers": w.layers,
                   "geometry_dtype": "f64", "attn_kernel": variant,
                   "attn_plan": nga.attn_plan(dtype_code, n, w.sel, w.c, w.heads)},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": traffic,
                     "kernel": variant, "flops_per_launch": flops, "launch_ms": attn_ms,
                     "peak_basis": peak_basis},
        "parts_ms": {"nl_build": nl_ms, "edge_csr": csr_ms, "block_attn_forward": attn_ms},
        "timing": timing,
        "nl_hbm": {"algorithmic_bytes": nl_bytes, "achieved_gbs": nl_gbs,
                   "frac": nl_gbs / PEAK_HBM_GBS,
                   # nl_build's own HBM bytes from the committed FETCH_SIZE / WRITE_SIZE
                   # summary, over nl_build's time alone
                   "counter_bytes": nl_counter,
                   "counter_gbs": None if nl_counter is None else nl_counter / (nl_ms * 1e-3) / 1e9},
        "csr_hbm": {"algorithmic_bytes": csr_bytes, "achieved_gbs": csr_gbs,
                    "frac": csr_gbs / PEAK_HBM_GBS},
    }
    if graph_rec is not None:
        rec["graph"] = graph_rec
    if reuse_rec is not None:
        rec["nl_reuse"] = reuse_rec
    if batch_rec is not None:
        rec["nl_batch"] = batch_rec
    if smooth_rec is not None:
        rec["smooth"] = smooth_rec
    if local_rec is not None:
        rec["local_atten"] = local_rec
    if pair_rec is not None:
        rec["pair_axis"] = pair_rec
    if split_rec is not None:
        rec["split16"] = split_rec
    if gs_rec is not None:
        rec["gather_scatter"] = gs_rec
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, pos_np, box, rp, x_np, wt_np, args.cpu_seconds)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
