#!/usr/bin/env python3
"""Benchmark of the Atom copy/reduce collectives on one MI355X.

A step is one pass over every collective of the hot path, each on its own
resident synthetic input (bf16):

  copy    Atom copy of one 256 MiB input (also the counters' calibration kernel)
  rs_c1   ReduceScatter of Figure 4's layout at P = 4, 4 x 65536 fp32 per input
          (U[-1,1], seed 1): cache-resident, timed for its microseconds
  rs8     8-way ReduceScatter, 8 x 256 MiB (N(0,1), seed 2)
  ar      fused one-shot AllReduce of the same 8 x 256 MiB
  a2av    AllToAllV MoE dispatch, 8 x 4096 x 7168 (Dirichlet-multinomial counts, seed 3)
  ag_zs   AllGather, zero staging, 8 partitions of 64 MiB (U[-1,1], seed 4)
  ag_snac AllGather through SNAC, same input, 512 KiB chunks, 64-slot ring
  ar_snac composed AllReduce through SNAC (Figure 6) of the 8 x 256 MiB, 2 MiB
          chunks, 16-slot ring
  dec     decode AllReduce, 8 x b x 7168 for b in 1, 2, 4, 8, 16 (N(0,0.02), seed 5)
  rsv_zipf ReduceScatterV of the 8 x 256 MiB, Zipf(0.125) partitions (Figure 16)
  agv_zipf AllGatherV of 512 MiB in Zipf(0.125) partitions
  rsv_zipf_snac, agv_zipf_snac
          the same two through SNAC (the library's default staged plan)
  ag_8k   AllGather, zero staging, 8 partitions of 8 KiB
  moe_route, moe_dispatch, moe_combine
          expert-parallel MoE (Table 2): routing of 8 ranks x 512 tokens, top-8
          of 256 experts (seed 6), dispatch of the 7168-wide bf16 token rows to
          the experts and the weighted combine of same-shape expert outputs

`value` is the step's credited bytes (every input element read once, every
output element written once, a reduced element counted with its P reads)
over the step time, in GB/s. Per-collective GB/s and fraction of the 8 TB/s
HBM peak (from the median of the row's event-timed samples; samples above
1.5x the median are counted as outliers), the 8 KiB AllGather p50/p99
latency (an event pair around each launch), zero-staging and staged, their
time per call back to back, the zero-staging one's in a HIP graph, and the
dominant kernel's roofline are reported
alongside; the CPU oracle is timed on the same step as a baseline, and on
the P = 4 ReduceScatter alone.

`--ceilings` measures instead the cold rate of each traffic pattern on this
chip (streaming read, write, copy, 1 -> 8 fan-out and its variants) with
the measurement kernels of libatom_ceiling.so, a 1 GiB streaming fill
before each run.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12           # MI355X HBM3E, bytes/s
MiB = 1 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--lat-iters", type=int, default=10000,
                    help="event-timed samples of the 8 KiB AllGather and of each decode AllReduce")
    ap.add_argument("--ag-mib", type=int, default=64, help="AllGather partition size (MiB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=3)
    ap.add_argument("--study", action="store_true",
                    help="instead of the step: Atom copy bandwidth vs workgroups (CUs used) "
                         "and vs pipeline depth, one JSON line per point")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the step: AllGather (zero-staging and SNAC with 512 KiB, "
                         "1 MiB, 2 MiB chunks) over 8 KiB..1 GiB partitions, ReduceScatter, "
                         "AllReduce and AllToAll over 8 KiB..256 MiB inputs, MoE over 1..4096 "
                         "tokens per rank; one JSON line per point")
    ap.add_argument("--ceilings", action="store_true",
                    help="instead of the step: cold HBM rates of streaming read, write, copy and "
                         "1 -> 8 fan-out (plain, rotated store order, pure writes, one allocation "
                         "at several spacings); one JSON line per point")
    ap.add_argument("--snac-trace", action="store_true",
                    help="instead of the step: phase analysis of the staged (SNAC) path from its "
                         "per-task device-clock stamps (AllGather 8 x 64 MiB and 8 x 1 GiB at each "
                         "chunk size and lead, composed AllReduce, Zipf RSV/AGV, 8 KiB calls); one "
                         "JSON line per run")
    ap.add_argument("--ring-sweep", action="store_true",
                    help="instead of the step: the staged AllGather of 8 x 64 MiB and 8 x 1 GiB "
                         "at ring depths 2, 4, 8 and the default, each chunk size; one JSON line "
                         "per point")
    ap.add_argument("--snac-sweep", action="store_true",
                    help="instead of the step: staged-path launch choices (chunk x lead x piece) "
                         "for the AllGather 8 x 64 MiB, composed AllReduce 8 x 256 MiB, Zipf RSV/AGV, "
                         "and the AllGather 8 x 1 GiB (chunk x lead), cold; one JSON line per point")
    ap.add_argument("--xcd-order", action="store_true",
                    help="zero-staging kernels give each XCD one contiguous range of tiles")
    ap.add_argument("--no-snac", dest="snac", action="store_false",
                    help="leave out the SNAC-staged AllGather and AllReduce")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the P ranks are P buffers in one device's HBM "
              "and no collective crosses GPUs; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from reduce_atom_03_amd import atom as A
    from reduce_atom_03_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    if args.study:
        study(A, synth, torch, dev)
        return
    if args.sweep:
        sweep(A, synth, torch, dev)
        return
    if args.ceilings:
        ceilings(torch, dev)
        return
    if args.snac_trace:
        snac_trace(A, synth, torch, dev)
        return
    if args.ring_sweep:
        ring_sweep(A, synth, torch, dev)
        return
    if args.snac_sweep:
        snac_sweep(A, synth, torch, dev)
        return

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    def empty(n):
        return torch.empty(n, dtype=torch.bfloat16, device=dev)

    P = 8
    t0 = time.time()
    log("generating inputs ...")
    # ReduceScatter of Figure 4's layout, P = 4, 4 x 65536 fp32 per input
    c1 = synth.c1_inputs()
    x1 = [torch.from_numpy(x).to(dev) for x in c1]
    y1 = [torch.empty(65536, dtype=torch.float32, device=dev) for _ in range(4)]
    # 8-way reduce / AllReduce: 8 x 256 MiB
    c2 = synth.c2_inputs()
    x2 = [up(x) for x in c2]
    del c2
    N2 = 1 << 27
    n2 = N2 // P
    ys = [empty(n2) for _ in range(P)]
    ar_out = [empty(N2) for _ in range(P)]
    # AllToAllV
    C3 = synth.c3_counts()
    c3 = synth.c3_inputs()
    x3 = [up(x) for x in c3]
    del c3
    R3 = C3.sum(axis=0)
    a2a_out = [empty(int(R3[j]) * synth.HIDDEN) for j in range(P)]
    # AllGather
    S = args.ag_mib * MiB
    z4 = [up(z) for z in synth.c4_inputs(S, P)]
    ag_out = [empty(P * S // 2) for _ in range(P)]
    snac_cfg = A.config(flags=A.F_STAGED)     # chunk, ring and grid: the library's defaults
    # AllGatherV: 8 x 64 MiB in total, Zipf(0.125) partitions
    cnt_ag = synth.zipf_partition(P * S // 2, P, 0.125, 8) // 8
    zv = [up(synth.draw(4, k, int(cnt_ag[k]) * 8, "uniform", synth.BF16)) for k in range(P)]
    agv_out = [empty(P * S // 2) for _ in range(P)]
    # decode AllReduce
    x5 = {b: [up(x) for x in synth.c5_inputs(b)] for b in (1, 2, 4, 8, 16)}
    o5 = {b: [empty(b * synth.HIDDEN) for _ in range(P)] for b in (1, 2, 4, 8, 16)}
    # 8 KiB AllGather
    z8 = [up(z) for z in synth.c4_inputs(8 << 10, P)]
    o8 = [empty(P * 4096) for _ in range(P)]
    # MoE dispatch / combine
    moe_ids, moe_w = synth.moe_routing(6, P, synth.MOE_TOKENS, synth.MOE_EXPERTS, synth.MOE_TOPK)
    moe_rt = A.moe_alloc_routing([torch.from_numpy(a).to(dev) for a in moe_ids],
                                 synth.MOE_EXPERTS, synth.MOE_TOPK)
    A.atom_moe_route(moe_rt)
    moe_cap = int(moe_rt.recv_t.max().item())
    moe_x = [up(x) for x in synth.moe_inputs()]
    moe_w = [torch.from_numpy(a).to(dev) for a in moe_w]
    moe_disp = [empty(moe_cap * synth.HIDDEN) for _ in range(P)]
    moe_out = [empty(synth.MOE_TOKENS * synth.HIDDEN) for _ in range(P)]
    torch.cuda.synchronize()
    log(f"inputs resident in HBM ({time.time() - t0:.1f} s)")

    # Each row: (name, callable, credited bytes per call); CUs used per row
    # is min(workgroups launched, 256).
    cus = {}

    def plan_bytes(lin, lout, op, cfg=None, name=None):
        st, info = A.atom_plan_query(lin, lout, op, cfg)
        assert st == A.OK
        cus[name] = min(256, info.num_wgs)
        return info.credited_bytes

    L = A.layout
    zs_cfg = A.config(flags=A.F_XCD_ORDER) if args.xcd_order else None
    rows = []
    copy_out = empty(N2)
    rows.append(("copy", lambda: A.atom_copy(copy_out, x2[0]), 2 * N2 * 2))
    cus["copy"] = 256
    lay1 = (L(A.PARTITIONED, x1, 65536), L(A.SHARD, y1, 65536))
    rs_c1 = lambda l=lay1: A.atom_collective(l[0], l[1], A.OP_SUM)
    rows.append(("rs_c1", rs_c1, plan_bytes(lay1[0], lay1[1], A.OP_SUM, name="rs_c1")))
    lay = (L(A.PARTITIONED, x2, n2), L(A.SHARD, ys, n2))
    rows.append(("rs8", lambda l=lay: A.atom_collective(l[0], l[1], A.OP_SUM, zs_cfg),
                 plan_bytes(lay[0], lay[1], A.OP_SUM, zs_cfg, name="rs8")))
    lay = (L(A.PARTITIONED, x2, n2), L(A.GATHERED, ar_out, n2))
    rows.append(("ar", lambda l=lay: A.atom_collective(l[0], l[1], A.OP_SUM, zs_cfg),
                 plan_bytes(lay[0], lay[1], A.OP_SUM, zs_cfg, name="ar")))
    lay = (L(A.PARTITIONED, x3, 0, C3, synth.HIDDEN), L(A.TRANSPOSED, a2a_out, 0, None, synth.HIDDEN))
    rows.append(("a2av", lambda l=lay: A.atom_collective(l[0], l[1], A.OP_COPY, zs_cfg),
                 plan_bytes(lay[0], lay[1], A.OP_COPY, zs_cfg, name="a2av")))
    lay = (L(A.SHARD, z4, S // 2), L(A.GATHERED, ag_out, S // 2))
    rows.append(("ag_zs", lambda l=lay: A.atom_collective(l[0], l[1], A.OP_COPY, zs_cfg),
                 plan_bytes(lay[0], lay[1], A.OP_COPY, zs_cfg, name="ag_zs")))
    if args.snac:
        rows.append(("ag_snac", lambda l=lay: A.atom_collective(l[0], l[1], A.OP_COPY, snac_cfg),
                     plan_bytes(lay[0], lay[1], A.OP_COPY, snac_cfg, name="ag_snac")))
        lay = (L(A.PARTITIONED, x2, n2), L(A.GATHERED, ar_out, n2))
        rows.append(("ar_snac", lambda l=lay: A.atom_collective(l[0], l[1], A.OP_SUM, snac_cfg),
                     plan_bytes(lay[0], lay[1], A.OP_SUM, snac_cfg, name="ar_snac")))
    for b in (1, 2, 4, 8, 16):
        lay = (L(A.PARTITIONED, x5[b], b * 896), L(A.GATHERED, o5[b], b * 896))
        rows.append((f"dec_b{b}", lambda l=lay: A.atom_collective(l[0], l[1], A.OP_SUM),
                     plan_bytes(lay[0], lay[1], A.OP_SUM, name=f"dec_b{b}")))
    # Variable-length ReduceScatter / AllGather with Zipf(0.125) partitions
    cnt_rs = synth.zipf_partition(N2, P, 0.125, 8) // 8
    rsv_out = [empty(int(c) * 8) for c in cnt_rs]
    lay = (L(A.PARTITIONED, x2, 0, cnt_rs, 8), L(A.SHARD, rsv_out, 0, None, 8))
    rows.append(("rsv_zipf", lambda l=lay: A.atom_collective(l[0], l[1], A.OP_SUM, zs_cfg),
                 plan_bytes(lay[0], lay[1], A.OP_SUM, zs_cfg, name="rsv_zipf")))
    lay = (L(A.SHARD, zv, 0, cnt_ag, 8), L(A.GATHERED, agv_out, 0, None, 8))
    rows.append(("agv_zipf", lambda l=lay: A.atom_collective(l[0], l[1], A.OP_COPY, zs_cfg),
                 plan_bytes(lay[0], lay[1], A.OP_COPY, zs_cfg, name="agv_zipf")))
    if args.snac:
        # the same two through SNAC: Figure 16 runs them on ordinary buffers
        lay = (L(A.PARTITIONED, x2, 0, cnt_rs, 8), L(A.SHARD, rsv_out, 0, None, 8))
        rows.append(("rsv_zipf_snac", lambda l=lay: A.atom_collective(l[0], l[1], A.OP_SUM, snac_cfg),
                     plan_bytes(lay[0], lay[1], A.OP_SUM, snac_cfg, name="rsv_zipf_snac")))
        lay = (L(A.SHARD, zv, 0, cnt_ag, 8), L(A.GATHERED, agv_out, 0, None, 8))
        rows.append(("agv_zipf_snac", lambda l=lay: A.atom_collective(l[0], l[1], A.OP_COPY, snac_cfg),
                     plan_bytes(lay[0], lay[1], A.OP_COPY, snac_cfg, name="agv_zipf_snac")))
    lay8 = (L(A.SHARD, z8, 4096), L(A.GATHERED, o8, 4096))
    ag8 = lambda l=lay8: A.atom_collective(l[0], l[1], A.OP_COPY)
    rows.append(("ag_8k", ag8, plan_bytes(lay8[0], lay8[1], A.OP_COPY, name="ag_8k")))
    # MoE: the routing (metadata only), then dispatch into the experts'
    # buffers, then the combine of those buffers (standing in for the expert
    # outputs, same shape) back to the tokens.
    mb = moe_bytes(P, synth.MOE_TOKENS, synth.MOE_EXPERTS, synth.MOE_TOPK, synth.HIDDEN * 2)
    rows.append(("moe_route", lambda: A.atom_moe_route(moe_rt), mb["route"]))
    rows.append(("moe_dispatch", lambda: A.atom_moe_dispatch(moe_rt, moe_x, moe_disp, moe_cap,
                                                             synth.HIDDEN), mb["dispatch"]))
    rows.append(("moe_combine", lambda: A.atom_moe_combine(moe_rt, moe_disp, moe_w, moe_out, moe_cap,
                                                           synth.HIDDEN), mb["combine"]))
    nch = -(-synth.MOE_TOKENS * synth.MOE_TOPK // 256)
    cus.update({"moe_route": min(256, P * nch), "moe_dispatch": min(256, P * synth.MOE_TOKENS),
                "moe_combine": min(256, P * synth.MOE_TOKENS)})

    step_bytes = sum(r[2] for r in rows)

    for _ in range(args.warmup):
        for _, fn, _ in rows:
            fn()
    assert A.atom_sync_status() == A.OK

    K = args.steps
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in rows] for _ in range(K)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(K):
        for i, (_, fn, _) in enumerate(rows):
            ev[k][i][0].record(stream)
            fn()
            ev[k][i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    assert A.atom_sync_status() == A.OK

    per_row = {}
    for i, (name, _, nbytes) in enumerate(rows):
        ms = np.array([ev[k][i][0].elapsed_time(ev[k][i][1]) for k in range(K)])
        p50 = float(np.median(ms))
        per_row[name] = {"ms": round(p50, 5), "ms_mean": round(float(ms.mean()), 5),
                         "outliers": int((ms > 1.5 * p50).sum()), "credited_bytes": int(nbytes),
                         "GBps": round(nbytes / (p50 * 1e-3) / 1e9, 1),
                         "frac_hbm": round(nbytes / (p50 * 1e-3) / HBM_PEAK, 4)}
    ms_step = wall * 1e3 / K
    value = step_bytes / (ms_step * 1e-3) / 1e9

    # 8 KiB AllGather latency: event pair around each launch.
    lat = []
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.lat_iters)]
    for a, b in pairs:
        a.record(stream)
        ag8()
        b.record(stream)
    torch.cuda.synchronize()
    lat = np.array([a.elapsed_time(b) * 1e3 for a, b in pairs])
    # The same 8 KiB AllGather through SNAC (the staged path's latency): a
    # small call hands off through tagged words by default; ATOM_F_COUNTED
    # gives the slot-count hand-off of larger calls, for comparison.
    snac8 = lambda l=lay8: A.atom_collective(l[0], l[1], A.OP_COPY, snac_cfg)
    counted_cfg = A.config(flags=A.F_STAGED | A.F_COUNTED)
    snac8c = lambda l=lay8: A.atom_collective(l[0], l[1], A.OP_COPY, counted_cfg)

    def event_lat(fn):
        fn()
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(args.lat_iters)]
        for a, b in pairs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        assert A.atom_sync_status() == A.OK
        return np.array([a.elapsed_time(b) * 1e3 for a, b in pairs])
    lat_snac = event_lat(snac8)
    lat_snac_counted = event_lat(snac8c)
    # Decode AllReduce latency per batch size (event pairs, as above).
    dec_lat = {}
    for b in (1, 2, 4, 8, 16):
        lay = (L(A.PARTITIONED, x5[b], b * 896), L(A.GATHERED, o5[b], b * 896))
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(args.lat_iters)]
        for a, e in pairs:
            a.record(stream)
            A.atom_collective(lay[0], lay[1], A.OP_SUM)
            e.record(stream)
        torch.cuda.synchronize()
        v = np.array([a.elapsed_time(e) * 1e3 for a, e in pairs])
        dec_lat[f"b{b}"] = {"p50_us": round(float(np.percentile(v, 50)), 2),
                            "p99_us": round(float(np.percentile(v, 99)), 2)}
    # The P = 4 ReduceScatter alone: event pairs around lone launches.
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.lat_iters)]
    for a, b in pairs:
        a.record(stream)
        rs_c1()
        b.record(stream)
    torch.cuda.synchronize()
    c1_us = np.array([a.elapsed_time(b) * 1e3 for a, b in pairs])
    # Launch floor: the same event pair around a 16-byte atom_copy.
    tiny_src, tiny_dst = empty(8), empty(8)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.lat_iters)]
    for a, b in pairs:
        a.record(stream)
        A.atom_copy(tiny_dst, tiny_src, 16)
        b.record(stream)
    torch.cuda.synchronize()
    floor = np.array([a.elapsed_time(b) * 1e3 for a, b in pairs])
    # The same AllGather captured 100 times into one HIP graph: the per-call
    # cost once launch overhead is amortized (a serving loop's view).
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for _ in range(100):
                ag8()
    stream.wait_stream(side)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    gl = []
    for _ in range(20):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        b.record(stream)
        b.synchronize()
        gl.append(a.elapsed_time(b) * 1e3 / 100)
    graph_us = float(np.median(gl))
    # Back to back: 200 calls queued behind a spin kernel (so that the host's
    # submission, slower than the GPU per call, does not pace them) with one
    # event pair around all of them: the GPU time per call of a loop of
    # collectives, the convention of collective benchmarks' time per op. A
    # batch of 200 fits in the runtime's command queue (with 400 the host
    # blocks until the spin ends and the batch's tail is host-paced); the
    # spin is about 20 ms at the calibrated rate against ~1.5 ms of enqueue.
    # Batches whose enqueue outlasted half the spin are counted
    # (`back_to_back_host_paced_batches`, of `back_to_back_batches`); each
    # figure is the median over its 9 batches.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1000000)
    e0.record(stream)
    torch.cuda._sleep(1000000)
    e1.record(stream)
    e1.synchronize()
    ms_per_mcycle = max(e0.elapsed_time(e1), 1e-3)
    spin_ms = 20.0
    spin = int(1e6 * spin_ms / ms_per_mcycle)
    paced = []

    def back_to_back_us(fn, n=200, reps=9):
        v = []
        for _ in range(reps):
            torch.cuda._sleep(spin)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            h0 = time.perf_counter()
            a.record(stream)
            for _ in range(n):
                fn()
            b.record(stream)
            if (time.perf_counter() - h0) * 1e3 > spin_ms / 2:
                paced.append(1)
            b.synchronize()
            v.append(a.elapsed_time(b) * 1e3 / n)
        return round(float(np.median(v)), 2)

    b2b = {"ag_8KiB": back_to_back_us(ag8), "ag_8KiB_snac": back_to_back_us(snac8),
           "ag_8KiB_snac_counted": back_to_back_us(snac8c),
           "copy_16B": back_to_back_us(lambda: A.atom_copy(tiny_dst, tiny_src, 16))}
    for b in (1, 2, 4, 8, 16):
        lay = (L(A.PARTITIONED, x5[b], b * 896), L(A.GATHERED, o5[b], b * 896))
        b2b[f"dec_b{b}"] = back_to_back_us(lambda l=lay: A.atom_collective(l[0], l[1], A.OP_SUM))
    # Host-side time per call of the same launch (submission cost).
    t = time.perf_counter()
    for _ in range(args.lat_iters):
        ag8()
    host_us = (time.perf_counter() - t) / args.lat_iters * 1e6
    torch.cuda.synchronize()

    # Dominant kernel: the collective taking the most time per step.
    dom = max(per_row, key=lambda r: per_row[r]["ms"])
    d = per_row[dom]
    achieved = d["credited_bytes"] / (d["ms"] * 1e-3) / 1e9
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                "peak": HBM_PEAK / 1e9, "unit": "GB/s", "frac": round(achieved * 1e9 / HBM_PEAK, 4),
                "traffic": measured_traffic(dom)}

    cpu = None
    c1_oracle = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, C3, S, step_bytes)
        c1_oracle = c1_oracle_ms(c1)

    out = {
        "metric": "achieved HBM GB/s (% of peak) for 8-way reduce & AllToAll; p50 us at 8 KiB",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": ("one pass over: copy of 256 MiB; 8-way ReduceScatter and fused AllReduce of 8 x 256 MiB bf16; "
                         "AllToAllV 8 x 4096 x 7168 bf16 (Dirichlet-multinomial counts); "
                         f"AllGather 8 x {args.ag_mib} MiB (zero-staging"
                         + (" and SNAC, 512 KiB chunks, 64-slot ring); SNAC-composed AllReduce of the "
                            "8 x 256 MiB (2 MiB chunks, 16-slot ring); " if args.snac else "); ") +
                         "ReduceScatterV and AllGatherV with Zipf(0.125) partitions of the same totals"
                         + (", zero-staging and SNAC; " if args.snac else "; ") +
                         "decode AllReduce 8 x b x 7168 bf16, b = 1..16; AllGather 8 x 8 KiB; "
                         "MoE route, dispatch and combine of 8 x 512 tokens x 7168 bf16 "
                         "(256 experts, top-8)"),
            "P": P, "step_credited_bytes": int(step_bytes),
        },
        "reduce8_GBps": per_row["rs8"]["GBps"],
        "reduce8_frac": per_row["rs8"]["frac_hbm"],
        "a2a_GBps": per_row["a2av"]["GBps"],
        "a2a_frac": per_row["a2av"]["frac_hbm"],
        "p50_us_8KiB": round(float(np.percentile(lat, 50)), 2),
        "p99_us_8KiB": round(float(np.percentile(lat, 99)), 2),
        "p50_us_8KiB_snac": round(float(np.percentile(lat_snac, 50)), 2),
        "p99_us_8KiB_snac": round(float(np.percentile(lat_snac, 99)), 2),
        "p50_us_8KiB_snac_counted": round(float(np.percentile(lat_snac_counted, 50)), 2),
        "p99_us_8KiB_snac_counted": round(float(np.percentile(lat_snac_counted, 99)), 2),
        "host_us_per_call_8KiB": round(host_us, 2),
        "graph_us_per_call_8KiB": round(graph_us, 2),
        "back_to_back_us_per_call": b2b,
        "back_to_back_host_paced_batches": len(paced),
        "back_to_back_batches": 9 * len(b2b),
        "decode_allreduce_latency": dec_lat,
        "c1_gpu_us": {"p50": round(float(np.percentile(c1_us, 50)), 2),
                      "p99": round(float(np.percentile(c1_us, 99)), 2),
                      "samples": int(c1_us.size),
                      "workload": "ReduceScatter P=4, 4 x 65536 fp32 per input, event pair per launch"},
        "c1_oracle_ms": c1_oracle,
        "latency_samples": args.lat_iters,
        "p50_us_launch_floor_16B_copy": round(float(np.percentile(floor, 50)), 2),
        "cus_used": cus,
        "rows": per_row,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def study(A, synth, torch, dev):
    """Atom copy of 256 MiB (a one-rank AllGather, so the launch shape can be
    set): GB/s against workgroups launched (CUs used = min(WGs, 256)) and
    against pipeline depth (16-byte slots in flight per lane) at every grid
    from 8 workgroups to the full one-tile-per-workgroup grid, the one-GPU
    counterparts of the pages' SM-count and pipeline-depth studies
    (Figures 3 and 11); then GB/s against workgroups for the 8-way reduce
    and the 1 -> 8 fan-out. Cold: a 1 GiB streaming fill of another buffer
    (libatom_ceiling.so) precedes every timed call, so neither the caches
    nor the memory-side cache hold the call's data; median of 7 calls."""
    import ctypes
    clib = ctypes.CDLL(os.path.join(ROOT, "reduce_atom_03_amd", "libatom_ceiling.so"))
    clib.ceil_fill.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    stream = torch.cuda.current_stream()
    sp = int(stream.cuda_stream)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)

    def cold_ms(fn, reps=7):
        t = []
        for _ in range(reps):
            if clib.ceil_fill(flush.data_ptr(), 1 << 30, 256, 4, sp) != 0:
                raise RuntimeError("ceiling fill kernel failed")
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            t.append(e0.elapsed_time(e1))
        return float(np.median(t))

    n = 1 << 27
    src = torch.from_numpy(synth.draw(2, 0, n, "normal", synth.BF16).view(np.int16)).view(
        torch.bfloat16).to(dev)
    dst = torch.empty(n, dtype=torch.bfloat16, device=dev)
    lin, lout = A.layout(A.SHARD, [src], n), A.layout(A.GATHERED, [dst], n)

    def point(wgs, stages):
        cfg = A.config(num_wgs=wgs, stages=stages)
        A.atom_collective(lin, lout, A.OP_COPY, cfg)
        ms = cold_ms(lambda: A.atom_collective(lin, lout, A.OP_COPY, cfg))
        st, info = A.atom_plan_query(lin, lout, A.OP_COPY, cfg)
        gbs = 4 * n / ms / 1e6
        print(json.dumps({"study": "atom_copy_256MiB", "workgroups": info.num_wgs,
                          "cus_used": min(256, info.num_wgs), "stages": stages,
                          "ms": round(ms, 4), "GBps": round(gbs, 1),
                          "frac_hbm": round(gbs * 1e9 / HBM_PEAK, 4)}), flush=True)

    for wgs in (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096, 0):
        point(wgs, 4)
    for wgs in (8, 16, 64, 256, 1024, 4096, 16384, 65536, 0):
        for stages in (1, 2, 4, 8):
            point(wgs, stages)

    # The same CUs-used curve for the two other shapes of the hot path: the
    # 8-way reduce (8 x 256 MiB -> 256 MiB, ReduceScatter layout) and the
    # 1 -> 8 fan-out (AllGather of 8 x 64 MiB).
    P = 8
    del src, dst
    xs = [torch.randn(n, device=dev).to(torch.bfloat16) for _ in range(P)]
    ys = [torch.empty(n // P, dtype=torch.bfloat16, device=dev) for _ in range(P)]
    zs = [t[:n // 4] for t in xs]
    ag = [torch.empty(P * n // 4, dtype=torch.bfloat16, device=dev) for _ in range(P)]
    shapes = {
        "reduce8_8x256MiB": (A.layout(A.PARTITIONED, xs, n // P), A.layout(A.SHARD, ys, n // P),
                             A.OP_SUM, (P + 1) * n * 2),
        "fanout8_8x64MiB": (A.layout(A.SHARD, zs, n // 4), A.layout(A.GATHERED, ag, n // 4),
                            A.OP_COPY, (1 + P) * P * (n // 4) * 2),
    }
    for name, (li, lo, op, nbytes) in shapes.items():
        for wgs in (8, 16, 32, 64, 128, 256, 512, 1024, 4096, 0):
            cfg = A.config(num_wgs=wgs)
            A.atom_collective(li, lo, op, cfg)
            ms = cold_ms(lambda: A.atom_collective(li, lo, op, cfg), reps=5)
            st, info = A.atom_plan_query(li, lo, op, cfg)
            gbs = nbytes / ms / 1e6
            print(json.dumps({"study": name, "workgroups": info.num_wgs,
                              "cus_used": min(256, info.num_wgs), "stages": 0,
                              "ms": round(ms, 4), "GBps": round(gbs, 1),
                              "frac_hbm": round(gbs * 1e9 / HBM_PEAK, 4)}), flush=True)


def snac_decode(t, G, E, Q):
    """(produce, chunk, piece) of tickets t in the staged kernel's ticket
    order: producers of chunks 0..E-1; then, for each later chunk q, the
    consumers of chunk q-E followed by the producers of chunk q; then the
    consumers of the last E chunks (G pieces per chunk, Q chunks)."""
    warm = min(Q, E) * G
    mid = max(Q - E, 0) * 2 * G
    prod = np.zeros(t.size, dtype=bool)
    chunk = np.zeros(t.size, dtype=np.int64)
    a = t < warm
    prod[a], chunk[a] = True, t[a] // G
    b = (t >= warm) & (t < warm + mid)
    u = t[b] - warm
    q = E + u // (2 * G)
    w = u - (q - E) * 2 * G
    prod[b] = w >= G
    chunk[b] = np.where(w >= G, q, q - E)
    c = t >= warm + mid
    prod[c], chunk[c] = False, max(Q - E, 0) + (t[c] - warm - mid) // G
    return prod, chunk


def snac_trace(A, synth, torch, dev):
    """Where a staged call spends its time, from the stamps each task writes
    (atom_config.trace: ticket taken, wait over, work done, on the device's
    constant-rate clock). Per run: the kernel span; workgroup-time shares of
    producer and consumer waits and work and of the claim/notify gaps
    between tasks; per-task work times; the hand-off latency of each chunk
    (its last piece staged -> its first consumer past the wait) and of each
    slot reuse (the chunk D places earlier fully consumed -> the producer
    past its wait); the ramp (span start -> first consume) and the drain
    (last stage -> span end). The same call without the trace is timed
    alongside (event pairs, median), as is its credited rate."""
    P = 8
    L = A.layout
    us = 1e3 / A.atom_device_clock_khz()           # microseconds per clock tick

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    def timed(fn, reps):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ev]))

    def q(x, p):
        return round(float(np.percentile(x, p)), 2) if x.size else None

    def run(name, li, lo, op, reps=5, flags=0, **kw):
        cfg = A.config(flags=A.F_STAGED | flags, **kw)
        st, info = A.atom_plan_query(li, lo, op, cfg)
        assert st == A.OK and info.staged == 1, (name, st)
        n = int(info.snac_tasks)
        G, E, Q = n // (2 * int(info.num_chunks)), int(info.snac_lead), int(info.num_chunks)
        fn = lambda: A.atom_collective(li, lo, op, cfg)
        fn()
        ms = timed(fn, reps)
        tr = torch.zeros(4 * n, dtype=torch.int64, device=dev)
        tcfg = A.config(flags=A.F_STAGED | flags, trace=tr.data_ptr(), **kw)
        tfn = lambda: A.atom_collective(li, lo, op, tcfg)
        ms_traced = timed(tfn, 1)
        assert A.atom_sync_status() == A.OK, name
        e = tr.cpu().numpy().reshape(n, 4)
        c0, c1, c2 = e[:, 0], e[:, 1], e[:, 2]
        wg = e[:, 3] & 0xFFFFFFFF
        prod = ((e[:, 3] >> 32) & 1).astype(bool)
        assert not ((e[:, 3] >> 33) & 1).any() and (c0 > 0).all(), name
        dprod, chunk = snac_decode(np.arange(n, dtype=np.int64), G, E, Q)
        assert (dprod == prod).all(), name
        t0 = c0.min()
        span = (c2.max() - t0) * us
        wait, work = (c1 - c0) * us, (c2 - c1) * us
        # gaps between a workgroup's tasks: notify, next ticket, barriers
        o = np.lexsort((c0, wg))
        same = wg[o][1:] == wg[o][:-1]
        gaps = ((c0[o][1:] - c2[o][:-1]) * us)[same]
        nwg = int(np.unique(wg).size)
        wg_time = span * nwg
        staged_at = np.full(Q, -1, dtype=np.int64)
        np.maximum.at(staged_at, chunk[prod], c2[prod])
        cons_start = np.full(Q, np.iinfo(np.int64).max, dtype=np.int64)
        np.minimum.at(cons_start, chunk[~prod], c1[~prod])
        consumed_at = np.full(Q, -1, dtype=np.int64)
        np.maximum.at(consumed_at, chunk[~prod], c2[~prod])
        handoff = (cons_start - staged_at) * us
        D = int(info.ring_slots)
        reuse = np.array([], dtype=np.float64)
        if Q > D:
            pstart = np.full(Q, np.iinfo(np.int64).max, dtype=np.int64)
            np.minimum.at(pstart, chunk[prod], c1[prod])
            reuse = (pstart[D:] - consumed_at[:-D]) * us
        line = {
            "snac_trace": name, "chunk_bytes": int(info.chunk_bytes), "pieces": G,
            "ring_slots": D, "lead": E, "workgroups": nwg, "lanes": int(info.lanes), "tasks": n,
            "ms": round(ms, 4), "ms_traced": round(ms_traced, 4),
            "credited_GBps": round(info.credited_bytes / ms / 1e6, 1),
            "span_us": round(span, 1),
            "share": {k: round(float(v) / wg_time, 4) for k, v in (
                ("producer_wait", wait[prod].sum()), ("producer_work", work[prod].sum()),
                ("consumer_wait", wait[~prod].sum()), ("consumer_work", work[~prod].sum()),
                ("gaps", gaps.sum()))},
            "producer_work_us": {"p50": q(work[prod], 50), "p90": q(work[prod], 90)},
            "consumer_work_us": {"p50": q(work[~prod], 50), "p90": q(work[~prod], 90)},
            "producer_wait_us": {"p50": q(wait[prod], 50), "p90": q(wait[prod], 90)},
            "consumer_wait_us": {"p50": q(wait[~prod], 50), "p90": q(wait[~prod], 90)},
            "gap_us": {"p50": q(gaps, 50), "p90": q(gaps, 90)},
            "handoff_us": {"p50": q(handoff, 50), "p90": q(handoff, 90), "max": q(handoff, 100)},
            "slot_reuse_us": {"p50": q(reuse, 50), "p90": q(reuse, 90)},
            "ramp_us": round(float((cons_start.min() - t0) * us), 2),
            "drain_us": round(float((c2.max() - staged_at.max()) * us), 2),
            "first_stage_done_us": round(float((staged_at.min() - t0) * us), 2),
        }
        print(json.dumps(line), flush=True)

    MiB = 1 << 20
    # AllGather 8 x 64 MiB: each chunk size; the 512 KiB one at smaller leads
    S = 64 * MiB
    z = [up(a) for a in synth.c4_inputs(S, P)]
    o = [torch.empty(P * S // 2, dtype=torch.bfloat16, device=dev) for _ in range(P)]
    li, lo = L(A.SHARD, z, S // 2), L(A.GATHERED, o, S // 2)
    for chunk in (512 << 10, 1 << 20, 2 << 20):
        run(f"ag_8x64MiB_chunk{chunk >> 10}K", li, lo, A.OP_COPY, chunk_bytes=chunk)
    for lead in (32, 16, 8):
        run(f"ag_8x64MiB_chunk512K_lead{lead}", li, lo, A.OP_COPY, chunk_bytes=512 << 10, snac_lead=lead)
    for lead in (8, 4):
        run(f"ag_8x64MiB_chunk2048K_lead{lead}", li, lo, A.OP_COPY, chunk_bytes=2 << 20, snac_lead=lead)
    del z, o
    # composed AllReduce 8 x 256 MiB, default plan
    N2 = 1 << 27
    x = [torch.randn(N2, device=dev).to(torch.bfloat16) for _ in range(P)]
    ar = [torch.empty(N2, dtype=torch.bfloat16, device=dev) for _ in range(P)]
    run("ar_8x256MiB", L(A.PARTITIONED, x, N2 // P), L(A.GATHERED, ar, N2 // P), A.OP_SUM)
    for lead in (8, 4):
        run(f"ar_8x256MiB_lead{lead}", L(A.PARTITIONED, x, N2 // P), L(A.GATHERED, ar, N2 // P),
            A.OP_SUM, snac_lead=lead)
    del ar
    # Zipf ReduceScatterV / AllGatherV, default staged plans
    cnt = synth.zipf_partition(N2, P, 0.125, 8) // 8
    ys = [torch.empty(int(c) * 8, dtype=torch.bfloat16, device=dev) for c in cnt]
    run("rsv_zipf_8x256MiB", L(A.PARTITIONED, x, 0, cnt, 8), L(A.SHARD, ys, 0, None, 8), A.OP_SUM)
    del ys, x
    T = P * 64 * MiB // 2
    cnt = synth.zipf_partition(T, P, 0.125, 8) // 8
    zv = [torch.empty(int(c) * 8, dtype=torch.bfloat16, device=dev).uniform_(-1, 1) for c in cnt]
    ov = [torch.empty(T, dtype=torch.bfloat16, device=dev) for _ in range(P)]
    run("agv_zipf_512MiB", L(A.SHARD, zv, 0, cnt, 8), L(A.GATHERED, ov, 0, None, 8), A.OP_COPY)
    del zv, ov
    # small calls: 8 KiB AllGather and AllReduce, default plans (tagged
    # words), and through the slot counts
    z8 = [torch.empty(4096, dtype=torch.bfloat16, device=dev).uniform_(-1, 1) for _ in range(P)]
    o8 = [torch.empty(P * 4096, dtype=torch.bfloat16, device=dev) for _ in range(P)]
    x8 = [torch.randn(4096, device=dev).to(torch.bfloat16) for _ in range(P)]
    for sfx, fl in (("", 0), ("_counted", A.F_COUNTED)):
        run("ag_8x8KiB" + sfx, L(A.SHARD, z8, 4096), L(A.GATHERED, o8, 4096), A.OP_COPY, reps=200, flags=fl)
        run("ar_8x8KiB" + sfx, L(A.PARTITIONED, x8, 512), L(A.GATHERED, o8, 512), A.OP_SUM, reps=200,
            flags=fl)
    del z8, o8, x8
    # AllGather 8 x 1 GiB: each chunk size
    S = 1024 * MiB
    z = [torch.empty(S // 2, dtype=torch.bfloat16, device=dev).uniform_(-1, 1) for _ in range(P)]
    o = [torch.empty(P * S // 2, dtype=torch.bfloat16, device=dev) for _ in range(P)]
    li, lo = L(A.SHARD, z, S // 2), L(A.GATHERED, o, S // 2)
    for chunk in (512 << 10, 1 << 20, 2 << 20):
        run(f"ag_8x1GiB_chunk{chunk >> 10}K", li, lo, A.OP_COPY, reps=3, chunk_bytes=chunk)


def snac_sweep(A, synth, torch, dev):
    """Launch choices of the staged path, cold (a 1 GiB copy between calls;
    median of event-timed calls): for each chunk size (512 KiB, 1 MiB,
    2 MiB, the ring kept at 32 MiB), leads of D, D/2, D/4 and D/8 chunks and
    pieces of 32, 64 and 128 KiB, on the AllGather of 8 x 64 MiB, the
    composed AllReduce and the Zipf(0.125) ReduceScatterV of 8 x 256 MiB and
    the Zipf AllGatherV of 512 MiB; then the AllGather of 8 x 1 GiB at each
    chunk size and leads D, D/2, D/4 (default piece)."""
    P, MiB = 8, 1 << 20
    L = A.layout
    scrub_a = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev)
    scrub_b = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev)

    def timed(fn, reps):
        ts = []
        for _ in range(reps):
            scrub_b.copy_(scrub_a)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    def point(name, li, lo, op, reps, **kw):
        cfg = A.config(flags=A.F_STAGED, **kw)
        st, info = A.atom_plan_query(li, lo, op, cfg)
        assert st == A.OK, (name, kw, st)
        fn = lambda: A.atom_collective(li, lo, op, cfg)
        fn()
        ms = timed(fn, reps)
        assert A.atom_sync_status() == A.OK, name
        print(json.dumps({"snac_sweep": name, "chunk_bytes": int(info.chunk_bytes),
                          "lead": int(info.snac_lead), "ring_slots": int(info.ring_slots),
                          "piece_bytes": kw.get("piece_bytes", 0), "workgroups": int(info.num_wgs),
                          "ms": round(ms, 4), "GBps": round(info.credited_bytes / ms / 1e6, 1)}), flush=True)

    def grid(name, li, lo, op, reps):
        for chunk in (512 << 10, 1 << 20, 2 << 20):
            D = max(4, min(64, (32 << 20) // chunk))
            for lead in (D, D // 2, D // 4, D // 8):
                for piece in (32 << 10, 64 << 10, 128 << 10):
                    point(name, li, lo, op, reps, chunk_bytes=chunk, snac_lead=lead, piece_bytes=piece)

    S = 64 * MiB
    z = [torch.empty(S // 2, dtype=torch.bfloat16, device=dev).uniform_(-1, 1) for _ in range(P)]
    o = [torch.empty(P * S // 2, dtype=torch.bfloat16, device=dev) for _ in range(P)]
    grid("ag_8x64MiB", L(A.SHARD, z, S // 2), L(A.GATHERED, o, S // 2), A.OP_COPY, 7)
    del z, o
    N2 = 1 << 27
    x = [torch.randn(N2, device=dev).to(torch.bfloat16) for _ in range(P)]
    ar = [torch.empty(N2, dtype=torch.bfloat16, device=dev) for _ in range(P)]
    grid("ar_8x256MiB", L(A.PARTITIONED, x, N2 // P), L(A.GATHERED, ar, N2 // P), A.OP_SUM, 5)
    del ar
    cnt = synth.zipf_partition(N2, P, 0.125, 8) // 8
    ys = [torch.empty(int(c) * 8, dtype=torch.bfloat16, device=dev) for c in cnt]
    grid("rsv_zipf_8x256MiB", L(A.PARTITIONED, x, 0, cnt, 8), L(A.SHARD, ys, 0, None, 8), A.OP_SUM, 5)
    del ys, x
    T = P * 64 * MiB // 2
    cnt = synth.zipf_partition(T, P, 0.125, 8) // 8
    zv = [torch.empty(int(c) * 8, dtype=torch.bfloat16, device=dev).uniform_(-1, 1) for c in cnt]
    ov = [torch.empty(T, dtype=torch.bfloat16, device=dev) for _ in range(P)]
    grid("agv_zipf_512MiB", L(A.SHARD, zv, 0, cnt, 8), L(A.GATHERED, ov, 0, None, 8), A.OP_COPY, 7)
    del zv, ov
    S = 1024 * MiB
    z = [torch.empty(S // 2, dtype=torch.bfloat16, device=dev).uniform_(-1, 1) for _ in range(P)]
    o = [torch.empty(P * S // 2, dtype=torch.bfloat16, device=dev) for _ in range(P)]
    for chunk in (512 << 10, 1 << 20, 2 << 20):
        D = max(4, min(64, (32 << 20) // chunk))
        for lead in (D, D // 2, D // 4):
            point("ag_8x1GiB", L(A.SHARD, z, S // 2), L(A.GATHERED, o, S // 2), A.OP_COPY, 3,
                  chunk_bytes=chunk, snac_lead=lead)


def ring_sweep(A, synth, torch, dev):
    """Ring depth of the staged AllGather (the SNAC slots; the lead is half
    the depth, pieces the default), cold as in snac_sweep: 8 x 64 MiB and
    8 x 1 GiB partitions, chunks of 512 KiB, 1 MiB and 2 MiB, depths 2, 4, 8
    and the library's default (a 32 MiB ring)."""
    P, MiB = 8, 1 << 20
    L = A.layout
    scrub_a = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev)
    scrub_b = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev)
    for S, reps in ((64 * MiB, 7), (1024 * MiB, 3)):
        z = [torch.empty(S // 2, dtype=torch.bfloat16, device=dev).uniform_(-1, 1) for _ in range(P)]
        o = [torch.empty(P * S // 2, dtype=torch.bfloat16, device=dev) for _ in range(P)]
        li, lo = L(A.SHARD, z, S // 2), L(A.GATHERED, o, S // 2)
        for chunk in (512 << 10, 1 << 20, 2 << 20):
            for D in (2, 4, 8, 0):
                cfg = A.config(flags=A.F_STAGED, chunk_bytes=chunk, ring_slots=D)
                st, info = A.atom_plan_query(li, lo, A.OP_COPY, cfg)
                assert st == A.OK, (S, chunk, D, st)
                A.atom_collective(li, lo, A.OP_COPY, cfg)
                ts = []
                for _ in range(reps):
                    scrub_b.copy_(scrub_a)
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record()
                    A.atom_collective(li, lo, A.OP_COPY, cfg)
                    b.record()
                    torch.cuda.synchronize()
                    ts.append(a.elapsed_time(b))
                assert A.atom_sync_status() == A.OK, (S, chunk, D)
                ms = float(np.median(ts))
                print(json.dumps({"ring_sweep": f"ag_8x{S >> 20}MiB", "chunk_bytes": chunk,
                                  "ring_slots": int(info.ring_slots), "default_depth": D == 0,
                                  "lead": int(info.snac_lead), "workgroups": int(info.num_wgs),
                                  "ms": round(ms, 4),
                                  "GBps": round(info.credited_bytes / ms / 1e6, 1)}), flush=True)
        del z, o


def sweep(A, synth, torch, dev):
    """Message-size sweeps of the pages' collective benchmarks (one JSON line
    per point): AllGather of 8 partitions from 8 KiB to 1 GiB each, zero
    staging and SNAC with 512 KiB, 1 MiB and 2 MiB chunks; ReduceScatter,
    the fused and SNAC AllReduce and the uniform AllToAll of 8 inputs from
    8 KiB to 256 MiB each; the ReduceScatterV and AllGatherV with Zipf(0.125)
    partitions in units of 8 and of 1 element, zero-staging and staged, at
    16, 64 and 256 MiB per input (output); the MoE route, dispatch and
    combine for 1 to 4096 tokens per rank (256 experts, top-8, 7168-wide
    rows).
    Median of event-timed launches (more samples for small messages); GB/s
    on credited bytes. Where one call's footprint is under 1 GiB, successive
    launches rotate over several disjoint buffer sets (at least 4, enough for
    1 GiB up to 64) so that the 256 MB memory-side cache does not serve a
    call from the one before."""
    P = 8
    L = A.layout
    stream = torch.cuda.current_stream()

    def view(t, a, b):
        """t[a:b], refusing a slice that would run past the allocation (the
        library takes bare pointers and sizes)."""
        if b > t.numel():
            raise ValueError(f"view [{a}, {b}) past a buffer of {t.numel()} elements")
        return t[a:b]

    def nsets(footprint):
        return 1 if footprint >= (1 << 30) else min(64, max(4, -(-(1 << 30) // footprint)))

    def timed(fns, nbytes):
        fns = fns if isinstance(fns, list) else [fns]
        reps = 200 if nbytes < (1 << 24) else (20 if nbytes < (1 << 30) else 5)
        reps = max(reps, len(fns))
        for fn in fns + fns[:3]:
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for i, (a, b) in enumerate(ev):
            a.record(stream)
            fns[i % len(fns)]()
            b.record(stream)
        torch.cuda.synchronize()
        assert A.atom_sync_status() == A.OK
        return float(np.median([a.elapsed_time(b) for a, b in ev]))

    def emit(coll, mode, size, ms, credited, unit="bytes_per_rank"):
        print(json.dumps({"sweep": coll, "mode": mode, unit: size,
                          "us": round(ms * 1e3, 2), "GBps": round(credited / ms / 1e6, 1),
                          "frac_hbm": round(credited / ms / 1e6 * 1e9 / HBM_PEAK, 4)}), flush=True)

    # AllGather: inputs and outputs for the largest size, smaller sizes use views
    top = 1 << 30
    z = [torch.empty(top // 2, dtype=torch.bfloat16, device=dev).uniform_(-1, 1) for _ in range(P)]
    out = [torch.empty(P * top // 2, dtype=torch.bfloat16, device=dev) for _ in range(P)]
    size = 8 << 10
    while size <= top:
        n = size // 2
        cred = (1 + P) * P * size
        sets = [(L(A.SHARD, [view(t, i * n, (i + 1) * n) for t in z], n),
                 L(A.GATHERED, [view(t, i * P * n, (i + 1) * P * n) for t in out], n))
                for i in range(nsets(cred))]
        emit("allgather", "zero-staging", size,
             timed([lambda l=l: A.atom_collective(l[0], l[1], A.OP_COPY) for l in sets], size * P), cred)
        for chunk in (512 << 10, 1 << 20, 2 << 20):
            cfg = A.config(flags=A.F_STAGED, chunk_bytes=chunk)
            emit("allgather", f"snac_{chunk >> 10}KiB", size,
                 timed([lambda l=l: A.atom_collective(l[0], l[1], A.OP_COPY, cfg) for l in sets],
                       size * P), cred)
        size *= 2
    del z, out
    torch.cuda.empty_cache()
    # ReduceScatter / AllReduce of P inputs of `size` bytes each
    top = 256 << 20
    x = [torch.randn(top // 2, dtype=torch.float32, device=dev).to(torch.bfloat16) for _ in range(P)]
    ys = [torch.empty(top // 2 // P, dtype=torch.bfloat16, device=dev) for _ in range(P)]
    ar = [torch.empty(top // 2, dtype=torch.bfloat16, device=dev) for _ in range(P)]
    size = 8 << 10
    while size <= top:
        n = size // 2 // P
        m = P * n                                   # elements per rank
        cred_ar = 2 * P * P * n * 2
        sets = []
        for i in range(nsets(cred_ar)):
            lin = L(A.PARTITIONED, [view(t, i * m, (i + 1) * m) for t in x], n)
            sets.append((lin, L(A.SHARD, [view(t, i * n, (i + 1) * n) for t in ys], n),
                         L(A.GATHERED, [view(t, i * m, (i + 1) * m) for t in ar], n),
                         L(A.TRANSPOSED, [view(t, i * m, (i + 1) * m) for t in ar], n)))
        emit("reducescatter", "zero-staging", size,
             timed([lambda l=l: A.atom_collective(l[0], l[1], A.OP_SUM) for l in sets], size * P),
             (P + 1) * P * n * 2)
        emit("allreduce", "fused", size,
             timed([lambda l=l: A.atom_collective(l[0], l[2], A.OP_SUM) for l in sets], size * P), cred_ar)
        for chunk in (512 << 10, 1 << 20, 2 << 20):
            cfg = A.config(flags=A.F_STAGED, chunk_bytes=chunk)
            emit("allreduce", f"snac_{chunk >> 10}KiB", size,
                 timed([lambda l=l: A.atom_collective(l[0], l[2], A.OP_SUM, cfg) for l in sets],
                       size * P), cred_ar)
        # uniform AllToAll of the same inputs (partition j of every source to j)
        emit("alltoall", "zero-staging", size,
             timed([lambda l=l: A.atom_collective(l[0], l[3], A.OP_COPY) for l in sets], size * P), cred_ar)
        size *= 2
    # the uniform AllToAll of 8 x 4096 rows of 7168 bf16 (512 rows from every
    # source to every destination), plain and as a V call with uniform counts
    H = synth.HIDDEN
    rows = 512
    m = P * rows * H
    C = np.full((P, P), rows, dtype=np.int64)
    sets = [(L(A.PARTITIONED, [view(t, i * m, (i + 1) * m) for t in x], rows * H),
             L(A.TRANSPOSED, [view(t, i * m, (i + 1) * m) for t in ar], rows * H),
             L(A.PARTITIONED, [view(t, i * m, (i + 1) * m) for t in x], 0, C, H),
             L(A.TRANSPOSED, [view(t, i * m, (i + 1) * m) for t in ar], 0, None, H))
            for i in range(nsets(2 * P * m * 2))]
    emit("alltoall", "uniform", rows * H * 2 * P,
         timed([lambda l=l: A.atom_collective(l[0], l[1], A.OP_COPY) for l in sets], m * 2 * P),
         2 * P * m * 2)
    emit("alltoall", "v_uniform_counts", rows * H * 2 * P,
         timed([lambda l=l: A.atom_collective(l[2], l[3], A.OP_COPY) for l in sets], m * 2 * P),
         2 * P * m * 2)
    # Zipf(0.125) partitions (Figure 16): the ReduceScatterV of the 8 inputs
    # and the AllGatherV of the same total into the 8 outputs, partitions
    # counted in units of 8 elements and of single elements (partitions off
    # 16-byte alignment: the shifted vector path), zero-staging and staged.
    top_n = top // 2
    zv_all = torch.empty(top_n, dtype=torch.bfloat16, device=dev).uniform_(-1, 1)
    yv_all = [torch.empty(top_n, dtype=torch.bfloat16, device=dev) for _ in range(P)]
    size = 16 << 20
    while size <= top:
        N = size // 2                                   # elements per input / output
        for unit in (8, 1):
            cnt = synth.zipf_partition(N, P, 0.125, unit) // unit
            offs = np.concatenate([[0], np.cumsum(cnt * unit)])
            cred_rs = (P + 1) * N * 2
            cred_ag = (P + 1) * N * 2
            sets = []
            for i in range(nsets(cred_ag)):
                lo_i = i * N
                xs_v = [view(t, lo_i, lo_i + N) for t in x]
                ys_v = [view(yv_all[k], lo_i, lo_i + int(cnt[k]) * unit) for k in range(P)]
                zs_v = [view(zv_all, lo_i + int(offs[k]), lo_i + int(offs[k + 1])) for k in range(P)]
                os_v = [view(t, lo_i, lo_i + N) for t in ar]
                sets.append((L(A.PARTITIONED, xs_v, 0, cnt, unit), L(A.SHARD, ys_v, 0, None, unit),
                             L(A.SHARD, zs_v, 0, cnt, unit), L(A.GATHERED, os_v, 0, None, unit)))
            for mode, cfg in (("zero-staging", None), ("snac", A.config(flags=A.F_STAGED))):
                emit("reducescatterv_zipf", f"{mode}_unit{unit}", size,
                     timed([lambda l=l, c=cfg: A.atom_collective(l[0], l[1], A.OP_SUM, c) for l in sets],
                           size * P), cred_rs)
                emit("allgatherv_zipf", f"{mode}_unit{unit}", size,
                     timed([lambda l=l, c=cfg: A.atom_collective(l[2], l[3], A.OP_COPY, c) for l in sets],
                           size * P), cred_ag)
        size *= 4
    del x, ys, ar, zv_all, yv_all
    torch.cuda.empty_cache()
    # MoE route, dispatch and combine by tokens per rank (256 experts, top-8,
    # 7168-wide bf16 rows): decode-sized batches up to prefill-sized ones
    E, k, H = synth.MOE_EXPERTS, synth.MOE_TOPK, synth.HIDDEN
    for T in (1, 4, 16, 64, 256, 1024, 4096):
        ids, w = synth.moe_routing(6, P, T, E, k)
        rt = A.moe_alloc_routing([torch.from_numpy(a).to(dev) for a in ids], E, k)
        A.atom_moe_route(rt)
        cap = max(int(rt.recv_t.max().item()), 1)
        xs = [torch.randn(T * H, device=dev).to(torch.bfloat16) for _ in range(P)]
        ws = [torch.from_numpy(a).to(dev) for a in w]
        disp = [torch.empty(cap * H, dtype=torch.bfloat16, device=dev) for _ in range(P)]
        outs = [torch.empty(T * H, dtype=torch.bfloat16, device=dev) for _ in range(P)]
        mb = moe_bytes(P, T, E, k, H * 2)
        emit("moe", "route", T, timed(lambda: A.atom_moe_route(rt), 1), mb["route"], "tokens_per_rank")
        emit("moe", "dispatch", T, timed(lambda: A.atom_moe_dispatch(rt, xs, disp, cap, H), mb["dispatch"] // P),
             mb["dispatch"], "tokens_per_rank")
        emit("moe", "combine", T, timed(lambda: A.atom_moe_combine(rt, disp, ws, outs, cap, H), mb["combine"] // P),
             mb["combine"], "tokens_per_rank")


def ceilings(torch, dev):
    """Cold HBM rates of the traffic patterns the Atom kernels move, measured
    with libatom_ceiling.so's kernels (one tile per workgroup, non-temporal
    loads and stores): streaming read and write of 2 GiB, a 2 GiB copy, the
    1 -> 8 fan-out of 256 MiB into 8 separate allocations (stores in order,
    and rotated by tile), the same 8 x 256 MiB as pure writes, the fan-out
    in blocked order (one output at a time per block of 1-64 MiB, the source
    block loaded once per output) and the fan-out into one allocation at
    spacings of exactly 256 MiB and 256 MiB plus 4352 bytes. A 1 GiB streaming fill of another buffer precedes each
    run, so no run starts with the previous one's data or dirty lines in the
    caches; the median of 7 runs, event-timed, is reported."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "reduce_atom_03_amd", "libatom_ceiling.so"))
    vp = ctypes.c_void_p
    lib.ceil_fill.argtypes = [vp, ctypes.c_int64, ctypes.c_int, ctypes.c_int, vp]
    lib.ceil_read.argtypes = [vp, ctypes.c_int64, vp, ctypes.c_int, ctypes.c_int, vp]
    lib.ceil_fanout.argtypes = [ctypes.POINTER(vp), ctypes.c_int, vp, ctypes.c_int64, ctypes.c_int,
                                ctypes.c_int, ctypes.c_int, vp]
    lib.ceil_fanout_blocked.argtypes = [ctypes.POINTER(vp), ctypes.c_int, vp, ctypes.c_int64,
                                        ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    stream = torch.cuda.current_stream()
    sp = int(stream.cuda_stream)
    GiB, MiB256 = 1 << 30, 256 << 20

    def buf(nbytes):
        return torch.empty(nbytes, dtype=torch.uint8, device=dev)

    flush_buf = buf(GiB)
    big_a, big_b = buf(2 * GiB), buf(2 * GiB)
    big_b.fill_(1)
    sink = buf(256)
    outs = [buf(MiB256) for _ in range(8)]
    one = buf(8 * MiB256 + 8 * 4352)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def chk(rc):
        if rc != 0:
            raise RuntimeError(f"ceiling kernel refused its arguments or failed ({rc})")

    def timeit(fn, nbytes, **point):
        t = []
        for _ in range(7):
            chk(lib.ceil_fill(flush_buf.data_ptr(), GiB, 256, 4, sp))
            e0.record(stream)
            chk(fn())
            e1.record(stream)
            e1.synchronize()
            t.append(e0.elapsed_time(e1))
        ms = float(np.median(t))
        print(json.dumps({"ceiling": point.pop("pattern"), **point, "bytes": int(nbytes),
                          "ms": round(ms, 4), "GBps": round(nbytes / ms / 1e6, 1),
                          "frac_hbm": round(nbytes / ms / 1e6 * 1e9 / HBM_PEAK, 4)}), flush=True)

    def ptrs(ts):
        return (vp * len(ts))(*[int(t) if isinstance(t, int) else t.data_ptr() for t in ts])

    for lanes in (64, 256):
        for U in (1, 2, 4):
            timeit(lambda: lib.ceil_read(big_b.data_ptr(), 2 * GiB, sink.data_ptr(), lanes, U, sp),
                   2 * GiB, pattern="read", lanes=lanes, U=U)
            timeit(lambda: lib.ceil_fill(big_a.data_ptr(), 2 * GiB, lanes, U, sp),
                   2 * GiB, pattern="write", lanes=lanes, U=U)
            dst = ptrs([big_a])
            timeit(lambda: lib.ceil_fanout(dst, 1, big_b.data_ptr(), 2 * GiB, 0, lanes, U, sp),
                   4 * GiB, pattern="copy", lanes=lanes, U=U)
    src = big_b.data_ptr()
    sep = ptrs(outs)
    for lanes, U in ((64, 1), (64, 2), (256, 1)):
        for rot in (0, 1):
            timeit(lambda: lib.ceil_fanout(sep, 8, src, MiB256, rot, lanes, U, sp), 9 * MiB256,
                   pattern="fanout8", lanes=lanes, U=U, rotate=rot, dst="8 allocations")
            timeit(lambda: lib.ceil_fanout(sep, 8, None, MiB256, rot, lanes, U, sp), 8 * MiB256,
                   pattern="write8", lanes=lanes, U=U, rotate=rot, dst="8 allocations")
    # Blocked order: the chip writes one output at a time, block by block, and
    # loads each source tile once per output (streaming loads, or ordinary
    # ones that leave the block in the caches for the next output's loads).
    for lanes, U in ((64, 1), (256, 1), (256, 2)):
        for block in (1 << 20, 4 << 20, 16 << 20, 64 << 20):
            for cached in (0, 1):
                timeit(lambda: lib.ceil_fanout_blocked(sep, 8, src, MiB256, block, cached, lanes, U, sp),
                       9 * MiB256, pattern="fanout8_blocked", lanes=lanes, U=U, block=block,
                       cached_loads=cached, dst="8 allocations")
    base = one.data_ptr()
    base += (-base) % 4096
    for spacing in (MiB256, MiB256 + 4352):
        d = ptrs([base + q * spacing for q in range(8)])
        timeit(lambda: lib.ceil_fanout(d, 8, src, MiB256 - 4096, 0, 64, 1, sp), 9 * (MiB256 - 4096),
               pattern="fanout8", lanes=64, U=1, rotate=0, dst=f"one allocation, spacing {spacing}")


def measured_traffic(row):
    """HBM bytes per launch of `row` from the committed rocprofv3 counter
    summary (bytes leaving the L2s, from the TCC_EA0 read and write request
    counters by request size; the 256 MiB copy reads 1.0001x its bytes with
    no calibration), or None when the summary is missing or any kernel
    source changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    csrc = os.path.join(ROOT, "reduce_atom_03_amd", "csrc")
    hashes = d.get("sources", {})
    if set(hashes) != set(os.listdir(csrc)):     # every source file must be covered
        return None
    for fn, h in hashes.items():
        src = os.path.join(csrc, fn)
        try:
            with open(src, "rb") as f:
                if hashlib.sha256(f.read()).hexdigest()[:16] != h:
                    return None
        except OSError:
            return None
    row_d = d.get("rows", {}).get(row)
    return int(row_d["traffic_bytes"]) if row_d else None


def moe_bytes(P, T, E, k, row_bytes):
    """Algorithmic bytes of the MoE rows. Route: the ids read, the positions
    written, the counts and rows-received written. Dispatch: each token row
    read once and written once per choice, plus the ids and positions read.
    Combine: each choice's row read once and the token row written once, plus
    the ids, positions and weights read."""
    n = P * T * k
    return {"route": n * 8 + P * E * 4 + P * 8,
            "dispatch": P * T * (k + 1) * row_bytes + n * 8,
            "combine": P * T * (k + 1) * row_bytes + n * 12}


def c1_oracle_ms(c1):
    """The oracle's P = 4 ReduceScatter (4 x 65536 fp32 per input) on this
    host: median of 100 calls, with the threads it used and on one thread."""
    import oracle
    def med(reps=100):
        t = []
        for _ in range(reps):
            t0 = time.perf_counter()
            oracle.reduce_scatter(c1)
            t.append(time.perf_counter() - t0)
        return float(np.median(t)) * 1e3
    cores = oracle.threads()
    many = med()
    oracle.set_threads(1)
    try:
        one = med()
    finally:
        oracle.set_threads(cores)
    return {"ms": round(many, 4), "cores": cores, "ms_one_core": round(one, 4)}


def cpu_baseline(args, C3, S, credited):
    """The oracle, as it stands, on the same step (same seeds and shapes, its
    own OpenMP threads, then once on one thread); GB/s on the same credited
    bytes, with the host's CPU count, model and memory."""
    import oracle
    from reduce_atom_03_amd import synth
    log("timing the CPU oracle ...")
    P = 8
    c1 = synth.c1_inputs()
    c2 = synth.c2_inputs()
    c3 = synth.c3_inputs()
    z4 = synth.c4_inputs(S, P)
    x5 = {b: synth.c5_inputs(b) for b in (1, 2, 4, 8, 16)}
    z8 = synth.c4_inputs(8 << 10, P)
    cnt_rs = synth.zipf_partition(1 << 27, P, 0.125, 8) // 8
    cnt_ag = synth.zipf_partition(P * S // 2, P, 0.125, 8) // 8
    zv = [synth.draw(4, k, int(cnt_ag[k]) * 8, "uniform", synth.BF16) for k in range(P)]
    moe_ids, moe_w = synth.moe_routing(6, P, synth.MOE_TOKENS, synth.MOE_EXPERTS, synth.MOE_TOPK)
    moe_x = synth.moe_inputs()
    def step():
        t = time.perf_counter()
        oracle.all_gather([c2[0]])          # P = 1 AllGather: a copy
        oracle.reduce_scatter(c1)
        oracle.reduce_scatter(c2)
        oracle.all_reduce(c2)
        oracle.all_to_all_v(c3, C3, synth.HIDDEN)
        oracle.all_gather(z4)
        if args.snac:
            oracle.all_gather(z4)
            oracle.all_reduce(c2)
        for b in (1, 2, 4, 8, 16):
            oracle.all_reduce(x5[b])
        oracle.reduce_scatter_v(c2, cnt_rs * 8)
        oracle.all_gather_v(zv)
        if args.snac:
            oracle.reduce_scatter_v(c2, cnt_rs * 8)
            oracle.all_gather_v(zv)
        oracle.all_gather(z8)
        E, k, H = synth.MOE_EXPERTS, synth.MOE_TOPK, synth.HIDDEN
        pos, _, recv = oracle.moe_route(moe_ids, E, k)
        disp = oracle.moe_dispatch(moe_x, moe_ids, pos, E, k, H, int(recv.max()))
        oracle.moe_combine(disp, moe_ids, pos, moe_w, E, k, H, int(recv.max()))
        return time.perf_counter() - t

    best = float(np.median([step() for _ in range(args.cpu_reps)]))
    cores = oracle.threads()
    oracle.set_threads(1)                   # the same step once on one core
    try:
        one = step()
    finally:
        oracle.set_threads(cores)
    return {"value": round(credited / best / 1e9, 2), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"the full step (same shapes and seeds), median of {args.cpu_reps} runs, "
                      f"{best:.2f} s per step",
            "one_core": {"value": round(credited / one / 1e9, 2), "unit": "GB/s",
                         "sample": f"the same step once on 1 thread, {one:.2f} s"},
            "host": host_info()}


def host_info():
    """The host the oracle ran on: logical CPUs, CPU model, memory."""
    info = {"nproc": os.cpu_count()}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemTotal:"):
                    info["mem_gib"] = round(int(line.split()[1]) / (1 << 20), 1)
                    break
    except OSError:
        pass
    return info


if __name__ == "__main__":
    main()
