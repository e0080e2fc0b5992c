#!/usr/bin/env python
"""Benchmark of the mixed-depth weight-read hot path on one MI355X.

A step is one pass of the hot path over one batch of synthetic input:
build the per-block level map from the lens rules, then read every matrix of
the workload at its blocks' depths.  For a weight field both happen in one
grouped launch (every wavefront computes its block's rung, writes it to the
map and reads the block at that depth); --separate-map gives the map its own
launch first.  Steps are issued eagerly and timed by the wall clock.
Packing is offline and untimed.  Inputs are resident in HBM before the timed
region starts.

Default workload: the large streaming layer stack (8 layers of 8192x28672
and 28672x8192 int8, 4,608 blocks of 64 rows, block coordinates uniform on
the unit square, 4 lenses, g = 1, glass D2, sum, focus_area calibrated by the
oracle to a mean of 4.0 bits/weight), batch 1: the largest workload that fits
one GPU.  The same run reports, as extra keys, the Gemma-E2B-scale weight
field at 4.0 bits (30 synthetic decoder layers, 9,360 blocks) and the
Qwen3-0.6B-shaped decode (tokens/s), each beside the CPU oracle.

Prints ONE JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
CALIBRATION = os.path.join(ROOT, "tests", "golden", "calibration.json")
COUNTERS = os.path.join(ROOT, "profiles", "hbm_counters.json")
KERNEL_SRC = os.path.join(ROOT, "query_adaptive_mixed_amd", "csrc", "qmatvec.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash(src: str = KERNEL_SRC) -> str:
    with open(src, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def measured_traffic(key: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current source of the kernel they measure (else None)."""
    try:
        with open(COUNTERS) as fh:
            d = json.load(fh)
    except (OSError, ValueError):
        return None
    ent = d.get(key)
    if not ent:
        return None
    src = os.path.join(ROOT, "query_adaptive_mixed_amd", "csrc", ent.get("kernel_src", "qmatvec.hip"))
    if ent.get("kernel_sha") != kernel_hash(src):
        return None
    return ent.get("bytes_per_launch")


# ----------------------------------------------------------------- workloads

def build_field(fld, lens, B, torch, Q, dev, sample_blocks=0):
    """Pack every matrix of a field; returns (items, algorithmic byte counts).
    With sample_blocks > 0 the codes of each matrix's first sample_blocks
    blocks are kept on the host (the CPU oracle's bounded sample)."""
    coords = torch.from_numpy(fld.coords).to(dev)
    lv = Q.build_level_map(coords, lens.centres, lens.radii, lens.f, lens.g, lens.combine, lens.glass)
    torch.cuda.synchronize()
    lv_h = lv.cpu().numpy()
    items, sample = [], []
    wbytes = other = 0
    offs = fld.block_offsets()
    t0 = time.time()
    for i, m in enumerate(fld.matrices):
        Wh = fld.codes(i)
        if sample_blocks > 0:
            sample.append(Wh[:64 * min(sample_blocks, m.n_blocks)].copy())
        W = torch.from_numpy(Wh).to(dev)
        del Wh
        sc = torch.from_numpy(fld.scales(i)).to(dev)
        pm = Q.pack_slices(W, sc)
        del W
        x = torch.from_numpy(fld.x(i, B)).to(dev)
        y = torch.empty((B, m.N), dtype=torch.float32, device=dev)
        sub = lv[offs[i]:offs[i] + m.n_blocks]
        items.append((pm, x, y, sub, coords[offs[i]:offs[i] + m.n_blocks]))
        mb, wb = Q.map_weight_bytes(lv_h[offs[i]:offs[i] + m.n_blocks], m.K)
        wbytes += wb
        nz = int(np.count_nonzero(lv_h[offs[i]:offs[i] + m.n_blocks]))
        other += nz * 64 * 4 + B * m.K * 4 + B * m.N * 4 + m.n_blocks
        if i % 30 == 0 or len(fld.matrices) <= 16:
            log(f"  packed {i + 1}/{len(fld.matrices)} matrices ({time.time() - t0:.1f} s)")
    torch.cuda.synchronize()
    return coords, lv, lv_h, items, wbytes, other, sample


def run_field(args, torch, Q, WL, workload=None, batch=None, sample_blocks=0):
    """A weight field's step at its calibrated map; workload / batch default
    to the command line's."""
    workload = workload or args.workload
    batch = batch or args.batch
    dev = torch.device("cuda:0")
    cal = json.load(open(CALIBRATION))
    if workload == "e2b_field":
        fld = WL.e2b_field(0)
        c = cal["e2b_field"]
        f = c["target_4.0"]["f"] if args.mean_bits == 4.0 else 0.5
        lens = WL.e2b_lenses(fld, f=f, g=c["g"])
        desc = "e2b_field: 30 layers x {q,k,v,o 1536x1536; gate,up 6144x1536; down 1536x6144} int8, 9360 blocks"
    else:
        fld = WL.streaming_stack(0)
        c = cal["streaming_stack"][f"glass{args.glass}_target{float(args.mean_bits)}"]
        cen, rad = WL.stack_lenses(fld)
        lens = WL.LensParams(centres=cen, radii=rad, f=c["f"], g=1.0, combine="sum", glass=args.glass)
        desc = "streaming_stack: 8 x {8192x28672, 28672x8192} int8, 4608 blocks"
    log(f"workload {desc}; f={lens.f:.6f} g={lens.g} glass={lens.glass}")
    coords, lv, lv_h, items, wbytes, other, sample = build_field(fld, lens, batch, torch, Q, dev, sample_blocks)
    w = fld.block_weights()
    if args.uniform_map:
        # the same mean bits with every block at one depth (3 bits: D2 and D4
        # alternating by block parity, every matrix having an even block count)
        mb = float(args.mean_bits)
        if mb == 3.0:
            u = np.where(np.arange(fld.n_blocks) % 2 == 0, 1, 2).astype(np.uint8)
        else:
            u = np.full(fld.n_blocks, int(mb) // 2, np.uint8)
        lv.copy_(torch.from_numpy(u).to(dev))
        lv_h = u
        offs = fld.block_offsets()
        wbytes = other = 0
        for i, m in enumerate(fld.matrices):
            ui = u[offs[i]:offs[i] + m.n_blocks]
            wbytes += Q.map_weight_bytes(ui, m.K)[1]
            other += int(np.count_nonzero(ui)) * 64 * 4 + batch * (m.K + m.N) * 4 + m.n_blocks
        desc += f"; uniform map at {mb:g} bits (no lenses)"
    mean_bits = float(np.sum(w * np.array(Q.LADDER_BITS)[lv_h]) / np.sum(w))
    group = Q.GroupedQmatvec(items, device=dev, tuning=json.loads(args.tuning) if args.tuning else None)
    rules = Q.LensRules(lens.centres, lens.radii, lens.f, lens.g, lens.combine, lens.glass)
    # a lens map on the staged route is built inside the product launch (one
    # launch per step): each block's coordinates are read (16 bytes) and its
    # rung written, in place of reading the rung
    fused = not args.uniform_map and not args.separate_map and group.route == "staged"
    if fused:
        other += 16 * fld.n_blocks

    def build_map():
        if not args.uniform_map:
            Q.build_level_map(coords, None, None, None, None, out=lv, rules=rules)

    def step():
        if fused:
            group.run_lens(rules)
        else:
            build_map()
            group.run()

    # Kernel durations from HIP events on the stream the kernels run on: the
    # map launch alone (events around it), and the product launch from events
    # the launch itself records at the kernel's start and end (events around
    # a launch would add the dispatch latency ahead of it), or, for a two-
    # kernel launch, the spacing of events after back-to-back launches.
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = []
    for _ in range(args.steps):
        a, b = (torch.cuda.Event(enable_timing=True) for _ in range(2))
        a.record()
        build_map()
        b.record()
        ev.append((a, b))
    torch.cuda.synchronize()
    map_ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
    import ctypes as C
    from query_adaptive_mixed_amd import _lib as L
    if fused:
        times = (C.c_float * args.steps)()
        L.check(L.lib().qam_group_lens_launch_times(
            C.byref(group.desc), rules.lenses, rules.n_lenses, C.byref(rules.params), C.cast(rules.ladder, C.c_void_p),
            rules.n_rungs, rules.glass, args.steps, C.cast(times, C.c_void_p),
            C.c_void_p(torch.cuda.current_stream().cuda_stream)))
        kern_ms = float(np.median(list(times)))
        kern_timing = ("median over launches of HIP events recorded at the kernel's start and end "
                       "(hipExtLaunchKernel); the launch builds the level map and runs the product")
    elif group.route == "staged":
        # HIP events recorded at the kernel's own start and end (one launch each)
        times = (C.c_float * args.steps)()
        L.check(L.lib().qam_group_launch_times(C.byref(group.desc), args.steps, C.cast(times, C.c_void_p),
                                                C.c_void_p(torch.cuda.current_stream().cuda_stream)))
        kern_ms = float(np.median(list(times)))
        kern_timing = "median over launches of HIP events recorded at the kernel's start and end (hipExtLaunchKernel)"
    else:
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        group.run()
        marks[0].record()
        for i in range(args.steps):
            group.run()
            marks[i + 1].record()
        torch.cuda.synchronize()
        kern_ms = float(np.median([marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)]))
        kern_timing = "median spacing of HIP events recorded after each of back-to-back launches"

    # The byte-budget regulator on this field (outside the timed step): the
    # largest focus area whose map reads at most the bytes of a 4-bit mean.
    regulator = None
    if not args.uniform_map:
        wt = torch.from_numpy(fld.block_weights().astype(np.int64)).to(dev)
        budget = int(np.sum(fld.block_weights())) * 4 // 8
        torch.cuda.synchronize()
        r0 = time.perf_counter()
        f_fit, b_fit, _ = Q.fit_focus_area(coords, wt, lens.centres, lens.radii, lens.g, budget,
                                           combine=lens.combine, glass=lens.glass, iters=40)
        regulator = {"budget_bytes": budget, "focus_area_f": f_fit, "bytes": b_fit, "bisection_steps": 40,
                     "ms": round((time.perf_counter() - r0) * 1e3, 3)}

    # Whole-step throughput: wall clock over K steps issued from the host (map
    # + grouped product each), so the host's per-call overhead is inside the
    # timed region wherever the host falls behind the GPU.  With --graph, one
    # step captured as a HIP graph and replayed instead (on this stack each
    # replay leaves the GPU idle for about 8.5 us between steps, where eager
    # launches queue back to back).
    graph = None
    if args.graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(args.warmup):
            graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert np.array_equal(lv.cpu().numpy(), lv_h), "level map changed between steps"
    ms = wall * 1e3 / args.steps
    # lens coverage: the share of blocks lifted above the glass (the stack's
    # workload names lenses covering 10-60% of blocks; points outside that
    # range are flagged, not dropped)
    lifted = lv_h > lens.glass
    coverage = {"blocks_lifted_fraction": round(float(np.mean(lifted)), 6),
                "weights_lifted_fraction": round(float(np.sum(w[lifted]) / np.sum(w)), 6),
                "within_10_60_percent": bool(0.10 <= float(np.mean(lifted)) <= 0.60)}
    return dict(desc=desc, mean_bits=mean_bits, wbytes=wbytes, other=other, ms=ms, kern_ms=kern_ms, map_ms=map_ms,
                kern_timing=kern_timing, fused=fused, regulator=regulator, coverage=coverage, sample=sample,
                batch=batch, workload=workload,
                variant=Q.last_variant(), lens=lens, fld=fld, lv_h=lv_h, n_items=len(items),
                key=f"{workload}_{args.mean_bits}_g{lens.glass}_b{batch}" + ("_uniform" if args.uniform_map else "")
                + ("_lens" if fused else ""))


# ----------------------------------------------------------------- batched per-request layer

MALL_BYTES = 256 << 20   # MI355X Infinity Cache


def n_rotation_copies(step_bytes: int) -> int:
    """Copies of a working set to rotate through so that more than twice the
    256 MB Infinity Cache passes between two reads of one copy."""
    return max(2, int(math.ceil(2 * MALL_BYTES / max(step_bytes, 1))) + 1)


class Rotate:
    """Calls fns[0], fns[1], ... in turn, one per call."""

    def __init__(self, fns):
        self.fns, self.i = list(fns), 0

    def __call__(self):
        fn = self.fns[self.i]
        self.i = (self.i + 1) % len(self.fns)
        return fn()


def run_batched(args, torch, Q, WL):
    """One layer (4096x4096, 14336x4096, 4096x14336) for B requests, each with
    its own level map from 3 lenses (f calibrated per request to a mean of 4
    bits): one grouped matrix-core launch pair (limb pre-pass + product).
    Every block is read once, to the deepest slice any request needs."""
    dev = torch.device("cuda:0")
    cal = json.load(open(CALIBRATION))["batched_layer"]
    fld = WL.batched_layer(0)
    B = args.batch
    reqs = WL.request_lenses(fld, B)
    coords = torch.from_numpy(fld.coords).to(dev)
    maps = torch.empty((B, fld.n_blocks), dtype=torch.uint8, device=dev)
    fs = [cal["requests"][r]["f"] for r in range(B)]
    sets = Q.LensSets(reqs, fs, g=1.0, combine="sum", glass=1)

    def build_maps():
        Q.build_level_maps(coords, out=maps, sets=sets)

    build_maps()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(10):
        build_maps()
    torch.cuda.synchronize()
    map_ms = (time.perf_counter() - t0) * 1e3 / 10
    lv = maps.cpu().numpy()
    offs = fld.block_offsets()
    bits = np.array(Q.LADDER_BITS)
    union = per_req = other = 0
    xdt = torch.bfloat16 if args.x_dtype == "bf16" else torch.float32
    xs, ys = [], []
    for i, m in enumerate(fld.matrices):
        xs.append(torch.from_numpy(fld.x(i, B)).to(dev).to(xdt).contiguous())
        ys.append(torch.empty((B, m.N), dtype=torch.float32, device=dev))
        sub = lv[:, offs[i]:offs[i] + m.n_blocks]
        union += int(np.sum(64 * m.K * bits[sub.max(axis=0)]) // 8)
        per_req += int(np.sum(64 * m.K * bits[sub]) // 8)
        nz = int(np.count_nonzero(sub.max(axis=0)))
        other += nz * 64 * 4 + B * m.K * xs[i].element_size() + B * m.N * 4 + B * m.n_blocks
    # copies of the layer's packed weights, run in turn, so that the layer a
    # step reads was last read more than 512 MB of traffic ago (out of the cache)
    n_copies = n_rotation_copies(union)
    groups = []
    for c in range(n_copies):
        items = []
        for i, m in enumerate(fld.matrices):
            pm = Q.pack_slices(torch.from_numpy(fld.codes(i)).to(dev), torch.from_numpy(fld.scales(i)).to(dev))
            items.append((pm, xs[i], ys[i], maps[:, offs[i]:offs[i] + m.n_blocks]))   # rows of the [B, 352] maps
        groups.append(Q.GroupedQmatvec(items, device=dev, tuning=json.loads(args.tuning) if args.tuning else None))
    torch.cuda.synchronize()
    run = Rotate([g.run for g in groups])
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    ev = []
    for _ in range(args.steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        run()
        b.record()
        ev.append((a, b))
    torch.cuda.synchronize()
    kern_ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
    group = groups[0]

    def step():
        build_maps()
        run()

    # eager launches timed by the wall clock (--graph: replays of a captured step)
    graph = None
    if args.graph:
        graphs = []
        for g in groups:
            def one(g=g):
                build_maps()
                g.run()
            st = torch.cuda.Stream()
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                one()
            torch.cuda.current_stream().wait_stream(st)
            torch.cuda.synchronize()
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                one()
            graphs.append(gr.replay)
        graph = Rotate(graphs)
    for _ in range(args.warmup):
        graph() if graph is not None else step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph() if graph is not None else step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    assert np.array_equal(maps.cpu().numpy(), lv), "level maps changed between steps"
    w = fld.block_weights()
    mean_req = float(np.mean([np.sum(w * bits[lv[r]]) / np.sum(w) for r in range(B)]))
    mean_union = float(np.sum(w * bits[lv.max(axis=0)]) / np.sum(w))
    flops = 2.0 * B * sum(m.N * m.K for m in fld.matrices)
    return dict(desc="batched_layer: {4096x4096, 14336x4096, 4096x14336} int8, 352 blocks, per-request maps",
                wbytes=union, per_req_bytes=per_req, other=other, ms=ms, kern_ms=kern_ms, map_ms=map_ms,
                mean_bits=mean_union, mean_bits_per_request=mean_req, variant=Q.last_variant(), flops=flops,
                n_items=3, n_copies=n_copies, key=f"batched_layer_b{B}_{args.x_dtype}")


def run_layer(args, torch, Q, WL):
    """The layer that decides its own depths, on the batched layer's three
    matrices for B requests: per matrix, the product at the glass (D2, a
    uniform map), the reduced scores and the share rule on the device (the
    top third of each request's blocks rise to D8: a mean of 4 bits per
    request), then the product at those per-request maps.  Timed beside the
    same products with the maps held fixed (the fixed mixed layout)."""
    dev = torch.device("cuda:0")
    fld = WL.batched_layer(0)
    B = args.batch
    rule = Q.LayerRule(share=1.0 / 3.0, g=1.0, glass=1)
    xs = [torch.from_numpy(fld.x(i, B)).to(dev).contiguous() for i in range(len(fld.matrices))]
    # copies of the layer run in turn: a step's weights were last read more
    # than 512 MB of traffic ago (the base pass and the refinement of a step
    # each read about 110-140 MB at these maps)
    n_copies = n_rotation_copies(sum(m.N * m.K for m in fld.matrices) // 2)
    grps = []
    for c in range(n_copies):
        items = []
        for i, m in enumerate(fld.matrices):
            pm = Q.pack_slices(torch.from_numpy(fld.codes(i)).to(dev), torch.from_numpy(fld.scales(i)).to(dev))
            items.append((pm, xs[i], torch.empty((B, m.N), dtype=torch.float32, device=dev)))
        grps.append(Q.LayerDecidesGroup(items, rule, device=dev))
    grp = grps[0]
    step, fixed, levels_only = Rotate([g.run for g in grps]), Rotate([g.second.run for g in grps]), grp.decide
    if args.graph:
        # each timed function as replays of its own captured graphs, one per copy
        def captured(fn):
            st = torch.cuda.Stream()
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                fn()
            torch.cuda.current_stream().wait_stream(st)
            torch.cuda.synchronize()
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                fn()
            return gr.replay
        step = Rotate([captured(g.run) for g in grps])
        fixed = Rotate([captured(g.second.run) for g in grps])

    def wall(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps

    step_ms = wall(step)
    lv = [l.cpu().numpy() for l in grp.levels]
    grp.base.run()            # the base outputs again (the refinement adds into them)
    ev = []
    for _ in range(args.steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        levels_only()
        b.record()
        ev.append((a, b))
    torch.cuda.synchronize()
    levels_ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
    assert all(np.array_equal(a.cpu().numpy(), l) for a, l in zip(grp.levels, lv)), "maps changed"
    fixed_ms = wall(fixed)
    bits = np.array(Q.LADDER_BITS)
    base_bytes = sum(m.N * m.K * 2 // 8 for m in fld.matrices)
    union = sum(int(np.sum(64 * m.K * bits[l.max(axis=0)]) // 8) for m, l in zip(fld.matrices, lv))
    above = sum(int(np.sum(64 * m.K * (bits[l.max(axis=0)] - bits[1])) // 8) for m, l in zip(fld.matrices, lv))
    w = fld.block_weights()
    allv = np.concatenate(lv, axis=1)
    mean_req = float(np.mean([np.sum(w * bits[allv[r]]) / np.sum(w) for r in range(B)]))
    return dict(step_ms=step_ms, fixed_ms=fixed_ms, levels_ms=levels_ms, base_bytes=base_bytes, n_copies=n_copies,
                union_bytes=above if grp.refine else union, fixed_bytes=union, refine=grp.refine, mean_bits_per_request=mean_req,
                mean_bits_union=float(np.sum(w * bits[allv.max(axis=0)]) / np.sum(w)))


# ----------------------------------------------------------------- decode

QWEN = dict(n_layers=28, hidden=1024, q_dim=2048, kv_dim=1024, ffn=3072, vocab=151936)


def run_decode(args, torch, Q, WL):
    """Qwen3-0.6B-shaped decode: T steps, each every block at D4 (top 4 bits),
    the 16% most uncertain steps (seeded synthetic scores) run again at D8.
    Each rung's step is one captured HIP graph of 4 x 28 + 1 fused products."""
    from query_adaptive_mixed_amd.decode import build_decoder
    c = QWEN
    T = args.decode_steps
    fld = WL.qwen_decode_field(0)
    t0 = time.time()
    dec = build_decoder(fld, c["n_layers"], c["hidden"], c["q_dim"], c["kv_dim"], c["ffn"], eps=1e-6,
                        target_waves=args.decode_waves, waves_per_block=args.decode_ksplit,
                        max_chunk_tiles=args.decode_max_chunk,
                        progress=lambda l: log(f"  packed layer {l + 1}/28 ({time.time() - t0:.1f} s)") if l % 7 == 6 else None)
    xs = torch.from_numpy(WL.decode_inputs(0, T, c["hidden"])).cuda()
    esc = Q.escalation_schedule(WL.escalation_scores(0, T), 0.16)
    n_esc = int(esc.sum())
    wb = {r: sum(64 * m.K * m.n_blocks * Q.LADDER_BITS[r] // 8 for m in fld.matrices) for r in (2, 4)}
    dec.capture(2)
    dec.capture(4)
    # per-rung step time: events around replays on the launch stream
    per = {}
    for rung in (2, 4):
        for _ in range(5):
            dec.hidden.copy_(xs[0])
            dec.replay(rung)
        ev = []
        for i in range(30):
            dec.hidden.copy_(xs[i % T])
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            dec.replay(rung)
            b.record()
            ev.append((a, b))
        torch.cuda.synchronize()
        per[rung] = float(np.median([a.elapsed_time(b) for a, b in ev]))
    # the decode run: T tokens, escalated steps re-run at D8
    for t in range(min(T, 8)):
        dec.hidden.copy_(xs[t])
        dec.replay(2)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(T):
        dec.hidden.copy_(xs[t])
        dec.replay(2)
        if esc[t]:
            dec.hidden.copy_(xs[t])
            dec.replay(4)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total = T * wb[2] + n_esc * wb[4]

    # The same decode with the gate decided on the device: the entropy of
    # each step's D4 output ([PoD]: escalate when the entropy is above a
    # threshold), the threshold set between the n_esc-th and the next largest
    # entropy of a first D4 pass so that the rate matches; per step the D4
    # graph, the gate launch, one small device-to-host read, then the D8
    # graph if the gate fired.
    gate = Q.Gate(dec.logits.numel())
    ents = []
    for t in range(T):
        dec.hidden.copy_(xs[t])
        dec.replay(2)
        gate.run(dec.logits)
        ents.append(gate.result()["entropy"])
    srt = sorted(ents, reverse=True)
    tau = 0.5 * (srt[n_esc - 1] + srt[n_esc]) if 0 < n_esc < T else (math.inf if n_esc == 0 else -math.inf)
    # the loop inside the library (one C call for all T steps) ...
    dec.decode_gated(xs[:min(T, 8)], gate, tau)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    flags = dec.decode_gated(xs, gate, tau)
    torch.cuda.synchronize()
    gwall = time.perf_counter() - t0
    fired = int(flags.sum())
    gtotal = T * wb[2] + fired * wb[4]
    # ... and the same loop driven from Python, step by step, for comparison
    py_fired = 0
    t0 = time.perf_counter()
    for t in range(T):
        dec.hidden.copy_(xs[t])
        dec.replay(2)
        gate.run(dec.logits, tau)
        if gate.result()["escalate"]:
            py_fired += 1
            dec.hidden.copy_(xs[t])
            dec.replay(4)
    torch.cuda.synchronize()
    pywall = time.perf_counter() - t0
    if py_fired != fired:
        raise RuntimeError(f"gated decode: the library loop escalated {fired} steps, the Python loop {py_fired}")
    # ... and with the decision kept on the device: the D8 step as a graph of
    # products predicated on the gate's flag, no synchronisation per step
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dec.decode_gated_async(xs[:min(T, 8)], gate, tau)
        side.synchronize()
        t0 = time.perf_counter()
        aflags = dec.decode_gated_async(xs, gate, tau)
        side.synchronize()
        awall = time.perf_counter() - t0
        # the predicated D8 graph alone when it does not fire: its floor cost per step
        gate.run(dec.logits, math.inf)
        never = []
        for i in range(12):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            dec.decode_gated_async(xs[:1], gate, math.inf)
            b.record()
            never.append((a, b))
        side.synchronize()
    torch.cuda.current_stream().wait_stream(side)
    a_fired = int(aflags.sum().item())
    if a_fired != fired:
        raise RuntimeError(f"gated decode: the device-decided loop escalated {a_fired} steps, the synchronising one {fired}")
    never_ms = float(np.median([a.elapsed_time(b) for a, b in never[2:]]))
    spec = run_speculation(args, torch, Q, WL, dec, wb) if args.spec_tokens > 0 else None
    return {
        "workload": "qwen_decode",
        "description": "Qwen3-0.6B-shaped decode: 28 x {q|k|v 4096x1024, o 1024x2048, gate|up 6144x1024, "
                       "down 1024x3072} + lm_head 151936x1024, int8; batch 1",
        "steps": T,
        "escalated_steps": n_esc,
        "tokens_per_s": round(T / wall, 2),
        "ms_per_token": round(wall * 1e3 / T, 5),
        "weight_bytes_per_token": int(total // T),
        "mean_bits_read_per_token": round(8.0 * total / T / wb[4], 6),
        "byte_ratio_vs_all_8bit": round(total / (T * wb[4]), 8),
        "achieved_weight_GBps": round(total / wall / 1e9, 2),
        "d4_step_ms": round(per[2], 5), "d8_step_ms": round(per[4], 5),
        "d4_step_GBps": round(wb[2] / per[2] / 1e6, 2), "d8_step_GBps": round(wb[4] / per[4] / 1e6, 2),
        "launches_per_step": 4 * c["n_layers"] + 1,
        "timing": "HIP graph per rung (captured by libqam), replayed per step; wall clock over all steps",
        "device_gate": {
            "rule": "entropy of the D4 output > tau (nats), tau between the 41st and 42nd largest entropies of a "
                    "first D4 pass",
            "tau_nats": round(tau, 6), "escalated_steps": fired,
            "tokens_per_s": round(T / gwall, 2), "ms_per_token": round(gwall * 1e3 / T, 5),
            "weight_bytes_per_token": int(gtotal // T),
            "gate_cost_ms_per_token": round((gwall - wall) * 1e3 / T, 5),
            "python_loop_tokens_per_s": round(T / pywall, 2),
            "no_sync": {
                "tokens_per_s": round(T / awall, 2), "ms_per_token": round(awall * 1e3 / T, 5),
                "escalated_steps": a_fired,
                "step_ms_when_not_fired": round(never_ms, 5),
                "timing": "qam_decoder_decode_gated_async, one call for all steps, one synchronisation at the "
                          "end; per step: D4 graph, gate, flag byte, predicated copy, then the D8 graph whose "
                          "113 products each read the gate's flag and exit at once when it is 0. "
                          "step_ms_when_not_fired: one such step with the gate forced off (events)",
            },
            "timing": "qam_decoder_decode_gated, one call for all steps; per step: D4 graph replay, gate launch, "
                      "device-to-host read of its result (a stream synchronisation), D8 graph replay when it "
                      "fired; wall clock over the call. python_loop_tokens_per_s: the same steps driven from "
                      "Python",
        },
        "speculation": spec,
        "_fld": fld, "_esc": esc, "_wb": wb,
    }


def run_speculation(args, torch, Q, WL, dec, wb):
    """Greedy draft-and-verify on the same decoder ([PoD] abstract: verified
    speculation): k D4 draft steps, then one batched D8 verify pass over the
    k + 1 positions; the token-feedback stand-in feeds back a seeded
    embedding row of each emitted token.  Bytes per token against one D8
    step, beside the gated schedule's ratio."""
    c = QWEN
    E = torch.from_numpy(WL.embedding_table(0, c["vocab"], c["hidden"])).cuda()
    ks = [int(v) for v in args.spec_k.split(",") if v]
    ver = Q.Verifier(dec, max(ks) + 1)
    n = args.spec_tokens
    out = {"tokens": n, "first_token": 0, "draft_rung": 2, "verify_rung": 4,
           "feedback": "embedding row of the emitted token, N(0,1) fp32 [151936, 1024] seeded table",
           "timing": "qam_decoder_speculate, one call; per round the D4 draft graphs, a device argmax and "
                     "embedding copy per draft, one batched D8 verify pass (graph replay), a device argmax and "
                     "accept kernel, "
                     "and one read of the round's tokens; wall clock over the call", "by_k": {}}
    for k in ks:
        ver.capture(4, k + 1)
        Q.speculate(dec, ver, E, 0, 4, k)                      # warm-up
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        toks, st = Q.speculate(dec, ver, E, 0, n, k)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        # one verify pass alone, timed with events on the launch stream
        ev = []
        for i in range(6):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            ver.replay(4, k + 1)
            b.record()
            ev.append((a, b))
        torch.cuda.synchronize()
        vms = float(np.median([a.elapsed_time(b) for a, b in ev[1:]]))
        nbytes = st["draft_steps"] * wb[2] + st["rounds"] * wb[4]
        out["by_k"][str(k)] = {
            "rounds": st["rounds"], "accepted_of_drafted": f"{st['accepted']}/{st['drafted']}",
            "acceptance": round(st["accepted"] / max(1, st["drafted"]), 4),
            "tokens_per_round": round(st["emitted"] / max(1, st["rounds"]), 4),
            "weight_bytes_per_token": int(nbytes // n),
            "byte_ratio_vs_all_8bit": round(nbytes / (n * wb[4]), 6),
            "tokens_per_s": round(n / wall, 2), "ms_per_token": round(wall * 1e3 / n, 5),
            "verify_pass_ms": round(vms, 5),
        }
    del ver, E
    return out


def decode_cpu_baseline(res, args):
    """The oracle's decode step (fp64 products + glue) on 2 of 28 layers and the
    head, scaled to the whole step; tokens/s at the same escalation rate."""
    import oracle as O
    from threadpoolctl import threadpool_limits
    from query_adaptive_mixed_amd.decode import interleave_gate_up, stack_rows
    threads = _blas_threads()
    import workloads as WL
    fld = res["_fld"]
    c = QWEN
    n_sample = 2
    mats = []
    for l in range(n_sample):
        cc = [fld.codes(7 * l + j) for j in range(7)]
        ss = [fld.scales(7 * l + j) for j in range(7)]
        mats.append([(stack_rows(cc[0], cc[1], cc[2]), stack_rows(ss[0], ss[1], ss[2])), (cc[3], ss[3]),
                     (interleave_gate_up(cc[4], cc[5]), interleave_gate_up(ss[4], ss[5])), (cc[6], ss[6])])
    Wl, sl = fld.codes(7 * c["n_layers"]), fld.scales(7 * c["n_layers"])
    x0 = WL.decode_inputs(0, 1, c["hidden"])

    def step(rung):
        lv = lambda W: np.full(W.shape[0] // 64, rung, np.uint8)
        h = x0.astype(np.float64)
        t0 = time.perf_counter()
        for (Wq, sq), (Wo, so), (Wg, sg), (Wd, sd) in mats:
            qkv = O.qmatvec_ref(Wq, sq, O.rmsnorm_ref(h), lv(Wq))
            h = h + O.qmatvec_ref(Wo, so, qkv[:, :c["q_dim"]], lv(Wo))
            gu = O.qmatvec_ref(Wg, sg, O.rmsnorm_ref(h), lv(Wg)).reshape(-1, 64)
            m = O.silu_mul_ref(gu[:, :32].reshape(1, -1), gu[:, 32:].reshape(1, -1))
            h = h + O.qmatvec_ref(Wd, sd, m, lv(Wd))
        t_layers = time.perf_counter() - t0
        t0 = time.perf_counter()
        O.qmatvec_ref(Wl, sl, O.rmsnorm_ref(h), lv(Wl))
        t_head = time.perf_counter() - t0
        return t_layers * c["n_layers"] / n_sample + t_head, t_layers + t_head

    T, n_esc = res["steps"], res["escalated_steps"]
    step(2)   # warm-up
    t4, s4 = step(2)
    t8, s8 = step(4)
    per_token = (T * t4 + n_esc * t8) / T
    with threadpool_limits(limits=1):
        u4, r4 = step(2)
        u8, r8 = step(4)
    per_token1 = (T * u4 + n_esc * u8) / T
    return {"value": round(1.0 / per_token, 4), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "host_cpu_count": os.cpu_count(), "value_one_core": round(1.0 / per_token1, 4),
            "sample": f"one fp64 oracle step at D4 and one at D8 over {n_sample} of 28 layers plus the full "
                      f"lm_head ({s4 + s8:.1f} s of CPU on all cores, {r4 + r8:.1f} s on one, after one warm-up "
                      f"step), scaled to 28 layers and to {n_esc} of {T} steps re-run at D8"}


# ----------------------------------------------------------------- CPU baseline

def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([int(p.get("num_threads", 1)) for p in threadpool_info()] or [1])
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline(res, args):
    """The oracle, as it stands, on a bounded sample of the same workload:
    the level map over every block, then the fp64 product of the first
    blocks of every matrix (the rows kept while packing), scaled to the whole
    workload by weight bytes.  Warm-up 1, median of 3, on all host cores
    (BLAS threads) and again limited to one core."""
    import oracle as O
    from threadpoolctl import threadpool_limits
    fld, lens, lv_h, sample = res["fld"], res["lens"], res["lv_h"], res["sample"]
    offs = fld.block_offsets()
    xs = [fld.x(i, res["batch"]) for i in range(len(fld.matrices))]
    scs = [fld.scales(i) for i in range(len(fld.matrices))]
    bits = np.array((0, 2, 4, 6, 8))

    def one_pass():
        t0 = time.perf_counter()
        O.level_map(fld.coords, lens.centres, lens.radii, lens.f, lens.g, lens.combine, 5, lens.glass)
        t_map = time.perf_counter() - t0
        done, t_prod = 0, 0.0
        for i, W in enumerate(sample):
            nb = W.shape[0] // 64
            sub = lv_h[offs[i]:offs[i] + nb]
            t0 = time.perf_counter()
            O.qmatvec_ref(W, scs[i][:W.shape[0]], xs[i], sub)
            t_prod += time.perf_counter() - t0
            done += int(np.sum(64 * W.shape[1] * bits[sub]) // 8)
        return t_map, t_prod, done

    def timed(reps):
        one_pass()
        runs = sorted((one_pass() for _ in range(reps)), key=lambda r: r[0] + r[1] * res["wbytes"] / max(r[2], 1))
        return runs[len(runs) // 2]

    t_map, t_prod, done = timed(3)
    frac = done / res["wbytes"]
    gbs = res["wbytes"] / (t_map + t_prod / frac) / 1e9
    with threadpool_limits(limits=1):
        t_map1, t_prod1, _ = timed(1)
    gbs1 = res["wbytes"] / (t_map1 + t_prod1 / frac) / 1e9
    nb = sample[0].shape[0] // 64 if sample else 0
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": _blas_threads(), "kind": "oracle",
            "host_cpu_count": os.cpu_count(),
            "value_one_core": round(gbs1, 4),
            "sample": f"level map over all {len(lv_h)} blocks + fp64 oracle product of the first {nb} blocks of "
                      f"each of the {len(sample)} matrices ({100 * frac:.1f}% of the weight bytes; "
                      f"{t_map + t_prod:.2f} s per sampled pass on all cores, {t_map1 + t_prod1:.2f} s on one), "
                      f"scaled to the whole workload by weight bytes; warm-up 1, median of 3 (one core: 1 timed)"}


def run_stack_file(args, torch, Q, WL):
    """The stored stack on disk: the E2B-shaped field's 210 packed matrices
    written once to a stack file, then read back at 2, 4, 6 and 8 bits into
    device memory (a read at depth d moves the first d/2 plane sections and
    the scales).  Reads are timed from the page cache (the file was just
    written), host file reads through pinned staging into HBM."""
    import tempfile
    fld = WL.e2b_field(0)
    dev = torch.device("cuda:0")
    mats = []
    for i, m in enumerate(fld.matrices):
        mats.append(Q.pack_slices(torch.from_numpy(fld.codes(i)).to(dev), torch.from_numpy(fld.scales(i)).to(dev)))
    torch.cuda.synchronize()
    out = {"workload": "stack_file", "matrices": len(mats),
           "description": "E2B-shaped field (30 x {q,k,v,o 1536x1536; gate,up 6144x1536; down 1536x6144}) as one "
                          "stack file; reads into caller device buffers, planes below the depth zero-filled",
           "reads": {}}
    with tempfile.TemporaryDirectory(dir=os.environ.get("TMPDIR", "/tmp")) as d:
        path = os.path.join(d, "e2b.qamstack")
        t0 = time.perf_counter()
        Q.stack_write(path, mats, [m.name for m in fld.matrices])
        wall = time.perf_counter() - t0
        size = os.path.getsize(path)
        out["file_bytes"] = size
        out["write_GBps"] = round(size / wall / 1e9, 3)
        dst, _ = Q.stack_read(path, 8)                               # destination buffers of the reads
        for bits in (2, 4, 6, 8):
            Q.stack_read(path, bits, out=dst)                       # warm the page cache for this prefix
            times = []
            for _ in range(3):
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                _, nread = Q.stack_read(path, bits, out=dst)
                times.append(time.perf_counter() - t0)
            best = min(times)
            out["reads"][str(bits)] = {"bytes_read": int(nread), "ms": round(best * 1e3, 3),
                                       "GBps": round(nread / best / 1e9, 3)}
        ok = all(torch.equal(a.buf, b.buf) for a, b in zip(dst, mats))   # the 8-bit read is the packed field
        out["round_trip_8bit_equal"] = bool(ok)
    return out


def copy_probe(args, torch):
    """A plain 1 GiB device-to-device copy: the known-size reference against which
    the FETCH_SIZE / WRITE_SIZE counters are scaled to bytes."""
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    print(json.dumps({"metric": "copy GB/s (read + write)", "value": round(2 * n / ms / 1e6, 2), "unit": "GB/s",
                      "bytes_read_per_copy": n, "bytes_written_per_copy": n, "ms_per_copy": round(ms, 4)}))


# ----------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="streaming_stack",
                    choices=["e2b_field", "streaming_stack", "batched_layer", "layer_decides", "qwen_decode",
                             "stack_file", "copy_probe"])
    ap.add_argument("--mean-bits", type=float, default=4.0)
    ap.add_argument("--glass", type=int, default=1)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--x-dtype", default="f32", choices=["f32", "bf16"], help="activations (batched_layer)")
    ap.add_argument("--uniform-map", action="store_true",
                    help="streaming_stack: every block at one depth, the same mean bits as the lens map")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true", help="time replays of a captured step instead of eager launches")
    ap.add_argument("--separate-map", action="store_true",
                    help="build the lens map with its own launch before the product (else inside the product launch)")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode tokens/s leg of the default run")
    ap.add_argument("--no-extras", action="store_true",
                    help="default run: skip the extra legs (E2B-scale field, decode)")
    ap.add_argument("--sample-blocks", type=int, default=32,
                    help="CPU oracle sample: the first blocks of every matrix")
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--decode-waves", type=int, default=0, help="decoder launch width goal (0 = library default)")
    ap.add_argument("--decode-ksplit", type=int, default=0, help="waves per block in the decoder (0 = default)")
    ap.add_argument("--decode-max-chunk", type=int, default=0,
                    help="decoder: longest column chunk in tiles (0 = default)")
    ap.add_argument("--tuning", default="", help="field and batched runs: launch plan of the group as JSON "
                    "(qam_tuning fields, e.g. '{\"set_max\": 8}'); empty = the library's defaults")
    ap.add_argument("--spec-tokens", type=int, default=64, help="draft-and-verify leg: tokens (0 = skip)")
    ap.add_argument("--spec-k", default="1,2,3", help="draft-and-verify leg: drafts per round, comma-separated")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        msg = ("bench.py measures one GPU only: the product would split by output-row blocks with no "
               "collective within a pass, but no multi-GPU path exists; run with --gpus 1")
        print(msg, file=sys.stderr)
        sys.exit(2)

    import torch
    import query_adaptive_mixed_amd as Q
    import workloads as WL

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    log(f"device: {torch.cuda.get_device_name(0)}")
    if args.workload == "copy_probe":
        return copy_probe(args, torch)
    if args.workload == "stack_file":
        r = run_stack_file(args, torch, Q, WL)
        r4 = r["reads"]["4"]
        print(json.dumps({"metric": "stack file read GB/s (page cache to HBM) at 4 bits", "value": r4["GBps"],
                          "unit": "GB/s", "n_gpus": 1, "steps": 3, "warmup": 1, "ms_per_step": r4["ms"],
                          "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u8",
                          "data": "synthetic (seeded codes and scales)", "config": r}), flush=True)
        return
    if args.workload == "qwen_decode":
        d = run_decode(args, torch, Q, WL)
        out = {
            "metric": "achieved HBM GB/s (% of peak) and decode tokens/s at mean bits/weight",
            "value": d["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": d["steps"], "warmup": 8,
            "ms_per_step": d["ms_per_token"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "int8 codes x fp32 activations (exact i8 MFMA on 24-bit fixed-point x in 3 int8 limbs), fp32 out",
            "data": "synthetic (seeded codes, scales, step inputs and escalation scores)",
            "config": {k: v for k, v in d.items() if not k.startswith("_")},
        }
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = decode_cpu_baseline(d, args)
        print(json.dumps(out), flush=True)
        return
    if args.workload == "layer_decides":
        res = run_layer(args, torch, Q, WL)
        step_bytes = res["base_bytes"] + res["union_bytes"]   # the second read: slices above the glass if refined
        gbs = step_bytes / (res["step_ms"] * 1e-3) / 1e9
        out = {
            "metric": "achieved HBM GB/s (% of peak) and decode tokens/s at mean bits/weight",
            "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(res["step_ms"], 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None,
            "dtype": "int8 codes x fp32 activations (exact int8 MFMA on 24-bit fixed-point x), fp64 scores, fp32 out",
            "data": "synthetic (seeded codes, scales and activations)",
            "config": {
                "workload": "layer_decides", "batch": args.batch,
                "description": "batched_layer matrices {4096x4096, 14336x4096, 4096x14336}; per matrix: product "
                               "at D2, reduced draft scores + top-third share to D8 on the device, product at the "
                               "per-request maps; the two products grouped over the three matrices (one launch "
                               "pair each), " + ("HIP graph replays" if args.graph else "eager launches")
                               + ", wall clock",
                "mean_bits_per_request": round(res["mean_bits_per_request"], 6),
                "mean_bits_union": round(res["mean_bits_union"], 6),
                "weight_bytes_base_pass": int(res["base_bytes"]),
                "second_pass": "lifted blocks' slices above the glass, added to the base outputs"
                               if res["refine"] else "full product at the per-request maps",
                "weight_bytes_second_pass_union": int(res["union_bytes"]),
                "weight_bytes_fixed_map_products": int(res["fixed_bytes"]),
                "step_ms": round(res["step_ms"], 5),
                "fixed_map_products_ms": round(res["fixed_ms"], 5),
                "layer_decides_over_fixed": round(res["step_ms"] / res["fixed_ms"], 4),
                "levels_ms_three_matrices": round(res["levels_ms"], 5),
                "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
                "rotated_copies": res["n_copies"],
            },
        }
        print(json.dumps(out), flush=True)
        return
    if args.workload == "batched_layer":
        res = run_batched(args, torch, Q, WL)
        gbs = res["wbytes"] / (res["ms"] * 1e-3) / 1e9
        kb = res["wbytes"] + res["other"]
        achieved = kb / (res["kern_ms"] * 1e-3) / 1e9
        out = {
            "metric": "achieved HBM GB/s (% of peak) and decode tokens/s at mean bits/weight",
            "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(res["ms"], 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": f"int8 codes x {args.x_dtype} activations (exact int8 MFMA on 24-bit fixed-point x), fp32 out",
            "data": "synthetic (seeded codes, scales, activations, block coordinates and per-request lenses)",
            "config": {
                "workload": "batched_layer", "description": res["desc"], "batch": args.batch,
                "x_dtype": args.x_dtype,
                "mean_bits_union": round(res["mean_bits"], 6),
                "mean_bits_per_request": round(res["mean_bits_per_request"], 6),
                "weight_bytes_per_step_union": int(res["wbytes"]),
                "weight_bytes_if_read_per_request": int(res["per_req_bytes"]),
                "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
                "requests_x_passes_per_s": round(args.batch * 1e3 / res["ms"], 1),
                "level_maps_ms_all_requests": round(res["map_ms"], 5),
                "step": "per-request level maps (one call, launches of 8 maps) + grouped limb pre-pass + "
                        "matrix-core product over the 3 matrices, "
                        + ("one HIP graph replay" if args.graph else "eager launches, wall clock"),
                "kernel": res["variant"],
                "useful_TOPs": round(res["flops"] / (res["kern_ms"] * 1e-3) / 1e12, 2),
                "rotated_copies": res["n_copies"],
            },
            "roofline": {
                "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(res["key"]),
                "kernel_ms": round(res["kern_ms"], 5), "algorithmic_bytes_per_launch": int(kb),
            },
        }
        print(json.dumps(out), flush=True)
        return
    default_run = args.workload == "streaming_stack" and args.batch == 1 and not args.no_extras
    res = run_field(args, torch, Q, WL, sample_blocks=0 if args.no_cpu_baseline else args.sample_blocks)
    out = field_line(args, res)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        out["cpu_baseline"] = cpu_baseline(res, args)
    del res
    if default_run:
        log("extra leg: the Gemma-E2B-scale field at 4.0 bits ...")
        r2 = run_field(args, torch, Q, WL, workload="e2b_field", batch=1, sample_blocks=0)
        e2 = field_line(args, r2)
        out["e2b_field"] = {"value": e2["value"], "unit": "GB/s", "ms_per_step": e2["ms_per_step"],
                            "config": e2["config"], "roofline": e2["roofline"]}
        del r2
        if not args.no_decode:
            log("extra leg: Qwen3-0.6B-shaped decode, 256 steps ...")
            d = run_decode(args, torch, Q, WL)
            out["decode"] = {k: v for k, v in d.items() if not k.startswith("_")}
            if not args.no_cpu_baseline:
                log("timing the CPU oracle's decode step ...")
                out["decode"]["cpu_baseline"] = decode_cpu_baseline(d, args)
    print(json.dumps(out), flush=True)


def field_line(args, res):
    """The JSON line of a weight-field run."""
    gbs = res["wbytes"] / (res["ms"] * 1e-3) / 1e9
    kern_bytes = res["wbytes"] + res["other"]
    achieved = kern_bytes / (res["kern_ms"] * 1e-3) / 1e9
    return {
        "metric": "achieved HBM GB/s (% of peak) and decode tokens/s at mean bits/weight",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 codes x fp32 activations (exact i8 MFMA on fixed-point x), fp64 sums, fp32 out",
        "data": "synthetic (seeded codes, scales, activations, block coordinates and lenses)",
        "config": {
            "workload": res["workload"],
            "description": res["desc"],
            "batch": res["batch"],
            "mean_bits": round(res["mean_bits"], 6),
            "weight_bytes_per_step": int(res["wbytes"]),
            "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
            "map": "uniform" if args.uniform_map else "lens",
            "focus_area_f": res["lens"].f, "focus_strength_g": res["lens"].g, "glass_rung": res["lens"].glass,
            "lens_coverage": res["coverage"],
            "matrices_per_launch": res["n_items"],
            "level_map": ("built inside the product launch" if res["fused"] else "own launch before the product"),
            "level_map_alone_ms": round(res["map_ms"], 5),
            "regulator": res["regulator"],
            "step_timing": "HIP graph replay of one step" if args.graph else "eager launches, wall clock",
            "kernel": res["variant"],
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(res["key"]),
            "kernel_ms": round(res["kern_ms"], 5),
            "kernel_timing": res["kern_timing"],
            "algorithmic_bytes_per_launch": int(kern_bytes),
        },
    }


if __name__ == "__main__":
    main()
