#!/usr/bin/env python3
"""Benchmark: one MoE layer's dispatch + combine on one MI355X.

A step is one pass of the whole hot path over one batch: layout (routing ->
counts, offsets, rows), dispatch (token rows -> per-expert or relay rows,
bf16 or fp8) and combine (k expert outputs per token -> weighted bf16 sum).
The expert computation between dispatch and combine is outside the path; its
outputs are a fixed synthetic bf16 tensor resident in HBM.

Default workload: 4096 tokens, hidden 7168, 256 experts, top-8 uniform, 16
ranks on 2 hosts, per-expert mode, bf16. Inputs are resident in HBM before
timing starts. Prints one JSON line.

Timing: W warm-up steps, then K steps bracketed by torch.cuda.synchronize();
HIP events on the launch stream around each kernel group give per-kernel
averages. `value` is algorithmic bytes of the layer / time per layer.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, public specification
COPY_BYTES = 256 << 20       # size of the calibration copy
EVICT_BYTES = 512 << 20      # scratch read before each step under --cold
CEILING_BYTES = 512 << 20    # device copy timed beside the peak (read + write = 1 GiB)


def algorithmic_bytes(T, k, H, hidden, rows, relay, fp8):
    """Bytes each kernel must move at minimum (each byte once, at DRAM).

    dispatch: read x (T*h*2) and each token's destinations (T*D*4, D = k
              slots or H relay slots); write the rows (rows*h*2 for bf16, or
              rows*(h + h/128*4) for fp8 codes + float32 scales).
    combine:  read the T*k expert rows (T*k*h*2), slots and weights
              (T*k*8); write out (T*h*2).
    layout:   read topk_idx twice (count and assign passes, 2*T*k*4); write
              slot and row_token (2*T*k*4); relay mode also writes relay_slot
              (T*H*4) and relay_token, fan-out and mask for every relay row
              up to the capacity (cap*(k+2)*4).
    """
    D = H if relay else k
    row_bytes = hidden + (hidden // 128) * 4 if fp8 else hidden * 2
    dispatch = T * hidden * 2 + T * D * 4 + rows * row_bytes
    combine = T * k * hidden * 2 + T * k * 8 + T * hidden * 2
    layout = 4 * T * k * 4
    if relay:
        layout += T * H * 4 + T * min(k, H) * (k + 2) * 4
    return {"dispatch": dispatch, "combine": combine, "layout": layout}


def group_bytes(idx, E, R, m, hidden, fp8):
    """Algorithmic bytes of each expert group's dispatch and combine.

    Pairs of group g: expert local index (e mod E/R) // (E/R/m) == g.
    dispatch g: read x for the tokens with a pair in g, the whole slot array
                (T*k*4: the group's pairs must be found), write the group's
                rows.
    combine g:  read the group's rows (bf16), slots (T*k*4) and the group's
                weights; read the float32 carry for tokens that had pairs in
                an earlier group, write it for tokens with pairs in a later
                group, write bf16 out for tokens whose last group is g.
    """
    T, k = idx.shape
    epr = E // R
    grp = (idx % epr) // (epr // m)
    row_bytes = hidden + (hidden // 128) * 4 if fp8 else hidden * 2
    out = {}
    for g in range(m):
        pairs = int((grp == g).sum())
        in_g = (grp == g).any(axis=1)
        prior = int((in_g & (grp < g).any(axis=1)).sum())
        later = int((in_g & (grp > g).any(axis=1)).sum())
        final = int(in_g.sum()) - later
        out[f"dispatch_g{g}"] = int(in_g.sum()) * hidden * 2 + T * k * 4 + pairs * row_bytes
        out[f"combine_g{g}"] = (pairs * hidden * 2 + T * k * 4 + pairs * 4 + prior * hidden * 4
                                + later * hidden * 4 + final * hidden * 2)
    return out


GRAPH_STEPS = 16   # layers captured in one graph under --graph

KERNEL_SOURCE = {"dispatch_bf16_kernel": "epx_dispatch.hip", "dispatch_fp8_kernel": "epx_dispatch.hip",
                 "combine_kernel": "epx_combine.hip", "relay_fanout_kernel": "epx_relay.hip",
                 "relay_partials_kernel": "epx_relay.hip", "relay_finish_kernel": "epx_relay.hip",
                 "combine_group_kernel": "epx_combine.hip", "plan_swaps_kernel": "epx_balance.hip",
                 "layout_dispatch_kernel": "epx_fused.hip", "assign_copy_kernel": "epx_layout.hip",
                 "layout_small_kernel": "epx_layout.hip", "layout_count_kernel": "epx_layout.hip",
                 "layout_scan_kernel": "epx_layout.hip", "layout_assign_kernel": "epx_layout.hip"}


def relay_receive_bytes(T, k, H, hidden, rows, fp8, f32_partials):
    """Algorithmic bytes of the relay receive side and the two-level combine.

    fan-out:  read the relay rows in use, write the T*k per-expert rows (same
              payload), read fan-out lists, slots and row tokens.
    partials: read the T*k expert-output rows (bf16) and slots/weights; write
              one partial row per relay row in use (fp32 or bf16).
    finish:   read the partial rows in use and the relay slots, write out.
    """
    row = hidden + (hidden // 128) * 4 if fp8 else hidden * 2
    prow = hidden * (4 if f32_partials else 2)
    return {"relay_fanout": rows * row + T * k * row + rows * (k + 1) * 4 + T * k * 4,
            "relay_partials": T * k * hidden * 2 + T * k * 8 + rows * (k + 1) * 4 + rows * prow,
            "relay_finish": rows * prow + T * H * 4 + T * hidden * 2}


def kernel_sources_hash(kernel: str = "") -> str:
    """Hash of the source file holding `kernel` (plus the shared internal
    headers); of every kernel source when the kernel is not listed."""
    csrc = os.path.join(ROOT, "combine_epx_get_amd", "csrc")
    if kernel in KERNEL_SOURCE:
        files = [os.path.join(csrc, f) for f in (KERNEL_SOURCE[kernel], "epx_internal.h", "epx_device.h")]
    else:
        files = sorted(glob.glob(os.path.join(csrc, "*")))
    h = hashlib.sha256()
    for f in files:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def fused_kernel(T, k, E, relay, fp8):
    """The kernel that copies the rows in an epx_layout_dispatch call: the
    single-launch kernel at decode sizes, the assign-and-copy launch for
    larger batches with k <= 16 (bf16, or fp8 in relay mode), else the plain
    dispatch kernel."""
    if T <= 1024 and T * k <= 4096 and k <= 16 and E <= 512:
        return "layout_dispatch_kernel"
    if k <= 16 and (relay or not fp8):
        return "assign_copy_kernel"
    return "dispatch_fp8_kernel" if fp8 else "dispatch_bf16_kernel"


def load_counter_traffic(kernel: str, tag: str):
    """HBM traffic per launch from a committed rocprofv3 counter summary for
    this kernel and workload tag (workload_mode_payload), if it was taken on
    the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"counters_{kernel}_{tag}.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("sources_hash") != kernel_sources_hash(kernel):
        return None
    return d.get("hbm_bytes_per_launch")


KERNEL_NAMES = ("dispatch_bf16_kernel", "dispatch_fp8_kernel", "combine_kernel",
                "relay_fanout_kernel", "relay_partials_kernel", "relay_finish_kernel",
                "layout_small_kernel", "layout_count_kernel", "layout_scan_kernel",
                "layout_assign_kernel", "combine_group_kernel", "plan_swaps_kernel",
                "layout_dispatch_kernel", "assign_copy_kernel")


def ingest_counters(fetch_csv: str, write_csv: str, tag: str, command: str) -> list:
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE; KiB per
    dispatch) of `bench.py --copy-calibration` into per-kernel HBM traffic
    summaries under profiles/. The calibration copy (COPY_BYTES read and
    written) fixes the scale from each counter to bytes."""
    import csv

    def load(path):
        rows = list(csv.DictReader(open(path)))
        return {r["Dispatch_Id"]: r for r in rows}

    fetch, write = load(fetch_csv), load(write_csv)

    # the calibration copy: the copy dispatch whose WRITE_SIZE is nearest
    # COPY_BYTES; the same dispatch id in the FETCH_SIZE run (same sequence)
    copies = [r for r in write.values() if "copyBuffer" in r["Kernel_Name"]]
    if not copies:
        raise SystemExit("calibration copy not found in the counter csv")
    cw = min(copies, key=lambda r: abs(float(r["Counter_Value"]) * 1024 - COPY_BYTES))
    cf = fetch[cw["Dispatch_Id"]]
    if "copyBuffer" not in cf["Kernel_Name"]:
        raise SystemExit("the two counter runs do not list the same dispatches")
    f_factor = COPY_BYTES / (float(cf["Counter_Value"]) * 1024)
    w_factor = COPY_BYTES / (float(cw["Counter_Value"]) * 1024)
    out = []
    for kname in KERNEL_NAMES:
        fv = [float(r["Counter_Value"]) for r in fetch.values() if kname in r["Kernel_Name"]]
        wv = [float(r["Counter_Value"]) for r in write.values() if kname in r["Kernel_Name"]]
        if not fv or not wv:
            continue
        fk, wk = sum(fv) / len(fv), sum(wv) / len(wv)
        d = {"kernel": kname, "workload": tag, "sources_hash": kernel_sources_hash(kname),
             "command": command,
             "launches": {"fetch_run": len(fv), "write_run": len(wv)},
             "fetch_size_kib_per_launch": round(fk, 3), "write_size_kib_per_launch": round(wk, 3),
             "calibration": {"copy_bytes": COPY_BYTES,
                             "copy_fetch_size_kib": float(cf["Counter_Value"]),
                             "copy_write_size_kib": float(cw["Counter_Value"]),
                             "fetch_factor": round(f_factor, 5), "write_factor": round(w_factor, 5)},
             "hbm_read_bytes_per_launch": round(fk * 1024 * f_factor),
             "hbm_write_bytes_per_launch": round(wk * 1024 * w_factor)}
        d["hbm_bytes_per_launch"] = d["hbm_read_bytes_per_launch"] + d["hbm_write_bytes_per_launch"]
        path = os.path.join(ROOT, "profiles", f"counters_{kname}_{tag}.json")
        with open(path, "w") as f:
            json.dump(d, f, indent=1)
        out.append(path)
    return out


def copy_ceiling(torch, dev, reps: int = 5) -> float:
    """A plain device copy of CEILING_BYTES (read + write), timed with events:
    the best of `reps` in GB/s, the copy rate this memory system reaches in
    the same run."""
    src = torch.ones(CEILING_BYTES // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    best = float("inf")
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        best = min(best, a.elapsed_time(b))
    del src, dst
    return 2 * CEILING_BYTES / (best * 1e-3) / 1e9


def cpu_baseline(w, d, y_bits, relay=False, fp8=False, min_seconds=12.0, max_reps=64):
    """The oracle as it stands (single-threaded C loops) on full layers of the
    same workload: layout + dispatch (per-expert or relay, bf16 or fp8) +
    combine of the same expert outputs the GPU combines, repeated until about
    min_seconds of CPU time have been spent. Returns (seconds per layer,
    layers timed)."""
    import oracle
    T, k = d["topk_idx"].shape
    reps, t_total = 0, 0.0
    while reps < max_reps and (t_total < min_seconds or reps < 2):
        t0 = time.perf_counter()
        lay = oracle.layout(d["topk_idx"], w.num_experts, w.num_ranks, w.num_hosts, w.my_rank, relay=relay)
        if fp8:
            oracle.dispatch_fp8(d["x"], lay, k, w.num_hosts, relay)
        else:
            oracle.dispatch_bf16(d["x"], lay, k, w.num_hosts, relay)
        oracle.combine(y_bits, lay, d["topk_weights"])
        t_total += time.perf_counter() - t0
        reps += 1
    return t_total / reps, reps


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="large_batch")
    ap.add_argument("--mode", choices=["per_expert", "relay"], default=None)
    ap.add_argument("--dtype", choices=["bf16", "fp8"], default=None)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU time spent timing the oracle for the baseline (0: skip)")
    ap.add_argument("--relay-receive", action="store_true",
                    help="relay mode: step = layout, relay dispatch, fan-out to per-expert rows, "
                         "per-host partials and the source-side finish (instead of the flat combine)")
    ap.add_argument("--partials", choices=["f32", "bf16"], default="f32",
                    help="wire form of the relay partials (with --relay-receive)")
    ap.add_argument("--swap-planner", type=int, default=None, metavar="TAU",
                    help="also run the per-step intra-host swap planner on the layout's expert counts "
                         "(threshold TAU tokens) between layout and dispatch")
    ap.add_argument("--groups", type=int, default=1, metavar="M",
                    help="expert groups (per-expert overlap): step = grouped layout, M group "
                         "dispatches, M group combines (per-expert mode)")
    ap.add_argument("--fused", action="store_true",
                    help="layout and dispatch in one call (epx_layout_dispatch: one launch for "
                         "decode-sized batches, assignment and copies in one launch above)")
    ap.add_argument("--graph", action=argparse.BooleanOptionalAction, default=None,
                    help="also time layers captured in a HIP graph (16 per graph) and replayed: the "
                         "layer time without per-launch host overhead (default: on, except with "
                         "--swap-planner)")
    ap.add_argument("--event-every", type=int, default=4, metavar="N",
                    help="record the per-kernel HIP events on every N-th timed step (1: all)")
    ap.add_argument("--cold", action="store_true",
                    help="read a 512 MiB scratch buffer before every step (evicts the 256 MB "
                         "Infinity Cache and L2); per-kernel and layer times then exclude the flush")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device-to-device copy (counter calibration)")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/counters_*.json from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--ingest-command", default="", help="the profiling command, recorded verbatim")
    args = ap.parse_args(argv)

    if args.ingest_counters:
        w0 = args.workload
        from combine_epx_get_amd import workloads as W0
        tag0 = f"{w0}_{args.mode or W0.WORKLOADS[w0].modes[0]}_{args.dtype or W0.WORKLOADS[w0].dtypes[0]}"
        if args.groups > 1:
            tag0 += f"_g{args.groups}"
        if args.fused:
            tag0 += "_fused"
        for pth in ingest_counters(*args.ingest_counters, tag0, args.ingest_command):
            print(pth)
        return 0

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this path has no "
              f"multi-GPU transport: every GPU would run the same independent single-rank layer).",
              file=sys.stderr)
        return 2

    import torch
    from combine_epx_get_amd import epx
    from combine_epx_get_amd import workloads as W

    w = W.WORKLOADS[args.workload]
    mode = args.mode or ("relay" if args.relay_receive else w.modes[0])
    dtype = args.dtype or w.dtypes[0]
    relay = mode == "relay"
    fp8 = dtype == "fp8"
    torch.cuda.set_device(0)
    dev = "cuda"

    d = W.make_inputs(w)
    T, k, hidden = d["T"], w.topk, w.hidden
    m = args.groups
    if m > 1 and relay:
        print("--groups needs per-expert mode", file=sys.stderr)
        return 2
    fused = args.fused
    if fused and (m > 1 or args.swap_planner is not None):
        print("--fused runs layout and dispatch as one call: no groups, no swap planner between them",
              file=sys.stderr)
        return 2
    p = epx.make_problem(T, k, w.num_experts, w.num_ranks, w.num_hosts, w.my_rank,
                         epx.MODE_HOST_RELAY if relay else epx.MODE_PER_EXPERT, m)
    L = epx.Layout(p, dev)
    idx = torch.from_numpy(d["topk_idx"]).to(dev)
    x = torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16).to(dev)
    wts = torch.from_numpy(d["topk_weights"]).to(dev)
    cap = epx.relay_capacity(p) if relay else T * k
    if fp8:
        recv = torch.empty((cap, hidden), dtype=torch.uint8, device=dev)
        scales = torch.empty((cap, hidden // 128), dtype=torch.float32, device=dev)
    else:
        recv = torch.empty((cap, hidden), dtype=torch.bfloat16, device=dev)
        scales = None
    y_np = W.random_bf16((T * k, hidden), seed=1000 + w.seed)   # stand-in expert outputs
    y = torch.from_numpy(y_np.view(np.int16)).view(torch.bfloat16).to(dev)
    out = torch.empty((T, hidden), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    out_dtype = epx.FP8_E4M3 if fp8 else epx.BF16

    receive = args.relay_receive
    if receive:
        if not relay:
            print("--relay-receive needs relay mode", file=sys.stderr)
            return 2
        # the relay GPU's per-expert rows, its partials (the return wire) and the output
        fan = torch.empty((T * k, hidden), dtype=recv.dtype, device=dev)
        fan_sc = torch.empty((T * k, hidden // 128), dtype=torch.float32, device=dev) if fp8 else None
        part = torch.empty((cap, hidden), dtype=torch.float32 if args.partials == "f32" else torch.bfloat16,
                           device=dev)

    if m > 1:
        carry = torch.empty((T, hidden), dtype=torch.float32, device=dev)
    planner = args.swap_planner is not None
    if planner:
        # the placement ping-pongs between two buffers: each step plans from
        # the previous step's placement
        E, R, H = w.num_experts, w.num_ranks, w.num_hosts
        places = [torch.arange(E, dtype=torch.int32, device=dev), torch.empty(E, dtype=torch.int32, device=dev)]
        plan_out = {"slot_expert": None, "load_before": torch.empty(R, dtype=torch.int32, device=dev),
                    "load_after": torch.empty(R, dtype=torch.int32, device=dev),
                    "swaps": torch.empty((H * ((R // H) // 2), 7), dtype=torch.int32, device=dev),
                    "host_bad": torch.empty(H, dtype=torch.int32, device=dev)}
        n_plans = [0]

    def step(ev=None):
        # launches go to the current stream (a capture stream under --graph)
        stream = torch.cuda.current_stream()

        def rec(i):
            if ev is not None:
                ev[i].record(stream)

        rec(0)
        if fused:
            # layout and dispatch in one call: its time is events 0 -> 1
            epx.epx_layout_dispatch(p, idx, L, x, out_dtype, recv, scales, stream)
            rec(1)
        else:
            epx.epx_get_layout(p, idx, L, stream)
            rec(1)
        if planner:
            i = n_plans[0] % 2
            plan_out["slot_expert"] = places[1 - i]
            epx.epx_plan_swaps(E, R, H, L["expert_count"], places[i], args.swap_planner, plan_out, stream)
            n_plans[0] += 1
        rec(6)
        if m > 1:
            # per-expert overlap order without the expert GEMMs: every group's
            # dispatch, then every group's combine (events 7.. per launch)
            for g in range(m):
                epx.epx_dispatch_group(p, L, g, x, out_dtype, recv, scales, stream)
                rec(7 + g)
            rec(2)
            for g in range(m):
                epx.epx_combine_group(p, L, g, y, wts, carry, out, stream)
                rec(7 + m + g)
            rec(3)
            return
        if not fused:
            epx.epx_dispatch(p, L, x, out_dtype, recv, scales, stream)
        rec(2)
        if receive:
            epx.epx_relay_fanout(p, L, recv, fan, scales, fan_sc, stream)
            rec(4)
            epx.epx_combine_relay_partials(p, L, y, wts, part, stream)
            rec(5)
            epx.epx_combine_relay_finish(p, L, part, out, stream)
        else:
            epx.epx_combine(p, L, y, wts, out, stream)
        rec(3)

    if args.copy_calibration:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE readings give
        # the scale from counter units to HBM bytes
        src = torch.ones(COPY_BYTES // 4, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # --cold: read a 512 MiB buffer before each step. Reading (not writing)
    # leaves clean lines in the caches, so the dirty lines of the previous
    # step are written back during the flush and none is left for the next
    # kernel to write back inside its own time.
    scratch = torch.ones(EVICT_BYTES // 4, dtype=torch.int32, device=dev) if args.cold else None

    def flush(i):
        if scratch is not None:
            scratch.max()

    for i in range(args.warmup):
        flush(i)
        step()
    torch.cuda.synchronize()
    assert epx.epx_read_error(L) == 0
    totals = L["totals"].cpu().numpy()
    rows = int(totals[1] if relay else totals[0])

    # Per-kernel events on every step would slow the step they measure (each
    # record is a marker the stream waits for: about 17 µs per large-batch
    # step), so they are recorded on the last step of every `event_every`
    # timed steps only (never on the first, which starts on an idle queue);
    # the other steps run as a caller would run them.
    every = max(1, min(args.event_every, args.steps))
    timed = [i for i in range(args.steps) if i % every == every - 1]
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(7 + 2 * m)] for _ in timed]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        flush(i)
        step(evs[i // every] if i % every == every - 1 else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    del scratch

    graph_us = None
    if args.graph and planner:
        print("--graph does not capture the swap planner's alternating placement", file=sys.stderr)
        return 2

    def time_graph(layer):
        """µs per layer from replays of GRAPH_STEPS layers captured in one
        HIP graph, so that one replay's host cost is spread over many layers
        and the time is the GPU's."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            layer()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(GRAPH_STEPS):
                layer()
        replays = max(1, args.steps // GRAPH_STEPS)
        for _ in range(max(1, args.warmup // GRAPH_STEPS)):
            graph.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(replays):
            graph.replay()
        g1.record()
        torch.cuda.synchronize()
        del graph
        return g0.elapsed_time(g1) * 1e3 / (replays * GRAPH_STEPS)

    graph_fused_us = None
    if args.graph if args.graph is not None else not planner:
        graph_us = time_graph(step)
        if not fused and m == 1 and not receive:
            # the same layer with layout and dispatch as one epx_layout_dispatch call
            def fused_layer():
                stream = torch.cuda.current_stream()
                epx.epx_layout_dispatch(p, idx, L, x, out_dtype, recv, scales, stream)
                epx.epx_combine(p, L, y, wts, out, stream)
            graph_fused_us = time_graph(fused_layer)

    lay_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    plan_ms = np.array([e[1].elapsed_time(e[6]) for e in evs])
    dis_ms = np.array([e[6].elapsed_time(e[2]) for e in evs])
    if receive:
        fan_ms = np.array([e[2].elapsed_time(e[4]) for e in evs])
        par_ms = np.array([e[4].elapsed_time(e[5]) for e in evs])
        fin_ms = np.array([e[5].elapsed_time(e[3]) for e in evs])
        com_ms = par_ms + fin_ms
    else:
        com_ms = np.array([e[2].elapsed_time(e[3]) for e in evs])
    step_ms = np.array([e[0].elapsed_time(e[3]) for e in evs])
    # the flush is not part of the layer: under --cold the step time comes
    # from the events around the layer, otherwise from the wall clock
    ms_per_step = float(step_ms.mean()) if args.cold else wall * 1e3 / args.steps

    nbytes = algorithmic_bytes(T, k, w.num_hosts, hidden, rows, relay, fp8)
    if receive:
        nbytes.update(relay_receive_bytes(T, k, w.num_hosts, hidden, rows, fp8, args.partials == "f32"))
        del nbytes["combine"]
    if m > 1:
        nbytes = {"layout": nbytes["layout"],
                  **group_bytes(d["topk_idx"], w.num_experts, w.num_ranks, m, hidden, fp8)}
    layer_bytes = sum(nbytes.values())
    us_layer = float(step_ms.mean() * 1e3)
    value = layer_bytes / (ms_per_step * 1e-3) / 1e9

    def kern(ms, nb):
        """Event times of one kernel over the timed steps (µs): mean (the
        roofline's figure), median, min and max."""
        us = np.asarray(ms, dtype=np.float64) * 1e3
        return {"us": float(us.mean()), "us_median": float(np.median(us)), "us_min": float(us.min()),
                "us_max": float(us.max()), "bytes": nb}

    if fused:
        per_kernel = {"layout_dispatch": kern(lay_ms, nbytes["layout"] + nbytes["dispatch"])}
    else:
        per_kernel = {"layout": kern(lay_ms, nbytes["layout"])}
    if m == 1 and not fused:
        per_kernel["dispatch"] = kern(dis_ms, nbytes["dispatch"])
    if m > 1:
        for g in range(m):
            d0 = 6 if g == 0 else 7 + g - 1
            c0 = 2 if g == 0 else 7 + m + g - 1
            per_kernel[f"dispatch_g{g}"] = kern([e[d0].elapsed_time(e[7 + g]) for e in evs],
                                                nbytes[f"dispatch_g{g}"])
            per_kernel[f"combine_g{g}"] = kern([e[c0].elapsed_time(e[7 + m + g]) for e in evs],
                                               nbytes[f"combine_g{g}"])
    if planner:
        # counts and placement in, placement, loads, pair records and flags out
        npair = H * ((R // H) // 2)
        per_kernel["swap_planner"] = kern(plan_ms, 4 * (3 * E + 2 * R + 7 * npair + H))
    if receive:
        per_kernel["relay_fanout"] = kern(fan_ms, nbytes["relay_fanout"])
        per_kernel["relay_partials"] = kern(par_ms, nbytes["relay_partials"])
        per_kernel["relay_finish"] = kern(fin_ms, nbytes["relay_finish"])
    elif m == 1:
        per_kernel["combine"] = kern(com_ms, nbytes["combine"])
    for v in per_kernel.values():
        v["GBs"] = v["bytes"] / (v["us"] * 1e-6) / 1e9
        v["frac_peak"] = v["GBs"] / PEAK_HBM_GBS
    dom = max((n for n in per_kernel if n not in ("layout", "swap_planner")), key=lambda n: per_kernel[n]["us"])
    kname = {"dispatch": "dispatch_fp8_kernel" if fp8 else "dispatch_bf16_kernel",
             "combine": "combine_kernel", "relay_fanout": "relay_fanout_kernel",
             "relay_partials": "relay_partials_kernel", "relay_finish": "relay_finish_kernel",
             "dispatch_g": "dispatch_fp8_kernel" if fp8 else "dispatch_bf16_kernel",
             "combine_g": "combine_group_kernel",
             "layout_dispatch": fused_kernel(T, k, w.num_experts, relay, fp8)}[dom.rstrip("0123456789")]
    tag = f"{args.workload}_{mode}_{dtype}" + (f"_g{m}" if m > 1 else "") + ("_fused" if fused else "")
    traffic = load_counter_traffic(kname, tag)
    roofline = {"bound": "hbm", "kernel": kname,
                "achieved": round(per_kernel[dom]["GBs"], 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(per_kernel[dom]["frac_peak"], 4), "traffic": traffic,
                "algorithmic_bytes": per_kernel[dom]["bytes"],
                "copy_ceiling_GBs": round(copy_ceiling(torch, dev), 1)}

    cpu = None
    if args.cpu_seconds > 0 and not receive and m == 1:
        cpu_s, reps = cpu_baseline(w, d, y_np, relay, fp8, args.cpu_seconds)
        cpu = {"value": round(layer_bytes / cpu_s / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "us_per_layer": round(cpu_s * 1e6, 1),
               "sample": f"{reps} full layers (layout + {mode.replace('_', '-')} {dtype} dispatch + combine) "
                         f"of the {args.workload} workload, single-threaded C oracle"}

    line = {
        "metric": "dispatch+combine µs/layer and HBM GB/s (% of MI355X peak) at 4096 tok, h=7168",
        "value": round(value, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if not fp8 else "fp8-e4m3 dispatch / bf16 combine",
        "data": "synthetic",
        "config": {"workload": args.workload, "tokens": T, "hidden": hidden, "experts": w.num_experts,
                   "topk": k, "ranks": w.num_ranks, "hosts": w.num_hosts, "routing": w.routing,
                   "mode": mode + ("+receive" if receive else ""), "payload": dtype,
                   **({"partials": args.partials} if receive else {}),
                   **({"swap_tau": args.swap_planner} if planner else {}),
                   **({"expert_groups": m} if m > 1 else {}),
                   **({"fused_layout_dispatch": True} if fused else {})},
        "cache": "cold (512 MiB scratch read before each step)" if args.cold else "warm (back-to-back steps)",
        "event_every": every,
        "us_per_layer": round(us_layer, 2),
        **({"us_per_layer_graph": round(graph_us, 2)} if graph_us is not None else {}),
        **({"us_per_layer_graph_fused": round(graph_fused_us, 2)} if graph_fused_us is not None else {}),
        "pct_of_peak_layer": round(100 * layer_bytes / (us_layer * 1e-6) / 1e9 / PEAK_HBM_GBS, 2),
        "kernels": {n: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for n, v in per_kernel.items()},
        "layer_bytes": layer_bytes, "rows": rows,
        "imbalance_ratio": round(float(totals[2]) / (T * k / w.num_experts), 3),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
