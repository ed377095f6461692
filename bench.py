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


def workload_tag(args) -> str:
    """workload_mode_payload[_gM][_fused]: the name of a configuration's
    committed profile summaries."""
    from combine_epx_get_amd import workloads as W0
    w0 = W0.WORKLOADS[args.workload]
    mode = args.mode or ("relay" if args.relay_receive else w0.modes[0])
    tag = f"{args.workload}_{mode}_{args.dtype or w0.dtypes[0]}"
    if args.groups > 1:
        tag += f"_g{args.groups}"
    if args.relay_receive:
        tag += "_receive" + ("_bf16partials" if args.partials == "bf16" else "")
    if args.swap_planner is not None:
        tag += f"_swap{args.swap_planner}"
    if args.fused:
        tag += "_fused"
    return tag


def short_kernel_name(name: str) -> str:
    """A demangled kernel name without namespaces, template arguments or
    parameters (combine_kernel<2>(...) -> combine_kernel)."""
    n = name[5:] if name.startswith("void ") else name
    n = n.replace("(anonymous namespace)::", "").replace("epx::", "")
    depth = 0
    for i, ch in enumerate(n):
        if ch == "<":
            if depth == 0 and i > 0:
                return n[:i]
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return n[:i]
    return n


def ingest_trace(stats_csv: str, tag: str, command: str) -> str:
    """Write profiles/<tag>.md from a rocprofv3 --kernel-trace --stats run:
    the per-kernel call counts and durations, stamped with the hash of the
    kernel sources they were taken on, plus the HBM traffic of the same
    workload's committed counter summaries that are current."""
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    out = [f"# {tag}: rocprofv3 kernel trace", "",
           f"sources_hash: {kernel_sources_hash()} (every file of combine_epx_get_amd/csrc; bench.py "
           f"reports these averages only while the sources hash to it)", "",
           "Command ($REPO is the repository root, run on an MI355X):", "", "    " + command, "",
           "| kernel | calls | average µs | min µs | max µs | % of GPU time |", "|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| {short_kernel_name(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                   f"{float(r['Percentage']):.1f} |")
    counters = []
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", f"counters_*_{tag}.json"))):
        d = json.load(open(path))
        if d.get("sources_hash") == kernel_sources_hash(d["kernel"]):
            counters.append(d)
    if counters:
        out += ["", "HBM traffic per launch (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE, scaled by a "
                    "plain copy of known size in the same runs; from profiles/counters_*_" + tag + ".json):",
                "", "| kernel | read MB | write MB | total MB | fetch factor | write factor |",
                "|---|---|---|---|---|---|"]
        for d in counters:
            cal = d["calibration"]
            out.append(f"| {d['kernel']} | {d['hbm_read_bytes_per_launch'] / 1e6:.2f} | "
                       f"{d['hbm_write_bytes_per_launch'] / 1e6:.2f} | {d['hbm_bytes_per_launch'] / 1e6:.2f} | "
                       f"{cal['fetch_factor']} | {cal['write_factor']} |")
        out += ["", "Counter commands:", ""] + ["    " + c for c in counters[0]["command"].split("  ;  ")]
    path = os.path.join(ROOT, "profiles", f"{tag}.md")
    with open(path, "w") as f:
        f.write("\n".join(out) + "\n")
    return path


def load_trace_average(kernel: str, tag: str):
    """The committed trace's average µs for `kernel` on this workload, if the
    trace was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"{tag}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    stamp = [l for l in text.splitlines() if l.startswith("sources_hash: ")]
    if not stamp or stamp[0].split()[1] != kernel_sources_hash():
        return None
    for line in text.splitlines():
        cells = [c.strip() for c in line.split("|")]
        if len(cells) > 4 and cells[1] == kernel:
            return float(cells[3])
    return None


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


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime this process already uses
    (torch's), for the library's measurement hook (epx_time_next_call): the
    events are bound to the library's kernels, so torch's own event objects,
    which only know their own records, cannot read them."""

    def __init__(self):
        import ctypes
        self._ct = ctypes
        self._hip = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD)
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                  ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self._events = []
        self._free = []

    def _new(self) -> int:
        ev = self._ct.c_void_p()
        if self._hip.hipEventCreate(self._ct.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        self._events.append(ev.value)
        return ev.value

    def reserve(self, pairs: int):
        """Create event pairs ahead of a timed loop, which then only takes them."""
        self._free += [(self._new(), self._new()) for _ in range(pairs)]

    def pair(self):
        return self._free.pop() if self._free else (self._new(), self._new())

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = self._ct.c_float()
        rc = self._hip.hipEventElapsedTime(self._ct.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc}): a timed call launched no kernel?")
        return float(ms.value)

    def release(self):
        for e in self._events:
            self._hip.hipEventDestroy(e)
        self._events = []


def host_cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_threads() -> int:
    """Host threads for the threaded baseline: the cores this process may
    run on, at most 16 (one GPU's share of the host)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def cpu_layer(w, d, y_bits, relay, fp8, pool=None, nthreads=1):
    """One full layer through the oracle as it stands: layout (sequential),
    dispatch and combine. With a pool, dispatch and combine run the same
    oracle functions on nthreads contiguous token slices at once (ctypes
    releases the GIL); every slice writes its own rows of the shared
    outputs, so the result is the same bytes."""
    import oracle
    T, k = d["topk_idx"].shape
    H, hidden = w.num_hosts, d["x"].shape[1]
    lay = oracle.layout(d["topk_idx"], w.num_experts, w.num_ranks, w.num_hosts, w.my_rank, relay=relay)
    rows = int(lay["totals"][1] if relay else lay["totals"][0])
    if pool is None:
        if fp8:
            oracle.dispatch_fp8(d["x"], lay, k, H, relay)
        else:
            oracle.dispatch_bf16(d["x"], lay, k, H, relay)
        return oracle.combine(y_bits, lay, d["topk_weights"])
    if fp8:
        recv = (np.zeros((rows, hidden), np.uint8), np.zeros((rows, hidden // 128), np.float32))
    else:
        recv = np.zeros((rows, hidden), np.uint16)
    out = np.zeros((T, hidden), np.uint16)
    cuts = np.linspace(0, T, nthreads + 1).astype(int)
    slices = [(int(a), int(b)) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]

    def disp(sl):
        a, b = sl
        sub = {"slot": lay["slot"][a * k:b * k]}
        if relay:
            sub["relay_slot"] = lay["relay_slot"][a * H:b * H]
        f = oracle.dispatch_fp8 if fp8 else oracle.dispatch_bf16
        f(d["x"][a:b], sub, k, H, relay, rows=rows, out=recv)

    def comb(sl):
        a, b = sl
        oracle.combine(y_bits, {"slot": lay["slot"][a * k:b * k]}, d["topk_weights"][a:b], out=out[a:b])

    list(pool.map(disp, slices))
    list(pool.map(comb, slices))
    return out


def cpu_baseline(w, d, y_bits, layer_bytes, relay=False, fp8=False, min_seconds=12.0, max_reps=64):
    """The oracle as it stands on full layers of the same workload, on the
    host of this GPU: single-threaded, then with dispatch and combine sharded
    over the host's cores (cpu_layer); about min_seconds of CPU work in all.
    Both runs give the same output bytes (checked)."""
    from concurrent.futures import ThreadPoolExecutor
    n = cpu_threads()

    def timed(fn, budget):
        reps, t_total, res = 0, 0.0, None
        while reps < max_reps and (t_total < budget or reps < 2):
            t0 = time.perf_counter()
            res = fn()
            t_total += time.perf_counter() - t0
            reps += 1
        return t_total / reps, reps, res

    s1, r1, out1 = timed(lambda: cpu_layer(w, d, y_bits, relay, fp8), min_seconds * 0.6)
    with ThreadPoolExecutor(max_workers=n) as pool:
        sn, rn, outn = timed(lambda: cpu_layer(w, d, y_bits, relay, fp8, pool, n), min_seconds * 0.4)
    assert np.array_equal(out1, outn), "threaded oracle layer differs from the single-threaded one"
    what = f"layout + {'relay' if relay else 'per-expert'} {'fp8' if fp8 else 'bf16'} dispatch + combine"
    return {"value": round(layer_bytes / sn / 1e9, 3), "unit": "GB/s", "cores": n, "kind": "oracle",
            "us_per_layer": round(sn * 1e6, 1),
            "single_thread": {"value": round(layer_bytes / s1 / 1e9, 3), "us_per_layer": round(s1 * 1e6, 1),
                              "layers": r1},
            "cpu_model": host_cpu_model(),
            "sample": f"{rn} full layers ({what}) of the {w.name} workload with dispatch and combine on "
                      f"{n} token slices in {n} threads (layout sequential), beside {r1} single-threaded "
                      f"layers; the C oracle unchanged"}


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
                    help="arm the per-call kernel events on every N-th timed step (1: all); kernels "
                         "launched with bound events leave larger gaps behind them, so armed steps "
                         "run slower by the wall clock")
    ap.add_argument("--cold", action="store_true",
                    help="headline from cold steps: a 512 MiB scratch buffer read before every step "
                         "(evicts the 256 MB Infinity Cache and L2; the flush is outside every "
                         "timing). Either way the line also carries the other cache state's "
                         "per-kernel times")
    ap.add_argument("--other-cache", action=argparse.BooleanOptionalAction, default=True,
                    help="also time the other cache state (cold beside a warm headline, warm beside "
                         "a cold one); profiling runs turn it off so that the trace covers the "
                         "headline's steps only")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device-to-device copy (counter calibration)")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/counters_*.json from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--ingest-trace", metavar="KERNEL_STATS_CSV",
                    help="write profiles/<workload tag>.md from a rocprofv3 --kernel-trace --stats "
                         "run (its kernel_stats.csv) and exit")
    ap.add_argument("--ingest-command", default="", help="the profiling command, recorded verbatim")
    args = ap.parse_args(argv)

    if args.ingest_counters or args.ingest_trace:
        tag0 = workload_tag(args)
        if args.ingest_trace:
            print(ingest_trace(args.ingest_trace, tag0, args.ingest_command))
        else:
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
    hipev = HipEvents()

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

    def step(rec=None):
        """One layer on the current stream (a capture stream under --graph).
        With `rec` (a list), every library call first arms the measurement
        hook with a fresh pair of HIP events, bound to the call's own
        kernels, and (name, start, stop) is appended to rec."""
        stream = torch.cuda.current_stream()

        def arm(name):
            if rec is not None:
                a, b = hipev.pair()
                rec.append((name, a, b))
                epx.epx_time_next_call(a, b)

        if fused:
            arm("layout_dispatch")
            epx.epx_layout_dispatch(p, idx, L, x, out_dtype, recv, scales, stream)
        else:
            arm("layout")
            epx.epx_get_layout(p, idx, L, stream)
        if planner:
            i = n_plans[0] % 2
            plan_out["slot_expert"] = places[1 - i]
            arm("swap_planner")
            epx.epx_plan_swaps(E, R, H, L["expert_count"], places[i], args.swap_planner, plan_out, stream)
            n_plans[0] += 1
        if m > 1:
            # per-expert overlap order without the expert GEMMs: every group's
            # dispatch, then every group's combine
            for g in range(m):
                arm(f"dispatch_g{g}")
                epx.epx_dispatch_group(p, L, g, x, out_dtype, recv, scales, stream)
            for g in range(m):
                arm(f"combine_g{g}")
                epx.epx_combine_group(p, L, g, y, wts, carry, out, stream)
            return
        if not fused:
            arm("dispatch")
            epx.epx_dispatch(p, L, x, out_dtype, recv, scales, stream)
        if receive:
            arm("relay_fanout")
            epx.epx_relay_fanout(p, L, recv, fan, scales, fan_sc, stream)
            arm("relay_partials")
            epx.epx_combine_relay_partials(p, L, y, wts, part, stream)
            arm("relay_finish")
            epx.epx_combine_relay_finish(p, L, part, out, stream)
        else:
            arm("combine")
            epx.epx_combine(p, L, y, wts, out, stream)

    if args.copy_calibration:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE readings give
        # the scale from counter units to HBM bytes
        src = torch.ones(COPY_BYTES // 4, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # Cold steps read a 512 MiB buffer first. Reading (not writing) leaves
    # clean lines in the caches, so the dirty lines of the previous step are
    # written back during the flush and none is left for the next kernel to
    # write back inside its own time. The flush is outside every timing.
    scratch = torch.ones(EVICT_BYTES // 4, dtype=torch.int32, device=dev)

    def flush():
        scratch.max()

    for _ in range(args.warmup):
        if args.cold:
            flush()
        step()
    torch.cuda.synchronize()
    assert epx.epx_read_error(L) == 0
    totals = L["totals"].cpu().numpy()
    rows = int(totals[1] if relay else totals[0])

    calls_per_step = (1 + (1 if planner else 0) +
                      (2 * m if m > 1 else (0 if fused else 1) + (3 if receive else 1)))

    def timed_steps(n, cold):
        """n steps, the kernel events armed on every `event_every`-th one.
        Returns (wall seconds, [records of the timed steps])."""
        every = max(1, min(args.event_every, n))
        recs = []
        hipev.reserve((n // every) * calls_per_step)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n):
            if cold:
                flush()
            r = [] if i % every == every - 1 else None
            step(r)
            if r is not None:
                recs.append(r)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, recs

    wall, recs = timed_steps(args.steps, args.cold)
    # the other cache state, for the same kernels: cold steps (flush before
    # each) beside a warm headline, warm steps beside a cold one
    recs_other = timed_steps(args.steps, not args.cold)[1] if args.other_cache else None
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

    nbytes = algorithmic_bytes(T, k, w.num_hosts, hidden, rows, relay, fp8)
    if receive:
        nbytes.update(relay_receive_bytes(T, k, w.num_hosts, hidden, rows, fp8, args.partials == "f32"))
        del nbytes["combine"]
    if m > 1:
        nbytes = {"layout": nbytes["layout"],
                  **group_bytes(d["topk_idx"], w.num_experts, w.num_ranks, m, hidden, fp8)}
    if fused:
        nbytes = {"layout_dispatch": nbytes["layout"] + nbytes["dispatch"],
                  **{n: v for n, v in nbytes.items() if n not in ("layout", "dispatch")}}
    if planner:
        # counts and placement in, placement, loads, pair records and flags out
        npair = H * ((R // H) // 2)
        nbytes["swap_planner"] = 4 * (3 * E + 2 * R + 7 * npair + H)
    layer_bytes = sum(v for n, v in nbytes.items() if n != "swap_planner")

    def kernel_times(records):
        """Per call: µs of its kernels (mean, median, min, max), bytes, GB/s
        and fraction of peak; and the layer µs (first kernel's start to the
        last kernel's end) of every timed step."""
        per, layer = {}, []
        for r in records:
            for name, a, b in r:
                per.setdefault(name, []).append(hipev.elapsed_ms(a, b) * 1e3)
            layer.append(hipev.elapsed_ms(r[0][1], r[-1][2]) * 1e3)
        out = {}
        for name, us in per.items():
            us = np.asarray(us, dtype=np.float64)
            nb = nbytes[name]
            v = {"us": float(us.mean()), "us_median": float(np.median(us)), "us_min": float(us.min()),
                 "us_max": float(us.max()), "bytes": nb}
            v["GBs"] = nb / (v["us"] * 1e-6) / 1e9
            v["frac_peak"] = v["GBs"] / PEAK_HBM_GBS
            out[name] = v
        return out, np.asarray(layer, dtype=np.float64)

    per_kernel, layer_us = kernel_times(recs)
    other_kernel, other_layer_us = kernel_times(recs_other) if recs_other else (None, None)
    hipev.release()
    # the flush is not part of the layer: cold steps take their time from the
    # kernel events, warm steps from the wall clock
    ms_per_step = float(layer_us.mean() / 1e3) if args.cold else wall * 1e3 / args.steps
    us_layer = float(layer_us.mean())
    value = layer_bytes / (ms_per_step * 1e-3) / 1e9

    dom = max((n for n in per_kernel if n not in ("layout", "swap_planner")), key=lambda n: per_kernel[n]["us"])
    kname = {"dispatch": "dispatch_fp8_kernel" if fp8 else "dispatch_bf16_kernel",
             "combine": "combine_kernel", "relay_fanout": "relay_fanout_kernel",
             "relay_partials": "relay_partials_kernel", "relay_finish": "relay_finish_kernel",
             "dispatch_g": "dispatch_fp8_kernel" if fp8 else "dispatch_bf16_kernel",
             "combine_g": "combine_group_kernel",
             "layout_dispatch": fused_kernel(T, k, w.num_experts, relay, fp8)}[dom.rstrip("0123456789")]
    tag = workload_tag(args)
    traffic = load_counter_traffic(kname, tag)
    trace_us = load_trace_average(kname, tag)
    roofline = {"bound": "hbm", "kernel": kname,
                "achieved": round(per_kernel[dom]["GBs"], 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(per_kernel[dom]["frac_peak"], 4), "traffic": traffic,
                "algorithmic_bytes": per_kernel[dom]["bytes"],
                "timing": "HIP events bound to the kernels' dispatch packets (hipExtLaunchKernel)",
                "profile": ({"file": f"profiles/{tag}.md", "trace_avg_us": trace_us,
                             "event_avg_us": round(per_kernel[dom]["us"], 3)}
                            if trace_us is not None else None),
                "copy_ceiling_GBs": round(copy_ceiling(torch, dev), 1)}

    def rounded(pk):
        return {n: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                for n, v in pk.items()}

    other = None
    if other_kernel is not None:
        other = {"cache": "warm (back-to-back steps)" if args.cold else
                 "cold (512 MiB scratch read before each step)",
                 "us_per_layer": round(float(other_layer_us.mean()), 2),
                 "kernels": {n: {"us": round(v["us"], 3), "frac_peak": round(v["frac_peak"], 4)}
                             for n, v in other_kernel.items()}}

    cpu = None
    if args.cpu_seconds > 0 and not receive and m == 1:
        cpu = cpu_baseline(w, d, y_np, layer_bytes, relay, fp8, args.cpu_seconds)

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
        "event_every": max(1, min(args.event_every, args.steps)),
        "us_per_layer": round(us_layer, 2),
        **({"us_per_layer_graph": round(graph_us, 2)} if graph_us is not None else {}),
        **({"us_per_layer_graph_fused": round(graph_fused_us, 2)} if graph_fused_us is not None else {}),
        "pct_of_peak_layer": round(100 * layer_bytes / (us_layer * 1e-6) / 1e9 / PEAK_HBM_GBS, 2),
        "kernels": rounded(per_kernel),
        "cold" if not args.cold else "warm": other,
        "layer_bytes": layer_bytes, "rows": rows,
        "imbalance_ratio": round(float(totals[2]) / (T * k / w.num_experts), 3),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
