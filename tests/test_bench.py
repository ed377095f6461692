"""bench.py's contract: one GPU only, the algorithmic byte counts, and (on a
GPU) one JSON line with the metric, roofline and CPU-baseline objects."""
import io
import json
import os
import subprocess
import sys
from contextlib import redirect_stdout

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_large_batch():
    T, k, H, h = 4096, 8, 2, 7168
    b = bench.algorithmic_bytes(T, k, H, h, T * k, relay=False, fp8=False)
    assert b["dispatch"] == T * h * 2 + T * k * 4 + T * k * h * 2
    assert b["combine"] == T * k * h * 2 + T * k * 8 + T * h * 2
    assert b["layout"] == 4 * T * k * 4
    f = bench.algorithmic_bytes(T, k, H, h, 1000, relay=True, fp8=True)
    assert f["dispatch"] == T * h * 2 + T * H * 4 + 1000 * (h + h // 128 * 4)


def test_group_bytes_one_group_and_conservation():
    rng = np.random.Generator(np.random.PCG64(3))
    T, k, E, R, h, m = 300, 8, 64, 8, 256, 4
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    one = bench.group_bytes(idx, E, R, 1, h, False)
    # one group: the whole dispatch (x read once) and a combine with no carry
    assert one["dispatch_g0"] == T * h * 2 + T * k * 4 + T * k * h * 2
    assert one["combine_g0"] == T * k * h * 2 + T * k * 4 + T * k * 4 + T * h * 2
    b = bench.group_bytes(idx, E, R, m, h, False)
    grp = (idx % (E // R)) // (E // R // m)
    touched = sum(int((grp == g).any(axis=1).sum()) for g in range(m))   # (token, group) pairs
    # dispatch: x once per (token, group), the slots once per group, every row once
    assert sum(b[f"dispatch_g{g}"] for g in range(m)) == touched * h * 2 + m * T * k * 4 + T * k * h * 2
    # combine: every row and weight once, slots once per group, out once per
    # token; the rest is the float32 carry, 2 x h x 4 bytes per group boundary
    # a token crosses
    rest = sum(b[f"combine_g{g}"] for g in range(m)) - (T * k * h * 2 + m * T * k * 4 + T * k * 4 + T * h * 2)
    crossings = touched - T
    assert rest == crossings * 2 * h * 4


@pytest.mark.parametrize("relay,fp8", [(False, False), (True, True)])
def test_threaded_cpu_layer_equals_single_threaded(relay, fp8):
    """The threaded baseline runs the unchanged oracle on token slices; the
    layer's output is the same bytes as the single-threaded run."""
    from concurrent.futures import ThreadPoolExecutor
    from combine_epx_get_amd import workloads as W
    w = W.WORKLOADS["tiny"]
    d = W.make_inputs(w)
    y = W.random_bf16((w.num_tokens * w.topk, w.hidden), seed=3)
    one = bench.cpu_layer(w, d, y, relay, fp8)
    with ThreadPoolExecutor(max_workers=5) as pool:
        many = bench.cpu_layer(w, d, y, relay, fp8, pool, 5)
    assert np.array_equal(one, many)


@pytest.mark.gpu
def test_bench_prints_one_json_line():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible GPU")
    buf = io.StringIO()
    with redirect_stdout(buf):
        rc = bench.main(["--workload", "tiny", "--mode", "per_expert", "--steps", "3", "--warmup", "1",
                         "--cpu-seconds", "0.2"])
    assert rc == 0
    lines = [l for l in buf.getvalue().splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["config"]["workload"] == "tiny"
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["peak"] == 8000.0 and r["unit"] == "GB/s"
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert 0 < r["copy_ceiling_GBs"] < 2 * r["peak"]
    assert d["cache"].startswith("warm") and d["event_every"] == 3   # at most the step count
    assert r["timing"].startswith("HIP events bound")
    for v in d["kernels"].values():
        assert v["us_min"] <= v["us_median"] <= v["us_max"] and v["us_min"] <= v["us"] <= v["us_max"]
    # the cold-cache figures of the same kernels ride along
    assert d["cold"]["cache"].startswith("cold") and set(d["cold"]["kernels"]) == set(d["kernels"])
    assert all(v["us"] > 0 for v in d["cold"]["kernels"].values())
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["cores"] == bench.cpu_threads() and c["value"] > 0
    assert c["single_thread"]["value"] > 0 and c["cpu_model"]


@pytest.mark.gpu
def test_bench_cold_cache_and_fused_lines():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible GPU")
    for extra in (["--cold"], ["--fused", "--graph"]):
        buf = io.StringIO()
        with redirect_stdout(buf):
            rc = bench.main(["--workload", "tiny", "--mode", "relay", "--steps", "16", "--warmup", "2",
                             "--cpu-seconds", "0", *extra])
        assert rc == 0
        d = json.loads(buf.getvalue().strip().splitlines()[-1])
        if "--cold" in extra:
            assert d["cache"].startswith("cold") and d["warm"]["cache"].startswith("warm")
            # under --cold the step time is the layer's event time
            assert abs(d["ms_per_step"] * 1e3 - d["us_per_layer"]) < 0.02 * d["us_per_layer"] + 0.01
        else:
            assert "layout_dispatch" in d["kernels"] and d["us_per_layer_graph"] > 0
            assert d["config"]["fused_layout_dispatch"] is True
