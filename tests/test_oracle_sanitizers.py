"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

The oracle's library is rebuilt with -fsanitize=address,undefined (gcc, host
code only; nothing here touches a GPU) and every entry point is driven
through the oracle's own Python wrappers on small random shapes and on the
edge cases: T = 0 and 1, k = 1 and k = E, one host, one rank per host,
duplicate ids in a row, every token on one expert, out-of-range ids, expert
groups, the relay receive side and the swap planner. Any out-of-bounds
access, use after free or undefined arithmetic aborts the child process.
The inputs are drawn with numpy only, so that the child loads nothing but
numpy and the oracle next to the sanitizer runtime.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

DRIVER = r'''
import sys
import numpy as np
sys.path.insert(0, sys.argv[1])
import oracle

lib = oracle.load(sys.argv[2])
rng = np.random.Generator(np.random.PCG64(11))


def bf16(shape):
    # finite bf16 patterns: float32 values truncated to their upper half
    return (rng.standard_normal(shape, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def routing(T, k, E, dup=False):
    if dup:
        return rng.integers(0, E, size=(T, k)).astype(np.int32)
    return np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)


SHAPES = [
    # T, k, E, R, H, s, hidden
    (0, 2, 16, 4, 2, 1, 128),
    (1, 1, 8, 8, 8, 5, 128),
    (7, 3, 12, 4, 2, 3, 256),
    (33, 6, 6, 3, 1, 1, 128),       # k = E, one host
    (40, 2, 16, 16, 16, 15, 128),   # one rank per host
    (25, 8, 64, 8, 4, 2, 384),
]
for (T, k, E, R, H, s, h) in SHAPES:
    for dup in (False, True):
        idx = routing(T, k, E, dup)
        x = bf16((T, h))
        w = rng.random((T, k), dtype=np.float32)
        for relay in (False, True):
            lay = oracle.layout(idx, E, R, H, s, relay=relay, lib=lib)
            oracle.dispatch_bf16(x, lay, k, H, relay, lib=lib)
            oracle.dispatch_fp8(x, lay, k, H, relay, lib=lib)
        lay = oracle.layout(idx, E, R, H, s, relay=True, lib=lib)
        y = bf16((T * k, h))
        oracle.combine(y, lay, w, lib=lib)
        rows = oracle.dispatch_bf16(x, lay, k, H, True, lib=lib)
        oracle.relay_fanout(rows, lay, idx, E, R, H, lib=lib)
        q, sc = oracle.dispatch_fp8(x, lay, k, H, True, lib=lib)
        oracle.relay_fanout(q, lay, idx, E, R, H, relay_scales=sc, lib=lib)
        for b in (False, True):
            part = oracle.relay_partials(y, lay, idx, w, E, R, H, bf16=b, lib=lib)
            oracle.relay_finish(part, lay, T, H, lib=lib)
        epr = E // R
        for m in [g for g in (2, 4) if epr % g == 0]:
            glay = oracle.layout_grouped(idx, E, R, m, lib=lib)
            for g in range(m):
                oracle.dispatch_group(x, glay, idx, E, R, m, g, lib=lib)
                oracle.dispatch_group(x, glay, idx, E, R, m, g, fp8=True, lib=lib)
            oracle.combine_grouped(y, glay, idx, w, E, R, m, lib=lib)

# every token on one expert
idx = np.full((50, 4), 5, np.int32)
lay = oracle.layout(idx, 16, 4, 2, 0, relay=True, lib=lib)
oracle.dispatch_fp8(bf16((50, 128)), lay, 4, 2, True, lib=lib)

# out-of-range ids: reported, nothing else computed
for bad in (-1, 16, 1 << 30):
    idx = routing(20, 2, 16)
    idx[7, 1] = bad
    try:
        oracle.layout(idx, 16, 4, 2, 0, relay=True, lib=lib)
        raise SystemExit("bad id not reported")
    except oracle.OracleError as e:
        assert e.code != 0

# swap planner, including a host whose slots hold a bad id
for (E, R, H) in ((16, 4, 2), (64, 8, 1), (256, 32, 4), (24, 6, 3)):
    counts = rng.integers(0, 50, size=E).astype(np.int32)
    oracle.plan_swaps(counts, R, H, 1, lib=lib)
    slots = np.arange(E, dtype=np.int32)
    slots[0] = E + 3
    slots[1] = -1
    got = oracle.plan_swaps(counts, R, H, 0, slot_expert=slots, lib=lib)
    assert got["host_bad"][0] == 2 and not got["host_bad"][1:].any()

# conversions over special values
v = np.array([0.0, -0.0, 1e-30, -1e-30, 448.0, 449.0, -3e38, 2.0 ** -9, 2.0 ** -10, 1.0,
              np.inf, -np.inf], np.float32)
oracle.f32_to_e4m3(v, lib=lib)
oracle.f32_to_bf16(v, lib=lib)
oracle.e4m3_to_f32(np.arange(256, dtype=np.uint8), lib=lib)
print("sanitized oracle ok", flush=True)
'''


def _runtime(name):
    gcc = shutil.which("gcc")
    if gcc is None:
        return None
    out = subprocess.run([gcc, f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None or _runtime("libubsan.so") is None:
        pytest.skip("gcc sanitizer runtimes are not installed")
    sys.path.insert(0, ROOT)
    import oracle
    lib = str(tmp_path / "liboracle_san.so")
    oracle.build(lib, extra_flags=("-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                                   "-fno-omit-frame-pointer", "-g"))
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", DRIVER, ROOT, lib], capture_output=True, text=True,
                       env=env, timeout=600)
    assert r.returncode == 0 and "sanitized oracle ok" in r.stdout, (r.returncode, r.stdout[-2000:],
                                                                     r.stderr[-4000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
